"""ctypes binding of libkie.so (include/kie.h).  Argument marshalling only:
every step of the decode path runs in the HIP library.  PyTorch provides the
device buffers and the stream.

The binding never falls back to anything else: if the library is missing it
raises, so a run without the native code fails loudly.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

from .config import ModelConfig
from .inputs import LAYER_TENSORS

_PKG = os.path.dirname(os.path.abspath(__file__))
# KIE_LIBRARY selects another build of the same library (the sanitized
# host-only build that the CPU tests of the C ABI use)
LIB_PATH = os.environ.get("KIE_LIBRARY") or os.path.join(_PKG, "libkie.so")

KIE_OK = 0
STATUS = {0: "ok", -1: "invalid argument", -2: "HIP error", -3: "capacity", -4: "state",
          -5: "timeout", -6: "unsupported", -7: "bad token", -8: "fp16 range"}


class KieError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"kie status {status} ({STATUS.get(status, '?')}): {msg}")
        self.status = status


class ModelConfigC(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("d_model", C.c_int32), ("n_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn_dim", C.c_int32),
                ("vocab", C.c_int32), ("rms_eps", C.c_float), ("rope_base", C.c_double),
                ("n_lanes", C.c_int32), ("lane_delay", C.c_int32), ("parallel_block", C.c_int32),
                ("max_ctx", C.c_int32)]


_P16 = C.POINTER(C.c_uint16)
_PP16 = C.POINTER(_P16)


class WeightsC(C.Structure):
    _fields_ = [("embed", _P16), ("lm_head", _P16), ("final_norm", _P16),
                ("attn_norm", _PP16), ("wq", _PP16), ("wk", _PP16), ("wv", _PP16), ("wo", _PP16),
                ("mlp_norm", _PP16), ("w_gate", _PP16), ("w_up", _PP16), ("w_down", _PP16)]


_lib = None


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = C.CDLL(LIB_PATH)
        vp, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
        L.kie_create.argtypes = [C.POINTER(ModelConfigC), C.c_int, C.POINTER(vp)]
        L.kie_query_sizes.argtypes = [vp, C.POINTER(sz), C.POINTER(sz), C.POINTER(sz)]
        L.kie_bind_memory.argtypes = [vp, vp, vp, vp]
        L.kie_load_weights.argtypes = [vp, C.POINTER(WeightsC), vp]
        L.kie_prefill.argtypes = [vp, vp, i32, vp, vp, vp]
        L.kie_prefill_scratch_bytes.argtypes = [vp, i32, C.POINTER(sz)]
        L.kie_prefill_batched.argtypes = [vp, vp, i32, vp, vp, vp, sz, vp]
        L.kie_prefill_batched_noalloc.argtypes = [vp, vp, i32, vp, vp, vp]
        L.kie_decode.argtypes = [vp, i32, vp, vp, vp, vp]
        L.kie_set_position.argtypes = [vp, i32, i32, vp]
        L.kie_sync_status.argtypes = [vp, vp]
        L.kie_set_timeout_us.argtypes = [vp, C.c_uint64]
        L.kie_set_debug_flags.argtypes = [vp, C.c_uint32]
        L.kie_set_sampling.argtypes = [vp, C.c_float, C.c_uint64]
        L.kie_set_launch_steps.argtypes = [vp, i32]
        L.kie_set_trace.argtypes = [vp, vp, i32]
        L.kie_pack_weights_host.argtypes = [C.POINTER(ModelConfigC), C.POINTER(WeightsC), vp]
        L.kie_launch_info.argtypes = [vp, C.POINTER(i32), C.POINTER(i32), C.POINTER(i32),
                                      C.POINTER(C.c_int64), C.POINTER(C.c_int64)]
        L.kie_validate_schedule.argtypes = [C.POINTER(ModelConfigC), i32, i32, C.c_char_p, sz]
        L.kie_phase_order.argtypes = [C.POINTER(ModelConfigC), i32, C.POINTER(i32), C.POINTER(i32), i32]
        L.kie_ring_depth.argtypes = [C.POINTER(ModelConfigC), i32, C.POINTER(i32)]
        L.kie_position.argtypes = [vp]
        L.kie_position.restype = i32
        L.kie_status_string.argtypes = [C.c_int]
        L.kie_status_string.restype = C.c_char_p
        L.kie_last_error.argtypes = [vp]
        L.kie_last_error.restype = C.c_char_p
        L.kie_destroy.argtypes = [vp]
        L.kie_destroy.restype = None
        for name in ("kie_create", "kie_query_sizes", "kie_bind_memory", "kie_load_weights",
                     "kie_prefill", "kie_prefill_scratch_bytes", "kie_prefill_batched", "kie_prefill_batched_noalloc",
                     "kie_decode", "kie_set_position", "kie_sync_status",
                     "kie_set_timeout_us", "kie_set_debug_flags", "kie_set_sampling", "kie_set_launch_steps",
                     "kie_set_trace",
                     "kie_pack_weights_host", "kie_launch_info", "kie_validate_schedule", "kie_phase_order",
                     "kie_ring_depth"):
            getattr(L, name).restype = C.c_int
        _lib = L
    return _lib


def unload() -> None:
    """Unload the library (its kernels' code objects are unregistered from
    the HIP runtime now, while the runtime is fully up, rather than by exit
    handlers at interpreter teardown).  Every context must be destroyed
    first; lib() loads it again."""
    global _lib
    if _lib is None:
        return
    import _ctypes
    h = _lib._handle
    _lib = None
    _ctypes.dlclose(h)


def config_c(cfg: ModelConfig, max_ctx: Optional[int] = None) -> ModelConfigC:
    return ModelConfigC(cfg.n_layers, cfg.d_model, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim,
                        cfg.ffn_dim, cfg.vocab, float(cfg.rms_eps), float(cfg.rope_base),
                        int(cfg.n_lanes), int(cfg.lane_delay), 0 if cfg.sequential else 1,
                        int(max_ctx if max_ctx is not None else cfg.max_ctx))


class _WeightRefs:
    """kie_weights pointing into numpy fp16 arrays (kept alive here)"""

    def __init__(self, cfg: ModelConfig, w: Dict[str, np.ndarray]):
        self.keep = []

        def p(a):
            a = np.ascontiguousarray(a)
            if a.dtype != np.float16:
                raise TypeError("weights must be float16")
            self.keep.append(a)
            return a.ctypes.data_as(_P16)

        def arr(name):
            ptrs = (_P16 * cfg.n_layers)(*[p(w[f"layers.{l}.{name}"]) for l in range(cfg.n_layers)])
            self.keep.append(ptrs)
            return C.cast(ptrs, _PP16)

        self.c = WeightsC(p(w["embed"]), p(w["lm_head"]), p(w["final_norm"]),
                          *[arr(n) for n in LAYER_TENSORS])


def _check(status: int, ctx=None):
    if status != KIE_OK:
        msg = lib().kie_last_error(ctx).decode() if ctx else ""
        raise KieError(status, msg)


# --------------------------------------------------------------------------
# host-only helpers (no GPU needed)
# --------------------------------------------------------------------------
def query_sizes(cfg: ModelConfig, max_ctx: Optional[int] = None) -> Tuple[int, int, int]:
    L = lib()
    ctx = C.c_void_p()
    c = config_c(cfg, max_ctx)
    _check(L.kie_create(C.byref(c), -1, C.byref(ctx)))
    try:
        a, b, d = C.c_size_t(), C.c_size_t(), C.c_size_t()
        _check(L.kie_query_sizes(ctx, C.byref(a), C.byref(b), C.byref(d)), ctx)
        return a.value, b.value, d.value
    finally:
        L.kie_destroy(ctx)


def pack_weights_host(cfg: ModelConfig, weights: Dict[str, np.ndarray]) -> np.ndarray:
    packed_bytes, _, _ = query_sizes(cfg, 1)
    out = np.zeros(packed_bytes // 2, dtype=np.uint16)
    refs = _WeightRefs(cfg, weights)
    c = config_c(cfg, 1)
    _check(lib().kie_pack_weights_host(C.byref(c), C.byref(refs.c), out.ctypes.data_as(C.c_void_p)))
    return out


def validate_schedule(cfg: ModelConfig, n_workgroups: int, n_ctx: int) -> None:
    buf = C.create_string_buffer(256)
    c = config_c(cfg)
    s = lib().kie_validate_schedule(C.byref(c), n_workgroups, n_ctx, buf, 256)
    if s != KIE_OK:
        raise KieError(s, buf.value.decode())


PHASE_KIND_NAMES = ("QKV", "attention", "O", "gate/up", "down", "LM head")


def phase_order(cfg: ModelConfig, n_workgroups: int) -> list:
    """[(kind, layer)] of the phases of one decode step, in the kernel's
    order (kind: 0 QKV, 1 attention, 2 O, 3 gate/up, 4 down, 5 LM head)"""
    n = 5 * cfg.n_layers + 1
    kind = (C.c_int32 * n)()
    layer = (C.c_int32 * n)()
    _check(lib().kie_phase_order(C.byref(config_c(cfg)), n_workgroups, kind, layer, n))
    return list(zip(kind, layer))


def ring_depth(cfg: ModelConfig, n_workgroups: int) -> int:
    """LDS ring slots per wave of the decode kernel build a context for cfg
    on n_workgroups workgroups launches (8 or 10)"""
    d = C.c_int32()
    _check(lib().kie_ring_depth(C.byref(config_c(cfg)), n_workgroups, C.byref(d)))
    return d.value


def lane_placement(cfg: ModelConfig, n_workgroups: int):
    """(lo, hi): int32 arrays [3, n_workgroups] of the lowest and highest lane
    of each workgroup's QKV rows (0), attention head (1) and gate/up rows (2),
    -1 where it has none"""
    f = lib().kie_lane_placement
    f.argtypes = [C.POINTER(ModelConfigC), C.c_int32, C.POINTER(C.c_int32), C.POINTER(C.c_int32)]
    f.restype = C.c_int
    n = 3 * n_workgroups
    lo = (C.c_int32 * n)()
    hi = (C.c_int32 * n)()
    _check(f(C.byref(config_c(cfg)), n_workgroups, lo, hi))
    return (np.array(lo, dtype=np.int32).reshape(3, n_workgroups),
            np.array(hi, dtype=np.int32).reshape(3, n_workgroups))


def kernel_name(cfg: ModelConfig, n_workgroups: int) -> str:
    """the decode kernel's symbol as profilers print it"""
    g = cfg.n_heads // cfg.n_kv_heads
    par = "false" if cfg.sequential else "true"
    return f"kie::ring{ring_depth(cfg, n_workgroups)}::kie_monokernel<{g}, {par}>"


def create_status(cfg: ModelConfig, device: int = -1, max_ctx: Optional[int] = None) -> int:
    """status of kie_create (the context is destroyed again)"""
    L = lib()
    ctx = C.c_void_p()
    c = config_c(cfg, max_ctx)
    s = L.kie_create(C.byref(c), device, C.byref(ctx))
    if s == KIE_OK:
        L.kie_destroy(ctx)
    return s


# --------------------------------------------------------------------------
# GPU engine
# --------------------------------------------------------------------------
class Engine:
    """One decoding context on one GPU.  Device memory comes from PyTorch."""

    def __init__(self, cfg: ModelConfig, device: int = 0, max_ctx: Optional[int] = None):
        import torch
        self.torch = torch
        self.cfg = cfg
        self.device = device
        self.dev = torch.device("cuda", device)
        self.L = lib()
        self.max_ctx = int(max_ctx if max_ctx is not None else cfg.max_ctx)
        self.ctx = C.c_void_p()
        c = config_c(cfg, self.max_ctx)
        _check(self.L.kie_create(C.byref(c), device, C.byref(self.ctx)))
        a, b, d = C.c_size_t(), C.c_size_t(), C.c_size_t()
        _check(self.L.kie_query_sizes(self.ctx, C.byref(a), C.byref(b), C.byref(d)), self.ctx)
        self.packed_bytes, self.kv_bytes, self.ws_bytes = a.value, b.value, d.value
        u8 = torch.uint8
        self.d_packed = torch.empty(self.packed_bytes, dtype=u8, device=self.dev)
        self.d_kv = torch.empty(self.kv_bytes, dtype=u8, device=self.dev)
        self.d_ws = torch.empty(self.ws_bytes, dtype=u8, device=self.dev)
        _check(self.L.kie_bind_memory(self.ctx, self.d_packed.data_ptr(), self.d_kv.data_ptr(),
                                      self.d_ws.data_ptr()), self.ctx)

    # -- plumbing --------------------------------------------------------
    def stream(self):
        return C.c_void_p(self.torch.cuda.current_stream(self.dev).cuda_stream)

    def close(self):
        if self.ctx:
            self.L.kie_destroy(self.ctx)
            self.ctx = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def launch_info(self) -> Dict[str, int]:
        n, t, l = C.c_int32(), C.c_int32(), C.c_int32()
        q, m = C.c_int64(), C.c_int64()
        _check(self.L.kie_launch_info(self.ctx, C.byref(n), C.byref(t), C.byref(l), C.byref(q),
                                      C.byref(m)), self.ctx)
        return dict(n_workgroups=n.value, threads=t.value, lds_bytes=l.value,
                    qkv_offset=q.value, lm_offset=m.value)

    def set_timeout_us(self, us: int):
        _check(self.L.kie_set_timeout_us(self.ctx, int(us)), self.ctx)

    def set_debug_flags(self, flags: int):
        _check(self.L.kie_set_debug_flags(self.ctx, int(flags)), self.ctx)

    def set_sampling(self, temperature: float, seed: int = 0):
        """kie_set_sampling: temperature 0 is greedy; else Gumbel-max draws
        from softmax(logits / temperature) with Philox noise keyed by seed"""
        _check(self.L.kie_set_sampling(self.ctx, float(temperature), int(seed) & 0xFFFFFFFFFFFFFFFF), self.ctx)

    TRACE_PHASES = 5 * 64 + 2

    def set_trace(self, steps: int):
        """allocate a trace buffer for the first `steps` steps of each launch
        (0 turns tracing off); read it back with trace()"""
        t = self.torch
        if steps <= 0:
            self._trace = None
            _check(self.L.kie_set_trace(self.ctx, None, 0), self.ctx)
            return
        nwg = self.launch_info()["n_workgroups"]
        self._trace = t.zeros(steps * self.TRACE_PHASES * nwg * 4, dtype=t.int64, device=self.dev)
        self._trace_shape = (steps, self.TRACE_PHASES, nwg, 4)
        _check(self.L.kie_set_trace(self.ctx, self._trace.data_ptr(), steps), self.ctx)

    def trace(self) -> np.ndarray:
        """[steps, phases, workgroups, 4] wall-clock stamps (100 MHz ticks)"""
        return self._trace.cpu().numpy().reshape(self._trace_shape)

    def set_launch_steps(self, n: int):
        _check(self.L.kie_set_launch_steps(self.ctx, int(n)), self.ctx)

    @property
    def position(self) -> int:
        return int(self.L.kie_position(self.ctx))

    def sync(self):
        _check(self.L.kie_sync_status(self.ctx, self.stream()), self.ctx)

    # -- the path ----------------------------------------------------------
    def load_weights(self, weights: Dict[str, np.ndarray]):
        refs = _WeightRefs(self.cfg, weights)
        _check(self.L.kie_load_weights(self.ctx, C.byref(refs.c), self.stream()), self.ctx)

    def _ids(self, ids) -> "object":
        t = self.torch
        a = np.ascontiguousarray(np.asarray(ids, dtype=np.int32))
        return t.from_numpy(a).to(self.dev)

    def prefill(self, prompt: Sequence[int], want_logits: bool = False):
        t = self.torch
        d_prompt = self._ids(prompt)
        d_next = t.empty(1, dtype=t.int32, device=self.dev)
        d_logits = t.empty(self.cfg.vocab, dtype=t.float32, device=self.dev) if want_logits else None
        _check(self.L.kie_prefill(self.ctx, d_prompt.data_ptr(), len(prompt), d_next.data_ptr(),
                                  d_logits.data_ptr() if d_logits is not None else None,
                                  self.stream()), self.ctx)
        self.sync()
        tok = int(d_next.cpu()[0])
        if want_logits:
            return tok, d_logits.cpu().numpy()
        return tok

    def prefill_scratch_bytes(self, chunk: int) -> int:
        nbytes = C.c_size_t()
        _check(self.L.kie_prefill_scratch_bytes(self.ctx, int(chunk), C.byref(nbytes)), self.ctx)
        return int(nbytes.value)

    def prefill_batched_device(self, d_prompt, n: int, d_next, scratch, d_logits=None):
        """asynchronous kie_prefill_batched on caller-provided device tensors"""
        _check(self.L.kie_prefill_batched(self.ctx, d_prompt.data_ptr(), int(n),
                                          d_next.data_ptr() if d_next is not None else None,
                                          d_logits.data_ptr() if d_logits is not None else None,
                                          scratch.data_ptr(), scratch.numel() * scratch.element_size(),
                                          self.stream()), self.ctx)

    def prefill_batched(self, prompt: Sequence[int], want_logits: bool = False, chunk: int = 2048):
        """kie_prefill_batched with a scratch buffer for `chunk` tokens"""
        t = self.torch
        d_prompt = self._ids(prompt)
        nbytes = C.c_size_t()
        _check(self.L.kie_prefill_scratch_bytes(self.ctx, int(chunk), C.byref(nbytes)), self.ctx)
        scratch = t.empty(max(int(nbytes.value) // 4, 4), dtype=t.float32, device=self.dev)
        d_next = t.empty(1, dtype=t.int32, device=self.dev)
        d_logits = t.empty(self.cfg.vocab, dtype=t.float32, device=self.dev) if want_logits else None
        _check(self.L.kie_prefill_batched(self.ctx, d_prompt.data_ptr(), len(prompt), d_next.data_ptr(),
                                          d_logits.data_ptr() if d_logits is not None else None,
                                          scratch.data_ptr(), int(nbytes.value), self.stream()), self.ctx)
        self.sync()
        tok = int(d_next.cpu()[0])
        if want_logits:
            return tok, d_logits.cpu().numpy()
        return tok

    def prefill_batched_noalloc(self, prompt: Sequence[int], want_logits: bool = False):
        """kie_prefill_batched_noalloc: the batched prefill on the library's
        own fixed scratch (no device allocation inside the call)"""
        t = self.torch
        d_prompt = self._ids(prompt)
        d_next = t.empty(1, dtype=t.int32, device=self.dev)
        d_logits = t.empty(self.cfg.vocab, dtype=t.float32, device=self.dev) if want_logits else None
        _check(self.L.kie_prefill_batched_noalloc(self.ctx, d_prompt.data_ptr(), len(prompt), d_next.data_ptr(),
                                                  d_logits.data_ptr() if d_logits is not None else None,
                                                  self.stream()), self.ctx)
        self.sync()
        tok = int(d_next.cpu()[0])
        if want_logits:
            return tok, d_logits.cpu().numpy()
        return tok

    def decode_device(self, n: int, d_out, d_forced=None, d_logits=None):
        """asynchronous decode into caller-provided device tensors"""
        _check(self.L.kie_decode(self.ctx, int(n), d_out.data_ptr() if d_out is not None else None,
                                 d_forced.data_ptr() if d_forced is not None else None,
                                 d_logits.data_ptr() if d_logits is not None else None,
                                 self.stream()), self.ctx)

    def decode(self, n: int, forced: Optional[Sequence[int]] = None, want_logits: bool = False):
        t = self.torch
        d_out = t.empty(n, dtype=t.int32, device=self.dev)
        d_forced = self._ids(forced) if forced is not None else None
        if d_forced is not None and d_forced.numel() < n:
            raise ValueError("forced must hold n tokens")
        d_logits = t.empty((n, self.cfg.vocab), dtype=t.float32, device=self.dev) if want_logits else None
        self.decode_device(n, d_out, d_forced, d_logits)
        self.sync()
        toks = d_out.cpu().numpy()
        if want_logits:
            return toks, d_logits.cpu().numpy()
        return toks

    def set_position(self, pos: int, next_token: int):
        _check(self.L.kie_set_position(self.ctx, int(pos), int(next_token), self.stream()), self.ctx)
