"""Host logic of the C ABI, on the CPU: the library loads and exports every
declared symbol, configurations are validated, buffer sizes follow the
layout, the packer is a pure permutation of the weights, and the kernel's work
partition covers every row and key exactly once."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from decode_persistent_monokernel_amd import kie
from decode_persistent_monokernel_amd.config import CFG0, CFG1, CFG2, CFG3, CFG4, ModelConfig
from decode_persistent_monokernel_amd.inputs import gen_weights

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kie.h")

needs_lib = pytest.mark.skipif(not os.path.exists(kie.LIB_PATH), reason="libkie.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kie_[a-z_]+)\s*\(", text)))


@needs_lib
def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 18
    L = C.CDLL(kie.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


@needs_lib
@pytest.mark.parametrize("cfg", [CFG0, CFG1, CFG2, CFG3, CFG4], ids=lambda c: c.name)
def test_presets_are_accepted_host_only(cfg):
    assert kie.create_status(cfg, -1) == kie.KIE_OK


@needs_lib
@pytest.mark.parametrize("bad", [
    dict(n_layers=0), dict(n_heads=6, n_kv_heads=4), dict(head_dim=60), dict(ffn_dim=1020),
    dict(n_lanes=3), dict(lane_delay=2), dict(vocab=-1), dict(rope_base=1.0),
])
def test_invalid_configs_rejected(bad):
    assert kie.create_status(CFG0.with_(**bad), -1) == -1


@needs_lib
def test_unsupported_shapes_rejected():
    # 8 query heads per KV head and an FFN too wide for the LDS plan
    assert kie.create_status(CFG0.with_(n_heads=8, n_kv_heads=1, d_model=512), -1) == -6
    assert kie.create_status(CFG0.with_(ffn_dim=32768), -1) == -6


@needs_lib
def test_sizes_follow_layout():
    for cfg in (CFG0, CFG2, CFG4):
        packed, kvb, ws = kie.query_sizes(cfg)
        off = _offsets(cfg)
        assert packed == (off["embed"] + cfg.vocab * cfg.d_model + 127) // 128 * 256 + 1024
        if min(cfg.d_model, cfg.q_dim, cfg.ffn_dim) >= 512:
            params = cfg.param_elems() * 2
            assert params <= packed <= params + 4096 * (9 * cfg.n_layers + 3)
        # the cache itself, then one 1-KB chunk of slack
        assert kvb == cfg.n_layers * 2 * cfg.n_kv_heads * cfg.max_ctx * cfg.head_dim * 2 + 1024
        assert ws > cfg.max_ctx * cfg.head_dim * 4  # holds the RoPE table


@needs_lib
def test_host_only_context_refuses_gpu_calls():
    L = kie.lib()
    ctx = C.c_void_p()
    c = kie.config_c(CFG0)
    assert L.kie_create(C.byref(c), -1, C.byref(ctx)) == 0
    try:
        assert L.kie_bind_memory(ctx, 256, 256, 256) == -4
        assert L.kie_decode(ctx, 1, None, None, None, None) == -4
        assert L.kie_prefill(ctx, 256, 1, None, None, None) == -4
        assert L.kie_set_timeout_us(ctx, 0) == -1
        assert L.kie_set_launch_steps(ctx, 0) == -1
        # sampling settings are host state: checked without a GPU
        assert L.kie_set_sampling(ctx, -0.5, 1) == -1
        assert L.kie_set_sampling(ctx, float("nan"), 1) == -1
        assert L.kie_set_sampling(ctx, float("inf"), 1) == -1
        assert L.kie_set_sampling(ctx, 0.0, 0) == 0
        assert L.kie_set_sampling(ctx, 0.8, 2**64 - 1) == 0
        assert L.kie_position(ctx) == 0
        assert L.kie_status_string(-5) == b"wait timed out inside the kernel"
    finally:
        L.kie_destroy(ctx)


def _nb(k):
    """256-column blocks of a packed row"""
    return (k + 255) // 256


def _psize(rows, k):
    """packed elements of a rows x k matrix: one 512-element chunk per (row pair, block)"""
    return rows // 2 * _nb(k) * 512


def _full(flat, rows, k):
    """undo the row-pair chunk layout: chunk (p, b) = 256 columns of row 2p, then
    the same columns of row 2p+1; returns rows x (256 * blocks) with the pads"""
    c = flat[: _psize(rows, k)].reshape(rows // 2, _nb(k), 2, 256)
    return c.transpose(0, 2, 1, 3).reshape(rows, _nb(k) * 256)


def _mat(flat, rows, k):
    return _full(flat, rows, k)[:, :k]


def _unpack(cfg: ModelConfig, packed: np.ndarray, offsets):
    """invert the packed layout with the layout rules written out here"""
    d, H, Hkv, hd, F = cfg.d_model, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn_dim
    out = {}
    stride = offsets["layer_stride"]
    for l in range(cfg.n_layers):
        base = l * stride
        g = lambda off, n: packed[base + off: base + off + n]
        out[f"layers.{l}.attn_norm"] = g(offsets["attn_norm"], d)
        qkv = _mat(g(offsets["wqkv"], _psize((H + 2 * Hkv) * hd, d)), (H + 2 * Hkv) * hd, d)
        def unperm(block, heads):
            blk = block.reshape(heads, hd, d)
            o = np.empty_like(blk)
            o[:, : hd // 2] = blk[:, 0::2]
            o[:, hd // 2:] = blk[:, 1::2]
            return o.reshape(heads * hd, d)
        out[f"layers.{l}.wq"] = unperm(qkv[: H * hd], H)
        out[f"layers.{l}.wk"] = unperm(qkv[H * hd: (H + Hkv) * hd], Hkv)
        out[f"layers.{l}.wv"] = qkv[(H + Hkv) * hd:]
        out[f"layers.{l}.wo"] = _mat(g(offsets["wo"], _psize(d, H * hd)), d, H * hd)
        out[f"layers.{l}.mlp_norm"] = g(offsets["mlp_norm"], d)
        gu = _mat(g(offsets["wgu"], _psize(2 * F, d)), 2 * F, d)
        out[f"layers.{l}.w_gate"] = gu[0::2]
        out[f"layers.{l}.w_up"] = gu[1::2]
        out[f"layers.{l}.w_down"] = _mat(g(offsets["wd"], _psize(d, F)), d, F)
    out["final_norm"] = packed[offsets["final_norm"]: offsets["final_norm"] + d]
    out["lm_head"] = _mat(packed[offsets["lm_head"]:], cfg.vocab, d)
    out["embed"] = packed[offsets["embed"]: offsets["embed"] + cfg.vocab * d].reshape(cfg.vocab, d)
    return out


def _offsets(cfg):
    """256-byte aligned offsets (elements), written from the layout rules"""
    a = lambda x: (x + 127) // 128 * 128
    d, qd, kvd, F = cfg.d_model, cfg.q_dim, cfg.kv_dim, cfg.ffn_dim
    o = {}
    x = 0
    o["attn_norm"] = x; x = a(x + d)
    o["wqkv"] = x; x = a(x + _psize(qd + 2 * kvd, d))
    o["wo"] = x; x = a(x + _psize(d, qd))
    o["mlp_norm"] = x; x = a(x + d)
    o["wgu"] = x; x = a(x + _psize(2 * F, d))
    o["wd"] = x; x = a(x + _psize(d, F))
    o["layer_stride"] = x
    x = x * cfg.n_layers
    o["final_norm"] = x; x = a(x + d)
    o["lm_head"] = x; x = a(x + _psize(cfg.vocab, d))
    o["embed"] = x
    return o


@needs_lib
@pytest.mark.parametrize("cfg", [
    CFG0.with_(n_layers=2, vocab=512),
    CFG0.with_(n_layers=1, n_heads=8, n_kv_heads=2, head_dim=32, vocab=300, name="gqa"),
    CFG3.with_(n_layers=1, d_model=320, n_heads=4, n_kv_heads=4, head_dim=80, ffn_dim=864, vocab=100, n_lanes=4),
    CFG3.with_(n_layers=1, d_model=256, n_heads=4, n_kv_heads=2, head_dim=64, ffn_dim=512, vocab=100, n_lanes=2),
], ids=["mha", "gqa", "hd80", "lanes-gqa"])
def test_packer_is_a_permutation(cfg):
    w = gen_weights(cfg, std=0.5, threads=2)
    # distinct, recognisable norms
    for l in range(cfg.n_layers):
        w[f"layers.{l}.attn_norm"] = (np.arange(cfg.d_model) % 7 + 1).astype(np.float16)
        w[f"layers.{l}.mlp_norm"] = (np.arange(cfg.d_model) % 5 + 2).astype(np.float16)
    packed = kie.pack_weights_host(cfg, w)
    off = _offsets(cfg)
    assert packed.size * 2 >= (off["embed"] + cfg.vocab * cfg.d_model) * 2
    back = _unpack(cfg, packed, off)
    for k, v in w.items():
        assert np.array_equal(back[k], v.view(np.uint16)), k
    # the kernel streams whole 1-KB chunks: column pads and the tail slack are zeros
    assert not packed[-512:].any()
    d, qd, F = cfg.d_model, cfg.q_dim, cfg.ffn_dim
    rows = (cfg.n_heads + 2 * cfg.n_kv_heads) * cfg.head_dim
    for name, r, k in (("wqkv", rows, d), ("wo", d, qd), ("wgu", 2 * F, d), ("wd", d, F)):
        full = _full(packed[off[name]:], r, k)
        assert not full[:, k:].any(), name


# a shape whose O projection (d rows over the workgroups that are not
# attention mergers) gives a workgroup more rows than any other GEMV does
O_HEAVY = CFG0.with_(name="o-heavy", d_model=1024, n_heads=4, n_kv_heads=4, head_dim=64, ffn_dim=256, vocab=256)


@needs_lib
@pytest.mark.parametrize("cfg", [CFG0, CFG1, CFG2, CFG3, CFG4, O_HEAVY], ids=lambda c: c.name)
def test_schedule_covers_everything(cfg):
    ctxs = sorted({1, 2, 3, 17, cfg.prompt_len, cfg.prompt_len + 1, cfg.max_ctx})
    for nwg in (256, 80, 304):
        for n in ctxs:
            try:
                kie.validate_schedule(cfg, nwg, n)
            except kie.KieError as e:
                # other workgroup counts can overflow the LDS plan (MI355X has 256 CUs)
                assert nwg != 256 and "LDS" in str(e), str(e)


def _check_dependencies(cfg, order):
    """producers before consumers, read off the block's equations: x_l is
    x_0 for l <= delay (parallel block) and x_{l-1} + P_{l-delay-1} after,
    published by that layer's down projection"""
    L, par = cfg.n_layers, not cfg.sequential
    pos = {(k, l): i for i, (k, l) in enumerate(order[:5 * L])}
    assert len(pos) == 5 * L and order[-1] == (5, L)
    Q, A, O, G, D = 0, 1, 2, 3, 4
    for l in range(L):
        src = (l - cfg.lane_delay - 1) if par else (l - 1)
        for k in ((Q, G) if par else (Q,)):
            if src >= 0:
                assert pos[(D, src)] < pos[(k, l)]
        assert pos[(Q, l)] < pos[(A, l)] < pos[(O, l)]
        if not par:
            assert pos[(O, l)] < pos[(G, l)]
        assert pos[(G, l)] < pos[(D, l)] and pos[(O, l)] < pos[(D, l)]
    return pos


@needs_lib
def test_phase_order():
    """kie_phase_order: the sequential block runs layer by layer; the lane
    block with a delay of two layers or more runs its attention ahead of the
    next layer's QKV and gate/up, so two weight streams separate the
    attention output from O; every order respects the block's dependencies"""
    Q, A, O, G, D = 0, 1, 2, 3, 4
    seq = kie.phase_order(CFG2, 256)
    _check_dependencies(CFG2, seq)
    assert [k for k, _ in seq[:10]] == [Q, A, O, G, D] * 2
    pipe = kie.phase_order(CFG3, 256)
    pos = _check_dependencies(CFG3, pipe)
    assert [k for k, _ in pipe[:12]] == [Q, G, A, Q, G, O, D, A, Q, G, O, D]
    assert [l for _, l in pipe[:12]] == [0, 0, 0, 1, 1, 0, 0, 1, 2, 2, 1, 1]
    assert all(pos[(O, l)] - pos[(A, l)] == 3 for l in range(CFG3.n_layers - 1))
    lanes = CFG0.with_(name="lanes", n_layers=6, n_lanes=2, sequential=False)
    gqa4 = dict(n_heads=8, n_kv_heads=2, head_dim=32)  # four query heads per KV head: no staging
    for delay, shape, piped in ((0, {}, False), (1, {}, False), (2, {}, True), (3, dict(n_kv_heads=2), True),
                                (2, gqa4, False)):
        cfg = lanes.with_(lane_delay=delay, **shape)
        order = kie.phase_order(cfg, 256)
        _check_dependencies(cfg, order)
        assert ([k for k, _ in order[:4]] == [Q, G, A, Q]) == piped, (delay, shape)
    assert kie.lib().kie_phase_order(None, 256, None, None, 0) != kie.KIE_OK
    short = (C.c_int32 * 3)()
    assert kie.lib().kie_phase_order(C.byref(kie.config_c(CFG3)), 256, short, short, 3) != kie.KIE_OK


@needs_lib
def test_ring_depth():
    """kie_ring_depth: the sequential block runs ten LDS slots per wave when
    its other LDS buffers fit beside them, the lane block and the 8B shape's
    larger buffers keep eight; the kernel name carries the depth"""
    assert [kie.ring_depth(c, 256) for c in (CFG0, CFG1, CFG2, CFG3, CFG4)] == [10, 10, 10, 8, 8]
    assert kie.kernel_name(CFG2, 256) == "kie::ring10::kie_monokernel<1, false>"
    assert kie.kernel_name(CFG3, 256) == "kie::ring8::kie_monokernel<1, true>"
    assert kie.kernel_name(CFG4, 256) == "kie::ring8::kie_monokernel<4, false>"
    d = C.c_int32()
    assert kie.lib().kie_ring_depth(C.byref(kie.config_c(CFG2)), 256, None) == -1  # KIE_ERR_INVALID_ARG
    assert kie.lib().kie_ring_depth(None, 256, C.byref(d)) == -1  # KIE_ERR_INVALID_ARG
    assert kie.lib().kie_ring_depth(C.byref(kie.config_c(CFG2)), 0, C.byref(d)) == -1  # KIE_ERR_INVALID_ARG


@needs_lib
def test_lane_placement_maps_lanes_to_xcds():
    """The lane-structured 2.4B shape (8 lanes of 4 heads and 864 FFN columns)
    on 256 workgroups: workgroup w runs on XCD w // 32 (the kernel numbers its
    workgroups XCD by XCD), and every workgroup's attention head and gate/up
    rows belong to lane w // 32 alone, so lane j's attention and gate/up run
    on XCD j.  The QKV rows (all q, then all k, then all v) do not follow the
    lanes: the first three XCDs' workgroups compute the q rows of every lane."""
    lo, hi = kie.lane_placement(CFG3, 256)
    want = np.repeat(np.arange(8, dtype=np.int32), 32)
    for k, name in ((1, "attention"), (2, "gate/up")):
        assert np.array_equal(lo[k], want) and np.array_equal(hi[k], want), name
    # q rows: 2560 of the 7680 rows, 30 rows per workgroup; lane j's 320 q rows
    # on workgroups 320j/30 .. (320j + 319)/30
    rows = 30 * np.arange(256)
    assert np.array_equal(lo[0][:85], rows[:85] // 320)
    assert (lo[0][86:171] >= 0).all() and not np.array_equal(lo[0], want)
    # a lane block with two query heads per KV head and four lanes
    g2 = CFG3.with_(n_layers=2, n_kv_heads=16, n_lanes=4)
    lo, hi = kie.lane_placement(g2, 256)
    want4 = np.repeat(np.arange(4, dtype=np.int32), 64)
    for k in (1, 2):
        assert np.array_equal(lo[k], want4) and np.array_equal(hi[k], want4), k
    n = 3 * 256
    a = (C.c_int32 * n)()
    assert kie.lib().kie_lane_placement(C.byref(kie.config_c(CFG3)), 256, None, a) == -1  # KIE_ERR_INVALID_ARG
    assert kie.lib().kie_lane_placement(None, 256, a, a) == -1


@needs_lib
def test_schedule_validator_reports_problems():
    with pytest.raises(kie.KieError):
        kie.validate_schedule(CFG0, 2, 5)  # fewer workgroups than KV heads
