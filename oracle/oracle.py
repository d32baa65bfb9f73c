"""Plain fp64 CPU oracle for batch-1 decoding of a pre-norm decoder.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this module.  It shares no code with
the HIP path (it imports numpy and nothing else) and is never on the product
path.

What it computes.  The pages (Kog Inference Engine explainers: "Monokernel"
and results table) state the method is exact FP16 decoding at batch 1 with no
quantization, no speculative decoding and no pruning, run as one persistent
kernel.  The kernel changes where and when the work runs, not what is
computed, so the oracle is the textbook decoder written out in float64 from
the float16 weights (upcast exactly).  The block itself is not defined on the
pages; the reading used (Llama-style pre-norm: RMSNorm, rotate-half RoPE,
causal softmax attention with 1/sqrt(hd) scale, SwiGLU, untied embedding and
LM head, greedy argmax with the lowest id on ties) is listed with every other
reading in the design doc.

The lane-structured variant (the pages' Laneformer: 8 lanes aligned with
Delayed Tensor Parallelism, all-reduce delayed by two layers) is a parallel
block whose summed partial P_l = attn_l + mlp_l (both computed from x_l)
reaches the residual stream `delay` layers later: x_{l+1} = x_l + P_{l-delay};
the pending partials of the last `delay` layers are added before the final
RMSNorm.

Pins (tests/test_oracle_pins.py): brute-force scalar loops on tiny shapes,
KV-cached decode == no-cache recomputation, RoPE closed forms and the
relative-position identity, single-key attention returns V, softmax rows sum
to 1, GQA == MHA with duplicated KV heads, lane partials sum to the unsplit
layer, delay 0 == parallel block, argmax ties; for sampling, the published
Philox4x32-10 known-answer vectors, Gumbel-max frequencies against
softmax(logits / T) by a chi-square test, and T -> 0 reducing to greedy.  End-to-end logits of a model
are "parity unpinned" against the pages: they print no logits or tokens.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import numpy as np

f64 = np.float64


# --------------------------------------------------------------------------
# elementary pieces
# --------------------------------------------------------------------------
def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """g * x / sqrt(mean(x^2) + eps) over the last axis"""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def rope_angles(positions: np.ndarray, head_dim: int, base: float) -> np.ndarray:
    """theta[p, i] = p * base^(-2i/hd), i < hd/2"""
    i = np.arange(head_dim // 2, dtype=f64)
    inv_freq = np.power(f64(base), -2.0 * i / head_dim)
    return np.outer(np.asarray(positions, dtype=f64), inv_freq)


def apply_rope(u: np.ndarray, positions: np.ndarray, base: float) -> np.ndarray:
    """Rotate-half RoPE.  u: [n, heads, hd]; pair (i, i + hd/2) is rotated by
    +theta_i:  (a, b) -> (a cos - b sin, a sin + b cos)."""
    hd = u.shape[-1]
    half = hd // 2
    ang = rope_angles(positions, hd, base)
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    a = u[..., :half]
    b = u[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def softmax(s: np.ndarray, axis: int = -1) -> np.ndarray:
    m = np.max(s, axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """one query head over n keys: q [hd], K, V [n, hd] -> [hd]"""
    p = softmax(K @ q / np.sqrt(f64(q.shape[-1])))
    return p @ V


def greedy(logits: np.ndarray) -> int:
    """lowest id among exact maxima"""
    return int(np.argmax(logits))


# --------------------------------------------------------------------------
# stochastic LM-head sampling
# --------------------------------------------------------------------------
# The pages (Kog explainer, "Monokernel" section) place LM-head sampling inside
# the persistent kernel but do not say which sampler.  The reading used here:
# temperature sampling drawn with the Gumbel-max property (argmax of
# logits / T plus independent standard Gumbel noise is distributed as
# softmax(logits / T)), the noise taken from the counter-based generator
# Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
# easy as 1, 2, 3", SC 2011) keyed by the 64-bit seed, with counter
# (vocabulary row, position, 0, 0).  T = 0 is greedy decoding.
PHILOX_M = (0xD2511F53, 0xCD9E8D57)  # round multipliers
PHILOX_W = (0x9E3779B9, 0xBB67AE85)  # key increments between rounds


def philox4x32(counter, key, rounds: int = 10):
    """Philox4x32 with `rounds` rounds, elementwise over uint32 arrays.

    counter: four arrays (or ints) c0..c3; key: two ints k0, k1.  One round
    multiplies c0 and c2 by the two constants into 64-bit products and forms
    (hi(c2*M1) ^ c1 ^ k0, lo(c2*M1), hi(c0*M0) ^ c3 ^ k1, lo(c0*M0)); the key
    advances by the two Weyl increments after every round.  Returns the four
    output words as uint64 arrays holding 32-bit values."""
    m32 = np.uint64(0xFFFFFFFF)
    c = [np.asarray(x, dtype=np.uint64) & m32 for x in counter]
    k0, k1 = int(key[0]) & 0xFFFFFFFF, int(key[1]) & 0xFFFFFFFF
    for _ in range(rounds):
        p0 = np.uint64(PHILOX_M[0]) * c[0]
        p1 = np.uint64(PHILOX_M[1]) * c[2]
        c = [(p1 >> np.uint64(32)) ^ c[1] ^ np.uint64(k0), p1 & m32,
             (p0 >> np.uint64(32)) ^ c[3] ^ np.uint64(k1), p0 & m32]
        k0 = (k0 + PHILOX_W[0]) & 0xFFFFFFFF
        k1 = (k1 + PHILOX_W[1]) & 0xFFFFFFFF
    return c


def uniform_open(words: np.ndarray) -> np.ndarray:
    """(0, 1) from 32-bit words: the top 23 bits plus one half, times 2^-23
    (exact in float32 as well)"""
    return ((np.asarray(words, dtype=np.uint64) >> np.uint64(9)).astype(f64) + 0.5) * 2.0 ** -23


def gumbel_noise(seed: int, pos: int, n: int) -> np.ndarray:
    """standard Gumbel noise -log(-log(u)) for rows 0..n-1 at position pos"""
    rows = np.arange(n, dtype=np.uint64)
    w0 = philox4x32((rows, np.full(n, pos, np.uint64), 0, 0), (seed & 0xFFFFFFFF, seed >> 32))[0]
    return -np.log(-np.log(uniform_open(w0)))


def sample(logits: np.ndarray, temperature: float, seed: int, pos: int) -> int:
    """the token emitted after position pos: greedy for T = 0, else argmax of
    logits / T + Gumbel noise (lowest id among exact maxima)"""
    if temperature == 0:
        return greedy(logits)
    z = np.asarray(logits, dtype=f64) / f64(temperature) + gumbel_noise(seed, pos, len(logits))
    return int(np.argmax(z))


def sampling_scores(logits: np.ndarray, temperature: float, seed: int, pos: int) -> np.ndarray:
    """the perturbed scores whose argmax `sample` takes"""
    if temperature == 0:
        return np.asarray(logits, dtype=f64)
    return np.asarray(logits, dtype=f64) / f64(temperature) + gumbel_noise(seed, pos, len(logits))


# --------------------------------------------------------------------------
# model
# --------------------------------------------------------------------------
@dataclass
class Layer:
    attn_norm: np.ndarray
    wq: np.ndarray
    wk: np.ndarray
    wv: np.ndarray
    wo: np.ndarray
    mlp_norm: np.ndarray
    w_gate: np.ndarray
    w_up: np.ndarray
    w_down: np.ndarray


class KVCache:
    """fp64 K/V per layer: [Hkv, capacity, hd]"""

    def __init__(self, n_layers: int, n_kv: int, hd: int, capacity: int):
        self.K = [np.zeros((n_kv, capacity, hd)) for _ in range(n_layers)]
        self.V = [np.zeros((n_kv, capacity, hd)) for _ in range(n_layers)]
        self.capacity = capacity


class Oracle:
    """cfg: any object with n_layers, d_model, n_heads, n_kv_heads, head_dim,
    ffn_dim, vocab, rms_eps, rope_base, lane_delay, sequential, n_lanes.
    weights: dict of float16 arrays named as by the input generator."""

    def __init__(self, cfg, weights: Dict[str, np.ndarray], kv_fp16: bool = False):
        """kv_fp16: store K and V in the cache rounded to binary16 (round to
        nearest even), the cache of an FP16 model; arithmetic stays fp64.
        Default: the cache keeps fp64 values."""
        self.cfg = cfg
        self.kv_fp16 = bool(kv_fp16)
        up = lambda a: np.asarray(a).astype(f64)
        self.embed16 = weights["embed"]
        self.layers: List[Layer] = []
        for l in range(cfg.n_layers):
            w = lambda n: up(weights[f"layers.{l}.{n}"])
            self.layers.append(Layer(w("attn_norm"), w("wq"), w("wk"), w("wv"), w("wo"),
                                     w("mlp_norm"), w("w_gate"), w("w_up"), w("w_down")))
        self.final_norm = up(weights["final_norm"])
        self.lm_head = up(weights["lm_head"])
        self.H = cfg.n_heads
        self.Hkv = cfg.n_kv_heads
        self.hd = cfg.head_dim
        self.G = self.H // self.Hkv
        self.eps = float(cfg.rms_eps)
        self.base = float(cfg.rope_base)
        self.sequential = bool(getattr(cfg, "sequential", True))
        self.delay = int(getattr(cfg, "lane_delay", 0))

    # -- helpers ---------------------------------------------------------
    def cache_round(self, a: np.ndarray) -> np.ndarray:
        return a.astype(np.float16).astype(f64) if self.kv_fp16 else a

    def embed(self, tokens) -> np.ndarray:
        return self.embed16[np.asarray(tokens)].astype(f64)

    def mlp(self, L: Layer, h: np.ndarray) -> np.ndarray:
        return (silu(h @ L.w_gate.T) * (h @ L.w_up.T)) @ L.w_down.T

    def qkv(self, L: Layer, h: np.ndarray, positions: np.ndarray):
        n = h.shape[0]
        q = (h @ L.wq.T).reshape(n, self.H, self.hd)
        k = (h @ L.wk.T).reshape(n, self.Hkv, self.hd)
        v = (h @ L.wv.T).reshape(n, self.Hkv, self.hd)
        return apply_rope(q, positions, self.base), apply_rope(k, positions, self.base), v

    def causal_attention(self, q, k, v, positions):
        """q [n, H, hd] at `positions`; k, v [T, Hkv, hd] hold keys 0..T-1.
        Query at position p attends keys 0..p (itself included).  Query head
        i reads KV head i // G."""
        n = q.shape[0]
        T = k.shape[0]
        out = np.empty((n, self.H, self.hd))
        mask = np.arange(T)[None, :] > np.asarray(positions)[:, None]  # [n, T]
        scale = 1.0 / np.sqrt(f64(self.hd))
        for i in range(self.H):
            g = i // self.G
            s = (q[:, i, :] @ k[:, g, :].T) * scale
            s = np.where(mask, -np.inf, s)
            out[:, i, :] = softmax(s, axis=-1) @ v[:, g, :]
        return out

    def logits_from_hidden(self, x: np.ndarray) -> np.ndarray:
        return rmsnorm(x, self.final_norm, self.eps) @ self.lm_head.T

    # -- whole-sequence forward, no cache --------------------------------
    def forward_nocache(self, tokens: Sequence[int]) -> np.ndarray:
        """logits [n, V] of every position of `tokens` (positions 0..n-1)"""
        tokens = np.asarray(tokens)
        n = tokens.shape[0]
        pos = np.arange(n)
        x = self.embed(tokens)
        pending: Dict[int, np.ndarray] = {}
        for l, L in enumerate(self.layers):
            h = rmsnorm(x, L.attn_norm, self.eps)
            q, k, v = self.qkv(L, h, pos)
            a = self.causal_attention(q, k, v, pos).reshape(n, -1) @ L.wo.T
            if self.sequential:
                x = x + a
                x = x + self.mlp(L, rmsnorm(x, L.mlp_norm, self.eps))
            else:
                pending[l] = a + self.mlp(L, rmsnorm(x, L.mlp_norm, self.eps))
                if l - self.delay >= 0:
                    x = x + pending.pop(l - self.delay)
        if not self.sequential:
            for j in sorted(pending):
                x = x + pending[j]
        return self.logits_from_hidden(x)

    # -- cached path ------------------------------------------------------
    def new_cache(self, capacity: int) -> KVCache:
        return KVCache(len(self.layers), self.Hkv, self.hd, capacity)

    def prefill(self, cache: KVCache, tokens: Sequence[int], start: int = 0) -> np.ndarray:
        """Run `tokens` at positions start.., fill the cache, return the logits
        of the last position.  Batched over the prompt (plain GEMMs)."""
        tokens = np.asarray(tokens)
        n = tokens.shape[0]
        pos = np.arange(start, start + n)
        x = self.embed(tokens)
        pending: Dict[int, np.ndarray] = {}
        for l, L in enumerate(self.layers):
            h = rmsnorm(x, L.attn_norm, self.eps)
            q, k, v = self.qkv(L, h, pos)
            cache.K[l][:, start:start + n, :] = self.cache_round(k.transpose(1, 0, 2))
            cache.V[l][:, start:start + n, :] = self.cache_round(v.transpose(1, 0, 2))
            kk = cache.K[l][:, :start + n, :].transpose(1, 0, 2)
            vv = cache.V[l][:, :start + n, :].transpose(1, 0, 2)
            a = self.causal_attention(q, kk, vv, pos).reshape(n, -1) @ L.wo.T
            if self.sequential:
                x = x + a
                x = x + self.mlp(L, rmsnorm(x, L.mlp_norm, self.eps))
            else:
                pending[l] = a + self.mlp(L, rmsnorm(x, L.mlp_norm, self.eps))
                if l - self.delay >= 0:
                    x = x + pending.pop(l - self.delay)
        if not self.sequential:
            for j in sorted(pending):
                x = x + pending[j]
        return self.logits_from_hidden(x[-1])

    def step(self, cache: KVCache, token: int, pos: int) -> np.ndarray:
        """one decode token at position `pos`; appends K/V; returns logits"""
        x = self.embed([token])[0]
        pending: Dict[int, np.ndarray] = {}
        for l, L in enumerate(self.layers):
            h = rmsnorm(x, L.attn_norm, self.eps)
            q, k, v = self.qkv(L, h[None, :], np.array([pos]))
            cache.K[l][:, pos, :] = self.cache_round(k[0])
            cache.V[l][:, pos, :] = self.cache_round(v[0])
            o = np.empty((self.H, self.hd))
            for i in range(self.H):
                g = i // self.G
                o[i] = attend(q[0, i], cache.K[l][g, :pos + 1], cache.V[l][g, :pos + 1])
            a = o.reshape(-1) @ L.wo.T
            if self.sequential:
                x = x + a
                x = x + self.mlp(L, rmsnorm(x, L.mlp_norm, self.eps))
            else:
                pending[l] = a + self.mlp(L, rmsnorm(x, L.mlp_norm, self.eps))
                if l - self.delay >= 0:
                    x = x + pending.pop(l - self.delay)
        if not self.sequential:
            for j in sorted(pending):
                x = x + pending[j]
        return self.logits_from_hidden(x)

    # -- runs ---------------------------------------------------------------
    def run(self, prompt: Sequence[int], n_steps: int,
            forced: Optional[Sequence[int]] = None, keep_logits: bool = True,
            temperature: float = 0.0, seed: int = 0):
        """Prefill `prompt`, then n_steps decode steps.  Step k consumes
        forced[k] if given, else the previous emitted token (t1 from the
        prefill for k = 0), runs at position len(prompt) + k and emits
        sample(logits, temperature, seed, position) (argmax for T = 0; t1 is
        drawn at position len(prompt) - 1).
        Returns dict(t1, prefill_logits, inputs, tokens, logits)."""
        P = len(prompt)
        cache = self.new_cache(P + n_steps)
        lg0 = self.prefill(cache, prompt)
        t = sample(lg0, temperature, seed, P - 1)
        res = dict(t1=t, prefill_logits=lg0, inputs=[], tokens=[], logits=[])
        for k in range(n_steps):
            tin = int(forced[k]) if forced is not None else t
            lg = self.step(cache, tin, P + k)
            t = sample(lg, temperature, seed, P + k)
            res["inputs"].append(tin)
            res["tokens"].append(t)
            if keep_logits:
                res["logits"].append(lg)
        res["cache"] = cache
        return res


# --------------------------------------------------------------------------
# lane decomposition (for pinning the lane-structured variant)
# --------------------------------------------------------------------------
def lane_partials(orc: Oracle, l: int, x: np.ndarray, cache: KVCache, pos: int,
                  n_lanes: int) -> List[np.ndarray]:
    """Per-lane partial outputs of parallel layer l for one token at `pos`
    whose K/V are already in `cache`: lane j owns query heads
    [j*H/n, (j+1)*H/n) and FFN columns [j*F/n, (j+1)*F/n); its partial is
    Wo[:, its heads] o[its heads] + Wd[:, its cols] h[its cols]."""
    L = orc.layers[l]
    H, hd, G = orc.H, orc.hd, orc.G
    F = L.w_gate.shape[0]
    h = rmsnorm(x, L.attn_norm, orc.eps)
    q = (L.wq @ h).reshape(1, H, hd)
    q = apply_rope(q, np.array([pos]), orc.base)[0]
    o = np.empty((H, hd))
    for i in range(H):
        g = i // G
        o[i] = attend(q[i], cache.K[l][g, :pos + 1], cache.V[l][g, :pos + 1])
    h2 = rmsnorm(x, L.mlp_norm, orc.eps)
    act = silu(L.w_gate @ h2) * (L.w_up @ h2)
    hpl, fpl = H // n_lanes, F // n_lanes
    parts = []
    for j in range(n_lanes):
        hs = slice(j * hpl * hd, (j + 1) * hpl * hd)
        fs = slice(j * fpl, (j + 1) * fpl)
        parts.append(L.wo[:, hs] @ o.reshape(-1)[hs] + L.w_down[:, fs] @ act[fs])
    return parts
