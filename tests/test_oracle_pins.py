"""Pins of the fp64 oracle against what the mathematics fixes (CPU only).

Each check is a function returning an error figure so that the mutation tests
at the bottom can plant a plausible mistake in the oracle (on the CPU) and show
that at least one check catches it.
"""
import math

import numpy as np
import pytest

import oracle.oracle as O
from bruteforce import BruteDecoder
from decode_persistent_monokernel_amd.config import ModelConfig, CFG0
from decode_persistent_monokernel_amd.inputs import gen_weights, gen_prompt

TINY = ModelConfig(name="tiny", n_layers=2, d_model=8, n_heads=2, n_kv_heads=2, head_dim=4,
                   ffn_dim=16, vocab=11, prompt_len=3, decode_steps=3, seed_index=100)
TINY_GQA = TINY.with_(name="tiny_gqa", n_heads=4, n_kv_heads=2, d_model=12, seed_index=101)
TINY_LANES = TINY.with_(name="tiny_lanes", n_layers=4, n_heads=4, n_kv_heads=4, d_model=16,
                        n_lanes=2, lane_delay=2, sequential=False, seed_index=102)


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# ----------------------------------------------------------------------------
# checks
# ----------------------------------------------------------------------------
def check_bruteforce(cfg, std=0.5, n_steps=3, kv_fp16=False):
    w = gen_weights(cfg, std=std, threads=1)
    prompt = gen_prompt(cfg)
    orc = O.Oracle(cfg, w, kv_fp16=kv_fp16)
    res = orc.run(prompt, n_steps)
    bf = BruteDecoder(cfg, w, kv_fp16=kv_fp16)
    worst = 0.0
    lg = None
    for p, t in enumerate(prompt):
        lg = bf.token(int(t), p)
    worst = max(worst, rel(res["prefill_logits"], lg))
    for k in range(n_steps):
        lg = bf.token(res["inputs"][k], len(prompt) + k)
        worst = max(worst, rel(res["logits"][k], lg))
    return worst


def check_cached_vs_nocache(cfg, std=0.3, n_steps=6):
    w = gen_weights(cfg, std=std, threads=1)
    prompt = gen_prompt(cfg)
    orc = O.Oracle(cfg, w)
    res = orc.run(prompt, n_steps)
    seq = list(prompt) + res["inputs"]
    full = orc.forward_nocache(seq)
    P = len(prompt)
    worst = rel(res["prefill_logits"], full[P - 1])
    for k in range(n_steps):
        worst = max(worst, rel(res["logits"][k], full[P + k]))
    return worst


def check_rope_closed_form():
    # hd = 4, base = 100: theta_0 = p, theta_1 = p / 10
    u = np.array([[[1.0, 2.0, 3.0, 4.0]]])
    p = 3
    got = O.apply_rope(u, np.array([p]), 100.0)[0, 0]
    t0, t1 = 3.0, 0.3
    want = [1 * math.cos(t0) - 3 * math.sin(t0), 2 * math.cos(t1) - 4 * math.sin(t1),
            1 * math.sin(t0) + 3 * math.cos(t0), 2 * math.sin(t1) + 4 * math.cos(t1)]
    return float(np.max(np.abs(got - np.array(want))))


def check_rope_relative(hd=8, base=10000.0):
    rng = np.random.default_rng(0)
    q = rng.standard_normal((1, 1, hd))
    k = rng.standard_normal((1, 1, hd))
    worst = 0.0
    for m, n in [(5, 2), (17, 17), (40, 3), (1000, 999)]:
        lhs = np.sum(O.apply_rope(q, np.array([m]), base) * O.apply_rope(k, np.array([n]), base))
        rhs = np.sum(O.apply_rope(q, np.array([m - n]), base) * k)
        worst = max(worst, abs(lhs - rhs))
    return worst


def check_rmsnorm_closed_form():
    c, eps = 3.0, 1e-5
    g = np.array([1.0, 2.0, -1.0, 0.5])
    got = O.rmsnorm(np.full(4, c), g, eps)
    want = g * c / math.sqrt(c * c + eps)
    return float(np.max(np.abs(got - want)))


def check_gqa_equals_mha(cfg=TINY_GQA, std=0.4):
    """duplicate each KV head G times -> an MHA model with identical logits"""
    w = gen_weights(cfg, std=std, threads=1)
    G = cfg.n_heads // cfg.n_kv_heads
    hd = cfg.head_dim
    mha_cfg = cfg.with_(n_kv_heads=cfg.n_heads)
    w2 = dict(w)
    for l in range(cfg.n_layers):
        for n in ("wk", "wv"):
            W = w[f"layers.{l}.{n}"].reshape(cfg.n_kv_heads, hd, -1)
            w2[f"layers.{l}.{n}"] = np.repeat(W, G, axis=0).reshape(cfg.n_heads * hd, -1)
    prompt = gen_prompt(cfg)
    a = O.Oracle(cfg, w).run(prompt, 3)
    b = O.Oracle(mha_cfg, w2).run(prompt, 3, forced=a["inputs"])
    return max(rel(x, y) for x, y in zip(a["logits"] + [a["prefill_logits"]],
                                         b["logits"] + [b["prefill_logits"]]))


def check_argmax_ties():
    lg = np.array([0.5, 2.0, -1.0, 2.0, 2.0, 1.9])
    return O.greedy(lg)


# ----------------------------------------------------------------------------
# tests
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [TINY, TINY_GQA, TINY_LANES], ids=lambda c: c.name)
def test_bruteforce_tiny(cfg):
    assert check_bruteforce(cfg) < 1e-12


@pytest.mark.parametrize("cfg", [TINY, TINY_GQA, TINY_LANES], ids=lambda c: c.name)
def test_bruteforce_tiny_fp16_cache(cfg):
    """the fp16-cache reading: K/V rounded to binary16 (struct 'e' format in
    the brute force, numpy float16 in the oracle) before they are cached"""
    assert check_bruteforce(cfg, kv_fp16=True) < 1e-12
    # and the rounding really changes the result (so the option is live)
    w = gen_weights(cfg, std=0.5, threads=1)
    a = O.Oracle(cfg, w).run(gen_prompt(cfg), 2)["logits"][-1]
    b = O.Oracle(cfg, w, kv_fp16=True).run(gen_prompt(cfg), 2)["logits"][-1]
    assert 1e-7 < rel(a, b) < 1e-2


@pytest.mark.parametrize("cfg", [TINY, TINY_GQA, TINY_LANES], ids=lambda c: c.name)
def test_cached_equals_nocache_tiny(cfg):
    assert check_cached_vs_nocache(cfg) < 1e-12


def test_cached_equals_nocache_cfg0_shape():
    cfg = CFG0.with_(prompt_len=8, seed_index=7)
    assert check_cached_vs_nocache(cfg, std=0.05, n_steps=4) < 1e-12


def test_rope_identity_at_zero():
    rng = np.random.default_rng(1)
    u = rng.standard_normal((3, 2, 16))
    assert np.array_equal(O.apply_rope(u, np.zeros(3), 10000.0), u)


def test_rope_norm_preserved():
    rng = np.random.default_rng(2)
    u = rng.standard_normal((5, 3, 128))
    r = O.apply_rope(u, np.array([1, 7, 100, 2047, 32767]), 500000.0)
    assert np.allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(u, axis=-1), rtol=1e-13)


def test_rope_closed_form():
    assert check_rope_closed_form() < 1e-14


def test_rope_relative_position():
    assert check_rope_relative() < 1e-11


def test_rmsnorm_closed_form_and_scale():
    assert check_rmsnorm_closed_form() < 1e-14
    x = np.random.default_rng(3).standard_normal(64) * 5
    a = O.rmsnorm(x, np.ones(64), 0.0)
    b = O.rmsnorm(x * 7.5, np.ones(64), 0.0)
    assert np.allclose(a, b, rtol=1e-14)
    assert abs(np.sqrt(np.mean(a * a)) - 1.0) < 1e-14


def test_softmax_rows_sum_to_one():
    s = np.random.default_rng(4).standard_normal((7, 33)) * 30
    assert np.allclose(O.softmax(s).sum(-1), 1.0, atol=1e-14)


def test_single_key_returns_v():
    rng = np.random.default_rng(5)
    q, K, V = rng.standard_normal(8), rng.standard_normal((1, 8)), rng.standard_normal((1, 8))
    assert np.array_equal(O.attend(q, K, V), V[0])


def test_equal_scores_average_values():
    rng = np.random.default_rng(6)
    K = np.tile(rng.standard_normal((1, 8)), (5, 1))
    V = rng.standard_normal((5, 8))
    assert np.allclose(O.attend(rng.standard_normal(8), K, V), V.mean(0), rtol=1e-14)


def test_attention_key_permutation_invariant():
    rng = np.random.default_rng(7)
    q, K, V = rng.standard_normal(16), rng.standard_normal((9, 16)), rng.standard_normal((9, 16))
    perm = rng.permutation(9)
    assert np.allclose(O.attend(q, K, V), O.attend(q, K[perm], V[perm]), rtol=1e-13)


def test_split_lse_merge_equals_whole():
    """the split-context merge (m, l, O) -> O/L the decode kernel uses is exact"""
    rng = np.random.default_rng(8)
    q, K, V = rng.standard_normal(16), rng.standard_normal((40, 16)), rng.standard_normal((40, 16))
    s = K @ q / 4.0
    parts = []
    for a, b in [(0, 7), (7, 8), (8, 30), (30, 40)]:
        m = s[a:b].max()
        p = np.exp(s[a:b] - m)
        parts.append((m, p.sum(), p @ V[a:b]))
    M = max(p[0] for p in parts)
    L = sum(np.exp(m - M) * l for m, l, _ in parts)
    o = sum(np.exp(m - M) * acc for m, _, acc in parts) / L
    assert rel(o, O.attend(q, K, V)) < 1e-14


def test_silu_special_values():
    from scipy.special import expit
    z = np.linspace(-30, 30, 121)
    assert np.allclose(O.silu(z), z * expit(z), rtol=1e-14, atol=1e-300)
    assert O.silu(np.array([0.0]))[0] == 0.0


def test_gqa_equals_duplicated_mha():
    assert check_gqa_equals_mha() < 1e-12


def test_argmax_lowest_id_on_ties():
    assert check_argmax_ties() == 1


def test_causal_future_tokens_do_not_matter():
    w = gen_weights(TINY, std=0.5, threads=1)
    orc = O.Oracle(TINY, w)
    a = orc.forward_nocache([1, 2, 3, 4, 5])
    b = orc.forward_nocache([1, 2, 3, 9, 0])
    assert np.array_equal(a[:3], b[:3])
    assert not np.allclose(a[3], b[3])


def test_no_residual_update_reduces_to_lm_head():
    """Wo = Wd = 0 leaves the residual at the embedding: logits are
    W_lm rmsnorm(E[t]) for every position, whatever attention does"""
    cfg = TINY
    w = gen_weights(cfg, std=0.5, threads=1)
    for l in range(cfg.n_layers):
        w[f"layers.{l}.wo"][:] = 0
        w[f"layers.{l}.w_down"][:] = 0
    orc = O.Oracle(cfg, w)
    toks = [3, 1, 4, 1, 5]
    lg = orc.forward_nocache(toks)
    E = w["embed"].astype(np.float64)[toks]
    want = (E / np.sqrt((E * E).mean(-1, keepdims=True) + cfg.rms_eps)) @ w["lm_head"].astype(np.float64).T
    assert rel(lg, want) < 1e-14


def test_lane_partials_sum_to_layer_and_flush():
    """Lane decomposition of the parallel block: per-lane partials (computed lane
    by lane) sum to the unsplit layer output, and with the delayed update the
    final residual equals x0 + sum_l P_l."""
    cfg = TINY_LANES
    w = gen_weights(cfg, std=0.4, threads=1)
    orc = O.Oracle(cfg, w)
    prompt = [2, 7, 5]
    cache = orc.new_cache(4)
    orc.prefill(cache, prompt[:-1])
    pos = len(prompt) - 1
    # run the last token through the layers by hand, checking lane sums
    x = orc.embed([prompt[-1]])[0]
    x0 = x.copy()
    pend, total = {}, np.zeros_like(x)
    for l, L in enumerate(orc.layers):
        h = O.rmsnorm(x, L.attn_norm, orc.eps)
        k = O.apply_rope((L.wk @ h).reshape(1, orc.Hkv, orc.hd), np.array([pos]), orc.base)[0]
        cache.K[l][:, pos] = k
        cache.V[l][:, pos] = (L.wv @ h).reshape(orc.Hkv, orc.hd)
        parts = O.lane_partials(orc, l, x, cache, pos, cfg.n_lanes)
        q = O.apply_rope((L.wq @ h).reshape(1, orc.H, orc.hd), np.array([pos]), orc.base)[0]
        o = np.stack([O.attend(q[i], cache.K[l][i // orc.G, :pos + 1], cache.V[l][i // orc.G, :pos + 1])
                      for i in range(orc.H)])
        unsplit = L.wo @ o.reshape(-1) + orc.mlp(L, O.rmsnorm(x, L.mlp_norm, orc.eps))
        assert rel(sum(parts), unsplit) < 1e-13
        pend[l] = unsplit
        total += unsplit
        if l - cfg.lane_delay >= 0:
            x = x + pend.pop(l - cfg.lane_delay)
    for j in sorted(pend):
        x = x + pend[j]
    assert rel(x, x0 + total) < 1e-13
    # the oracle's own cached step agrees with this hand run
    cache2 = orc.new_cache(4)
    orc.prefill(cache2, prompt[:-1])
    assert rel(orc.step(cache2, prompt[-1], pos), orc.logits_from_hidden(x)) < 1e-13


def test_delay_zero_is_parallel_block():
    cfg = TINY_LANES.with_(lane_delay=0)
    w = gen_weights(cfg, std=0.4, threads=1)
    lg = O.Oracle(cfg, w).forward_nocache([4, 0, 9])
    # parallel block written out: x += attn(norm_a x) + mlp(norm_m x)
    orc = O.Oracle(cfg.with_(sequential=True), w)
    x = orc.embed([4, 0, 9])
    pos = np.arange(3)
    for L in orc.layers:
        q, k, v = orc.qkv(L, O.rmsnorm(x, L.attn_norm, orc.eps), pos)
        a = orc.causal_attention(q, k, v, pos).reshape(3, -1) @ L.wo.T
        x = x + a + orc.mlp(L, O.rmsnorm(x, L.mlp_norm, orc.eps))
    assert rel(lg, orc.logits_from_hidden(x)) < 1e-13


# ----------------------------------------------------------------------------
# planted mistakes: each must be caught by at least one check above
# ----------------------------------------------------------------------------
def _all_checks():
    errs = {
        "bf": max(check_bruteforce(c) for c in (TINY, TINY_GQA, TINY_LANES)),
        "cache": max(check_cached_vs_nocache(c) for c in (TINY, TINY_GQA, TINY_LANES)),
        "rope": check_rope_closed_form(),
        "rel": check_rope_relative(),
        "rms": check_rmsnorm_closed_form(),
        "gqa": check_gqa_equals_mha(),
    }
    return errs, check_argmax_ties()


def _caught(monkeypatch, **patches):
    for name, fn in patches.items():
        if "." in name:
            cls, attr = name.split(".")
            monkeypatch.setattr(getattr(O, cls), attr, fn)
        else:
            monkeypatch.setattr(O, name, fn)
    errs, tie = _all_checks()
    return any(e > 1e-9 for e in errs.values()) or tie != 1


def _rope_variant(sign=1.0, interleaved=False):
    def f(u, positions, base):
        hd = u.shape[-1]
        half = hd // 2
        ang = O.rope_angles(positions, hd, base)
        c = np.cos(ang)[:, None, :]
        s = sign * np.sin(ang)[:, None, :]
        if interleaved:
            a, b = u[..., 0::2], u[..., 1::2]
            out = np.empty_like(u)
            out[..., 0::2] = a * c - b * s
            out[..., 1::2] = a * s + b * c
            return out
        a, b = u[..., :half], u[..., half:]
        return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)
    return f


MUTANTS = {
    "rope_direction": dict(apply_rope=_rope_variant(sign=-1.0)),
    "rope_interleaved": dict(apply_rope=_rope_variant(interleaved=True)),
    "rmsnorm_eps_outside": dict(rmsnorm=lambda x, g, eps: x / (np.sqrt(np.mean(x * x, -1, keepdims=True)) + eps) * g),
    "silu_sigmoid": dict(silu=lambda z: 1.0 / (1.0 + np.exp(-z))),
    "argmax_last": dict(greedy=lambda lg: int(len(lg) - 1 - np.argmax(lg[::-1]))),
    "attn_scale_hd": dict(attend=lambda q, K, V: O.softmax(K @ q / q.shape[-1]) @ V),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_function_mistakes_are_caught(monkeypatch, name):
    assert _caught(monkeypatch, **MUTANTS[name])


def test_planted_gqa_mapping_mistake_is_caught(monkeypatch):
    orig = O.Oracle.causal_attention

    def wrong(self, q, k, v, positions):
        G = self.G
        self.G = 1 if self.Hkv < self.H else self.G  # i % Hkv style indexing
        try:
            kk = np.concatenate([k] * (self.H // self.Hkv), axis=1) if self.Hkv < self.H else k
            vv = np.concatenate([v] * (self.H // self.Hkv), axis=1) if self.Hkv < self.H else v
            return orig(self, q, kk, vv, positions)
        finally:
            self.G = G
    assert _caught(monkeypatch, **{"Oracle.causal_attention": wrong})


def test_planted_mask_mistake_is_caught(monkeypatch):
    def wrong(self, q, k, v, positions):
        n, T = q.shape[0], k.shape[0]
        out = np.empty((n, self.H, self.hd))
        mask = np.arange(T)[None, :] >= np.asarray(positions)[:, None]
        mask[:, 0] = False
        for i in range(self.H):
            g = i // self.G
            s = np.where(mask, -np.inf, (q[:, i] @ k[:, g].T) / np.sqrt(self.hd))
            out[:, i] = O.softmax(s) @ v[:, g]
        return out
    assert _caught(monkeypatch, **{"Oracle.causal_attention": wrong})


def test_planted_mlp_mistakes_are_caught(monkeypatch):
    swapped = lambda self, L, h: (O.silu(h @ L.w_up.T) * (h @ L.w_gate.T)) @ L.w_down.T
    assert _caught(monkeypatch, **{"Oracle.mlp": swapped})
    transposed = lambda self, L, h: (O.silu(h @ L.w_gate.T) * (h @ L.w_up.T)) @ L.w_down.T * 1.0001
    assert _caught(monkeypatch, **{"Oracle.mlp": transposed})


# --------------------------------------------------------------------------
# stochastic LM-head sampling (the oracle's reading: Gumbel-max over
# Philox4x32-10 noise)
# --------------------------------------------------------------------------
# Known-answer vectors of Philox4x32 with 10 rounds as published with the
# generator (Salmon et al., "Parallel random numbers: as easy as 1, 2, 3",
# SC 2011, and its reference implementation's test vectors): counter, key,
# output words.
PHILOX_KAT = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
    ((0xffffffff, 0xffffffff, 0xffffffff, 0xffffffff), (0xffffffff, 0xffffffff),
     (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
    ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
     (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
]


@pytest.mark.parametrize("ctr,key,want", PHILOX_KAT)
def test_philox_known_answers(ctr, key, want):
    got = O.philox4x32(ctr, key)
    assert tuple(int(x) for x in got) == want


def test_philox_is_elementwise_over_counters():
    # a vector of counters gives, word for word, the scalar results
    c0 = np.array([0, 0xffffffff, 0x243f6a88], dtype=np.uint64)
    rows = [O.philox4x32((int(c), 7, 9, 11), (3, 5)) for c in c0]
    vec = O.philox4x32((c0, 7, 9, 11), (3, 5))
    for i in range(3):
        assert [int(w[i]) for w in vec] == [int(w) for w in rows[i]]


def test_uniform_is_open_and_exact():
    u = O.uniform_open(np.array([0, 0xffffffff, 1 << 31], dtype=np.uint64))
    assert u[0] == 0.5 * 2.0 ** -23 and u[1] == 1 - 0.5 * 2.0 ** -23 and u[2] == 0.5 + 0.5 * 2.0 ** -23
    assert np.all(u.astype(np.float32).astype(np.float64) == u)  # representable in float32


def test_gumbel_max_matches_softmax_chi_square():
    # the oracle's sampler over many independent draws (positions 0..N-1 of
    # one seed) follows softmax(l/T): chi-square with 5 degrees of freedom
    l = np.array([1.3, 0.2, -0.5, 2.0, 1.9, -1.0])
    T, N = 0.7, 20000
    seed = 0x1234_5678_9abc
    picks = np.array([O.sample(l, T, seed, k) for k in range(N)])
    counts = np.bincount(picks, minlength=len(l))
    p = O.softmax(l / T)
    chi2 = float(np.sum((counts - N * p) ** 2 / (N * p)))
    assert chi2 < 25.7, (chi2, counts, N * p)  # 25.7 = chi-square(5) upper 1e-4 point


def test_sampling_low_temperature_is_greedy_and_zero_is_greedy():
    rng = np.random.default_rng(5)
    for _ in range(20):
        l = rng.normal(size=50)
        assert O.sample(l, 0.0, 99, 3) == O.greedy(l)
        # Gumbel noise is bounded by ~ -log(-log(1 - 2^-24)) < 17, so a
        # temperature that scales the top-2 gap above 40 cannot flip it
        s = np.sort(l)
        T = (s[-1] - s[-2]) / 40
        assert O.sample(l, T, 99, 3) == O.greedy(l)


def test_sampling_streams_differ_by_position_and_seed():
    a = O.gumbel_noise(1, 10, 64)
    assert not np.array_equal(a, O.gumbel_noise(1, 11, 64))
    assert not np.array_equal(a, O.gumbel_noise(2, 10, 64))
    assert not np.array_equal(a, O.gumbel_noise(1 << 32 | 1, 10, 64))  # the seed's upper half counts
    assert np.array_equal(a, O.gumbel_noise(1, 10, 64))


def test_planted_gumbel_sign_mistake_is_caught(monkeypatch):
    # +log(-log(u)) instead of -log(-log(u)): the chi-square pin must fail
    def wrong(seed, pos, n):
        rows = np.arange(n, dtype=np.uint64)
        w0 = O.philox4x32((rows, np.full(n, pos, np.uint64), 0, 0), (seed & 0xFFFFFFFF, seed >> 32))[0]
        return np.log(-np.log(O.uniform_open(w0)))
    monkeypatch.setattr(O, "gumbel_noise", wrong)
    with pytest.raises(AssertionError):
        test_gumbel_max_matches_softmax_chi_square()


def test_sampling_scores_argmax_is_the_sample():
    # the scores the GPU path maximises (logits / T plus the noise) pick the
    # same token as the sampler, over many seeds, positions and temperatures
    rng = np.random.default_rng(11)
    for k in range(300):
        l = rng.normal(size=97) * rng.uniform(0.1, 3.0)
        T = float(rng.choice([0.0, 0.3, 0.8, 2.5]))
        seed = int(rng.integers(0, 2 ** 63))
        pos = int(rng.integers(0, 40000))
        sc = O.sampling_scores(l, T, seed, pos)
        assert int(np.argmax(sc)) == O.sample(l, T, seed, pos)
        if T == 0:
            assert np.array_equal(sc, l)


def test_gumbel_noise_moments():
    # standard Gumbel: mean = Euler-Mascheroni constant, variance = pi^2 / 6
    # (200,000 rows of one position; 5 standard errors of slack)
    g = O.gumbel_noise(0xfeed, 123, 200_000)
    assert abs(g.mean() - 0.5772156649) < 0.015, g.mean()
    assert abs(g.var() - math.pi ** 2 / 6) < 0.04, g.var()
    # its distribution function exp(-exp(-x)) at a few points
    for x in (-1.0, 0.0, 1.0, 3.0):
        assert abs(np.mean(g <= x) - math.exp(-math.exp(-x))) < 0.005


def test_layer1_kv_helper_matches_the_prefill_cache():
    # the GPU tests' cheap layer-1 K/V reference (attention at sampled rows
    # only) equals the cache the oracle's full prefill writes
    from paritylib import layer1_kv_reference
    cfg = CFG0.with_(n_heads=4, n_kv_heads=2, seed_index=77)
    w = gen_weights(cfg, std=0.1)
    prompt = gen_prompt(cfg, n=40)
    for kv16 in (False, True):
        orc = O.Oracle(cfg, w, kv_fp16=kv16)
        cache = orc.new_cache(40)
        orc.prefill(cache, prompt)
        pos = np.array([0, 1, 17, 39])
        k1, v1 = (orc.cache_round(a) for a in layer1_kv_reference(orc, prompt, pos))
        assert rel(k1, cache.K[1][:, pos, :].transpose(1, 0, 2)) < 1e-12
        assert rel(v1, cache.V[1][:, pos, :].transpose(1, 0, 2)) < 1e-12
