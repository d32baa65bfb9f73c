"""GPU parity of the HIP decode path against the fp64 oracle (through the C ABI).

Every test prints its case before touching the GPU.  Each model here is small
enough for the oracle to follow every step; the large configurations are in
test_gpu_large.py."""
import numpy as np
import pytest

from decode_persistent_monokernel_amd.config import CFG0
from decode_persistent_monokernel_amd.inputs import gen_weights, gen_prompt
from oracle import Oracle
from paritylib import REL_TOL, say, teacher_forced, rel_l2

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

from decode_persistent_monokernel_amd.kie import Engine, KieError  # noqa: E402


def make_engine(cfg, max_ctx):
    e = Engine(cfg, device=0, max_ctx=max_ctx)
    e.set_timeout_us(2_000_000)
    return e


def check(rep, name):
    say(f"[{name}] worst rel-L2 {rep['worst_rel']:.3e}  token mismatches(margin>1e-2) {rep['bad_tokens']}"
        f"  self-argmax mismatches {rep['bad_self']}  t1 {rep['t1']}/{rep['ref_t1']}")
    assert rep["worst_rel"] <= REL_TOL
    assert rep["bad_tokens"] == 0
    assert rep["bad_self"] == 0


def test_cfg0_teacher_forced():
    cfg = CFG0
    say(f"case cfg0 full: P={cfg.prompt_len} N={cfg.decode_steps}")
    w = gen_weights(cfg)
    rep, eng = teacher_forced(cfg, w, gen_prompt(cfg), cfg.decode_steps, make_engine, Oracle)
    check(rep, "cfg0")
    eng.close()


def oracle_fp16_cache(cfg, w):
    """the oracle with K/V rounded to binary16 in the cache (the cache of an
    FP16 model); used where sharp attention would let the fp16 rounding of
    the cached keys alone exceed the bar against the fp64-cache oracle"""
    return Oracle(cfg, w, kv_fp16=True)


def test_cfg0_peaky_attention():
    """Wq, Wk with std 0.2 make the softmax sharp, so a misplaced key moves the
    logits (at std 0.02 attention is nearly uniform and hides such bugs)"""
    cfg = CFG0.with_(seed_index=10)
    say("case cfg0 peaky attention (wq, wk std 0.2)")
    w = gen_weights(cfg, overrides={"wq": 0.2, "wk": 0.2})
    rep, eng = teacher_forced(cfg, w, gen_prompt(cfg), cfg.decode_steps, make_engine, oracle_fp16_cache)
    check(rep, "cfg0-peaky")
    eng.close()


@pytest.mark.parametrize("hd,H,d", [(64, 4, 256), (80, 4, 320), (128, 2, 256), (32, 8, 256)])
def test_many_keys_per_wave(hd, H, d):
    """a 2.5K-token context spreads 4..20 keys over every wave, so every key
    slot of the split-context attention and its merges are exercised"""
    cfg = CFG0.with_(seed_index=17, d_model=d, n_heads=H, n_kv_heads=H, head_dim=hd, prompt_len=2500,
                     decode_steps=4, vocab=2048)
    say(f"case long context hd={hd} H={H} P=2500")
    w = gen_weights(cfg, overrides={"wq": 0.12, "wk": 0.12})
    rep, eng = teacher_forced(cfg, w, gen_prompt(cfg), cfg.decode_steps, make_engine, oracle_fp16_cache)
    check(rep, f"long-hd{hd}")
    eng.close()


@pytest.mark.parametrize("shape", [
    dict(n_heads=8, n_kv_heads=2, head_dim=32, name="gqa4"),
    dict(n_heads=8, n_kv_heads=4, head_dim=32, name="gqa2"),
    dict(d_model=320, n_heads=4, n_kv_heads=4, head_dim=80, ffn_dim=864, name="hd80"),
    dict(d_model=384, n_heads=6, n_kv_heads=6, head_dim=64, ffn_dim=1536, vocab=1000, name="ragged"),
    # rows of 864 and 1000 columns: 1-KB chunks straddle row ends in the
    # middle of a wave's range in every GEMV (several rows per workgroup)
    dict(d_model=864, n_heads=4, n_kv_heads=2, head_dim=64, ffn_dim=1000, vocab=3000, name="straddle"),
], ids=lambda s: s["name"])
def test_small_shapes_teacher_forced(shape):
    cfg = CFG0.with_(seed_index=11, prompt_len=9, decode_steps=12, **shape)
    say(f"case small shape {shape}")
    w = gen_weights(cfg, overrides={"wq": 0.1, "wk": 0.1})
    rep, eng = teacher_forced(cfg, w, gen_prompt(cfg), cfg.decode_steps, make_engine, oracle_fp16_cache)
    check(rep, shape["name"])
    eng.close()


@pytest.mark.parametrize("shape", [
    # delay 2: the pipelined phase order (attention ahead of the next layer's QKV and gate/up)
    dict(name="lanes-d2", n_layers=5, lane_delay=2, seed_index=12),
    # delay 3 with two query heads per KV head: pipelined, GQA attention
    dict(name="lanes-d3-gqa2", n_layers=6, lane_delay=3, n_kv_heads=2, seed_index=31),
    # no delay: layer by layer, every QKV polls the x the down projection before it wrote
    dict(name="lanes-d0", n_layers=4, lane_delay=0, seed_index=32),
], ids=lambda s: s["name"])
def test_lane_block_small(shape):
    cfg = CFG0.with_(n_lanes=2, sequential=False, prompt_len=7, decode_steps=10, **shape)
    say(f"case parallel block {shape}")
    w = gen_weights(cfg, overrides={"wq": 0.1, "wk": 0.1})
    rep, eng = teacher_forced(cfg, w, gen_prompt(cfg), cfg.decode_steps, make_engine, oracle_fp16_cache)
    check(rep, shape["name"])
    eng.close()


def test_lane_block_wide_ffn():
    """the parallel block when its O prologue cannot stage the down
    projection's input and the next layer's gains (a 12288-wide FFN leaves no
    LDS for them): the down, QKV and gate/up prologues fetch their own"""
    cfg = CFG0.with_(name="lanes-wide", n_layers=4, n_lanes=2, lane_delay=1, sequential=False, ffn_dim=12288,
                     seed_index=14, prompt_len=9, decode_steps=8)
    say("case parallel block, delay 1, FFN 12288 (no staging in the O prologue)")
    w = gen_weights(cfg, overrides={"wq": 0.1, "wk": 0.1})
    rep, eng = teacher_forced(cfg, w, gen_prompt(cfg), cfg.decode_steps, make_engine, oracle_fp16_cache)
    check(rep, "lanes-wide")
    eng.close()


def test_single_token_prompt_and_free_running():
    cfg = CFG0.with_(seed_index=13, prompt_len=1, decode_steps=20)
    say("case prompt of one token, free-running greedy")
    w = gen_weights(cfg)
    prompt = gen_prompt(cfg)
    ref = Oracle(cfg, w).run(prompt, cfg.decode_steps)
    eng = make_engine(cfg, cfg.max_ctx)
    eng.load_weights(w)
    t1 = eng.prefill(prompt)
    toks, lgs = eng.decode(cfg.decode_steps, want_logits=True)
    # free running: agree while every oracle step is decisive
    for k in range(cfg.decode_steps):
        lg = ref["logits"][k]
        top = np.sort(lg)[-2:]
        if top[1] - top[0] <= 1e-2:
            break
        assert toks[k] == ref["tokens"][k], k
        assert rel_l2(lgs[k], lg) <= REL_TOL
    assert t1 == ref["t1"]
    eng.close()


def test_deterministic_and_resumable():
    """bitwise-identical logits on a repeat, and decode(a) + decode(b) == decode(a + b)"""
    cfg = CFG0.with_(seed_index=14, prompt_len=11, decode_steps=24)
    say("case determinism / resume")
    w = gen_weights(cfg)
    prompt = gen_prompt(cfg)
    eng = make_engine(cfg, cfg.max_ctx)
    eng.load_weights(w)
    t1 = eng.prefill(prompt)
    a_tok, a_lg = eng.decode(24, want_logits=True)
    eng.set_position(len(prompt), t1)
    b_tok, b_lg = eng.decode(24, want_logits=True)
    assert np.array_equal(a_tok, b_tok) and np.array_equal(a_lg.view(np.uint32), b_lg.view(np.uint32))
    eng.set_position(len(prompt), t1)
    c1, l1 = eng.decode(9, want_logits=True)
    c2, l2 = eng.decode(15, want_logits=True)
    assert np.array_equal(np.concatenate([c1, c2]), a_tok)
    assert np.array_equal(np.concatenate([l1, l2]).view(np.uint32), a_lg.view(np.uint32))
    # launches split into short chunks give the same bits
    eng.set_position(len(prompt), t1)
    eng.set_launch_steps(5)
    d_tok, d_lg = eng.decode(24, want_logits=True)
    assert np.array_equal(d_lg.view(np.uint32), a_lg.view(np.uint32))
    eng.close()


@pytest.mark.parametrize("shape", [
    dict(name="mha", seed_index=17),
    dict(name="gqa4", n_heads=8, n_kv_heads=2, head_dim=32, seed_index=18),
    dict(name="lanes", n_layers=5, n_lanes=2, lane_delay=2, sequential=False, seed_index=19),
    dict(name="lanes-d3-gqa2", n_layers=6, n_lanes=2, lane_delay=3, n_kv_heads=2, sequential=False, seed_index=33),
    dict(name="lanes-d0", n_layers=4, n_lanes=2, lane_delay=0, sequential=False, seed_index=34),
], ids=lambda s: s["name"])
def test_jitter_keeps_results_bitwise(shape):
    """race detection: with every wave sleeping a pseudo-random time at every
    phase start (a different pattern in every launch), the logits of a
    teacher-forced decode stay bitwise identical to an undisturbed run; the
    first differing repeat fails"""
    cfg = CFG0.with_(prompt_len=9, decode_steps=12, **shape)
    say(f"case jitter bitwise repeat ({shape['name']})")
    w = gen_weights(cfg, overrides={"wq": 0.1, "wk": 0.1})
    prompt = gen_prompt(cfg)
    eng = make_engine(cfg, cfg.max_ctx)
    eng.load_weights(w)
    t1 = eng.prefill(prompt)
    forced = list(np.random.default_rng(3).integers(0, cfg.vocab, cfg.decode_steps))
    a_tok, a_lg = eng.decode(cfg.decode_steps, forced=forced, want_logits=True)
    eng.set_debug_flags(2)
    for rep in range(4):
        eng.set_position(len(prompt), t1)
        eng.set_launch_steps(cfg.decode_steps if rep % 2 == 0 else 5)
        b_tok, b_lg = eng.decode(cfg.decode_steps, forced=forced, want_logits=True)
        assert np.array_equal(a_lg.view(np.uint32), b_lg.view(np.uint32)), f"repeat {rep} differs"
        assert np.array_equal(a_tok, b_tok)
    eng.set_debug_flags(0)
    eng.close()


def random_shapes(n=12, seed=2024):
    """n model shapes drawn from a fixed seed: 1-3 layers, d_model 128..1024
    in steps of 8 (not only multiples of 64), head_dim 32..128 in steps of 8,
    1, 2 or 4 query heads per KV head, FFN widths and vocabularies that are
    not multiples of 256, the sequential block and the lane block with delay
    0..3, prompts of 1..40 tokens; shapes the host does not run are redrawn"""
    from decode_persistent_monokernel_amd import kie
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        G = (1, 2, 4)[len(out) % 3]
        hkv = int(rng.integers(1, 5))
        par = bool(rng.integers(0, 2))
        cfg = CFG0.with_(
            name=f"rand{len(out)}", n_layers=int(rng.integers(1, 4)), d_model=8 * int(rng.integers(16, 129)),
            n_heads=G * hkv, n_kv_heads=hkv, head_dim=8 * int(rng.integers(4, 17)),
            ffn_dim=8 * int(rng.integers(16, 385)), vocab=2 * int(rng.integers(250, 2501)),
            sequential=not par, n_lanes=1, lane_delay=int(rng.integers(0, 4)) if par else 0,
            prompt_len=int(rng.integers(1, 41)), decode_steps=6, seed_index=100 + len(out))
        try:
            kie.validate_schedule(cfg, 256, cfg.prompt_len + cfg.decode_steps + 1)
        except kie.KieError:
            continue
        out.append(cfg)
    return out


@pytest.mark.parametrize("cfg", random_shapes(), ids=lambda c: c.name)
def test_random_shapes_teacher_forced(cfg):
    say(f"case random shape {cfg.name}: L{cfg.n_layers} d{cfg.d_model} H{cfg.n_heads}/{cfg.n_kv_heads}x"
        f"{cfg.head_dim} F{cfg.ffn_dim} V{cfg.vocab} {'seq' if cfg.sequential else f'lanes d{cfg.lane_delay}'} "
        f"P{cfg.prompt_len}")
    w = gen_weights(cfg, overrides={"wq": 0.1, "wk": 0.1})
    rep, eng = teacher_forced(cfg, w, gen_prompt(cfg), cfg.decode_steps, make_engine, oracle_fp16_cache)
    check(rep, cfg.name)
    eng.close()


def test_bounded_wait_reports_timeout():
    """a workgroup waits on a word nobody writes: the launch must end with
    KIE_ERR_TIMEOUT, not hang, and the context must work again afterwards"""
    cfg = CFG0.with_(seed_index=15, prompt_len=4, decode_steps=4)
    say("case forced timeout (bounded wait)")
    w = gen_weights(cfg)
    eng = make_engine(cfg, cfg.max_ctx)
    eng.load_weights(w)
    t1 = eng.prefill(gen_prompt(cfg))
    eng.set_timeout_us(20_000)
    eng.set_debug_flags(1)
    with pytest.raises(KieError) as ei:
        eng.decode(2)
    assert ei.value.status == -5
    eng.set_debug_flags(0)
    eng.set_timeout_us(2_000_000)
    eng.set_position(cfg.prompt_len, t1)
    toks = eng.decode(2)
    assert toks.shape == (2,)
    eng.close()


def test_capacity_and_bad_token_errors():
    cfg = CFG0.with_(seed_index=16, prompt_len=4, decode_steps=4)
    say("case capacity / bad token")
    eng = make_engine(cfg, cfg.max_ctx)
    eng.load_weights(gen_weights(cfg))
    eng.prefill(gen_prompt(cfg))
    with pytest.raises(KieError) as ei:
        eng.decode(cfg.max_ctx)
    assert ei.value.status == -3
    with pytest.raises(KieError) as ei:
        eng.decode(1, forced=[cfg.vocab + 5])
    assert ei.value.status == -7
    eng.close()
