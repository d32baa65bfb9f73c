"""GPU checks of the batched (matrix-core) prefill, kie_prefill_batched.

Against the oracle on small and odd shapes, with chunks shorter than the
prompt: the prefill's logits and t1, then a teacher-forced decode from the
KV cache it wrote, to the greedy tests' bar (relative L2 <= 1e-3, the same
token where the oracle's top-2 margin exceeds 1e-2).  At the benchmark's
shape (cfg2, 2048-token prompt), where the oracle cannot follow, the batched
prefill is compared with the token-by-token prefill of the decode kernel:
every layer's K and V caches agree to relative L2 <= 1e-3 (the paths add in
different orders, and fp32 rounding differences grow through the layers),
and the last position's logits and t1 agree to the parity bar.

Every test prints its case before touching the GPU."""
import time

import numpy as np
import pytest

from decode_persistent_monokernel_amd.config import CFG0, CFG2
from decode_persistent_monokernel_amd.inputs import gen_weights, gen_prompt
from oracle import Oracle
from paritylib import REL_TOL, MARGIN, say, rel_l2, margin, compare_step

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

from decode_persistent_monokernel_amd.kie import Engine, KieError  # noqa: E402


def make_engine(cfg, max_ctx, timeout_us=2_000_000):
    e = Engine(cfg, device=0, max_ctx=max_ctx)
    e.set_timeout_us(timeout_us)
    return e


def kv_rows(eng, cfg, n_pos):
    """the cache's first n_pos positions as a float32 device tensor [L][2][Hkv][n_pos][hd]"""
    n = cfg.n_layers * 2 * cfg.n_kv_heads * eng.max_ctx * cfg.head_dim  # the buffer may end in padding
    a = eng.d_kv.view(torch.float16)[:n].view(cfg.n_layers, 2, cfg.n_kv_heads, eng.max_ctx, cfg.head_dim)
    return a[:, :, :, :n_pos].float()


def check_against_oracle(cfg, w, prompt, chunk, n_steps, kv_fp16):
    ref = Oracle(cfg, w, kv_fp16=kv_fp16).run(prompt, n_steps)
    eng = make_engine(cfg, len(prompt) + n_steps)
    eng.load_weights(w)
    t1, lg0 = eng.prefill_batched(prompt, want_logits=True, chunk=chunk)
    assert eng.position == len(prompt)
    worst = rel_l2(lg0, ref["prefill_logits"])
    assert margin(ref["prefill_logits"]) <= MARGIN or t1 == ref["t1"]
    toks, lgs = eng.decode(n_steps, forced=ref["inputs"], want_logits=True)
    bad = 0
    for k in range(n_steps):
        r, tok_ok, self_ok, _ = compare_step(ref["logits"][k], lgs[k], toks[k])
        worst = max(worst, r)
        bad += (not tok_ok) + (not self_ok)
    say(f"  worst rel-L2 {worst:.3e}, token mismatches {bad}")
    assert worst <= REL_TOL
    assert bad == 0
    eng.close()


@pytest.mark.parametrize("chunk", [1, 5, 64])
def test_cfg0_batched_prefill(chunk):
    cfg = CFG0.with_(seed_index=31, prompt_len=33, decode_steps=8)
    say(f"case batched prefill cfg0 P=33 chunk={chunk}")
    check_against_oracle(cfg, gen_weights(cfg), gen_prompt(cfg), chunk, cfg.decode_steps, kv_fp16=False)


@pytest.mark.parametrize("shape", [
    dict(n_heads=8, n_kv_heads=2, head_dim=32, name="gqa4"),
    dict(d_model=320, n_heads=4, n_kv_heads=4, head_dim=80, ffn_dim=864, name="hd80"),
    dict(d_model=864, n_heads=4, n_kv_heads=2, head_dim=64, ffn_dim=1000, vocab=3000, name="straddle"),
    dict(d_model=1024, n_heads=4, n_kv_heads=4, head_dim=256, ffn_dim=2048, vocab=1000, name="hd256"),
], ids=lambda s: s["name"])
def test_small_shapes_batched_prefill(shape):
    # 150 tokens: GEMM tiles of 64 rows with a ragged last tile, sharp attention
    cfg = CFG0.with_(seed_index=32, prompt_len=150, decode_steps=6, **shape)
    say(f"case batched prefill small shape {shape['name']} P=150 chunk=100")
    w = gen_weights(cfg, overrides={"wq": 0.1, "wk": 0.1})
    check_against_oracle(cfg, w, gen_prompt(cfg), 100, cfg.decode_steps, kv_fp16=True)


@pytest.mark.parametrize("chunk", [4, 64])
def test_lane_block_batched_prefill(chunk):
    # the parallel block with its residual delayed by 2 layers (5 layers, 2 lanes)
    cfg = CFG0.with_(name="lanes", n_layers=5, n_lanes=2, lane_delay=2, sequential=False, seed_index=33,
                     prompt_len=40, decode_steps=6)
    say(f"case batched prefill on the lane block, delay 2, chunk={chunk}")
    check_against_oracle(cfg, gen_weights(cfg), gen_prompt(cfg), chunk, cfg.decode_steps, kv_fp16=False)


def test_bad_token_in_batched_part_is_reported():
    cfg = CFG0.with_(seed_index=34, prompt_len=10, decode_steps=1)
    say("case batched prefill with an out-of-range id")
    eng = make_engine(cfg, 16)
    eng.load_weights(gen_weights(cfg))
    prompt = list(gen_prompt(cfg))
    prompt[3] = cfg.vocab + 7
    with pytest.raises(KieError) as ei:
        eng.prefill_batched(prompt, chunk=4)
    assert ei.value.status == -7
    eng.close()


def test_activation_beyond_fp16_range_is_reported():
    """RMSNorm gains of 30000 push the largest normalised activations (about
    three times the RMS) past 65504, which the batched prefill's fp16 split cannot
    carry: it latches KIE_ERR_RANGE instead of writing non-finite keys and
    values.  The token-by-token path keeps fp32 activations and stays
    finite on the same weights."""
    cfg = CFG0.with_(seed_index=35, prompt_len=10, decode_steps=1)
    say("case batched prefill with activations beyond the fp16 range")
    w = gen_weights(cfg)
    w["layers.0.attn_norm"] = np.full(cfg.d_model, 30000.0, dtype=np.float16)
    prompt = gen_prompt(cfg)
    eng = make_engine(cfg, 16)
    eng.load_weights(w)
    with pytest.raises(KieError) as ei:
        eng.prefill_batched(prompt, chunk=4)
    assert ei.value.status == -8  # KIE_ERR_RANGE
    eng.close()
    eng = make_engine(cfg, 16)
    eng.load_weights(w)
    _, lg = eng.prefill(prompt, want_logits=True)
    assert np.isfinite(lg).all()
    eng.close()


def test_cfg2_batched_equals_token_by_token_prefill():
    cfg = CFG2
    P = cfg.prompt_len
    say(f"case cfg2 batched vs token-by-token prefill, P={P}")
    w = gen_weights(cfg)
    prompt = gen_prompt(cfg)
    a = make_engine(cfg, P + 8, 5_000_000)
    a.load_weights(w)
    t0 = time.time()
    ta, la = a.prefill_batched(prompt, want_logits=True)
    tb_s = time.time() - t0
    kva = kv_rows(a, cfg, P)
    b = make_engine(cfg, P + 8, 5_000_000)
    b.load_weights(w)
    t0 = time.time()
    tb, lb = b.prefill(prompt, want_logits=True)
    tt_s = time.time() - t0
    kvb = kv_rows(b, cfg, P)
    say(f"  batched {tb_s:.3f} s, token by token {tt_s:.3f} s")
    r = rel_l2(la, lb)
    # per layer and K/V: relative L2 of the difference, and the share of
    # entries more than two binary16 ulps apart
    diff = (kva - kvb).double()
    num = diff.pow(2).sum(dim=(2, 3, 4)).sqrt()
    den = kvb.double().pow(2).sum(dim=(2, 3, 4)).sqrt()
    layer_rel = (num / den).cpu().numpy()
    far = ((kva - kvb).abs() > 2 * kvb.abs() * 2.0 ** -10).float().mean().item()
    say(f"  logits rel-L2 {r:.3e}, t1 {ta}/{tb}; KV rel-L2 per layer max {layer_rel.max():.3e} "
        f"(layer 0 {layer_rel[0].max():.3e}, last {layer_rel[-1].max():.3e}); entries > 2 ulp apart {far:.2%}")
    assert r <= REL_TOL
    assert margin(lb) <= MARGIN or ta == tb
    assert layer_rel.max() <= REL_TOL
    a.close()
    b.close()
