"""kie_prefill_batched_noalloc (the batched prefill on the library's own fixed
scratch, for callers that cannot allocate) against kie_prefill_batched with
a caller scratch buffer: two calls in a row, the second with a shorter
prompt, each compared on t1, the last position's logits and the KV cache of
every layer, to the parity bar (relative L2 <= 1e-3, the same t1 where the
top-2 margin exceeds 1e-2).  The fixed scratch holds 590 tokens of this
shape, so both prompts run in several chunks there and in one chunk with the
caller's buffer."""
import numpy as np
import pytest

from decode_persistent_monokernel_amd.config import CFG2
from decode_persistent_monokernel_amd.inputs import gen_weights, gen_prompt
from paritylib import REL_TOL, MARGIN, say, rel_l2, margin

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

from decode_persistent_monokernel_amd.kie import Engine  # noqa: E402


def kv_prefix(eng, cfg, n):
    n_all = cfg.n_layers * 2 * cfg.n_kv_heads * eng.max_ctx * cfg.head_dim
    a = eng.d_kv.view(torch.float16)[:n_all].view(cfg.n_layers, 2, cfg.n_kv_heads, eng.max_ctx, cfg.head_dim)
    return a[:, :, :, :n].float().cpu().numpy()


def test_noalloc_prefill_matches_caller_scratch_twice():
    cfg = CFG2.with_(name="cfg2-2L", n_layers=2, seed_index=61)
    w = gen_weights(cfg)
    prompt = gen_prompt(cfg, n=1500)
    eng = Engine(cfg, device=0, max_ctx=1600)
    eng.set_timeout_us(5_000_000)
    eng.load_weights(w)
    for n in (1500, 700):
        say(f"case no-allocation batched prefill, cfg2 shape with 2 layers, prompt {n}")
        p = prompt[:n]
        eng.set_position(0, 0)
        t_ref, lg_ref = eng.prefill_batched(p, want_logits=True, chunk=2048)
        kv_ref = kv_prefix(eng, cfg, n)
        eng.set_position(0, 0)
        t_na, lg_na = eng.prefill_batched_noalloc(p, want_logits=True)
        assert eng.position == n
        kv_na = kv_prefix(eng, cfg, n)
        r_lg, r_kv = rel_l2(lg_na, lg_ref), rel_l2(kv_na, kv_ref)
        bitwise = np.array_equal(lg_na.view(np.uint32), lg_ref.view(np.uint32))
        say(f"  logits rel-L2 {r_lg:.2e} (bitwise {bitwise}), KV rel-L2 {r_kv:.2e}, t1 {t_na}/{t_ref}")
        assert r_lg <= REL_TOL and r_kv <= REL_TOL
        assert margin(lg_ref) <= MARGIN or t_na == t_ref
        # decoding goes on from the state the no-allocation prefill left
        toks = eng.decode(3)
        assert toks.shape == (3,) and eng.position == n + 3
    eng.close()
