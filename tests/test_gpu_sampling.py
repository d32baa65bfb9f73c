"""GPU checks of in-kernel stochastic LM-head sampling (kie_set_sampling)
against the oracle's sampler (Gumbel-max over Philox4x32-10 noise).

Bar: logits as in the greedy tests (relative L2 <= 1e-3; they are not
perturbed), and at every step the token equals the argmax of the oracle's
perturbed scores logits / T + g wherever their top-1 / top-2 margin exceeds
1e-2 / T (the logits' own tolerance carried through the 1/T scaling).  The
kernel's token must also be the argmax of its own logits / T plus the same
noise, recomputed on the host, wherever that margin exceeds 1e-4.  The
sampled distribution at one fixed state is checked by a chi-square test over
many seeds."""
import numpy as np
import pytest

from decode_persistent_monokernel_amd.config import CFG0
from decode_persistent_monokernel_amd.inputs import gen_weights, gen_prompt
from oracle import Oracle
import oracle.oracle as O
from paritylib import REL_TOL, MARGIN, say, rel_l2, margin

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

from decode_persistent_monokernel_amd.kie import Engine  # noqa: E402


def make_engine(cfg, max_ctx):
    e = Engine(cfg, device=0, max_ctx=max_ctx)
    e.set_timeout_us(2_000_000)
    return e


@pytest.mark.parametrize("T,seed", [(0.8, 12345), (2.5, 2**63 + 77)])
def test_sampled_decode_matches_oracle(T, seed):
    cfg = CFG0.with_(seed_index=21, prompt_len=9, decode_steps=40)
    say(f"case sampled decode cfg0 T={T} seed={seed}")
    w = gen_weights(cfg)
    prompt = gen_prompt(cfg)
    ref = Oracle(cfg, w).run(prompt, cfg.decode_steps, temperature=T, seed=seed)
    P = len(prompt)
    eng = make_engine(cfg, P + cfg.decode_steps)
    eng.load_weights(w)
    eng.set_sampling(T, seed)
    t1, lg0 = eng.prefill(prompt, want_logits=True)
    # teacher forcing with the oracle's own sampled inputs keeps both on one path
    toks, lgs = eng.decode(cfg.decode_steps, forced=ref["inputs"], want_logits=True)
    steps = [(P - 1, ref["prefill_logits"], lg0, t1, ref["t1"])]
    steps += [(P + k, ref["logits"][k], lgs[k], toks[k], ref["tokens"][k]) for k in range(cfg.decode_steps)]
    worst, decided, distinct = 0.0, 0, set()
    for pos, rl, gl, gt, rt in steps:
        worst = max(worst, rel_l2(gl, rl))
        z = O.sampling_scores(rl, T, seed, pos)
        assert rt == int(np.argmax(z))
        if margin(z) > MARGIN / T:
            decided += 1
            assert int(gt) == rt, (pos, int(gt), rt)
        zg = np.asarray(gl, dtype=np.float64) / T + O.gumbel_noise(seed, pos, cfg.vocab)
        if margin(zg) > 1e-4:
            assert int(gt) == int(np.argmax(zg)), pos
        distinct.add(int(gt))
    say(f"  worst rel-L2 {worst:.3e}, decided steps {decided}/{len(steps)}, distinct tokens {len(distinct)}")
    assert worst <= REL_TOL
    assert decided >= len(steps) // 2
    eng.close()


def test_sampling_off_is_greedy_again():
    cfg = CFG0.with_(seed_index=22, prompt_len=5, decode_steps=12)
    say("case sampling switched on, then off")
    w = gen_weights(cfg)
    prompt = gen_prompt(cfg)
    eng = make_engine(cfg, len(prompt) + cfg.decode_steps)
    eng.load_weights(w)
    t_greedy = eng.prefill(prompt)
    a = eng.decode(cfg.decode_steps)
    eng.set_position(0, 0)
    eng.set_sampling(1.0, 9)
    eng.prefill(prompt)
    eng.set_sampling(0.0, 9)
    eng.set_position(len(prompt), t_greedy)
    b = eng.decode(cfg.decode_steps)
    assert list(a) == list(b)
    eng.close()


def _temperature_for_top(lg, target):
    """a temperature at which softmax(lg / T) has its largest probability ~target"""
    lo, hi = 1e-3, 1e3
    for _ in range(60):
        mid = np.sqrt(lo * hi)
        if O.softmax(lg / mid).max() > target:
            lo = mid
        else:
            hi = mid
    return float(np.sqrt(lo * hi))


def test_sampler_frequencies_chi_square():
    cfg = CFG0.with_(seed_index=23, prompt_len=7, decode_steps=1)
    say("case chi-square of the kernel's sampler at one state, 1500 seeds")
    w = gen_weights(cfg)
    prompt = gen_prompt(cfg)
    P = len(prompt)
    eng = make_engine(cfg, P + 1)
    eng.load_weights(w)
    t1 = eng.prefill(prompt)
    _, lg = eng.decode(1, want_logits=True)
    lg = np.asarray(lg[0], dtype=np.float64)
    T = _temperature_for_top(lg, 0.25)
    p = O.softmax(lg / T)
    N = 1500
    counts = np.zeros(cfg.vocab, dtype=np.int64)
    d_out = torch.empty(N, dtype=torch.int32, device=eng.dev)
    for s in range(N):
        eng.set_sampling(T, 1000 + s)
        eng.set_position(P, t1)
        eng.decode_device(1, d_out[s:s + 1])
    eng.sync()
    for t in d_out.cpu().numpy():
        counts[int(t)] += 1
    big = p * N >= 8
    obs = np.append(counts[big], counts[~big].sum())
    exp = np.append(p[big] * N, p[~big].sum() * N)
    keep = exp > 0
    chi2 = float(np.sum((obs[keep] - exp[keep]) ** 2 / exp[keep]))
    dof = int(keep.sum()) - 1
    # upper 1e-4 point of chi-square(dof) by the Wilson-Hilferty approximation
    z = 3.719
    crit = dof * (1 - 2 / (9 * dof) + z * np.sqrt(2 / (9 * dof))) ** 3
    say(f"  T={T:.4f} bins {len(obs)} chi2 {chi2:.1f} (critical {crit:.1f})")
    assert dof >= 2
    assert chi2 < crit
    eng.close()
