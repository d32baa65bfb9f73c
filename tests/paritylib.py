"""Shared helpers of the GPU parity tests: run the oracle and the HIP path on
the same seeded inputs and compare them step by step.

Bar (per decode step and for the prefill's last position): relative L2 error
of the logits <= 1e-3, and the same greedy token wherever the oracle's
top-1 / top-2 margin exceeds 1e-2 (where it does not, both tokens are
correct answers to the fp16 problem)."""
from __future__ import annotations

import sys
import time

import numpy as np

REL_TOL = 1e-3
MARGIN = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def margin(lg) -> float:
    top = np.partition(np.asarray(lg, dtype=np.float64), -2)[-2:]
    return float(top[1] - top[0])


def compare_step(ref_logits, gpu_logits, gpu_token):
    r = rel_l2(gpu_logits, ref_logits)
    m = margin(ref_logits)
    ref_tok = int(np.argmax(ref_logits))
    tok_ok = (m <= MARGIN) or (int(gpu_token) == ref_tok)
    # the GPU's own token must be the argmax of the logits it returned
    self_ok = int(gpu_token) == int(np.argmax(gpu_logits))
    return r, tok_ok, self_ok, m


def teacher_forced(cfg, weights, prompt, n_steps, engine_factory, oracle_factory, ref=None,
                   prefill="tokens", chunk=2048):
    """returns (report dict, engine) -- engine left open for further checks.
    prefill: "tokens" (kie_prefill, the decode kernel token by token) or
    "batched" (kie_prefill_batched in chunks of `chunk` tokens)"""
    t0 = time.time()
    if ref is None:
        ref = oracle_factory(cfg, weights).run(prompt, n_steps)
    t_or = time.time() - t0
    eng = engine_factory(cfg, len(prompt) + n_steps)
    eng.load_weights(weights)
    if prefill == "batched":
        t1, lg0 = eng.prefill_batched(prompt, want_logits=True, chunk=chunk)
    else:
        t1, lg0 = eng.prefill(prompt, want_logits=True)
    toks, lgs = eng.decode(n_steps, forced=ref["inputs"], want_logits=True)
    worst = rel_l2(lg0, ref["prefill_logits"])
    bad_tok = 0 if (margin(ref["prefill_logits"]) <= MARGIN or t1 == ref["t1"]) else 1
    bad_self = 0
    for k in range(n_steps):
        r, tok_ok, self_ok, _ = compare_step(ref["logits"][k], lgs[k], toks[k])
        worst = max(worst, r)
        bad_tok += 0 if tok_ok else 1
        bad_self += 0 if self_ok else 1
    rep = dict(worst_rel=worst, bad_tokens=bad_tok, bad_self=bad_self, n=n_steps, oracle_s=t_or,
               t1=t1, ref_t1=ref["t1"], toks=toks, logits=lgs, ref=ref)
    return rep, eng


def layer1_kv_reference(orc, tokens, positions):
    """K and V of layer 1 at prompt positions `positions`, from the oracle's
    own pieces (sequential pre-norm block): layer 0's keys and values for
    every position up to the largest one (rounded as the oracle's cache
    rounds them), layer 0's attention, O projection and MLP only at the rows
    asked for, then layer 1's QKV and RoPE there.  Returns (k, v), each
    [n, Hkv, hd], before the cache's own rounding (apply orc.cache_round to
    get the cached values).  Cheap where the whole prefill is not: attention
    runs for the sampled rows only."""
    from oracle.oracle import rmsnorm
    tokens = np.asarray(tokens)
    positions = np.asarray(positions)
    T = int(positions.max()) + 1
    L0, L1 = orc.layers[0], orc.layers[1]
    x0 = orc.embed(tokens[:T])
    h0 = rmsnorm(x0, L0.attn_norm, orc.eps)
    _, k0, v0 = orc.qkv(L0, h0, np.arange(T))
    k0, v0 = orc.cache_round(k0), orc.cache_round(v0)
    q0, _, _ = orc.qkv(L0, h0[positions], positions)
    o = orc.causal_attention(q0, k0, v0, positions).reshape(len(positions), -1)
    x1 = x0[positions] + o @ L0.wo.T
    x2 = x1 + orc.mlp(L0, rmsnorm(x1, L0.mlp_norm, orc.eps))
    h1 = rmsnorm(x2, L1.attn_norm, orc.eps)
    _, k1, v1 = orc.qkv(L1, h1, positions)
    return k1, v1
