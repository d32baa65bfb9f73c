"""How much layer 1's keys and values move when layer 0's keys and values
are computed in fp32 instead of fp64 before the fp16 cache rounds them.

TEST INFRASTRUCTURE ONLY (calls nothing but the oracle and the seeded input
generator).  The pages state FP16 decoding (Kog explainers, results table
"Laneformer 2B"): K and V are rounded to binary16 as they enter the cache.
An implementation that computes them in fp32 (a dot product over d terms,
relative error about 2^-24 * sqrt(d), ~4e-6 at d = 4096) rounds a fraction
of them to the other binary16 neighbour than the fp64 oracle does.  Those
one-ulp differences in layer 0's cache reach layer 1 through attention, O
projection and MLP, and some positions (where a few keys dominate the
softmax) amplify them.  This script perturbs the oracle's own layer-0 K and
V by relative Gaussian noise of that size before the rounding, recomputes
layer 1's K and V (before their own rounding) at every position, and records
the largest changes: the spread within which any fp32 implementation's
layer-1 cache must be accepted.

    python oracle/layer1_sensitivity.py --write tests/golden/layer1_sensitivity.json
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle.oracle import Oracle, rmsnorm  # noqa: E402


def sensitivity(cfg_name: str, layers: int, prompt: int, sigma: float, seeds) -> dict:
    from decode_persistent_monokernel_amd.config import preset
    from decode_persistent_monokernel_amd.inputs import gen_weights, gen_prompt
    cfg = preset(cfg_name).with_(name=f"{cfg_name}-{layers}L", n_layers=layers)
    w = gen_weights(cfg)
    tokens = gen_prompt(cfg, n=preset(cfg_name).prompt_len)[:prompt]
    orc = Oracle(cfg, w, kv_fp16=True)
    P = len(tokens)
    pos = np.arange(P)
    L0, L1 = orc.layers[0], orc.layers[1]
    x0 = orc.embed(tokens)
    h0 = rmsnorm(x0, L0.attn_norm, orc.eps)
    q0, k0, v0 = orc.qkv(L0, h0, pos)

    def layer1(k, v):
        k, v = orc.cache_round(k), orc.cache_round(v)
        o = orc.causal_attention(q0, k, v, pos).reshape(P, -1)
        x1 = x0 + o @ L0.wo.T
        x2 = x1 + orc.mlp(L0, rmsnorm(x1, L0.mlp_norm, orc.eps))
        _, k1, v1 = orc.qkv(L1, rmsnorm(x2, L1.attn_norm, orc.eps), pos)
        return k1, v1

    k1, v1 = layer1(k0, v0)
    rms = float(np.sqrt(np.mean(np.concatenate([k1.ravel(), v1.ravel()]) ** 2)))
    runs = []
    for seed in seeds:
        rng = np.random.default_rng(seed)
        kp = k0 * (1 + sigma * rng.standard_normal(k0.shape))
        vp = v0 * (1 + sigma * rng.standard_normal(v0.shape))
        flips = float(np.mean(np.concatenate([(orc.cache_round(kp) != orc.cache_round(k0)).ravel(),
                                              (orc.cache_round(vp) != orc.cache_round(v0)).ravel()])))
        k1p, v1p = layer1(kp, vp)
        elem = max(float(np.abs(k1p - k1).max()), float(np.abs(v1p - v1).max()))
        per_pos = np.maximum(np.linalg.norm((k1p - k1).reshape(P, -1), axis=1) / np.linalg.norm(k1.reshape(P, -1), axis=1),
                             np.linalg.norm((v1p - v1).reshape(P, -1), axis=1) / np.linalg.norm(v1.reshape(P, -1), axis=1))
        runs.append({"seed": int(seed), "flip_fraction": flips, "max_element_change_over_rms": elem / rms,
                     "max_position_rel_l2": float(per_pos.max()), "median_position_rel_l2": float(np.median(per_pos)),
                     "worst_position": int(per_pos.argmax())})
    return {"config": cfg_name, "layers": layers, "prompt": P, "sigma": sigma, "rms": rms, "runs": runs,
            "max_element_change_over_rms": max(r["max_element_change_over_rms"] for r in runs),
            "max_position_rel_l2": max(r["max_position_rel_l2"] for r in runs)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--write", default="")
    ap.add_argument("--prompt", type=int, default=4200)
    args = ap.parse_args()
    t0 = time.time()
    res = sensitivity("cfg4", 2, args.prompt, 4e-6, (1, 2, 3))
    res["seconds"] = round(time.time() - t0, 1)
    res["command"] = "python oracle/layer1_sensitivity.py --write tests/golden/layer1_sensitivity.json"
    print(json.dumps(res, indent=1))
    if args.write:
        with open(args.write, "w") as fh:
            json.dump(res, fh, indent=1)
            fh.write("\n")


if __name__ == "__main__":
    main()
