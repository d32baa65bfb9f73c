"""How far apart the two readings of the KV cache put the logits.

TEST INFRASTRUCTURE ONLY (calls nothing but the oracle and the seeded input
generator).  The pages state FP16 decoding with no quantization (Kog
explainers, results table "Laneformer 2B"); a model whose KV cache holds fp16
values rounds K and V to binary16 as they enter the cache.  The oracle can
keep the cache in fp64 (the plain textbook definition) or rounded to binary16
(`Oracle(kv_fp16=True)`).  This script measures, under teacher forcing on the
same inputs, the relative L2 distance between the logits of the two at every
step, so the choice of the fp16-cache oracle as the parity reference rests
on a recorded figure rather than prose.

    python oracle/kv_rounding_distance.py cfg1 --prompt 1024 --steps 8
    python oracle/kv_rounding_distance.py --write tests/golden/kv_rounding_distance.json

With --write it runs the recorded cases (cfg1 at its 1024-token prompt, the
~2.4B cfg2 at its 2048-token prompt and with one layer) and stores the
figures; tests/test_oracle_kv_rounding.py recomputes the cfg1 case and
compares.
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

from oracle.oracle import Oracle  # noqa: E402

# (config, prompt length, decode steps, layers or None for all)
RECORDED = [("cfg1", 1024, 8, None), ("cfg2", 2048, 4, 1), ("cfg2", 2048, 4, None)]


def rel_l2(a, b) -> float:
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / np.linalg.norm(np.asarray(b)))


def distance(cfg_name: str, prompt_len: int, steps: int, layers=None) -> dict:
    """per-step rel-L2 of fp16-cache logits against fp64-cache logits; both
    fed the fp64-cache run's greedy tokens"""
    from decode_persistent_monokernel_amd.config import preset
    from decode_persistent_monokernel_amd.inputs import gen_prompt, gen_weights
    cfg = preset(cfg_name)
    if layers is not None:
        cfg = cfg.with_(n_layers=layers)
    w = gen_weights(cfg)
    prompt = gen_prompt(cfg, n=prompt_len)
    t0 = time.time()
    orc = Oracle(cfg, w)  # the upcast weights are shared by both runs
    del w
    exact = orc.run(prompt, steps)
    orc.kv_fp16 = True
    rounded = orc.run(prompt, steps, forced=exact["inputs"])
    per = [rel_l2(rounded["prefill_logits"], exact["prefill_logits"])]
    per += [rel_l2(r, e) for r, e in zip(rounded["logits"], exact["logits"])]
    return {"config": cfg_name, "layers": cfg.n_layers, "prompt": prompt_len, "steps": steps,
            "rel_l2_per_step": per, "max": max(per), "seconds": round(time.time() - t0, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("config", nargs="?", default="cfg1")
    ap.add_argument("--prompt", type=int, default=1024)
    ap.add_argument("--steps", type=int, default=8)
    ap.add_argument("--layers", type=int, default=None)
    ap.add_argument("--write", metavar="JSON", help="run the recorded cases and store them")
    a = ap.parse_args()
    if a.write:
        out = {"what": "rel-L2 distance of fp16-KV-cache oracle logits from fp64-KV-cache oracle logits, "
                       "teacher-forced on the same tokens (entry 0: the prompt's last position)",
               "command": "python oracle/kv_rounding_distance.py --write tests/golden/kv_rounding_distance.json",
               "cases": []}
        for name, P, N, nl in RECORDED:
            r = distance(name, P, N, nl)
            print(json.dumps(r), flush=True)
            out["cases"].append(r)
        with open(a.write, "w") as fh:
            json.dump(out, fh, indent=1)
            fh.write("\n")
        return
    print(json.dumps(distance(a.config, a.prompt, a.steps, a.layers)))


if __name__ == "__main__":
    main()
