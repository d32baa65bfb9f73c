#!/usr/bin/env python3
"""Batch-1 decode throughput of the persistent monokernel on one MI355X.

A step is one decode token: the whole hot path (embedding, every layer's
RMSNorm / QKV / RoPE / KV append / attention / O / SwiGLU MLP, final norm,
LM head, greedy argmax) for one token of one request.  The default workload is
the ~2.4B-shaped fp16 decoder (28 layers, d 2560, 20x128 MHA, FFN 6912,
vocab 32000) after a 2048-token prompt, decoding 512 tokens.

Prints ONE JSON line.  `value` is decode tokens/s of the single request; the
`roofline` object prices the same timed launch against MI355X's 8 TB/s HBM
peak with the algorithmic bytes (every streamed fp16 weight once per token plus
the fp16 KV rows read and written); `cpu_baseline` times the fp64 oracle's
decode step on the host for a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "bs=1 decode tokens/s/request on 1 MI355X + achieved HBM GB/s vs peak"
PEAK_HBM_GBS = 8000.0


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("kie_kernel.hip", "kie_layout.h"):
        with open(os.path.join(ROOT, "decode_persistent_monokernel_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(cfg_name: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, only
    if it was taken on the kernel source as it is now"""
    p = os.path.join(ROOT, "profiles", f"traffic_{cfg_name}.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except Exception:
        return None
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, weights, pos: int, n_steps: int):
    """the fp64 oracle as it stands: n_steps decode steps at context pos..,
    with a random fp64 KV cache of the right shape in place of the prompt"""
    from oracle import Oracle
    orc = Oracle(cfg, weights)
    cache = orc.new_cache(pos + n_steps + 1)
    rng = np.random.default_rng(0)
    for l in range(cfg.n_layers):
        cache.K[l][:, :pos] = rng.standard_normal(cache.K[l][:, :pos].shape)
        cache.V[l][:, :pos] = rng.standard_normal(cache.V[l][:, :pos].shape)
    tok = 1
    orc.step(cache, tok, pos)  # one untimed step (first-touch)
    t0 = time.perf_counter()
    for k in range(n_steps):
        lg = orc.step(cache, tok, pos + 1 + k)
        tok = int(np.argmax(lg))
    dt = time.perf_counter() - t0
    threads = os.environ.get("OPENBLAS_NUM_THREADS") or os.environ.get("OMP_NUM_THREADS") or str(os.cpu_count())
    return dict(value=n_steps / dt, unit="tok/s", cores=int(threads), kind="oracle",
                sample=f"{n_steps} fp64 oracle decode steps of {cfg.name} at context {pos + 1}..{pos + n_steps} "
                       f"(random fp64 KV cache in place of the prompt; weight upcast not timed)")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--config", default="cfg2")
    ap.add_argument("--prompt", type=int, default=None, help="prompt length (default: the config's)")
    ap.add_argument("--cpu-steps", type=int, default=24)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--repeats", type=int, default=0, help="extra timed repeats for the launch-time spread")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "multi-GPU decode is not part of it", file=sys.stderr)
        sys.exit(2)

    import torch
    from decode_persistent_monokernel_amd.config import preset
    from decode_persistent_monokernel_amd.inputs import gen_weights, gen_prompt
    from decode_persistent_monokernel_amd.kie import Engine

    cfg = preset(args.config)
    P = args.prompt if args.prompt is not None else cfg.prompt_len
    K, W = args.steps, args.warmup
    max_ctx = P + max(K, W) + 1
    t_setup = time.time()
    w = gen_weights(cfg)
    prompt = gen_prompt(cfg, n=P)
    eng = Engine(cfg, device=0, max_ctx=max_ctx)
    eng.set_launch_steps(max(K, W, 1))
    eng.load_weights(w)
    t1 = eng.prefill(prompt)
    dev = eng.dev
    out = torch.empty(max(K, W), dtype=torch.int32, device=dev)
    print(f"bench: {cfg.name} setup {time.time() - t_setup:.1f}s (P={P}, t1={t1})", file=sys.stderr, flush=True)

    # warm-up, then rewind to the end of the prompt
    if W > 0:
        eng.decode_device(W, out)
        eng.sync()
    eng.set_position(P, t1)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    eng.decode_device(K, out)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    eng.sync()
    kernel_ms = ev0.elapsed_time(ev1)
    toks = out[:K].cpu().numpy()

    launch_ms = [kernel_ms]
    for _ in range(args.repeats):
        eng.set_position(P, t1)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        eng.decode_device(K, out)
        b.record(stream)
        torch.cuda.synchronize()
        launch_ms.append(a.elapsed_time(b))
        eng.sync()

    n_launches = (K + max(K, W, 1) - 1) // max(K, W, 1)
    algo_bytes = cfg.run_bytes(P, K)
    achieved = algo_bytes / (kernel_ms * 1e-3) / 1e9
    traffic = measured_traffic(cfg.name)
    value = K / wall
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(wall * 1e3 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: {cfg.description}; fp16 weights and KV, fp32 accumulation; "
                        f"prompt {P} tokens, greedy decode {K} tokens, batch 1",
            "prompt_len": P, "decode_tokens": K, "layers": cfg.n_layers, "d_model": cfg.d_model,
            "heads": cfg.n_heads, "kv_heads": cfg.n_kv_heads, "head_dim": cfg.head_dim,
            "ffn": cfg.ffn_dim, "vocab": cfg.vocab, "launches": n_launches,
            "workgroups": eng.launch_info()["n_workgroups"],
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": algo_bytes,
            "kernel_ms": round(kernel_ms, 3),
            "launch_ms_all": [round(x, 3) for x in launch_ms],
            "kernel": "kie::kie_monokernel<1>" if cfg.n_heads == cfg.n_kv_heads else
                      f"kie::kie_monokernel<{cfg.n_heads // cfg.n_kv_heads}>",
        },
        "tokens_head": [int(t) for t in toks[:8]],
    }
    eng.close()
    del eng
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, w, P, args.cpu_steps)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
