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
import csv
import glob
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


def measured_traffic(cfg_name: str, prompt: int, steps: int):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary of the
    same run (config, prompt, decode steps), only if it was taken on the
    kernel source as it is now"""
    p = os.path.join(ROOT, "profiles", f"traffic_{cfg_name}_P{prompt}_N{steps}.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except Exception:
        return None
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    if d.get("prompt") != prompt or d.get("decode_steps") != steps:
        return None
    return d.get("hbm_bytes_per_launch")


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [d.get("num_threads", 0) for d in threadpool_info() if d.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return int(os.environ.get("OPENBLAS_NUM_THREADS") or os.environ.get("OMP_NUM_THREADS") or os.cpu_count())


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
    return dict(value=round(n_steps / dt, 3), unit="tok/s", cores=blas_threads(), kind="oracle",
                sample=f"{n_steps} fp64 oracle decode steps of {cfg.name} at context {pos + 1}..{pos + n_steps} "
                       f"(random fp64 KV cache in place of the prompt; weight upcast not timed)")


# ---------------------------------------------------------------------------
# rocprofv3 summaries (written under profiles/; the commands are in them)
# ---------------------------------------------------------------------------
def _rows(d, suffix):
    fs = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not fs:
        raise SystemExit(f"no *{suffix} under {d}")
    with open(fs[0]) as fh:
        return list(csv.DictReader(fh))


def summarize_trace(d: str, command: str, profiler_rc: int = 0) -> str:
    """markdown: per-kernel stats and every monokernel dispatch (for a trace of
    the --prefill mode: per-kernel stats and the batched prefill's share)"""
    stats = _rows(d, "kernel_stats.csv")
    trace = _rows(d, "kernel_trace.csv")
    prefill = "--prefill" in command
    title = ("# rocprofv3 kernel trace of the batched prefill benchmark (cfg2, 2048-token prompt, chunks of 2048)"
             if prefill else
             "# rocprofv3 kernel trace of the default benchmark run (cfg2, 2048-token prompt, 512 decode steps)")
    out = [title, "", "Command (from the repository root, on an MI355X):", "", "```", command, "```", ""]
    if profiler_rc:
        out += [f"rocprofv3 exited with status {profiler_rc} after the program's last line and after the tool's "
                "finalization had written every result file.  The same happens to any process that has both "
                "torch's HIP runtime and this library's code object loaded (either alone exits 0 under the "
                "profiler; plain runs exit 0); the figures below are complete.", ""]
    out += ["| kernel | calls | total ms | average ms | min ms | max ms |", "|---|---|---|---|---|---|"]
    for r in stats:
        ns = lambda k: float(r[k]) / 1e6
        out.append(f"| `{r['Name'][:70]}` | {r['Calls']} | {ns('TotalDurationNs'):.3f} | {ns('AverageNs'):.3f} | "
                   f"{ns('MinNs'):.3f} | {ns('MaxNs'):.3f} |")
    if prefill:
        tot = sum(float(r["TotalDurationNs"]) for r in stats if "kie::" in r["Name"])
        out += ["", "Share of the kie kernels' time (two prefills: a warm-up and the timed one; in each, all "
                "prompt tokens but the last run through the batched kernels, the last through one decode-kernel "
                "launch):", "", "| kernel | share |", "|---|---|"]
        for r in stats:
            if "kie::" in r["Name"]:
                out.append(f"| `{r['Name'][:70]}` | {100 * float(r['TotalDurationNs']) / tot:.1f} % |")
        return "\n".join(out) + "\n"
    mk = [r for r in trace if "kie_monokernel" in r["Kernel_Name"]]
    out += ["", "Every launch of the persistent kernel, in order: the prompt's launches, the warm-up decode, "
            "then the timed decode (the last row; bench.py's HIP events time the same launch).", "",
            "| # | duration ms |", "|---|---|"]
    for i, r in enumerate(mk):
        out.append(f"| {i} | {(int(r['End_Timestamp']) - int(r['Start_Timestamp'])) / 1e6:.3f} |")
    return "\n".join(out) + "\n"


def summarize_traffic(fetch_dir: str, write_dir: str, copy_bytes: int, cfg_name: str, steps: int,
                      prompt: int, ea_dir: str = "") -> dict:
    """HBM bytes of the timed decode launch from FETCH_SIZE / WRITE_SIZE (KiB
    per dispatch), each scaled by what it reads for a plain copy of
    copy_bytes (read copy_bytes, write copy_bytes).  With ea_dir (a pass of
    TCC_EA0_RDREQ_{32B,64B,128B}_sum and TCC_EA0_RDREQ_sum), also the read
    bytes counted from the EA read requests by size, unscaled, for the kernel
    and the copy: a second counter family for the read figure."""
    def pick(d, counter, scale=1024.0):
        rows = [r for r in _rows(d, "counter_collection.csv") if r["Counter_Name"] == counter]
        mono = [r for r in rows if "kie_monokernel" in r["Kernel_Name"]]
        last_mono = max(int(r["Dispatch_Id"]) for r in mono) if mono else 0
        copies = [r for r in rows if int(r["Dispatch_Id"]) > last_mono]
        if not mono or not copies:
            raise SystemExit(f"{counter}: missing dispatches in {d}")
        timed = max(mono, key=lambda r: int(r["Dispatch_Id"]))
        copy = max(copies, key=lambda r: int(r["Dispatch_Id"]))  # the multiply that copies
        return float(timed["Counter_Value"]) * scale, float(copy["Counter_Value"]) * scale, copy["Kernel_Name"]
    f_k, f_c, f_name = pick(fetch_dir, "FETCH_SIZE")
    w_k, w_c, _ = pick(write_dir, "WRITE_SIZE")
    sf, sw = copy_bytes / f_c, copy_bytes / w_c
    from decode_persistent_monokernel_amd.config import preset
    algo = preset(cfg_name).run_bytes(prompt, steps)
    ea = {}
    if ea_dir:
        n = {k: pick(ea_dir, f"TCC_EA0_RDREQ{k}_sum", 1.0)[:2] for k in ("", "_32B", "_64B", "_128B")}
        by_size = lambda i: 32 * n["_32B"][i] + 64 * n["_64B"][i] + 128 * n["_128B"][i]
        ea = {
            "ea_read_requests": {k or "all": n[k][0] for k in n},
            "ea_read_bytes_per_launch": by_size(0),
            "ea_read_bytes_copy": by_size(1),
            "ea_copy_ratio": by_size(1) / copy_bytes,
            "ea_read_ratio_to_fetch_scaled": by_size(0) / (f_k * sf),
            "ea_unsized_requests": n[""][0] - n["_32B"][0] - n["_64B"][0] - n["_128B"][0],
        }
    return {
        "config": cfg_name, "prompt": prompt, "decode_steps": steps,
        "kernel_source_hash": kernel_source_hash(),
        "fetch_kib_raw": f_k / 1024, "write_kib_raw": w_k / 1024,
        "copy_kernel": f_name[:80], "copy_bytes": copy_bytes,
        "fetch_scale": sf, "write_scale": sw,
        "hbm_read_bytes_per_launch": f_k * sf, "hbm_write_bytes_per_launch": w_k * sw,
        "hbm_bytes_per_launch": f_k * sf + w_k * sw,
        "algorithmic_bytes_per_launch": algo,
        "ratio_to_algorithmic": (f_k * sf + w_k * sw) / algo,
        **ea,
    }


# ---------------------------------------------------------------------------
# per-phase critical path from the kernel's own wall-clock stamps
# ---------------------------------------------------------------------------
END_PHASE = 5 * 64 + 1


def phase_trace_summary(tr: np.ndarray, cfg, untraced_ms_per_token: float, command: str) -> str:
    """Markdown attribution of one token's time from kie_set_trace stamps
    tr[step, phase, workgroup, 4] (100 MHz ticks: phase start, input ready,
    stream done, phase end; attention: start, query ready, records stored,
    end after the merge).

    Critical path: for every phase, `hop` is the time from the previous
    phase's last end to this phase's last input-ready stamp (the dependency
    exchange the slowest consumer waited for), `work` from that to this
    phase's last end (its stream and epilogue).  The end of a step (release,
    token gather, acquire) follows the LM head.  Per workgroup: the share of
    its time spent between a phase's start and its input being ready (waiting
    on other workgroups), the analogue of a grid-synchronisation share."""
    from decode_persistent_monokernel_amd import kie
    tick_us = 0.01
    L = cfg.n_layers
    # phase index -> kind name, in the kernel's order (pipelined for the
    # lane block with a delayed residual)
    order = [kie.PHASE_KIND_NAMES[k] for k, _ in kie.phase_order(cfg, tr.shape[2])]
    names = tuple(dict.fromkeys(order[:5 * L]))
    steps = list(range(1, tr.shape[0]))  # the launch's first step also fills the ring: left out
    phases = list(range(5 * L)) + [5 * L]
    hop = {n: [] for n in names + ("LM head",)}
    work = {n: [] for n in names + ("LM head",)}
    wait_share, tok_us, end_us, first_hop = [], [], [], []
    per_phase_wait = {n: [] for n in names + ("LM head",)}
    for s in steps:
        t = tr[s].astype(np.float64)
        start = t[0, :, 0].min()
        prev_end = start
        waited = np.zeros(tr.shape[2])
        for ph in phases:
            nm = order[ph]
            st = t[ph]
            r_max, e_max = st[:, 1].max(), st[:, 3].max()
            hop[nm].append((r_max - prev_end) * tick_us)
            work[nm].append((e_max - r_max) * tick_us)
            w = st[:, 1] - st[:, 0]
            waited += w
            per_phase_wait[nm].append(w.mean() * tick_us)
            prev_end = e_max
        e = t[END_PHASE]
        step_end = e[:, 1].max()
        end_us.append((step_end - prev_end) * tick_us)
        nxt = tr[s + 1][0, :, 0].min() if s + 1 < tr.shape[0] else None
        total = ((nxt if nxt is not None else step_end) - start) * tick_us
        tok_us.append(total)
        wait_share.append(float(np.mean(waited * tick_us / total)))
    T = float(np.mean(tok_us))
    seq = " ".join(f"{n}_{l}" for n, l in zip(order[:12], [l for _, l in kie.phase_order(cfg, tr.shape[2])][:12]))
    out = [f"# Per-phase critical path of one decode token ({cfg.name}, {cfg.n_layers} layers)", "",
           "From the kernel's own phase stamps (`kie_set_trace`, wall clock at 100 MHz) over "
           f"{len(steps)} decode steps; the stamps are kept in LDS and written out at the end of each step.", "",
           f"Phase order of a step (`kie_phase_order`): {seq} ...", "",
           "Command (from the repository root, on an MI355X):", "", "```", command, "```", "",
           f"- traced token time: {T:.1f} us (untraced, same run: {untraced_ms_per_token * 1e3:.1f} us)",
           f"- per layer: {T / L:.2f} us",
           f"- share of a workgroup's time spent waiting for another workgroup's output (phase start to input "
           f"ready, summed over phases, mean over workgroups): **{100 * np.mean(wait_share):.1f} %**", "",
           "Critical path per token (sum over the layers of the phase; `hop` = previous phase's last end to "
           "this phase's last input ready, `work` = that to this phase's last end):", "",
           "| phase | hop us/token | work us/token | hop+work | share of token | mean wait per workgroup us/token |",
           "|---|---|---|---|---|---|"]
    nsteps = len(steps)
    tot_hop = tot_work = 0.0
    for nm in names + ("LM head",):
        h = sum(hop[nm]) / nsteps
        w = sum(work[nm]) / nsteps
        pw = sum(per_phase_wait[nm]) / nsteps
        tot_hop += h
        tot_work += w
        out.append(f"| {nm} | {h:.1f} | {w:.1f} | {h + w:.1f} | {100 * (h + w) / T:.1f} % | {pw:.1f} |")
    E = float(np.mean(end_us))
    out.append(f"| end of step (release, token gather, acquire) | {E:.1f} | - | {E:.1f} | {100 * E / T:.1f} % | - |")
    out += ["", f"Hops total {tot_hop + E:.1f} us/token ({100 * (tot_hop + E) / T:.1f} % of the token); "
            f"work total {tot_work:.1f} us/token ({100 * tot_work / T:.1f} %)."]
    return "\n".join(out) + "\n"


def release_engine(eng) -> None:
    """destroy the library context, then free the engine's device tensors and
    hand the cached blocks back to the runtime"""
    import torch
    eng.close()
    for name in ("d_packed", "d_kv", "d_ws", "_trace"):
        if hasattr(eng, name):
            setattr(eng, name, None)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


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
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after the timed decode, run one plain device copy of this many bytes (the reference "
                         "dispatch for scaling HBM counters)")
    ap.add_argument("--summarize-trace", metavar="DIR", help="write a markdown summary of a rocprofv3 "
                    "--kernel-trace --stats output directory to stdout and exit")
    ap.add_argument("--ea-dir", default="", help="with --summarize-traffic: a rocprofv3 --pmc run of "
                    "TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_32B_sum TCC_EA0_RDREQ_64B_sum TCC_EA0_RDREQ_128B_sum")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the JSON traffic summary of two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) "
                         "of this command with --copy-bytes and exit")
    ap.add_argument("--command", default="", help="the profiled command, recorded in a summary")
    ap.add_argument("--profiler-rc", type=int, default=0, help="rocprofv3's exit status, recorded in a summary")
    ap.add_argument("--launch-steps", type=int, default=0,
                    help="decode steps per kernel launch (default: all timed steps in one launch); 1 measures the "
                         "per-token launch cost the persistent kernel removes")
    ap.add_argument("--phase-trace", metavar="FILE", default="",
                    help="after the timed run, trace 16 decode steps and write the per-phase critical-path "
                         "summary (markdown) to FILE, and the raw stamps to FILE's stem + _stamps.npz")
    ap.add_argument("--prefill", action="store_true",
                    help="instead of the decode benchmark, time the batched prefill of the prompt and print "
                         "its own JSON line (matrix-core roofline)")
    args = ap.parse_args()

    if args.summarize_trace:
        sys.stdout.write(summarize_trace(args.summarize_trace, args.command, args.profiler_rc))
        return
    if args.summarize_traffic:
        from decode_persistent_monokernel_amd.config import preset
        P = args.prompt if args.prompt is not None else preset(args.config).prompt_len
        res = summarize_traffic(args.summarize_traffic[0], args.summarize_traffic[1], args.copy_bytes,
                                args.config, args.steps, P, args.ea_dir)
        res["command"] = args.command
        print(json.dumps(res, indent=1))
        return

    if args.gpus != 1:
        print(f"bench.py: decode runs on one GPU only (asked for --gpus {args.gpus}); "
              "multi-GPU decode is not implemented", file=sys.stderr)
        sys.exit(2)

    import torch
    from decode_persistent_monokernel_amd.config import preset
    from decode_persistent_monokernel_amd.inputs import gen_weights, gen_prompt
    from decode_persistent_monokernel_amd import kie
    from decode_persistent_monokernel_amd.kie import Engine

    cfg = preset(args.config)
    P = args.prompt if args.prompt is not None else cfg.prompt_len
    K, W = args.steps, args.warmup
    max_ctx = P + max(K, W) + 1
    t_setup = time.time()
    w = gen_weights(cfg)
    prompt = gen_prompt(cfg, n=P)
    eng = Engine(cfg, device=0, max_ctx=max_ctx)
    per_launch = args.launch_steps if args.launch_steps > 0 else max(K, W, 1)
    eng.set_launch_steps(per_launch)
    eng.load_weights(w)
    if args.prefill:
        prefill_bench(args, cfg, eng, prompt)
        return
    t1 = eng.prefill_batched(prompt)
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

    n_launches = (K + per_launch - 1) // per_launch
    algo_bytes = cfg.run_bytes(P, K)
    achieved = algo_bytes / (kernel_ms * 1e-3) / 1e9
    traffic = measured_traffic(cfg.name, P, K)
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
            "kernel": kie.kernel_name(cfg, eng.launch_info()["n_workgroups"]),
        },
        "tokens_head": [int(t) for t in toks[:8]],
    }
    if args.phase_trace:
        # 16 traced steps from the same position (a separate launch, after
        # the timed one)
        eng.set_position(P, t1)
        eng.set_launch_steps(16)
        eng.set_trace(16)
        eng.decode_device(16, out)
        eng.sync()
        tr = eng.trace()
        eng.set_trace(0)
        cmd = "python bench.py " + " ".join(a for a in sys.argv[1:])
        with open(args.phase_trace, "w") as fh:
            fh.write(phase_trace_summary(tr, cfg, wall * 1e3 / K, cmd))
        # the raw stamps beside the summary, for analyses of their own
        np.savez_compressed(os.path.splitext(args.phase_trace)[0] + "_stamps.npz", stamps=tr,
                            order=np.array(kie.phase_order(cfg, tr.shape[2]), dtype=np.int32))
    # release every device buffer while the runtime (and a profiler attached
    # to it) is still fully up: nothing is left for interpreter teardown
    del out
    release_engine(eng)
    del eng
    if args.copy_bytes > 0:
        src = torch.ones(args.copy_bytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)  # an elementwise kernel: reads and writes copy_bytes
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, w, P, args.cpu_steps)
    print(json.dumps(res), flush=True)


PEAK_FP16_MFMA_TFLOPS = 2500.0  # MI355X dense fp16 matrix rate (the prefill GEMMs' instructions)


def prefill_flops(cfg, n_tokens: int) -> float:
    """GEMM and attention FLOPs of pushing prompt tokens 0..n_tokens-1 through
    the layers (2 per multiply-add)"""
    d, hd, H, Hkv, F, L = cfg.d_model, cfg.head_dim, cfg.n_heads, cfg.n_kv_heads, cfg.ffn_dim, cfg.n_layers
    per_token_params = (H + 2 * Hkv) * hd * d + d * H * hd + 2 * F * d + d * F
    gemm = 2.0 * per_token_params * L * n_tokens
    attn = 4.0 * hd * H * L * (n_tokens * (n_tokens + 1) / 2)  # q.k and p.v over keys 0..i
    return gemm + attn


def prefill_bench(args, cfg, eng, prompt):
    """time kie_prefill_batched over the whole prompt (the batched part covers
    all tokens but the last, which runs through the decode kernel)"""
    import torch
    P = len(prompt)
    dev = eng.dev
    d_prompt = torch.tensor(np.asarray(prompt, dtype=np.int32), device=dev)
    d_next = torch.empty(1, dtype=torch.int32, device=dev)
    chunk = 2048
    scratch = torch.empty(eng.prefill_scratch_bytes(chunk) // 4, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    times = []
    for it in range(1 + max(1, args.repeats)):
        eng.set_position(0, 0)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        eng.prefill_batched_device(d_prompt, P, d_next, scratch)
        b.record(stream)
        torch.cuda.synchronize()
        eng.sync()
        if it > 0:  # the first run is a warm-up
            times.append(a.elapsed_time(b))
    ms = float(np.median(times))
    flops = prefill_flops(cfg, P - 1)
    achieved = flops / (ms * 1e-3) / 1e12
    res = {
        "metric": "batched prefill tokens/s on 1 MI355X + achieved matrix TFLOP/s vs the fp16 peak",
        "value": round(P / (ms * 1e-3), 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "ms": round(ms, 3),
        "higher_is_better": True,
        "dtype": "fp32 activations as fp16 hi + lo pairs, fp16 weights, fp32 accumulation",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.description}; batched prefill of a {P}-token prompt, "
                               f"chunks of {chunk}", "prompt_len": P},
        # each fp32 product is two fp16 MFMAs (hi and lo), so the split's own
        # ceiling is half the fp16 peak
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP16_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP16_MFMA_TFLOPS, 4), "traffic": None,
                     "frac_of_split_ceiling": round(2 * achieved / PEAK_FP16_MFMA_TFLOPS, 4),
                     "flops": flops, "all_ms": [round(x, 3) for x in times]},
        "next_token": int(d_next.cpu()[0]),
    }
    del d_prompt, d_next, scratch
    release_engine(eng)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
