#!/usr/bin/env python3
"""Benchmark of one GQA decode step (attention + o_proj) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Default workload: batch 1, 32 query / 8 KV heads, head_dim 128, 2048 cached
keys, o_proj 4096 x 4096 (the shape of the F-16 decode-attention page).
Inputs are seeded synthetic tensors already resident in HBM. To keep the
256 MB Infinity Cache from serving them, the loop cycles through R copies of
every buffer, R chosen so that at least 512 MiB of distinct data is touched
per cycle.

Prints ONE JSON line: the whole-step throughput (algorithmic bytes / time),
the roofline of the dominant kernel (HIP events on the stream the kernels run
on) and the CPU oracle timed on the host over a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "µs per decode step (attn+o_proj) and achieved HBM TB/s vs peak, 1×MI355X"
HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 * 1024 * 1024


def parse():
    import workloads

    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=workloads.PAGES.name, choices=[w.name for w in workloads.DECODE])
    ap.add_argument("--min-rotate-mib", type=float, default=512.0)
    ap.add_argument("--breakdown-steps", type=int, default=200, help="launches per kernel in the breakdown pass")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs on exactly one GPU; --gpus %d (WORLD_SIZE %d) is not supported. "
              "Multi-GPU sharding is described in DESIGN.md, not run." % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import decode_attention_output_amd as da
    import workloads

    wl = workloads.BY_NAME[args.workload]
    s = wl.shape
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    da.load_library()

    inp = workloads.decode_inputs(wl, poison=True)
    seq_lens = inp["seq_lens"]
    alg_bytes = workloads.algorithmic_bytes(s, seq_lens)
    D = s.head_dim
    kv_read = 2 * 2 * s.num_kv_heads * D * int(np.sum(seq_lens))
    w_bytes = 2 * s.o_in * s.hidden

    def to_dev(words):
        return torch.from_numpy(np.ascontiguousarray(words).view(np.int16)).view(torch.bfloat16).to(dev)

    base = {n: to_dev(inp[n]) for n in ("q", "k", "v", "o_weight")}
    sl = torch.from_numpy(seq_lens).to(dev)
    R = max(1, math.ceil(args.min_rotate_mib * 2 ** 20 / alg_bytes))
    sets = []
    for r in range(R):
        st = {n: (t if r == 0 else t.clone()) for n, t in base.items()}
        st["out"] = torch.empty((s.batch, s.hidden), dtype=torch.bfloat16, device=dev)
        st["flat"] = torch.empty((s.batch, s.o_in), dtype=torch.bfloat16, device=dev)
        st["ws"] = da.Workspace(dev)
        sets.append(st)
    del inp["k"], inp["v"]  # host copies of the cache are reloaded below only if needed
    stream = torch.cuda.current_stream()

    def step(st):
        da.decode_attn_fwd(st["q"], st["k"], st["v"], sl, st["o_weight"], out=st["out"], workspace=st["ws"])

    plan = da.decode_attn_plan(da.make_shape(s.batch, s.num_q_heads, s.num_kv_heads, s.max_seq_len, s.hidden))

    # ---- warm-up, then exactly `steps` timed steps ----
    for i in range(args.warmup):
        step(sets[i % R])
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        step(sets[i % R])
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_us = (t1 - t0) / args.steps * 1e6
    ev_us = [a.elapsed_time(b) * 1e3 for a, b in ev]
    step_us = statistics.median(ev_us)

    # ---- per-kernel pass: the attention launches and the projection launch ----
    n_b = args.breakdown_steps
    ev_a = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_b)]
    ev_o = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_b)]
    for i in range(n_b):
        st = sets[i % R]
        ev_a[i][0].record(stream)
        da.decode_attn_only(st["q"], st["k"], st["v"], sl, out=st["flat"], workspace=st["ws"])
        ev_a[i][1].record(stream)
    for i in range(n_b):
        st = sets[i % R]
        ev_o[i][0].record(stream)
        da.oproj_fwd(st["flat"], st["o_weight"], out=st["out"], workspace=st["ws"])
        ev_o[i][1].record(stream)
    torch.cuda.synchronize()
    attn_us = statistics.mean(a.elapsed_time(b) * 1e3 for a, b in ev_a)
    oproj_us = statistics.mean(a.elapsed_time(b) * 1e3 for a, b in ev_o)
    # restore the step's own output in set 0 for the parity check
    step(sets[0])
    torch.cuda.synchronize()

    attn_bytes = kv_read + 2 * s.batch * s.num_q_heads * D + 2 * s.batch * s.o_in
    proj_bytes = w_bytes + 2 * s.batch * s.o_in + 2 * s.batch * s.hidden
    if proj_bytes >= attn_bytes:
        dom = {"kernel": "gemv_kernel (o_proj, VALU)" if plan.oproj_path == 0 else "gemm_kernel (o_proj, MFMA)",
               "bytes": proj_bytes, "us": oproj_us}
    else:
        dom = {"kernel": "attn_split_kernel + attn_combine_kernel", "bytes": attn_bytes, "us": attn_us}
    achieved = dom["bytes"] / (dom["us"] * 1e-6) / 1e9

    result = {
        "metric": METRIC,
        "value": round(alg_bytes / (wall_us * 1e-6) / 1e12, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_us / 1e3, 6),
        "us_per_step": round(wall_us, 3),
        "us_per_step_events_median": round(step_us, 3),
        "frac_of_hbm_peak": round(alg_bytes / (wall_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "batch": s.batch, "num_q_heads": s.num_q_heads, "num_kv_heads": s.num_kv_heads,
            "head_dim": D, "max_seq_len": s.max_seq_len, "seq_lens_sum": int(np.sum(seq_lens)),
            "hidden": s.hidden, "algorithmic_bytes": alg_bytes, "rotation_sets": R,
            "split_len": plan.split_len, "num_splits": plan.num_splits, "oproj_path": int(plan.oproj_path),
            "fused": int(plan.fused),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": dom["kernel"],
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "avg_launch_us": round(dom["us"], 3),
            "alg_bytes_per_launch": dom["bytes"],
        },
        "breakdown_us": {"attention": round(attn_us, 3), "oproj": round(oproj_us, 3)},
    }

    if not args.no_parity or not args.no_cpu_baseline:
        import oracle

        full = workloads.decode_inputs(wl, poison=True)
    if not args.no_parity:
        ref = oracle.decode_step(full["q"], full["k"], full["v"], full["seq_lens"], full["o_weight"])
        got = torch.from_numpy(sets[0]["out"].cpu().view(torch.int16).numpy()).view(torch.bfloat16).double().numpy()
        err = np.abs(got - ref["out_ref"])
        mask = np.abs(ref["out_ref"]) >= 1e-2
        rel = float((err[mask] / np.abs(ref["out_ref"][mask])).max()) if mask.any() else 0.0
        ok = bool(np.all(np.isfinite(got)) and err.max() <= 1e-2 and rel <= 2.0 ** -7)
        result["parity"] = {"vs": "oracle", "ok": ok, "max_abs": float(err.max()), "max_rel": rel}
    if not args.no_cpu_baseline:
        threads = oracle.default_threads()
        n, t_cpu = 0, 0.0
        while n < 1 or (t_cpu < args.cpu_seconds and n < 1000):
            c0 = time.perf_counter()
            oracle.decode_step(full["q"], full["k"], full["v"], full["seq_lens"], full["o_weight"], nthreads=threads)
            t_cpu += time.perf_counter() - c0
            n += 1
        cpu_us = t_cpu / n * 1e6
        result["cpu_baseline"] = {
            "value": round(alg_bytes / (cpu_us * 1e-6) / 1e12, 6),
            "unit": "TB/s",
            "us_per_step": round(cpu_us, 1),
            "cores": threads,
            "kind": "oracle",
            "sample": "%d full decode steps of %s (fp64 C oracle, %d threads, %.1f s)" % (n, wl.name, threads, t_cpu),
        }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
