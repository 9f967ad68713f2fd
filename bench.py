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
on) and the CPU oracle timed on the host over a bounded sample. The line also
carries five more timed regions and their median, and a warm number taken on
one buffer set (caches may serve it).

    python bench.py --workload prefill_b4_t512_h32kv8_ctx8192

times the context (prefill) attention of a token chunk instead, in TFLOP/s
against the bf16 MFMA peak, and

    python bench.py --workload gemm_f16_256x512x1024

the dense fp16 GEMM check (integer-valued inputs, bit-exact against the
oracle) against the fp16 MFMA peak.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "µs per decode step (attn+o_proj) and achieved HBM TB/s vs peak, 1×MI355X"
CALIB_BYTES = 64 * 2 ** 20  # plain device-to-device copy whose HBM traffic is known (read + write)
PROFILES = os.path.join(ROOT, "profiles")
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix-core peak of one MI355X
PREFILL_METRIC = "TFLOP/s of context (prefill) attention of a token chunk vs bf16 MFMA peak, 1×MI355X"
MFMA_F16_PEAK_TFLOPS = 2500.0  # dense fp16 matrix-core peak of one MI355X
GEMM_METRIC = "TFLOP/s of the dense fp16 GEMM check (MFMA, bit-exact) vs fp16 MFMA peak, 1×MI355X"
SIMDS = 256 * 4  # SIMDs of one MI355X (256 compute units of 4)
PEAK_CLOCK_GHZ = 2.4  # peak engine clock of one MI355X
MALL_BYTES = 256 * 1024 * 1024


def kernel_source_hash() -> str:
    """Hash of the HIP sources: HBM-traffic counters taken from another build are not reused."""
    import glob
    import hashlib

    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "decode_attention_output_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload: str, kernel_prefix: str):
    """Measured HBM bytes per dispatch of the dominant kernel, from the committed
    rocprofv3 PMC summary of this workload, if it was taken on the current sources."""
    path = os.path.join(PROFILES, "%s_%s.txt" % (kernel_prefix, workload))
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_hash") != kernel_source_hash() or fields.get("kernel") != kernel_prefix:
        return None
    try:
        return int(float(fields["hbm_bytes_per_dispatch"]))
    except (KeyError, ValueError):
        return None


def workloads_alg_bytes(shape, seq_lens):
    import workloads

    return workloads.algorithmic_bytes(shape, seq_lens)


def dominant_kernel(wl, plan, seq_lens):
    """(kernel name, algorithmic bytes per launch) of the launch that moves the most bytes."""
    import numpy as np

    s = wl.shape
    D = s.head_dim
    attn_bytes = 2 * 2 * s.num_kv_heads * D * int(np.sum(seq_lens)) + 2 * s.batch * s.num_q_heads * D \
        + 2 * s.batch * s.o_in
    proj_bytes = 2 * s.o_in * s.hidden + 2 * s.batch * s.o_in + 2 * s.batch * s.hidden
    if plan.fused:
        # one launch carries the whole step: the small single-launch step (1), the large one (2)
        # or the tiny one (3)
        name = {1: "decode_step_kernel", 2: "decode_step_large_kernel", 3: "decode_step_tiny_kernel"}[plan.fused]
        return name, workloads_alg_bytes(s, seq_lens), "step"
    if proj_bytes >= attn_bytes:
        return ("gemv_kernel" if plan.oproj_path == 0 else "gemm_kernel"), proj_bytes, "oproj"
    return "attn_streamk_kernel", attn_bytes, "attention"


def repeat_and_warm(run_steps, steps, repeats=5):
    """GPU-event µs per step of `repeats` more timed regions over the rotation sets
    (their median) and of one region on set 0 alone (warm: caches may serve it)."""
    import statistics

    import torch

    res = []
    for _ in range(repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        res.append(run_steps(e0, e1, rotate=True) * 1e3 / steps)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    warm = run_steps(e0, e1, rotate=False) * 1e3 / steps
    return [round(x, 3) for x in res], round(statistics.median(res), 3), round(warm, 3)


def stream_floor(nbytes, stream, min_rotate_mib, launches=200):
    """The floor of a step of `nbytes`: the best time of a plain streaming read of that many bytes
    (decode_attn_read_probe, the attention's 1 KiB-per-instruction load pattern) over rotated
    buffers, back to back on the bench stream, for a few workgroup counts."""
    import torch

    import decode_attention_output_amd as da

    lib = da.load_library()
    nbytes = (nbytes + 15) // 16 * 16
    R = max(1, math.ceil(min_rotate_mib * 2 ** 20 / nbytes))
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(R)]
    sink = torch.empty(65536, dtype=torch.int32, device="cuda")
    best = None
    for wgs in (256, 512, 1024, 2048):
        def launch(i):
            rc = lib.decode_attn_read_probe(bufs[i % R].data_ptr(), nbytes, sink.data_ptr(), wgs, stream.cuda_stream)
            if rc != da.DA_OK:
                raise da.DecodeAttnError(rc, "decode_attn_read_probe")
        for i in range(50):
            launch(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(launches):
            launch(i)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / launches
        if best is None or us < best[0]:
            best = (us, wgs)
    del bufs
    tbs = nbytes / (best[0] * 1e-6) / 1e12
    return {"us": round(best[0], 3), "tb_s": round(tbs, 3), "frac_of_peak": round(tbs * 1e3 / HBM_PEAK_GBS, 4),
            "workgroups": best[1], "bytes": nbytes,
            "note": "a plain streaming read of as many bytes as the timed launch must move (decode_attn_read_probe), best of "
                    "256-2048 workgroups, rotated buffers, back-to-back launches"}


def oracle_single_thread(run_once, budget_s=3.0):
    """Seconds per call of an oracle function on one host thread, over a few calls."""
    n, t = 0, 0.0
    while n < 1 or (t < budget_s and n < 100):
        c0 = time.perf_counter()
        run_once()
        t += time.perf_counter() - c0
        n += 1
    return t / n, n


def prefill_alg_bytes(wl):
    """Bytes a chunk's attention must move at minimum: its queries, every cached
    K and V row once, and its bf16 output."""
    rows = wl.batch * wl.tokens * wl.num_q_heads * wl.head_dim
    return 2 * rows + 2 * 2 * wl.batch * wl.num_kv_heads * wl.ctx_len * wl.head_dim + 2 * rows


def bench_gemm(args, wl):
    """The dense fp16 GEMM check: C = A @ B with entries in {-1, 0, 1}, timed per launch."""
    import numpy as np
    import torch

    import decode_attention_output_amd as da
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = da.load_library()
    g = workloads.gemm_inputs(wl)
    M, N, K = g["m"], g["n"], g["k"]
    flops = 2 * M * N * K
    set_bytes = 2 * (M * K + K * N + M * N)
    R = max(1, math.ceil(args.min_rotate_mib * 2 ** 20 / set_bytes))

    def to_dev(words):
        return torch.from_numpy(np.ascontiguousarray(words).view(np.int16)).view(torch.float16).to(dev)

    a0, b0 = to_dev(g["a"]), to_dev(g["b"])
    stream = torch.cuda.Stream(device=dev)
    sets = []
    for r in range(R):
        a, b = (a0, b0) if r == 0 else (a0.clone(), b0.clone())
        c = torch.empty((M, N), dtype=torch.float16, device=dev)
        sets.append((a, b, c))
    handle = stream.cuda_stream

    def launch(i):
        a, b, c = sets[i % R]
        rc = lib.gemm_f16(a.data_ptr(), b.data_ptr(), c.data_ptr(), M, N, K, handle)
        if rc != da.DA_OK:
            raise da.DecodeAttnError(rc, "gemm_f16")

    # the streaming floor of the same bytes first: its launches also bring the GPU out of idle
    floor = None if args.no_floor else stream_floor(set_bytes, stream, args.min_rotate_mib)

    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            launch(i)
    torch.cuda.synchronize()

    # a plain elementwise copy of known size, outside the timed region: the HBM
    # counters of a profiled run are scaled by what they read for it
    calib_src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
    calib_dst = torch.empty_like(calib_src)
    torch.mul(calib_src, 1.0, out=calib_dst)
    torch.cuda.synchronize()
    del calib_src, calib_dst

    def run_steps(e0, e1, rotate):
        e0.record(stream)
        for i in range(args.steps):
            launch(i if rotate else 0)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    gpu_ms = run_steps(ev0, ev1, True)
    wall_us = (time.perf_counter() - t0) / args.steps * 1e6
    gpu_us = gpu_ms * 1e3 / args.steps
    repeats_us, median_us, warm_us = repeat_and_warm(run_steps, args.steps)
    launch(0)
    torch.cuda.synchronize()

    achieved = flops / (gpu_us * 1e-6) / 1e12
    result = {
        "metric": GEMM_METRIC,
        "value": round(achieved, 4),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(gpu_us / 1e3, 6),
        "us_per_step": round(gpu_us, 3),
        "us_per_step_wall": round(wall_us, 3),
        "us_per_step_repeats": repeats_us,
        "us_per_step_median": median_us,
        "us_per_step_warm": warm_us,
        "warm_note": "one buffer set, so the Infinity Cache and L2 may serve it; value uses rotated sets",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": wl.name, "m": M, "n": N, "k": K, "flops": flops, "rotation_sets": R},
        "roofline": {
            "bound": "mfma",
            "kernel": gemm_f16_kernel(M, N),
            "achieved": round(achieved, 3),
            "peak": MFMA_F16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 5),
            "traffic": traffic_from_profile(wl.name, gemm_f16_kernel(M, N)),
            "avg_launch_us": round(gpu_us, 3),
            "flops_per_launch": flops,
            "timing": "HIP events around the timed back-to-back launches on the bench stream",
            "note": "0.27 GFLOP over 1.8 MB: a single launch is bound by latency, not by the matrix cores",
        },
        "stream_floor": floor,
    }
    if not args.no_parity or not args.no_cpu_baseline:
        import oracle

        threads = oracle.default_threads()
        n, t_cpu, ref = 0, 0.0, None
        while n < 1 or (not args.no_cpu_baseline and t_cpu < args.cpu_seconds and n < 1000):
            c0 = time.perf_counter()
            ref, _ = oracle.gemm_f16(g["a"], g["b"], nthreads=threads)
            t_cpu += time.perf_counter() - c0
            n += 1
    if not args.no_parity:
        got = sets[0][2].cpu().view(torch.int16).numpy().view(np.uint16)
        result["parity"] = {"vs": "oracle", "ok": bool(np.array_equal(got, ref)), "bit_exact": True,
                            "mismatches": int(np.count_nonzero(got != ref))}
    if not args.no_cpu_baseline:
        cpu_us = t_cpu / n * 1e6
        result["cpu_baseline"] = {
            "value": round(flops / (cpu_us * 1e-6) / 1e12, 6),
            "unit": "TFLOP/s",
            "us_per_step": round(cpu_us, 1),
            "cores": threads,
            "kind": "oracle",
            "sample": "%d runs of the %dx%dx%d GEMM (fp64 C oracle, %d threads, %.1f s)" % (n, M, N, K, threads, t_cpu),
        }
        sec, n1 = oracle_single_thread(lambda: oracle.gemm_f16(g["a"], g["b"], nthreads=1))
        result["cpu_baseline"]["single_thread"] = {
            "value": round(flops / sec / 1e12, 6), "us_per_step": round(sec * 1e6, 1), "cores": 1,
            "sample": "%d runs of the GEMM on one thread" % n1}
    print(json.dumps(result), flush=True)


KNOWN_KERNELS = ("decode_step_large_kernel", "decode_step_tiny_kernel", "decode_step_kernel", "attn_streamk_kernel",
                 "gemm_kernel", "gemv_kernel", "gemm_narrow_kernel", "prefill_kernel", "read_probe_kernel")


def gemm_f16_kernel(m, n):
    """The kernel gemm_f16 launches for an m x n product: 16 x 32 tiles over all of K when fewer
    than 256 tiles of 128 columns x 16 rows would be launched, else the 128-column GEMM."""
    return "gemm_narrow_kernel" if -(-n // 128) * (m // 16) < 256 else "gemm_kernel"


def kernel_alg_bytes(args):
    """{kernel name: algorithmic bytes per dispatch} for the kernels a run of --workload launches,
    and the dominant kernel's name."""
    import decode_attention_output_amd as da
    import numpy as np
    import workloads

    wl = workloads.BY_NAME[args.workload]
    if isinstance(wl, workloads.PrefillWorkload):
        return {"prefill_kernel": prefill_alg_bytes(wl)}, "prefill_kernel"
    if isinstance(wl, workloads.GemmWorkload):
        kname = gemm_f16_kernel(wl.m, wl.n)
        return {kname: 2 * (wl.m * wl.k + wl.k * wl.n + wl.m * wl.n)}, kname
    s = wl.shape
    seq_lens = workloads.draw_seq_lens(wl, np.random.default_rng(wl.seed))
    tiles = json.loads(args.tiles) if args.tiles else None
    plan = da.decode_attn_plan(da.make_shape(s.batch, s.num_q_heads, s.num_kv_heads, s.max_seq_len, s.hidden,
                                             s.head_dim, tiles=tiles))
    kname, kbytes, _ = dominant_kernel(wl, plan, seq_lens)
    D = s.head_dim
    attn = 2 * 2 * s.num_kv_heads * D * int(np.sum(seq_lens)) + 2 * s.batch * s.num_q_heads * D + 2 * s.batch * s.o_in
    proj = 2 * s.o_in * s.hidden + 2 * s.batch * s.o_in + 2 * s.batch * s.hidden
    whole = workloads.algorithmic_bytes(s, seq_lens)
    return {"decode_step_large_kernel": whole, "decode_step_kernel": whole, "decode_step_tiny_kernel": whole,
            "attn_streamk_kernel": attn,
            "gemm_kernel": proj, "gemv_kernel": proj, "read_probe_kernel": (whole + 15) // 16 * 16,
            kname: kbytes}, kname


def summarize_profile(args):
    """profiles/<kernel>_<workload>[_<tag>].txt, for every kernel of the run, from a FETCH_SIZE run,
    a WRITE_SIZE run and a kernel-trace run of the same bench command."""
    import csv

    import workloads

    wl = workloads.BY_NAME[args.workload]
    alg, dominant = kernel_alg_bytes(args)

    def counter_avg(path, counter, match):
        vals = []
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") == counter and match(row.get("Kernel_Name", "")):
                    vals.append(float(row["Counter_Value"]))
        return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)

    is_cal = lambda n: "MulFunctor" in n
    fetch_cal, _ = counter_avg(args.summarize_profile[0], "FETCH_SIZE", is_cal)
    write_cal, _ = counter_avg(args.summarize_profile[1], "WRITE_SIZE", is_cal)
    f_scale = (CALIB_BYTES / 1024.0) / fetch_cal if fetch_cal else None
    w_scale = (CALIB_BYTES / 1024.0) / write_cal if write_cal else None
    stats = []
    with open(args.summarize_profile[2]) as f:
        for row in csv.DictReader(f):
            stats.append((row["Name"], int(row["Calls"]), float(row["AverageNs"]), float(row["MinNs"]),
                          float(row["MaxNs"])))
    present = []
    for name, *_ in stats:
        k = next((k for k in KNOWN_KERNELS if re.search(r"\b%s\b" % k, re.sub(r"[^A-Za-z0-9_]", " ", name))), None)
        if k and k not in present:
            present.append(k)
    extra = " --tiles '%s'" % args.tiles if args.tiles else ""
    cmd_tail = "--workload %s --no-cpu-baseline --no-parity --no-graph%s" % (wl.name, extra)
    os.makedirs(PROFILES, exist_ok=True)
    tag = ("_" + args.profile_tag) if args.profile_tag else ""
    for kname in present:
        match = lambda n, k=kname: re.search(r"\b%s\b" % k, re.sub(r"[^A-Za-z0-9_]", " ", n)) is not None
        fetch, nf = counter_avg(args.summarize_profile[0], "FETCH_SIZE", match)
        write, nw = counter_avg(args.summarize_profile[1], "WRITE_SIZE", match)
        rd = fetch * f_scale * 1024 if fetch is not None and f_scale else None
        wr = write * w_scale * 1024 if write is not None and w_scale else None
        kbytes = alg.get(kname)
        out = os.path.join(PROFILES, "%s_%s%s.txt" % (kname, wl.name, tag))
        with open(out, "w") as f:
            f.write("# rocprofv3 summary: %s, workload %s%s\n" % (kname, wl.name,
                                                                  (" (" + args.profile_tag + ")") if tag else ""))
            f.write("# commands (run from the repository root on one MI355X):\n")
            f.write("#   rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run -- python3 bench.py %s\n"
                    % cmd_tail)
            f.write("#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o fetch -- python3 bench.py %s "
                    "--steps 50\n" % cmd_tail)
            f.write("#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -o write -- python3 bench.py %s "
                    "--steps 50\n" % cmd_tail)
            f.write("#   python3 bench.py %s --summarize-profile <fetch csv> <write csv> <stats csv>%s\n"
                    % (cmd_tail, (" --profile-tag " + args.profile_tag) if tag else ""))
            f.write("# FETCH_SIZE / WRITE_SIZE are KiB per dispatch; each is scaled by what the same counter reads\n")
            f.write("# for a plain elementwise copy (torch mul by 1.0) of %d MiB read + %d MiB written.\n"
                    % (CALIB_BYTES >> 20, CALIB_BYTES >> 20))
            f.write("# kernel trace (per kernel: calls, average / min / max ns):\n")
            for name, calls, avg, mn, mx in stats:
                f.write("#   %-90s %6d %12.1f %12.1f %12.1f\n" % (name[:90], calls, avg, mn, mx))
            f.write("kernel = %s\n" % kname)
            f.write("dominant = %s\n" % (kname == dominant))
            f.write("source_hash = %s\n" % kernel_source_hash())
            f.write("algorithmic_bytes_per_dispatch = %s\n" % kbytes)
            f.write("dispatches_counted = %d / %d\n" % (nf, nw))
            f.write("fetch_kib_per_dispatch = %s\n" % fetch)
            f.write("write_kib_per_dispatch = %s\n" % write)
            f.write("fetch_scale = %s\nwrite_scale = %s\n" % (f_scale, w_scale))
            f.write("hbm_read_bytes_per_dispatch = %s\n" % (None if rd is None else int(rd)))
            f.write("hbm_write_bytes_per_dispatch = %s\n" % (None if wr is None else int(wr)))
            f.write("hbm_bytes_per_dispatch = %s\n" % (None if rd is None or wr is None else int(rd + wr)))
            dom_avg = [avg for name, _, avg, _, _ in stats if match(name)]
            f.write("trace_avg_ns = %s\n" % (dom_avg[0] if dom_avg else None))
            if dom_avg and kbytes:
                f.write("achieved_gb_s = %.1f\n" % (kbytes / dom_avg[0]))
        print(out)


def summarize_mfma(args):
    """profiles/<kernel>_<workload>_mfma.txt: matrix-core counters of one kernel from a
    --pmc run (SQ_INSTS_VALU_MFMA_MOPS_F16, SQ_INSTS_VALU_MFMA_MOPS_BF16,
    SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE) and a kernel-trace run."""
    import csv

    kname, pmc_csv, stats_csv = args.summarize_mfma
    vals = {}
    with open(pmc_csv) as f:
        for row in csv.DictReader(f):
            if kname in row.get("Kernel_Name", ""):
                vals.setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
    avg = {c: sum(v) / len(v) for c, v in vals.items()}
    full_name = None
    stats = []
    with open(stats_csv) as f:
        for row in csv.DictReader(f):
            stats.append((row["Name"], int(row["Calls"]), float(row["AverageNs"]), float(row["MinNs"]),
                          float(row["MaxNs"])))
            if kname in row["Name"] and full_name is None:
                full_name = row["Name"]
    trace_ns = next((a for n, _, a, _, _ in stats if kname in n), None)
    mops = avg.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0) + avg.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)
    # busy cycles are summed over the SIMDs; the kernel's own cycles come from its
    # trace duration at the peak clock (GRBM_GUI_ACTIVE is summed over the 8 XCDs and
    # spans the counter window around each dispatch, so it is only reported)
    busy = avg.get("SQ_VALU_MFMA_BUSY_CYCLES")
    util = 100.0 * busy / (trace_ns * PEAK_CLOCK_GHZ * SIMDS) if busy is not None and trace_ns else None
    mfma_flops = mops * 512
    stem = re.sub(r"[^A-Za-z0-9]+", "_", kname).strip("_")
    out = os.path.join(PROFILES, "%s_%s_mfma.txt" % (stem, args.workload))
    os.makedirs(PROFILES, exist_ok=True)
    tiles = getattr(args, "tiles", None)
    extra = " --tiles '%s'" % tiles if tiles else ""
    with open(out, "w") as f:
        f.write("# rocprofv3 matrix-core summary: %s, workload %s\n" % (kname, args.workload))
        f.write("# commands (run from the repository root on one MI355X):\n")
        f.write("#   rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run -- "
                "python3 bench.py --workload %s --no-cpu-baseline --no-parity --no-graph%s\n" % (args.workload, extra))
        f.write("#   rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES "
                "GRBM_GUI_ACTIVE --output-format csv -d <dir> -o mfma -- "
                "python3 bench.py --workload %s --no-cpu-baseline --no-parity --no-graph%s --steps 50\n"
                % (args.workload, extra))
        f.write("#   python3 bench.py --workload %s%s --summarize-mfma '%s' <mfma csv> <stats csv>\n"
                % (args.workload, extra, kname))
        f.write("# matrix-core busy %% = SQ_VALU_MFMA_BUSY_CYCLES (summed over SIMDs) / (trace duration x %.1f GHz x %d "
                "SIMDs)\n" % (PEAK_CLOCK_GHZ, SIMDS))
        f.write("# executed matrix flops = (MOPS_F16 + MOPS_BF16) x 512, per dispatch\n")
        f.write("# kernel trace (per kernel: calls, average / min / max ns):\n")
        for name, calls, a, mn, mx in stats:
            f.write("#   %-90s %6d %12.1f %12.1f %12.1f\n" % (name[:90], calls, a, mn, mx))
        f.write("kernel = %s\n" % (full_name or kname))
        f.write("source_hash = %s\n" % kernel_source_hash())
        f.write("dispatches_counted = %d\n" % max((len(v) for v in vals.values()), default=0))
        for c in sorted(avg):
            f.write("%s_per_dispatch = %.1f\n" % (c, avg[c]))
        f.write("mfma_flops_per_dispatch = %.0f\n" % mfma_flops)
        f.write("mfma_busy_pct_at_peak_clock = %s\n" % (None if util is None else round(util, 3)))
        f.write("trace_avg_ns = %s\n" % trace_ns)
        if trace_ns:
            f.write("executed_mfma_tflops = %.2f\n" % (mfma_flops / trace_ns / 1e3))
    print(out)


def parse():
    import workloads

    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=500,
                    help="untimed steps first (enough for the clock to settle: with 20 the first timed region ran ~9 %% slow)")
    ap.add_argument("--workload", default=workloads.PAGES.name,
                    choices=[w.name for w in workloads.DECODE + workloads.PREFILL + [workloads.GEMM]])
    ap.add_argument("--min-rotate-mib", type=float, default=512.0)
    ap.add_argument("--breakdown-steps", type=int, default=400, help="launches per kernel in the breakdown pass")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay measurement")
    ap.add_argument("--tiles", default=None,
                    help="JSON tile override of the decode step (decode_attn_tiles_t fields), e.g. "
                         "'{\"step_mode\": 2, \"proj_tile_n\": 256}'")
    ap.add_argument("--no-floor", action="store_true", help="skip the streaming-read floor of the step's bytes")
    ap.add_argument("--summarize-profile", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "TRACE_STATS_CSV"),
                    help="write the PMC/trace summary of a profiled run to profiles/ and exit")
    ap.add_argument("--profile-tag", default="", help="suffix of the summary file names (a tile variant)")
    ap.add_argument("--summarize-mfma", nargs=3, metavar=("KERNEL", "PMC_CSV", "TRACE_STATS_CSV"),
                    help="write the matrix-core counter summary of kernel KERNEL (a name prefix) in a profiled run "
                         "of --workload to profiles/ and exit")
    return ap.parse_args()


def main():
    args = parse()
    if args.summarize_profile:
        summarize_profile(args)
        return
    if args.summarize_mfma:
        summarize_mfma(args)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the decode step runs on exactly one GPU; --gpus %d (WORLD_SIZE %d) is not supported "
              "(sharding across GPUs is not implemented)." % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import decode_attention_output_amd as da
    import workloads

    wl = workloads.BY_NAME[args.workload]
    if isinstance(wl, workloads.PrefillWorkload):
        bench_prefill(args, wl)
        return
    if isinstance(wl, workloads.GemmWorkload):
        bench_gemm(args, wl)
        return
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
    # every launch goes to one dedicated stream (a graph must be captured on a non-default stream)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    torch.cuda.set_stream(stream)

    tiles = json.loads(args.tiles) if args.tiles else None
    for st in sets:
        st["step"] = da.DecodeStep(st["q"], st["k"], st["v"], sl, st["o_weight"], out=st["out"], workspace=st["ws"],
                                   stream=stream, tiles=tiles)

    plan = da.decode_attn_plan(da.make_shape(s.batch, s.num_q_heads, s.num_kv_heads, s.max_seq_len, s.hidden, s.head_dim,
                                             tiles=tiles))

    # the streaming floor first: its launches also bring the GPU out of idle before the warm-up
    floor = None if args.no_floor else stream_floor(alg_bytes, stream, args.min_rotate_mib)

    # ---- warm-up, then exactly `steps` timed steps (one prepared C-ABI call each) ----
    for i in range(args.warmup):
        sets[i % R]["step"]()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        sets[i % R]["step"]()
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_us = (t1 - t0) / args.steps * 1e6
    gpu_us = ev0.elapsed_time(ev1) * 1e3 / args.steps

    def run_steps(e0, e1, rotate):
        e0.record(stream)
        for i in range(args.steps):
            sets[i % R if rotate else 0]["step"]()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    repeats_us, median_us, warm_us = repeat_and_warm(run_steps, args.steps)

    # ---- the same steps replayed from a HIP graph (no host work per step) ----
    graph_us = None
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(args.steps):
                sets[i % R]["step"]()
        torch.cuda.synchronize()
        g.replay()  # first replay uploads the graph
        torch.cuda.synchronize()
        gv0, gv1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gv0.record(stream)
        g.replay()
        gv1.record(stream)
        torch.cuda.synchronize()
        graph_us = gv0.elapsed_time(gv1) * 1e3 / args.steps
        del g

    # ---- per-kernel pass: the attention launch alone and the projection launch alone ----
    # Each is timed like the step: n_b back-to-back launches on the bench stream between
    # two HIP events, cycling through the rotation sets; the average per launch is the
    # kernel's launch duration (the rocprofv3 kernel trace of the same command agrees).
    n_b = args.breakdown_steps
    for st in sets:
        st["attn"] = da.AttentionStep(st["q"], st["k"], st["v"], sl, out=st["flat"], workspace=st["ws"], stream=stream,
                                      tiles=tiles)
        st["proj"] = da.OprojStep(st["flat"], st["o_weight"], out=st["out"], workspace=st["ws"], stream=stream)

    def avg_launch_us(name):
        for i in range(min(R, 10)):
            sets[i % R][name]()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n_b):
            sets[i % R][name]()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n_b

    attn_us = avg_launch_us("attn")
    oproj_us = avg_launch_us("proj")
    step_us = gpu_us  # the timed region above
    # restore the step's own output in set 0 for the parity check
    sets[0]["step"]()
    torch.cuda.synchronize()
    # the single-launch steps' bounded waits never gave up in any of the calls above
    step_status = [da.decode_attn_step_status(st["ws"], stream) for st in sets]
    if any(rc != da.DA_OK for rc in step_status):
        raise da.DecodeAttnError(next(rc for rc in step_status if rc != da.DA_OK), "decode step (status)")

    kname, kbytes, which = dominant_kernel(wl, plan, seq_lens)
    dom_us = {"oproj": oproj_us, "attention": attn_us, "step": step_us}[which]
    achieved = kbytes / (dom_us * 1e-6) / 1e9
    traffic = traffic_from_profile(wl.name, kname)

    # a plain elementwise copy of known size, outside the timed region: the HBM
    # counters of a profiled run are scaled by what they read for it
    calib_src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
    calib_dst = torch.empty_like(calib_src)
    torch.mul(calib_src, 1.0, out=calib_dst)
    torch.cuda.synchronize()
    del calib_src, calib_dst

    result = {
        "metric": METRIC,
        "value": round(alg_bytes / (wall_us * 1e-6) / 1e12, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_us / 1e3, 6),
        "us_per_step": round(wall_us, 3),
        "us_per_step_gpu_events": round(gpu_us, 3),
        "us_per_step_graph_replay": None if graph_us is None else round(graph_us, 3),
        "us_per_step_repeats": repeats_us,
        "us_per_step_median": median_us,
        "us_per_step_warm": warm_us,
        "warm_note": "one buffer set, so the Infinity Cache and L2 may serve it; value uses rotated sets",
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
            "kernel": kname,
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "avg_launch_us": round(dom_us, 3),
            "alg_bytes_per_launch": kbytes,
            "timing": ("HIP events around the timed steps (one launch each) on the bench stream" if which == "step"
                       else "HIP events around %d back-to-back launches of this kernel alone on the bench stream"
                       % n_b),
        },
        "breakdown_us": {"step": round(step_us, 3), "attention_alone": round(attn_us, 3),
                         "oproj_alone": round(oproj_us, 3)},
        "stream_floor": floor,
        "step_status": "ok",
    }
    if tiles:
        result["config"]["tiles"] = tiles

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
        if wl.name in (workloads.TINY.name, workloads.PAGES.name):
            # the same oracle on one host thread
            sec, n1 = oracle_single_thread(lambda: oracle.decode_step(full["q"], full["k"], full["v"], full["seq_lens"],
                                                                      full["o_weight"], nthreads=1))
            result["cpu_baseline"]["single_thread"] = {
                "value": round(alg_bytes / sec / 1e12, 6), "us_per_step": round(sec * 1e6, 1), "cores": 1,
                "sample": "%d full decode steps on one thread" % n1}
    print(json.dumps(result), flush=True)


def bench_prefill(args, wl):
    """One step = the attention of one token chunk of every sequence (one launch)."""
    import numpy as np
    import torch

    import decode_attention_output_amd as da
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    da.load_library()
    inp = workloads.prefill_inputs(wl, poison=True)
    ctx = inp["ctx_lens"]
    flops = workloads.prefill_flops(wl.tokens, wl.num_q_heads, wl.head_dim, ctx)
    nbytes = prefill_alg_bytes(wl)

    def to_dev(words):
        return torch.from_numpy(np.ascontiguousarray(words).view(np.int16)).view(torch.bfloat16).to(dev)

    base = {n: to_dev(inp[n]) for n in ("q", "k", "v")}
    cl = torch.from_numpy(ctx).to(dev)
    R = max(1, math.ceil(args.min_rotate_mib * 2 ** 20 / nbytes))
    sets = []
    for r in range(R):
        st = {n: (t if r == 0 else t.clone()) for n, t in base.items()}
        st["out"] = torch.empty((wl.batch, wl.tokens, wl.num_q_heads * wl.head_dim), dtype=torch.bfloat16,
                                device=dev)
        sets.append(st)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    torch.cuda.set_stream(stream)

    def step(st):
        da.prefill_attn_fwd(st["q"], st["k"], st["v"], cl, out=st["out"], stream=stream)

    for i in range(args.warmup):
        step(sets[i % R])
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(sets[i % R])
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_us = (time.perf_counter() - t0) / args.steps * 1e6
    gpu_us = ev0.elapsed_time(ev1) * 1e3 / args.steps

    def run_steps(e0, e1, rotate):
        e0.record(stream)
        for i in range(args.steps):
            step(sets[i % R if rotate else 0])
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    repeats_us, median_us, warm_us = repeat_and_warm(run_steps, args.steps)
    step(sets[0])
    torch.cuda.synchronize()

    # the elementwise copy whose counters scale a profiled run's HBM bytes
    calib_src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
    calib_dst = torch.empty_like(calib_src)
    torch.mul(calib_src, 1.0, out=calib_dst)
    torch.cuda.synchronize()
    del calib_src, calib_dst

    achieved = flops / (gpu_us * 1e-6) / 1e12
    result = {
        "metric": PREFILL_METRIC,
        "value": round(flops / (wall_us * 1e-6) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_us / 1e3, 6),
        "us_per_step": round(wall_us, 3),
        "us_per_step_gpu_events": round(gpu_us, 3),
        "us_per_step_repeats": repeats_us,
        "us_per_step_median": median_us,
        "us_per_step_warm": warm_us,
        "warm_note": "one buffer set, so the Infinity Cache and L2 may serve it; value uses rotated sets",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "batch": wl.batch, "tokens": wl.tokens, "num_q_heads": wl.num_q_heads,
            "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim, "ctx_len": wl.ctx_len,
            "algorithmic_flops": flops, "algorithmic_bytes": nbytes, "rotation_sets": R,
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "prefill_kernel",
            "achieved": round(achieved, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": traffic_from_profile(wl.name, "prefill_kernel"),
            "avg_launch_us": round(gpu_us, 3),
            "alg_flops_per_launch": flops,
            "timing": "HIP events around the timed steps (one launch each) on the bench stream",
        },
    }
    if not args.no_parity or not args.no_cpu_baseline:
        # one bounded oracle sample serves both: the first sequence's chunk (its
        # output is compared element by element, and the runs are timed)
        import oracle

        threads = oracle.default_threads()
        sub = {n: np.ascontiguousarray(inp[n][:1]) for n in ("q", "k", "v")}
        sub_flops = workloads.prefill_flops(wl.tokens, wl.num_q_heads, wl.head_dim, ctx[:1])
        n, t_cpu, ref = 0, 0.0, None
        while n < 1 or (not args.no_cpu_baseline and t_cpu < args.cpu_seconds and n < 100):
            c0 = time.perf_counter()
            ref = oracle.prefill_attention(sub["q"], sub["k"], sub["v"], ctx[:1], nthreads=threads)["ref"]
            t_cpu += time.perf_counter() - c0
            n += 1
    if not args.no_parity:
        got = torch.from_numpy(sets[0]["out"][:1].cpu().view(torch.int16).numpy()).view(torch.bfloat16)
        got = got.double().numpy()
        err = np.abs(got - ref)
        mask = np.abs(ref) >= 1e-2
        rel = float((err[mask] / np.abs(ref[mask])).max()) if mask.any() else 0.0
        ok = bool(np.all(np.isfinite(got)) and err.max() <= 1e-2 and rel <= 2.0 ** -7)
        result["parity"] = {"vs": "oracle", "ok": ok, "max_abs": float(err.max()), "max_rel": rel,
                            "checked": "every output of the first sequence's chunk"}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = {
            "value": round(sub_flops * n / t_cpu / 1e12, 6),
            "unit": "TFLOP/s",
            "cores": threads,
            "kind": "oracle",
            "sample": "%d run(s) of the first sequence's %d-token chunk of %s (fp64 C oracle, %d threads, %.1f s)"
                      % (n, wl.tokens, wl.name, threads, t_cpu),
        }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
