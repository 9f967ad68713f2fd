"""Measured tile search for one decode-step shape.

The per-matmul tile lesson of "PyPTO 开箱性能调优实战：Decode Attention 多 Matmul
独立 TileShape 配置 F-16" (sections 核心原则 and 迭代过程) is that each matmul of
the step needs its own tile and that the right one is found by measuring. This
tool does that search on the GPU through the C ABI's tile override
(decode_attn_tiles_t), one matmul group at a time:

  1. attention (QK^T, softmax, attn x V): stream-K workgroups x pipeline depth,
     timed with decode_attn_only;
  2. projection (attn_output_flat x o_weight): column tile x K split, timed as
     the whole step in two launches with the best attention tiles;
  3. where the single-launch step supports the shape: its attention pieces x
     projection column tile, against two launches.

Every candidate is timed over rotated copies of the inputs (at least 512 MiB,
twice the Infinity Cache) with HIP events on one stream, median of several
repeats, and its output is compared with the built-in choice's output (two
correct results differ by at most a couple of bf16 ulps). The result is one
JSON line per candidate and a final line with the best tiles; with --emit the
best tiles become the shape's row of the measured tile table
(csrc/tile_table.inc), which the library consults for calls without an
override of their own (rebuild after emitting).

    python -m decode_attention_output_amd.autotune --workload decode_b4_h64kv8_L32768_o8192 --emit
"""
from __future__ import annotations

import argparse
import itertools
import json
import math
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _parse_list(text):
    return [int(x) for x in text.split(",") if x.strip()]


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", required=True)
    ap.add_argument("--attn-wgs", default="128,192,256,320,384,512,768")
    ap.add_argument("--attn-depth", default="1,2,3")
    ap.add_argument("--tile-n", default="64,128,256,512")
    ap.add_argument("--ksplit", default="0,1,2,4,8,16,32")
    ap.add_argument("--launches", type=int, default=100, help="timed launches per repeat")
    ap.add_argument("--repeats", type=int, default=5)
    ap.add_argument("--min-rotate-mib", type=float, default=512.0)
    ap.add_argument("--step-wgs", default="32,64,96,128,192,256",
                    help="attention workgroups aimed at in the single-launch step")
    ap.add_argument("--skip", default="", help="comma list of stages to skip: attn,proj,mode")
    ap.add_argument("--emit", action="store_true", help="write the best tiles into csrc/tile_table.inc")
    ap.add_argument("--table", default=TABLE, help=argparse.SUPPRESS)
    return ap.parse_args(argv)


TABLE = os.path.join(HERE, "csrc", "tile_table.inc")
TILE_FIELDS = ("attn_workgroups", "attn_depth", "proj_tile_n", "proj_ksplit", "step_mode")


def emit_entry(path, shape, tiles, note):
    """Insert or replace the table row of `shape` (a dict of batch, num_q_heads, num_kv_heads,
    head_dim, max_seq_len, hidden); the header comment and the other rows are kept, rows sorted
    by shape."""
    key = (shape["batch"], shape["num_q_heads"], shape["num_kv_heads"], shape["head_dim"], shape["max_seq_len"],
           shape["hidden"])
    head, rows = [], {}
    with open(path) as f:
        for line in f:
            if line.startswith("TILE_ENTRY("):
                vals = [int(v) for v in line[len("TILE_ENTRY("):line.index(")")].split(",")]
                rows[tuple(vals[:6])] = line
            else:
                head.append(line)
    vals = list(key) + [int(tiles.get(n, 0)) for n in TILE_FIELDS]
    rows[key] = "TILE_ENTRY(%s)  // %s\n" % (", ".join(str(v) for v in vals), note)
    with open(path, "w") as f:
        f.writelines(head)
        f.writelines(rows[k] for k in sorted(rows))


def main(argv=None):
    args = parse(argv)
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
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

    def to_dev(words):
        return torch.from_numpy(np.ascontiguousarray(words).view(np.int16)).view(torch.bfloat16).to(dev)

    base = {n: to_dev(inp[n]) for n in ("q", "k", "v", "o_weight")}
    del inp
    sl = torch.from_numpy(seq_lens).to(dev)
    R = max(1, math.ceil(args.min_rotate_mib * 2 ** 20 / alg_bytes))
    sets = []
    for r in range(R):
        st = {n: (t if r == 0 else t.clone()) for n, t in base.items()}
        st["out"] = torch.empty((s.batch, s.hidden), dtype=torch.bfloat16, device=dev)
        st["flat"] = torch.empty((s.batch, s.o_in), dtype=torch.bfloat16, device=dev)
        st["ws"] = da.Workspace(dev)
        sets.append(st)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    torch.cuda.set_stream(stream)

    def time_calls(calls):
        """Median µs per launch of the prepared calls, cycled over the rotation sets."""
        for i in range(max(10, len(calls))):
            calls[i % len(calls)]()
        torch.cuda.synchronize()
        res = []
        for _ in range(args.repeats):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(args.launches):
                calls[i % len(calls)]()
            e1.record(stream)
            torch.cuda.synchronize()
            res.append(e0.elapsed_time(e1) * 1e3 / args.launches)
        return statistics.median(res)

    def bf16_to_f64(t):
        return torch.from_numpy(t.cpu().view(torch.int16).numpy()).view(torch.bfloat16).double().numpy()

    def differs(got, ref):
        err = np.abs(got - ref)
        return bool(not np.all(np.isfinite(got)) or (err > 2.0 ** -6 * np.maximum(np.abs(ref), 1e-2)).any())

    def attn_calls(tiles):
        return [da.AttentionStep(st["q"], st["k"], st["v"], sl, out=st["flat"], workspace=st["ws"], stream=stream,
                                 tiles=tiles) for st in sets]

    def step_calls(tiles):
        return [da.DecodeStep(st["q"], st["k"], st["v"], sl, st["o_weight"], out=st["out"], workspace=st["ws"],
                              stream=stream, tiles=tiles) for st in sets]

    # outputs of the built-in choice: the reference every candidate must agree with
    attn_calls(None)[0]()
    step_calls(None)[0]()
    torch.cuda.synchronize()
    ref_flat = bf16_to_f64(sets[0]["flat"])
    ref_out = bf16_to_f64(sets[0]["out"])

    skip = set(x for x in args.skip.split(",") if x)
    rows = []

    def report(stage, tiles, us, ok, nbytes):
        row = {"stage": stage, "tiles": tiles, "us": round(us, 3), "tbs": round(nbytes / (us * 1e-6) / 1e12, 4),
               "ok": ok}
        rows.append(row)
        print(json.dumps(row), flush=True)

    def try_tiles(stage, tiles, calls_fn, ref, which, nbytes):
        try:
            calls = calls_fn(tiles)
        except da.DecodeAttnError:
            return None  # outside the ranges this shape allows
        us = time_calls(calls)
        calls[0]()
        torch.cuda.synchronize()
        ok = not differs(bf16_to_f64(sets[0][which]), ref)
        report(stage, tiles, us, ok, nbytes)
        return us if ok else None

    kv_bytes = 2 * 2 * s.num_kv_heads * s.head_dim * int(np.sum(seq_lens))
    best_attn, best_attn_us = {}, try_tiles("attn", {}, attn_calls, ref_flat, "flat", kv_bytes)
    if "attn" not in skip:
        for w, d in itertools.product(_parse_list(args.attn_wgs), _parse_list(args.attn_depth)):
            t = {"attn_workgroups": w, "attn_depth": d}
            us = try_tiles("attn", t, attn_calls, ref_flat, "flat", kv_bytes)
            if us is not None and us < best_attn_us:
                best_attn, best_attn_us = t, us

    two = dict(best_attn, step_mode=2)
    best_proj, best_proj_us = two, try_tiles("proj", two, step_calls, ref_out, "out", alg_bytes)
    if "proj" not in skip:
        for tn, ks in itertools.product(_parse_list(args.tile_n), _parse_list(args.ksplit)):
            t = dict(two, proj_tile_n=tn, proj_ksplit=ks)
            us = try_tiles("proj", t, step_calls, ref_out, "out", alg_bytes)
            if us is not None and (best_proj_us is None or us < best_proj_us):
                best_proj, best_proj_us = t, us

    best, best_us = best_proj, best_proj_us
    plan = da.decode_attn_plan(da.make_shape(s.batch, s.num_q_heads, s.num_kv_heads, s.max_seq_len, s.hidden, s.head_dim))
    if "mode" not in skip and plan.fused:
        # the single-launch step: attention workgroups aimed at x projection column tile
        for w, tn in itertools.product([0] + _parse_list(args.step_wgs), [0, 128, 256, 512]):
            t = {"step_mode": 1, "attn_workgroups": w, "proj_tile_n": tn}
            us = try_tiles("mode", t, step_calls, ref_out, "out", alg_bytes)
            if us is not None and us < best_us:
                best, best_us = t, us
    builtin_us = try_tiles("builtin", {}, step_calls, ref_out, "out", alg_bytes)
    shape = {"batch": s.batch, "num_q_heads": s.num_q_heads, "num_kv_heads": s.num_kv_heads,
             "max_seq_len": s.max_seq_len, "hidden": s.hidden, "head_dim": s.head_dim}
    print(json.dumps({"workload": wl.name, "best": best, "best_us": round(best_us, 3),
                      "builtin_us": None if builtin_us is None else round(builtin_us, 3), "shape": shape}),
          flush=True)
    if args.emit:
        emit_entry(args.table, shape, best, "%s: %.2f us (built-in %s us)" % (
            wl.name, best_us, "?" if builtin_us is None else "%.2f" % builtin_us))


if __name__ == "__main__":
    main()
