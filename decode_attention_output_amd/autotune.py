"""Measured tile search: per-shape table rows and built-in rules.

The per-matmul tile lesson of "PyPTO 开箱性能调优实战：Decode Attention 多 Matmul
独立 TileShape 配置 F-16" (sections 核心原则 and 迭代过程) is that each matmul of
the step needs its own tile and that the right one is found by measuring; the
page "CCCL → Triton 方法论迁移" (section 一) adds how a rule is chosen: run every
candidate on several problem sizes and keep the one with the best geometric
mean. This tool does both on the GPU through the C ABI's tile override
(decode_attn_tiles_t):

  search   one shape: attention tiles (stream-K workgroups x pipeline depth x
           the per-sequence charge), then projection tiles (column tile x K
           split) on top of the best of them, or the small single-launch
           step's own knobs, each timed as the whole step against the built-in
           choice. The winner is timed once more in alternation with the
           built-in choice; with --emit it becomes the shape's row of the
           measured tile table (csrc/tile_table.inc) only if it beats the
           built-in choice by more than the repeat spread of the two, and
           otherwise the shape's row is removed (the built-in rules serve it).
  rules    candidate settings applied to every shape of a set (by default the
           benchmarked decode workloads and the one-GPU shares of a sharded
           step); each candidate's time is divided by the built-in time of the
           same shape, and the candidate with the best geometric mean of those
           ratios is reported as the rule to build in.

"Built-in choice" means the library's rules alone: an override whose fields
are all zero bypasses the measured table as well. Every candidate is timed over
rotated copies of the inputs (at least 512 MiB, twice the Infinity Cache) with
HIP events on one stream; a measurement is the median of several repeats, its
spread the difference between the slowest and the fastest repeat. Every
candidate's output is compared with the built-in choice's (two correct results
differ by at most a couple of bf16 ulps).

    python -m decode_attention_output_amd.autotune search --workload decode_b4_h64kv8_L32768_o8192 --emit
    python -m decode_attention_output_amd.autotune rules
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
TABLE = os.path.join(HERE, "csrc", "tile_table.inc")
TILE_FIELDS = ("attn_workgroups", "attn_depth", "proj_tile_n", "proj_ksplit", "step_mode", "attn_seq_cost",
               "step_weight_delay")


def _parse_list(text):
    return [int(x) for x in text.split(",") if x.strip()]


# ---- selection logic (host only) ------------------------------------------

class Timing:
    """Repeat times of one measurement (µs per launch)."""

    def __init__(self, samples):
        self.samples = list(samples)

    @property
    def median(self):
        return statistics.median(self.samples)

    @property
    def spread(self):
        return max(self.samples) - min(self.samples)

    def as_dict(self):
        return {"median_us": round(self.median, 3), "spread_us": round(self.spread, 3),
                "samples": [round(x, 3) for x in self.samples]}


def significant(best: Timing, builtin: Timing) -> bool:
    """A candidate replaces the built-in choice only if its median is lower by more than
    the larger of the two repeat spreads (a smaller gap is inside the measurement noise)."""
    return builtin.median - best.median > max(best.spread, builtin.spread)


def geomean(values):
    values = list(values)
    return math.exp(sum(math.log(v) for v in values) / len(values))


def select_rule(times):
    """times: {candidate key: {shape: Timing}} with the built-in choice under key None.
    Returns (best key, {key: geometric mean of candidate / built-in medians}); a candidate
    must have run on every shape the built-in ran on (missing = not allowed there)."""
    base = times[None]
    ratios = {}
    for key, per_shape in times.items():
        if set(per_shape) != set(base):
            continue
        ratios[key] = geomean(per_shape[s].median / base[s].median for s in base)
    best = min(ratios, key=lambda k: (ratios[k], k is not None))
    return best, ratios


def emit_entry(path, shape, tiles, note):
    """Insert or replace the table row of `shape` (a dict of batch, num_q_heads, num_kv_heads,
    head_dim, max_seq_len, hidden); the header comment and the other rows are kept, rows sorted
    by shape. `tiles` None removes the shape's row."""
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
    if tiles is None:
        rows.pop(key, None)
    else:
        vals = list(key) + [int(tiles.get(n, 0)) for n in TILE_FIELDS]
        rows[key] = "TILE_ENTRY(%s)  // %s\n" % (", ".join(str(v) for v in vals), note)
    with open(path, "w") as f:
        f.writelines(head)
        f.writelines(rows[k] for k in sorted(rows))


# ---- measurement on the GPU ------------------------------------------------

class Bench:
    """Seeded inputs of one decode workload in rotated copies, and timers of prepared calls."""

    def __init__(self, wl, launches, repeats, min_rotate_mib):
        import numpy as np
        import torch

        import decode_attention_output_amd as da
        import workloads

        self.da, self.np, self.torch, self.wl = da, np, torch, wl
        self.launches, self.repeats = launches, repeats
        s = wl.shape
        dev = torch.device("cuda:0")
        inp = workloads.decode_inputs(wl, poison=True)
        self.seq_lens = inp["seq_lens"]
        self.alg_bytes = workloads.algorithmic_bytes(s, self.seq_lens)
        self.kv_bytes = 2 * 2 * s.num_kv_heads * s.head_dim * int(np.sum(self.seq_lens))

        def to_dev(words):
            return torch.from_numpy(np.ascontiguousarray(words).view(np.int16)).view(torch.bfloat16).to(dev)

        base = {n: to_dev(inp[n]) for n in ("q", "k", "v", "o_weight")}
        del inp
        self.sl = torch.from_numpy(self.seq_lens).to(dev)
        R = max(1, math.ceil(min_rotate_mib * 2 ** 20 / self.alg_bytes))
        self.sets = []
        for r in range(R):
            st = {n: (t if r == 0 else t.clone()) for n, t in base.items()}
            st["out"] = torch.empty((s.batch, s.hidden), dtype=torch.bfloat16, device=dev)
            st["ws"] = da.Workspace(dev)
            self.sets.append(st)
        self.stream = torch.cuda.Stream()
        torch.cuda.synchronize()
        self.step_calls(None)[0]()
        torch.cuda.synchronize()
        self.ref = self.bf16_to_f64(self.sets[0]["out"])

    def bf16_to_f64(self, t):
        torch, np = self.torch, self.np
        return torch.from_numpy(t.cpu().view(torch.int16).numpy()).view(torch.bfloat16).double().numpy()

    def step_calls(self, tiles):
        da = self.da
        return [da.DecodeStep(st["q"], st["k"], st["v"], self.sl, st["o_weight"], out=st["out"], workspace=st["ws"],
                              stream=self.stream, tiles=tiles) for st in self.sets]

    def _once(self, calls):
        torch = self.torch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        for i in range(self.launches):
            calls[i % len(calls)]()
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / self.launches

    def _warm(self, calls):
        for i in range(max(20, len(calls))):
            calls[i % len(calls)]()
        self.torch.cuda.synchronize()

    def time(self, calls):
        self._warm(calls)
        return Timing(self._once(calls) for _ in range(self.repeats))

    def time_pair(self, calls_a, calls_b, rounds):
        """Both call lists timed in alternation (a, b, a, b, ...), so that a drift of the clock
        or the temperature over the measurement falls on both alike."""
        self._warm(calls_a)
        self._warm(calls_b)
        ta, tb = [], []
        for _ in range(rounds):
            ta.append(self._once(calls_a))
            tb.append(self._once(calls_b))
        return Timing(ta), Timing(tb)

    def try_tiles(self, tiles):
        """Timing of the step under `tiles`, or None if the tiles are outside what the shape
        allows or change the result."""
        np = self.np
        try:
            calls = self.step_calls(tiles)
        except self.da.DecodeAttnError:
            return None
        t = self.time(calls)
        calls[0]()
        self.torch.cuda.synchronize()
        got, ref = self.bf16_to_f64(self.sets[0]["out"]), self.ref
        err = np.abs(got - ref)
        if not np.all(np.isfinite(got)) or (err > 2.0 ** -6 * np.maximum(np.abs(ref), 1e-2)).any():
            return None
        if any(self.da.decode_attn_step_status(st["ws"], self.stream) != self.da.DA_OK for st in self.sets):
            return None
        return t

    def shape(self):
        s = self.wl.shape
        return {"batch": s.batch, "num_q_heads": s.num_q_heads, "num_kv_heads": s.num_kv_heads,
                "max_seq_len": s.max_seq_len, "hidden": s.hidden, "head_dim": s.head_dim}


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    sub = ap.add_subparsers(dest="mode", required=True)
    for name in ("search", "rules"):
        p = sub.add_parser(name)
        p.add_argument("--launches", type=int, default=100, help="timed launches per repeat")
        p.add_argument("--repeats", type=int, default=7)
        p.add_argument("--min-rotate-mib", type=float, default=512.0)
    s = sub.choices["search"]
    s.add_argument("--workload", required=True)
    s.add_argument("--attn-wgs", default="128,144,160,176,192,224,256")
    s.add_argument("--attn-depth", default="1,2")
    s.add_argument("--seq-cost", default="1,3,6,12")
    s.add_argument("--tile-n", default="64,128,256,512")
    s.add_argument("--ksplit", default="0,2,4,8,16")
    s.add_argument("--step-wgs", default="64,96,128,192,256",
                   help="attention workgroups aimed at in the single-launch step")
    s.add_argument("--weight-delay", default="0,50,100", help="single-launch step: weight delay, 10 ns ticks")
    s.add_argument("--skip", default="", help="comma list of stages to skip: attn,proj,mode")
    s.add_argument("--emit", action="store_true", help="write (or remove) the shape's row of csrc/tile_table.inc")
    s.add_argument("--table", default=TABLE, help=argparse.SUPPRESS)
    r = sub.choices["rules"]
    r.add_argument("--shapes", default="", help="comma list of workload names (default: the benchmarked decode "
                                                 "workloads and the one-GPU shares of sharded steps)")
    r.add_argument("--candidates", default="", help="JSON list of tile dicts applied to every shape")
    return ap.parse_args(argv)


DEFAULT_RULE_CANDIDATES = [
    {"attn_workgroups": 160}, {"attn_workgroups": 224}, {"attn_workgroups": 256},
    {"attn_seq_cost": 1}, {"attn_seq_cost": 3}, {"attn_seq_cost": 12},
    {"proj_ksplit": 2}, {"proj_ksplit": 8},
]


def run_search(args):
    import workloads

    wl = workloads.BY_NAME[args.workload]
    b = Bench(wl, args.launches, args.repeats, args.min_rotate_mib)
    da = b.da
    skip = set(x for x in args.skip.split(",") if x)

    def report(stage, tiles, t):
        row = {"stage": stage, "tiles": tiles, "ok": t is not None}
        if t is not None:
            row.update(t.as_dict())
        print(json.dumps(row), flush=True)
        return t

    builtin = report("builtin", {}, b.try_tiles({}))
    best, best_t = {}, builtin
    plan = da.decode_attn_plan(da.make_shape(**b.shape()))
    if "attn" not in skip and plan.fused not in (1, 3):
        # attention tiles timed in the whole step: in the single-launch step the projection's
        # workgroups share the chip with the attention's, so the attention alone misleads
        best_a = {}
        for w, d, c in itertools.product(_parse_list(args.attn_wgs), _parse_list(args.attn_depth),
                                         _parse_list(args.seq_cost)):
            t = {"attn_workgroups": w, "attn_depth": d, "attn_seq_cost": c}
            tm = report("attn", t, b.try_tiles(t))
            if tm is not None and tm.median < best_t.median:
                best, best_t, best_a = t, tm, t
        for tn, ks in itertools.product(_parse_list(args.tile_n), _parse_list(args.ksplit)):
            t = dict(best_a, proj_tile_n=tn, proj_ksplit=ks)
            tm = report("proj", t, b.try_tiles(t))
            if tm is not None and tm.median < best_t.median:
                best, best_t = t, tm
    if "mode" not in skip and plan.fused in (1, 3):
        # (a tiny step, fused 3, has no tiles of its own: the small step's are its alternatives)
        for w, tn, dl in itertools.product([0] + _parse_list(args.step_wgs), [0, 128, 256, 512],
                                           _parse_list(args.weight_delay)):
            t = {"step_mode": 1, "attn_workgroups": w, "proj_tile_n": tn, "step_weight_delay": dl}
            tm = report("mode", t, b.try_tiles(t))
            if tm is not None and tm.median < best_t.median:
                best, best_t = t, tm
    # the winner again, beside the built-in choice, so that both spreads come from the same moment
    # the winner once more, in alternation with the built-in choice
    final_best, final_builtin = b.time_pair(b.step_calls(best), b.step_calls({}), 2 * args.repeats + 1)
    keep = bool(best) and significant(final_best, final_builtin)
    summary = {"workload": wl.name, "best": best, "best_timing": final_best.as_dict(),
               "builtin_timing": final_builtin.as_dict(), "significant": keep, "shape": b.shape()}
    print(json.dumps(summary), flush=True)
    if args.emit:
        emit_entry(args.table, b.shape(), best if keep else None, "%s: %.2f us (built-in %.2f us, spread %.2f)" % (
            wl.name, final_best.median, final_builtin.median, max(final_best.spread, final_builtin.spread)))


def run_rules(args):
    import workloads

    names = [x for x in args.shapes.split(",") if x] or [w.name for w in workloads.RULE_SHAPES]
    cands = json.loads(args.candidates) if args.candidates else DEFAULT_RULE_CANDIDATES
    times = {None: {}}
    for name in names:
        b = Bench(workloads.BY_NAME[name], args.launches, args.repeats, args.min_rotate_mib)
        t0 = b.try_tiles({})
        times[None][name] = t0
        print(json.dumps({"shape": name, "tiles": {}, **t0.as_dict()}), flush=True)
        for c in cands:
            t = b.try_tiles(c)
            key = json.dumps(c, sort_keys=True)
            if t is not None:
                times.setdefault(key, {})[name] = t
            print(json.dumps({"shape": name, "tiles": c, "ok": t is not None,
                              **(t.as_dict() if t is not None else {})}), flush=True)
        del b
    best, ratios = select_rule(times)
    print(json.dumps({"geomean_ratio_vs_builtin": {("builtin" if k is None else k): round(v, 4)
                                                   for k, v in sorted(ratios.items(), key=lambda kv: kv[1])},
                      "best": None if best is None else json.loads(best)}), flush=True)


def main(argv=None):
    args = parse(argv)
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import torch

    import decode_attention_output_amd as da

    torch.cuda.set_device(0)
    da.load_library()
    if args.mode == "search":
        run_search(args)
    else:
        run_rules(args)


if __name__ == "__main__":
    main()
