"""Host-side tools without a GPU: the tile-table writer of the measured tile
search and the benchmark's command-line contract."""
import os
import subprocess
import sys

import pytest

import decode_attention_output_amd as da
from decode_attention_output_amd import autotune

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _rows(path):
    with open(path) as f:
        return [l for l in f if l.startswith("TILE_ENTRY(")]


def test_emit_entry_inserts_replaces_and_sorts(tmp_path):
    table = tmp_path / "tile_table.inc"
    table.write_text(open(autotune.TABLE).read())
    head = [l for l in open(autotune.TABLE) if not l.startswith("TILE_ENTRY(")]
    big = dict(batch=64, num_q_heads=8, num_kv_heads=1, head_dim=128, max_seq_len=100, hidden=512)
    small = dict(batch=2, num_q_heads=8, num_kv_heads=1, head_dim=256, max_seq_len=100, hidden=512)
    n0 = len(_rows(table))
    autotune.emit_entry(str(table), big, {"attn_workgroups": 96, "step_mode": 2}, "first")
    autotune.emit_entry(str(table), small, {"proj_tile_n": 128}, "second")
    autotune.emit_entry(str(table), big, {"attn_workgroups": 64}, "replaced")
    rows = _rows(table)
    assert len(rows) == n0 + 2
    # the header comment is kept, rows are sorted by shape, a shape has one row
    assert [l for l in open(table) if not l.startswith("TILE_ENTRY(")] == head
    keys = [tuple(int(v) for v in r[len("TILE_ENTRY("):r.index(")")].split(",")[:6]) for r in rows]
    assert keys == sorted(keys) and len(set(keys)) == len(keys)
    mine = [r for r in rows if r.startswith("TILE_ENTRY(64, 8, 1, 128, 100, 512,")]
    assert mine == ["TILE_ENTRY(64, 8, 1, 128, 100, 512, 64, 0, 0, 0, 0, 0, 0)  // replaced\n"]
    assert "TILE_ENTRY(2, 8, 1, 256, 100, 512, 0, 0, 128, 0, 0, 0, 0)  // second\n" in rows
    # a row carries every field of the table, in the table's order; None removes the row
    autotune.emit_entry(str(table), small, {"attn_seq_cost": 3, "step_weight_delay": 50}, "all")
    assert "TILE_ENTRY(2, 8, 1, 256, 100, 512, 0, 0, 0, 0, 0, 3, 50)  // all\n" in _rows(table)
    autotune.emit_entry(str(table), small, None, "")
    assert not [r for r in _rows(table) if r.startswith("TILE_ENTRY(2, 8, 1, 256, 100, 512,")]
    assert len(_rows(table)) == n0 + 1


def test_tile_fields_follow_the_table_macro():
    # the table's row holds the shape, then the override fields in TILE_FIELDS order
    src = open(os.path.join(ROOT, "decode_attention_output_amd", "csrc", "abi.hip")).read()
    macro = src[src.index("#define TILE_ENTRY("):]
    args = [a.strip() for a in macro[len("#define TILE_ENTRY("):macro.index(")")].split(",")]
    assert len(args) == 6 + len(autotune.TILE_FIELDS)
    # the macro's body lists the decode_attn_tiles_t fields in order: a field the table sets takes
    # its argument, the others 0
    body = macro[macro.index("{", macro.index(")")):]
    body = body[body.index("{", 1) + 1:body.index("}")]
    values = [v.strip() for v in body.split(",")]
    struct = [n for n, _ in da.DecodeAttnTiles._fields_]
    assert len(values) == len(struct)
    for name, v in zip(struct, values):
        want = args[6 + autotune.TILE_FIELDS.index(name)] if name in autotune.TILE_FIELDS else "0"
        assert v == want, (name, v, want)


def test_significance_needs_a_gap_beyond_the_spread():
    T = autotune.Timing
    builtin = T([10.0, 10.2, 10.1])
    assert autotune.significant(T([9.5, 9.6, 9.55]), builtin)
    assert not autotune.significant(T([9.95, 10.0, 9.9]), builtin)       # faster, but inside the noise
    assert not autotune.significant(T([9.0, 10.5, 9.1]), builtin)        # its own spread swallows the gap
    assert builtin.median == 10.1 and abs(builtin.spread - 0.2) < 1e-12


def test_rule_selection_by_geometric_mean():
    T = autotune.Timing
    base = {"a": T([10.0]), "b": T([100.0]), "c": T([1.0])}
    times = {
        None: base,
        "fast_on_big": {"a": T([10.0]), "b": T([50.0]), "c": T([1.5])},    # ratios 1, 0.5, 1.5
        "even": {"a": T([9.0]), "b": T([90.0]), "c": T([0.9])},            # 0.9 on every shape
        "partial": {"a": T([1.0]), "b": T([1.0])},                         # not allowed on c: left out
    }
    best, ratios = autotune.select_rule(times)
    assert best == "even"
    assert abs(ratios["fast_on_big"] - (0.75) ** (1 / 3)) < 1e-12 and "partial" not in ratios
    assert ratios[None] == 1.0
    # with nothing better the built-in choice stays
    best, _ = autotune.select_rule({None: base, "slow": {k: T([v.median * 1.1]) for k, v in base.items()}})
    assert best is None


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_attention_only_workspace_covers_the_table_rows():
    # a table row can set the attention grid; an attention-only call (whose hidden size is not part
    # of the lookup, so it takes the row of the same attention shape) must fit the workspace that
    # the size query of the full step reports
    rows = [[int(v) for v in r[len("TILE_ENTRY("):r.index(")")].split(",")] for r in _rows(autotune.TABLE)]
    assert rows
    for row in rows:
        shape = dict(batch=row[0], num_q_heads=row[1], num_kv_heads=row[2], head_dim=row[3], max_seq_len=row[4])
        tiles = dict(zip(autotune.TILE_FIELDS, row[6:]))
        need_attn = da.decode_attn_workspace_size(da.make_shape(hidden=8, tiles=tiles, **shape))
        assert da.decode_attn_workspace_size(da.make_shape(hidden=row[5], **shape)) >= need_attn, row


def test_mfma_summary_from_counter_and_trace_csvs(tmp_path, monkeypatch):
    # two dispatches of the counted kernel, one of another; busy % is the summed
    # per-SIMD busy cycles over (trace duration x peak clock x SIMDs), flops are MOPS x 512
    import bench

    pmc = tmp_path / "mfma.csv"
    rows = ["Kernel_Name,Counter_Name,Counter_Value"]
    for kern in ("gemm_kernel<true, 1, 2>", "gemm_kernel<true, 1, 2>"):
        rows += ["%s,SQ_INSTS_VALU_MFMA_MOPS_F16,524288" % kern.replace(",", ";"),
                 "%s,SQ_VALU_MFMA_BUSY_CYCLES,102400" % kern.replace(",", ";"),
                 "%s,GRBM_GUI_ACTIVE,1000" % kern.replace(",", ";")]
    rows += ["other_kernel,SQ_INSTS_VALU_MFMA_MOPS_F16,7", "other_kernel,GRBM_GUI_ACTIVE,5"]
    pmc.write_text("\n".join(rows) + "\n")
    stats = tmp_path / "stats.csv"
    stats.write_text("Name,Calls,AverageNs,MinNs,MaxNs\n"
                     "gemm_kernel<true; 1; 2>,10,5000.0,4000.0,6000.0\nother_kernel,1,100.0,100.0,100.0\n")
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))

    class A:
        workload = "gemm_f16_256x512x1024"
        summarize_mfma = ("gemm_kernel", str(pmc), str(stats))

    bench.summarize_mfma(A())
    text = (tmp_path / "profiles" / "gemm_kernel_gemm_f16_256x512x1024_mfma.txt").read_text()
    assert "gemm_kernel<true; 1; 2>" in text
    fields = dict(l.split(" = ", 1) for l in text.splitlines() if " = " in l and not l.startswith("#"))
    assert fields["dispatches_counted"] == "2"
    assert float(fields["mfma_flops_per_dispatch"]) == 524288 * 512
    assert float(fields["mfma_busy_pct_at_peak_clock"]) == round(100.0 * 102400 / (5000.0 * 2.4 * 1024), 3)
    assert float(fields["trace_avg_ns"]) == 5000.0
    assert float(fields["executed_mfma_tflops"]) == round(524288 * 512 / 5000.0 / 1e3, 2)


def test_traffic_summaries_for_every_kernel_of_the_run(tmp_path, monkeypatch):
    # FETCH / WRITE KiB per dispatch of each kernel, scaled by what the counters read for the 64 MiB
    # calibration copy (here 2x too much read, exact write), one summary file per kernel
    import bench
    import workloads

    def pmc(path, counter, vals):
        rows = ["Kernel_Name,Counter_Name,Counter_Value"]
        rows += ["%s,%s,%s" % (k, counter, v) for k, v in vals]
        path.write_text("\n".join(rows) + "\n")

    attn = "void da::(anonymous namespace)::attn_streamk_kernel<4; 4; 1; 128>(da::AttnParams)"
    gemm = "void da::(anonymous namespace)::gemm_kernel<false; 1; 2>(da::GemmParams)"
    cal = "void at::native::elementwise_kernel<MulFunctor>"
    fetch, write, stats = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "s.csv"
    pmc(fetch, "FETCH_SIZE", [(attn, 1000.0), (attn, 3000.0), (gemm, 500.0), (cal, 2 * 65536.0)])
    pmc(write, "WRITE_SIZE", [(attn, 10.0), (attn, 30.0), (gemm, 5.0), (cal, 65536.0)])
    stats.write_text("Name,Calls,AverageNs,MinNs,MaxNs\n%s,5,50000.0,1.0,2.0\n%s,5,12000.0,1.0,2.0\n%s,1,9.0,9.0,9.0\n"
                     % (attn, gemm, cal))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))

    class A:
        workload = workloads.BATCHED.name
        tiles = '{"step_mode": 2}'
        profile_tag = "two_launches"
        summarize_profile = (str(fetch), str(write), str(stats))

    bench.summarize_profile(A())
    files = sorted(p.name for p in (tmp_path / "profiles").iterdir())
    assert files == ["attn_streamk_kernel_%s_two_launches.txt" % workloads.BATCHED.name,
                     "gemm_kernel_%s_two_launches.txt" % workloads.BATCHED.name]
    text = (tmp_path / "profiles" / files[0]).read_text()
    fields = dict(l.split(" = ", 1) for l in text.splitlines() if " = " in l and not l.startswith("#"))
    assert fields["kernel"] == "attn_streamk_kernel" and fields["dominant"] == "True"
    assert int(fields["hbm_read_bytes_per_dispatch"]) == 2000 * 512   # 2000 KiB at half scale
    assert int(fields["hbm_write_bytes_per_dispatch"]) == 20 * 1024
    assert float(fields["trace_avg_ns"]) == 50000.0
    assert "--tiles '{\"step_mode\": 2}'" in text
    gfields = dict(l.split(" = ", 1) for l in (tmp_path / "profiles" / files[1]).read_text().splitlines()
                   if " = " in l and not l.startswith("#"))
    assert gfields["dominant"] == "False" and int(gfields["hbm_read_bytes_per_dispatch"]) == 500 * 512


def test_gemm_f16_kernel_names_the_launched_kernel():
    # the rule of gemm_f16: fewer than 256 tiles of 16 rows x 128 columns -> 16 x 32 tiles over all of K
    import bench

    assert bench.gemm_f16_kernel(256, 512) == "gemm_narrow_kernel"    # the fp16 check: 64 wide tiles
    assert bench.gemm_f16_kernel(32, 1040) == "gemm_narrow_kernel"
    assert bench.gemm_f16_kernel(512, 1024) == "gemm_kernel"          # 256 wide tiles
    assert bench.gemm_f16_kernel(256, 4096) == "gemm_kernel"
