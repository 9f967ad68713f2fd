"""The C ABI without a GPU: the library loads, exports every declared entry
point, rejects bad arguments before touching the device, and plans one tile
per matmul of the step."""
import ctypes
import os
import re

import pytest

import decode_attention_output_amd as da

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "decode_attn.h")
GOLDEN = os.path.join(ROOT, "tests", "golden")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while", "for", "sizeof")))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(da.LIB_PATH):
        from decode_attention_output_amd import build
        build.build()
    return da.load_library()


def test_header_declares_the_binding_names():
    assert _declared_functions() == sorted(da.EXPORTED)


def test_header_constants_match_the_binding():
    # every integer #define of the header that the binding mirrors has the same value
    text = open(os.path.join(ROOT, "include", "decode_attn.h")).read()
    defines = {}
    for line in text.splitlines():
        parts = line.split(None, 2)
        if len(parts) == 3 and parts[0] == "#define" and parts[1].startswith("DA_"):
            value = parts[2].split("/*")[0].strip().replace("u", "")
            try:
                defines[parts[1]] = int(eval(value, {}))
            except SyntaxError:
                pass
    mirrored = [n for n in defines if hasattr(da, n)]
    assert {"DA_ERR_TIMEOUT", "DA_MAX_GROUP", "DA_FLAG_SEPARATE", "DA_HEAD_DIM_WIDE"} <= set(mirrored)
    for name in mirrored:
        assert getattr(da, name) == defines[name], name


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert isinstance(getattr(lib, name), ctypes._CFuncPtr)


def test_status_strings(lib):
    for code in (da.DA_OK, da.DA_ERR_NULL, da.DA_ERR_SHAPE, da.DA_ERR_ALIGN, da.DA_ERR_WORKSPACE, da.DA_ERR_LAUNCH,
                 da.DA_ERR_TIMEOUT):
        assert da.status_str(code) and da.status_str(code) != "unknown status"
    assert da.status_str(-99) == "unknown status"


FAKE = 0x10000  # 16- and 256-byte aligned, never dereferenced: every call below fails its checks first


def _shape(**kw):
    base = dict(batch=1, num_q_heads=32, num_kv_heads=8, max_seq_len=2048, hidden=4096)
    base.update(kw)
    return da.make_shape(**base)


def _fwd(lib, shape, q=FAKE, k=FAKE, v=FAKE, sl=FAKE, w=FAKE, out=FAKE):
    return lib.decode_attn_fwd(q, k, v, sl, w, out, ctypes.byref(shape), None)


@pytest.mark.parametrize("which", ["q", "k", "v", "sl", "w", "out"])
def test_null_pointers_are_rejected(lib, which):
    assert _fwd(lib, _shape(), **{which: None}) == da.DA_ERR_NULL
    assert lib.decode_attn_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == da.DA_ERR_NULL


@pytest.mark.parametrize("kw", [dict(head_dim=64), dict(head_dim=192), dict(head_dim=512),
                                dict(head_dim=256, tiles=dict(attn_depth=2)), dict(num_q_heads=30), dict(num_q_heads=8 * 17),
                                dict(batch=0), dict(max_seq_len=0), dict(hidden=0), dict(hidden=4100),
                                dict(num_kv_heads=0)])
def test_bad_shapes_are_rejected(lib, kw):
    s = _shape(**kw)
    assert _fwd(lib, s) == da.DA_ERR_SHAPE
    assert da.decode_attn_workspace_size(s) == 0


@pytest.mark.parametrize("which", ["q", "k", "v", "w", "out"])
def test_misaligned_pointers_are_rejected(lib, which):
    assert _fwd(lib, _shape(), **{which: FAKE + 2}) == da.DA_ERR_ALIGN


def test_workspace_is_required_and_checked(lib):
    s = _shape()
    need = da.decode_attn_workspace_size(s)
    assert need > 0
    assert _fwd(lib, s) == da.DA_ERR_WORKSPACE
    s.workspace, s.workspace_bytes = FAKE, need - 1
    assert _fwd(lib, s) == da.DA_ERR_WORKSPACE
    s.workspace, s.workspace_bytes = FAKE + 16, need
    assert _fwd(lib, s) == da.DA_ERR_ALIGN


def test_debug_pointers_required_with_the_flag(lib):
    s = _shape(flags=da.DA_FLAG_DEBUG_SCORES)
    s.workspace, s.workspace_bytes = FAKE, da.decode_attn_workspace_size(s)
    assert _fwd(lib, s) == da.DA_ERR_NULL


def test_oproj_and_gemm_argument_checks(lib):
    assert lib.oproj_fwd(None, FAKE, FAKE, 1, 4096, 4096, FAKE, 1 << 30, None) == da.DA_ERR_NULL
    assert lib.oproj_fwd(FAKE, FAKE, FAKE, 1, 4096, 4100, FAKE, 1 << 30, None) == da.DA_ERR_SHAPE
    assert lib.oproj_fwd(FAKE, FAKE, FAKE + 8, 1, 4096, 4096, FAKE, 1 << 30, None) == da.DA_ERR_ALIGN
    need = da.oproj_workspace_size(1, 4096, 4096)
    assert need > 0
    assert lib.oproj_fwd(FAKE, FAKE, FAKE, 1, 4096, 4096, FAKE, need - 1, None) == da.DA_ERR_WORKSPACE
    assert lib.oproj_fwd(FAKE, FAKE, FAKE, 16, 4100, 4096, FAKE, 1 << 30, None) == da.DA_ERR_SHAPE
    assert lib.gemm_f16(FAKE, None, FAKE, 256, 512, 1024, None) == da.DA_ERR_NULL
    assert lib.gemm_f16(FAKE, FAKE, FAKE, 250, 512, 1024, None) == da.DA_ERR_SHAPE
    assert lib.gemm_f16(FAKE, FAKE, FAKE, 256, 512, 1000, None) == da.DA_ERR_SHAPE


def test_step_status_argument_checks(lib):
    # all rejected before any HIP call (no device here)
    assert lib.decode_attn_step_status(FAKE, 65535, None) == da.DA_ERR_WORKSPACE
    assert lib.decode_attn_step_status(FAKE + 16, 1 << 20, None) == da.DA_ERR_ALIGN
    # a workspace the binding never allocated has seen no single-launch step
    assert da.decode_attn_step_status(da.Workspace()) == da.DA_OK


def test_noalloc_entry_checks_arguments_before_any_hip_call(lib):
    def call(shape, **kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, sl=FAKE, w=FAKE, out=FAKE)
        a.update(kw)
        return lib.decode_attn_fwd_noalloc(a["q"], a["k"], a["v"], a["sl"], a["w"], a["out"],
                                           ctypes.byref(shape) if shape is not None else None, None)
    assert call(None) == da.DA_ERR_NULL
    assert call(_shape(), w=None) == da.DA_ERR_NULL
    assert call(_shape(), out=FAKE + 4) == da.DA_ERR_ALIGN
    assert call(_shape(num_q_heads=30)) == da.DA_ERR_SHAPE
    # a step whose workspace exceeds the scratch array: 1024 sequences' attention partials
    big = _shape(batch=1024, max_seq_len=32768, hidden=8192)
    assert da.decode_attn_workspace_size(big) > 16 << 20
    assert call(big) == da.DA_ERR_WORKSPACE


def test_read_probe_argument_checks(lib):
    sink = FAKE + 256
    assert lib.decode_attn_read_probe(None, 1024, sink, 8, None) == da.DA_ERR_NULL
    assert lib.decode_attn_read_probe(FAKE, 1024, None, 8, None) == da.DA_ERR_NULL
    assert lib.decode_attn_read_probe(FAKE + 8, 1024, sink, 8, None) == da.DA_ERR_ALIGN
    assert lib.decode_attn_read_probe(FAKE, 1000, sink, 8, None) == da.DA_ERR_SHAPE
    assert lib.decode_attn_read_probe(FAKE, 1024, sink, 0, None) == da.DA_ERR_SHAPE


def test_step_wait_polls_in_range_is_accepted(lib):
    for polls in (1, 1000, 1 << 24):
        assert da.decode_attn_workspace_size(_shape(tiles=dict(step_wait_polls=polls))) > 0


def _golden_shapes():
    rows = {}
    for line in open(os.path.join(GOLDEN, "decode_attention_matmul_shapes.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            name, m, k, n = line.split()
            rows[name] = (int(m), int(k), int(n))
    return rows


def test_plan_reports_the_pages_matmul_shapes(lib):
    g = _golden_shapes()
    plan = da.decode_attn_plan(_shape())
    assert (plan.qk.m, plan.qk.k, plan.qk.n) == g["qk_t"]
    assert (plan.pv.m, plan.pv.k, plan.pv.n) == g["attn_v"]
    assert (plan.oproj.m, plan.oproj.k, plan.oproj.n) == g["output_proj"]


@pytest.mark.parametrize("cfg", [dict(batch=1, num_q_heads=4, num_kv_heads=1, max_seq_len=256, hidden=512),
                                 dict(batch=1, num_q_heads=32, num_kv_heads=8, max_seq_len=2048, hidden=4096),
                                 dict(batch=16, num_q_heads=32, num_kv_heads=8, max_seq_len=8192, hidden=4096),
                                 dict(batch=4, num_q_heads=64, num_kv_heads=8, max_seq_len=32768, hidden=8192)])
def test_plan_tiles_follow_the_per_matmul_rules(lib, cfg):
    plan = da.decode_attn_plan(da.make_shape(**cfg))
    G = cfg["num_q_heads"] // cfg["num_kv_heads"]
    # a short axis is not split: head_dim 128 stays whole in QK^T (its K) and PV (its N)
    assert plan.qk.tile_k == 128 and plan.pv.tile_n == 128
    # the tiny M (query group) sits in one 16-row operand and is not padded further
    assert plan.qk.tile_m == 16 and G <= plan.pv.tile_m <= 16
    # the long axis (keys) is streamed 32 keys per wave step and cut evenly over the workgroups
    assert plan.qk.tile_n == 32 and plan.pv.tile_k == 32
    keys = cfg["batch"] * cfg["num_kv_heads"] * cfg["max_seq_len"]
    if plan.fused == 3:
        # the tiny step: each workgroup streams every sequence whole (one piece), 16 columns each
        assert plan.num_splits == 1 and plan.split_len == cfg["max_seq_len"]
        assert plan.qk.workgroups == -(-cfg["hidden"] // 16)
    elif plan.fused == 1:
        # one launch: every sequence cut into the same pieces of a multiple of 128 keys
        assert plan.split_len % 128 == 0 and plan.num_splits == -(-cfg["max_seq_len"] // plan.split_len)
        assert plan.qk.workgroups == cfg["batch"] * cfg["num_kv_heads"] * plan.num_splits
        assert plan.qk.workgroups >= min(192, keys // 128)
    else:
        # stream-K: the keys of all sequences cut into equal ranges, one per workgroup
        assert plan.split_len % 32 == 0 and plan.split_len * plan.num_splits >= keys
        assert plan.split_len * (plan.num_splits - 1) < keys + 32 * plan.num_splits
        # the keys are spread over 176 workgroups (22 per XCD, the measured best over a set of
        # steps), or the count of the shape's measured table row, when the problem allows it,
        # but never so many that a workgroup streams fewer than 128 keys
        row = _table_tiles(cfg)
        want = row["attn_workgroups"] if row and row["attn_workgroups"] else 176
        assert plan.qk.workgroups >= min(want, keys // 128)
        assert plan.split_len >= min(128, 32 * (-(-keys // 32)))
        assert plan.oproj.workgroups >= min(256, (cfg["hidden"] // 128) * (cfg["num_q_heads"] * 128 // 128))
    # projection path: the single-launch small and tiny steps' own VALU projections, else the MFMA
    # GEMM at every batch (K = Hq*128), in the large single-launch step (fused 2) or a launch of its own
    assert plan.oproj_path == (0 if plan.fused in (1, 3) else 1)
    assert plan.workspace_bytes == da.decode_attn_workspace_size(da.make_shape(**cfg))


TINY = [dict(batch=1, num_q_heads=4, num_kv_heads=1, max_seq_len=256, hidden=512),
        dict(batch=2, num_q_heads=16, num_kv_heads=2, max_seq_len=128, hidden=256)]
SMALL = [dict(batch=1, num_q_heads=32, num_kv_heads=8, max_seq_len=2048, hidden=4096),
         dict(batch=2, num_q_heads=16, num_kv_heads=2, max_seq_len=256, hidden=256)]
LARGE = [dict(batch=3, num_q_heads=16, num_kv_heads=2, max_seq_len=128, hidden=256),
         dict(batch=16, num_q_heads=32, num_kv_heads=8, max_seq_len=8192, hidden=4096),
         dict(batch=4, num_q_heads=64, num_kv_heads=8, max_seq_len=32768, hidden=8192)]


@pytest.mark.parametrize("cfg", TINY + SMALL + LARGE)
def test_plan_one_launch_per_step(lib, cfg):
    # tiny steps (at most 256 KiB of K and V): every workgroup computes the whole attention
    # (fused 3); small steps: the single-launch step with its own projection (fused 1); larger
    # ones: the stream-K attention and the MFMA projection's items in one grid (fused 2)
    plan = da.decode_attn_plan(da.make_shape(**cfg))
    sep = da.decode_attn_plan(da.make_shape(flags=da.DA_FLAG_SEPARATE, **cfg))
    assert plan.fused == (3 if cfg in TINY else 1 if cfg in SMALL else 2)
    assert sep.fused == 0
    # the workspace does not depend on the launch choice
    assert plan.workspace_bytes == sep.workspace_bytes
    if plan.fused == 2:
        # the same attention split and projection tiles as two launches
        for name in ("qk", "pv", "oproj"):
            assert getattr(sep, name).as_dict() == getattr(plan, name).as_dict(), name
        assert sep.split_len == plan.split_len
    if plan.fused == 1:
        # every workgroup of the single launch is resident at once (two per compute unit)
        assert plan.qk.workgroups + plan.oproj.workgroups <= 512
        assert plan.oproj_path == 0 and plan.oproj.tile_n in (128, 256, 512)
    if plan.fused == 3:
        # one piece per sequence, 16 output columns over all of K per workgroup
        assert plan.num_splits == 1 and plan.oproj.tile_n == 16 and plan.oproj.split == 1
        assert plan.oproj.workgroups == -(-cfg["hidden"] // 16) == plan.qk.workgroups


@pytest.mark.parametrize("tiles", [dict(attn_workgroups=-1), dict(attn_workgroups=1025), dict(attn_depth=4),
                                   dict(attn_depth=-2), dict(proj_tile_n=96), dict(proj_tile_n=1024),
                                   dict(proj_ksplit=-1), dict(step_mode=5), dict(step_wait_polls=-1),
                                   dict(step_wait_polls=(1 << 24) + 1), dict(attn_seq_cost=-1),
                                   dict(attn_seq_cost=257)])
def test_tile_override_out_of_range_is_a_shape_error(lib, tiles):
    shape = _shape(tiles=tiles)
    assert da.decode_attn_workspace_size(shape) == 0
    assert _fwd(lib, shape) == da.DA_ERR_SHAPE
    with pytest.raises(da.DecodeAttnError):
        da.decode_attn_plan(shape)


def test_gemv_is_chosen_by_its_own_widths(lib):
    cfg = dict(batch=4, num_q_heads=64, num_kv_heads=8, max_seq_len=32768, hidden=8192)
    for tn, path in ((0, 1), (128, 1), (64, 0), (256, 0), (512, 0)):
        plan = da.decode_attn_plan(da.make_shape(tiles=dict(proj_tile_n=tn), **cfg))
        assert plan.oproj_path == path and (tn == 0 or plan.oproj.tile_n == tn), tn


def test_tile_override_gemv_width_limit(lib):
    # the GEMV holds tile_n columns for every (power-of-two padded) row: at most 2048 values
    assert da.decode_attn_workspace_size(_shape(batch=4, tiles=dict(proj_tile_n=512))) > 0
    assert da.decode_attn_workspace_size(_shape(batch=5, tiles=dict(proj_tile_n=512))) == 0
    # the MFMA GEMM (16 rows and more) has one column tile
    assert da.decode_attn_workspace_size(_shape(batch=16, max_seq_len=8192, tiles=dict(proj_tile_n=64))) == 0


def test_tile_override_reaches_the_plan(lib):
    cfg = dict(batch=4, num_q_heads=64, num_kv_heads=8, max_seq_len=32768, hidden=8192)
    base = da.decode_attn_plan(da.make_shape(**cfg))
    over = da.decode_attn_plan(da.make_shape(tiles=dict(attn_workgroups=320, proj_tile_n=128, proj_ksplit=8), **cfg))
    assert base.qk.workgroups != 320 and over.qk.workgroups == 320
    assert over.num_splits == 320 and over.split_len * 320 >= 4 * 8 * 32768
    assert over.oproj.tile_n == 128 and over.oproj.split == 8
    assert over.oproj.workgroups == (8192 // 128) * 8
    # zero fields keep the built-in choice (a shape without a row in the measured table)
    cfg2 = dict(cfg, max_seq_len=30000)
    base2 = da.decode_attn_plan(da.make_shape(**cfg2))
    same = da.decode_attn_plan(da.make_shape(tiles={}, **cfg2))
    assert (same.qk.workgroups, same.oproj.tile_n, same.oproj.split) == (base2.qk.workgroups, base2.oproj.tile_n,
                                                                         base2.oproj.split)
    # a grid wider than the blocks of the step is capped at one 32-key block per workgroup
    tiny = da.decode_attn_plan(da.make_shape(batch=1, num_q_heads=4, num_kv_heads=1, max_seq_len=256, hidden=512,
                                             tiles=dict(attn_workgroups=1024, step_mode=2)))
    assert tiny.fused == 0 and tiny.qk.workgroups == 8
    # step_mode 2 asks for two launches where the built-in choice fuses
    pages = dict(batch=1, num_q_heads=32, num_kv_heads=8, max_seq_len=2048, hidden=4096)
    assert da.decode_attn_plan(da.make_shape(**pages)).fused == 1
    assert da.decode_attn_plan(da.make_shape(tiles=dict(step_mode=2), **pages)).fused == 0
    # step_mode 3 asks for the large single-launch step, also where the small one would serve
    assert da.decode_attn_plan(da.make_shape(tiles=dict(step_mode=3), **pages)).fused == 2
    # step_mode 4 asks for the tiny step; where the K/V are too large for it, the built-in choice stays
    assert da.decode_attn_plan(da.make_shape(tiles=dict(step_mode=4), **pages)).fused == 1
    tiny_shape = dict(batch=1, num_q_heads=4, num_kv_heads=1, max_seq_len=256, hidden=512)
    assert da.decode_attn_plan(da.make_shape(**tiny_shape)).fused == 3
    assert da.decode_attn_plan(da.make_shape(tiles=dict(step_mode=1), **tiny_shape)).fused == 1
    assert da.decode_attn_plan(da.make_shape(tiles=dict(step_mode=2), **tiny_shape)).fused == 0


def _table_rows():
    rows = []
    with open(os.path.join(ROOT, "decode_attention_output_amd", "csrc", "tile_table.inc")) as f:
        for line in f:
            if line.startswith("TILE_ENTRY("):
                rows.append([int(v) for v in line[len("TILE_ENTRY("):line.index(")")].split(",")])
    return rows


def _table_tiles(cfg):
    """The tiles of the table row of a shape (head_dim 128 unless given), or None."""
    from decode_attention_output_amd import autotune

    key = (cfg["batch"], cfg["num_q_heads"], cfg["num_kv_heads"], cfg.get("head_dim", 128), cfg["max_seq_len"],
           cfg["hidden"])
    for row in _table_rows():
        if tuple(row[:6]) == key:
            return dict(zip(autotune.TILE_FIELDS, row[6:]))
    return None


def test_measured_tile_table_rows_are_valid_and_used(lib):
    from decode_attention_output_amd import autotune

    fields = autotune.TILE_FIELDS
    for row in _table_rows():
        assert len(row) == 6 + len(fields), row
        shape = dict(batch=row[0], num_q_heads=row[1], num_kv_heads=row[2], head_dim=row[3], max_seq_len=row[4],
                     hidden=row[5])
        tiles = dict(zip(fields, row[6:]))
        assert da.decode_attn_workspace_size(da.make_shape(**shape)) > 0, row
        # a call without an override plans exactly as one that passes the row's tiles
        a = da.decode_attn_plan(da.make_shape(**shape))
        b = da.decode_attn_plan(da.make_shape(tiles=tiles, **shape))
        for name in ("qk", "pv", "oproj"):
            assert getattr(a, name).as_dict() == getattr(b, name).as_dict(), (row, name)
        assert (a.fused, a.split_len, a.workspace_bytes) == (b.fused, b.split_len, b.workspace_bytes)


def test_head_dim_256_plans_two_launches(lib):
    # head_dim 256 runs the stream-K attention (QK^T with K = 256, attn x V with N = 256) and the
    # separate projection with K = Hq * 256; the single-launch step is built for 128 only
    cfg = dict(batch=1, num_q_heads=16, num_kv_heads=2, max_seq_len=2048, hidden=4096)
    plan = da.decode_attn_plan(da.make_shape(head_dim=256, **cfg))
    assert plan.fused == 0
    assert (plan.qk.m, plan.qk.k, plan.qk.n) == (8, 256, 2048) and plan.qk.tile_k == 256
    assert (plan.pv.m, plan.pv.k, plan.pv.n) == (8, 2048, 256) and plan.pv.tile_n == 256
    assert (plan.oproj.m, plan.oproj.k, plan.oproj.n) == (1, 16 * 256, 4096)
    # the attention partials and the bf16 attention output are twice as wide as at 128
    narrow = da.decode_attn_workspace_size(da.make_shape(head_dim=128, flags=da.DA_FLAG_SEPARATE, **cfg))
    assert plan.workspace_bytes > narrow


def _pre(lib, q=FAKE, k=FAKE, v=FAKE, cl=FAKE, out=FAKE, **kw):
    fields = dict(batch=2, num_tokens=16, num_q_heads=32, num_kv_heads=8, head_dim=128, max_seq_len=1024,
                  softmax_scale=0.0)
    fields.update(kw)
    s = da.PrefillAttnShape(**fields)
    return lib.prefill_attn_fwd(q, k, v, cl, out, ctypes.byref(s), None)


@pytest.mark.parametrize("which", ["q", "k", "v", "cl", "out"])
def test_prefill_null_pointers_are_rejected(lib, which):
    assert _pre(lib, **{which: None}) == da.DA_ERR_NULL
    assert lib.prefill_attn_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == da.DA_ERR_NULL


@pytest.mark.parametrize("which", ["q", "k", "v", "out"])
def test_prefill_misaligned_pointers_are_rejected(lib, which):
    assert _pre(lib, **{which: FAKE + 2}) == da.DA_ERR_ALIGN


@pytest.mark.parametrize("kw", [dict(head_dim=256), dict(head_dim=64), dict(num_q_heads=30), dict(batch=0),
                                dict(num_tokens=0), dict(num_tokens=2048), dict(num_kv_heads=1, num_q_heads=32),
                                dict(max_seq_len=1 << 24)])
def test_prefill_bad_shapes_are_rejected(lib, kw):
    assert _pre(lib, **kw) == da.DA_ERR_SHAPE
