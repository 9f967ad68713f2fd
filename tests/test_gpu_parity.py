"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Every case draws seeded inputs, runs the library on the GPU and the oracle on
the host, and compares element by element:
  * bf16 outputs: max |gpu - ref| <= 1e-2 and max relative error <= 2^-7 where
    |ref| >= 1e-2 (ref = the oracle's unrounded double result);
  * fp32 debug scores: |gpu - ref| <= 1e-4 * max(|ref|, 1);
  * integer-valued GEMMs and the closed-form special cases: bit-exact.
The four decode workloads run at their full sizes in the same launch
configuration the benchmark times (the library picks it from the shape).
Every call gets a workspace whose scratch data is NaN (PoisonedWorkspace), so
a partial result read before it was written shows up in the output, and
after every decode step the single-launch step's error word is read back.
"""
import math

import numpy as np
import pytest
import torch

import decode_attention_output_amd as da
import oracle
import workloads
from gpu_helpers import (COUNTER_BLOCK, PoisonedWorkspace, assert_bf16_close, assert_scores_close,
                         assert_within_fp32_sum_bound, bf16_words_to_f64, dev_bf16, dev_f16, dev_i32, host_words,
                         ulp_distance_bf16)

pytestmark = pytest.mark.gpu


def _status_ok(ws, what=""):
    rc = da.decode_attn_step_status(ws)
    assert rc == da.DA_OK, "%s: step status %d (%s)" % (what, rc, da.status_str(rc))


def _run_step(inp, ws=None, scale=0.0, debug=False):
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    sl, w = dev_i32(inp["seq_lens"]), dev_bf16(inp["o_weight"])
    ws = ws or PoisonedWorkspace()
    flat = da.decode_attn_only(q, k, v, sl, workspace=ws, softmax_scale=scale)
    out = da.decode_attn_fwd(q, k, v, sl, w, workspace=ws, softmax_scale=scale)
    _status_ok(ws)
    res = {"flat": host_words(flat), "out": host_words(out)}
    if debug:
        B, Hq, _ = inp["q"].shape
        Lmax = inp["k"].shape[2]
        dbg_s = torch.full((B, Hq, Lmax), float("nan"), dtype=torch.float32, device="cuda")
        dbg_l = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
        da.decode_attn_only(q, k, v, sl, workspace=ws, softmax_scale=scale, debug_scores=dbg_s, debug_lse=dbg_l)
        _status_ok(ws, "debug scores")
        res["scores"] = dbg_s.cpu().numpy()
        res["lse"] = dbg_l.cpu().numpy()
    torch.cuda.synchronize()
    return res


def _check_step(inp, res, scale=None, what=""):
    ref = oracle.decode_step(inp["q"], inp["k"], inp["v"], inp["seq_lens"], inp["o_weight"], scale=scale)
    assert_bf16_close(res["flat"], ref["attn_ref"], what + " attention output")
    assert_bf16_close(res["out"], ref["out_ref"], what + " projected output")
    # the projection in isolation: oracle o_proj of the GPU's own attention output. The GPU sums K
    # products in fp32 and rounds once to bf16, so |gpu - ref| <= K * 2^-24 * sum_k |x_k w_kn| (any
    # summation order) + one bf16 step of the result.
    _, iso_ref = oracle.oproj(res["flat"], inp["o_weight"])
    assert_within_fp32_sum_bound(res["out"], iso_ref, res["flat"], inp["o_weight"], what + " o_proj alone")
    # diagnostic only (not gated): bf16 steps between the GPU's words and the oracle's rounded result
    for name, got, want in (("attention", res["flat"], ref["flat"]), ("out", res["out"], ref["out"])):
        hist = np.bincount(np.minimum(ulp_distance_bf16(got, want).ravel(), 3), minlength=4)
        print("%s %s: bf16 steps from the rounded oracle 0/1/2/3+: %s" % (what, name, hist.tolist()))
    return ref


def test_device_is_gfx950(gpu):
    props = torch.cuda.get_device_properties(0)
    assert props.gcnArchName.startswith("gfx950")
    assert props.multi_processor_count == 256
    assert props.warp_size == 64


@pytest.mark.parametrize("wl", [workloads.TINY, workloads.PAGES], ids=lambda w: w.name)
def test_decode_workload_small(gpu, wl):
    inp = workloads.decode_inputs(wl, poison=True)
    res = _run_step(inp, debug=True)
    ref = _check_step(inp, res, what=wl.name)
    att = oracle.attention(inp["q"], inp["k"], inp["v"], inp["seq_lens"], want_scores=True)
    for b, L in enumerate(inp["seq_lens"]):
        assert_scores_close(res["scores"][b, :, :L], att["scores"][b, :, :L], wl.name + " scores")
    np.testing.assert_allclose(res["lse"], att["lse"], rtol=1e-5, atol=1e-5)
    assert ref is not None


@pytest.mark.parametrize("wl", [workloads.BATCHED, workloads.LONG, workloads.WIDE], ids=lambda w: w.name)
def test_decode_workload_large(gpu, wl):
    # full size, stream-K attention: pieces of one sequence span workgroups and meet in the merge;
    # the debug export gives every fp32 score and the log-sum-exp of every query head
    inp = workloads.decode_inputs(wl, poison=True)
    res = _run_step(inp, debug=True)
    _check_step(inp, res, what=wl.name)
    att = oracle.attention(inp["q"], inp["k"], inp["v"], inp["seq_lens"], want_scores=True)
    for b, L in enumerate(inp["seq_lens"]):
        assert_scores_close(res["scores"][b, :, :L], att["scores"][b, :, :L], wl.name + " scores")
        assert np.all(np.isnan(res["scores"][b, :, L:]))  # nothing written past the sequence
    np.testing.assert_allclose(res["lse"], att["lse"], rtol=1e-5, atol=1e-5)


def test_gemm_f16_workload_bit_exact(gpu):
    g = workloads.gemm_inputs()
    c = da.gemm_f16(dev_f16(g["a"]), dev_f16(g["b"]))
    ref, _ = oracle.gemm_f16(g["a"], g["b"])
    np.testing.assert_array_equal(host_words(c), ref)


def test_gemm_f16_all_ones_golden(gpu):
    g = workloads.gemm_inputs(all_ones=True)
    c = host_words(da.gemm_f16(dev_f16(g["a"]), dev_f16(g["b"])))
    assert np.all(c == 0x6400)  # every entry is exactly k = 1024


GEMM_SHAPES = [
    # (M, N, K): 16 x 32 tiles over all of K where 128-column tiles would not fill the chip
    (16, 16, 32),       # one tile, half of it past N
    (48, 80, 96),       # a ragged last column tile; three K-steps for four waves
    (32, 1040, 2048),   # deep K: more K-steps per wave than are requested at once
    (512, 1024, 64),    # 256 column tiles of 128: the wide tiles
    (256, 4096, 32),    # the wide tiles, one K-step
]


@pytest.mark.parametrize("shape", GEMM_SHAPES, ids=lambda c: "M%d_N%d_K%d" % c)
def test_gemm_f16_integer_shapes_bit_exact(gpu, shape):
    M, N, K = shape
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    a = rng.integers(-1, 1, endpoint=True, size=(M, K)).astype(np.float16).view(np.uint16)
    b = rng.integers(-1, 1, endpoint=True, size=(K, N)).astype(np.float16).view(np.uint16)
    c = da.gemm_f16(dev_f16(a), dev_f16(b))
    ref, _ = oracle.gemm_f16(a, b)
    np.testing.assert_array_equal(host_words(c), ref)


# ---- edge cases of the attention path ------------------------------------

EDGE = [
    # (batch, Hq, Hkv, seq_lens, max_seq_len)
    (1, 4, 1, [1], 1),
    (1, 4, 1, [2], 2),
    (1, 1, 1, [33], 40),
    (2, 2, 1, [16, 17], 17),
    (3, 8, 2, [1, 129, 700], 700),
    (2, 6, 2, [127, 128], 300),
    (2, 32, 2, [300, 5], 300),
    (1, 16, 2, [4096], 4096),
    (4, 24, 8, [255, 256, 257, 1000], 1024),
    (2, 8, 8, [513, 2], 600),
    (3, 16, 2, [5, 37, 100], 128),   # group 8: last 32-key blocks hold <= 16 keys
    (2, 16, 1, [17, 48], 48),
]


@pytest.mark.parametrize("case", EDGE, ids=lambda c: "B%d_H%d_KV%d_L%s_Lmax%d" % (c[0], c[1], c[2],
                                                                                  "-".join(map(str, c[3])), c[4]))
def test_edge_shapes(gpu, case):
    B, Hq, Hkv, sl, Lmax = case
    inp = workloads.custom_decode_inputs(B, Hq, Hkv, sl, max_seq_len=Lmax, hidden=256, seed=sum(sl) + Hq)
    res = _run_step(inp, debug=True)
    _check_step(inp, res, what=str(case))
    att = oracle.attention(inp["q"], inp["k"], inp["v"], inp["seq_lens"], want_scores=True)
    for b, L in enumerate(sl):
        assert_scores_close(res["scores"][b, :, :L], att["scores"][b, :, :L], "scores")
        assert np.all(np.isnan(res["scores"][b, :, L:]))  # nothing written past the sequence
    np.testing.assert_allclose(res["lse"], att["lse"], rtol=1e-5, atol=1e-5)


def test_single_key_is_bit_exact(gpu):
    inp = workloads.custom_decode_inputs(2, 8, 2, [1, 1], max_seq_len=9, seed=21)
    res = _run_step(inp)
    for b in range(2):
        for qh in range(8):
            np.testing.assert_array_equal(res["flat"][b, qh * 128:(qh + 1) * 128], inp["v"][b, qh // 4, 0])


def test_constant_values_are_bit_exact(gpu):
    inp = workloads.custom_decode_inputs(1, 8, 2, [3000], seed=22)
    for h in range(2):
        inp["v"][0, h, :] = inp["v"][0, h, 7]
    res = _run_step(inp)
    for qh in range(8):
        np.testing.assert_array_equal(res["flat"][0, qh * 128:(qh + 1) * 128], inp["v"][0, qh // 4, 7])


def test_softmax_scale_override(gpu):
    inp = workloads.custom_decode_inputs(2, 8, 2, [200, 77], seed=23)
    res = _run_step(inp, scale=0.05)
    _check_step(inp, res, scale=0.05, what="scale 0.05")


def test_near_one_hot_in_the_last_split(gpu):
    # large scores (q x 8) and the dominant key at the very end of a long sequence
    inp = workloads.custom_decode_inputs(1, 4, 1, [2000], seed=24)
    qf = bf16_words_to_f64(inp["q"]) * 8
    inp["q"] = workloads.bf16_words_from_float(qf.astype(np.float32))
    inp["k"][0, 0, 1999] = workloads.bf16_words_from_float((qf[0, 0] / 8).astype(np.float32))
    res = _run_step(inp)
    _check_step(inp, res, what="near one-hot")


def test_result_does_not_depend_on_the_split(gpu):
    # the same sequences under a larger max_seq_len get a different split length
    base = workloads.custom_decode_inputs(2, 8, 2, [1500, 900], max_seq_len=1500, seed=25)
    big = dict(base)
    Lbig = 70000  # 4 (batch, kv head) pairs x 547 splits of 128 exceed the workgroup target
    for key in ("k", "v"):
        a = np.full((2, 2, Lbig, 128), workloads.BF16_NAN, np.uint16)
        a[:, :, :1500] = base[key]
        big[key] = a
    p1 = da.decode_attn_plan(da.make_shape(2, 8, 2, 1500, 256))
    p2 = da.decode_attn_plan(da.make_shape(2, 8, 2, Lbig, 256))
    r1, r2 = _run_step(base), _run_step(big)
    ref = _check_step(base, r1, what="Lmax 1500")
    _check_step(big, r2, what="Lmax 70000")
    assert (p1.split_len, p1.num_splits) != (p2.split_len, p2.num_splits)
    assert ref is not None


def _counter_block_is_clear(ws):
    torch.cuda.synchronize()
    assert int(ws.buf[:COUNTER_BLOCK].count_nonzero()) == 0, "arrival counters left non-zero"


def test_repeat_calls_are_deterministic_and_reuse_the_workspace(gpu):
    ws = PoisonedWorkspace()
    a = workloads.custom_decode_inputs(3, 16, 4, [700, 1, 333], seed=26)
    b = workloads.custom_decode_inputs(1, 4, 1, [4000], hidden=512, seed=27)
    r1 = _run_step(a, ws)
    _counter_block_is_clear(ws)
    r2 = _run_step(b, ws)   # different shape, same (now dirty) workspace
    _counter_block_is_clear(ws)
    r3 = _run_step(a, ws)
    _counter_block_is_clear(ws)
    np.testing.assert_array_equal(r1["out"], r3["out"])
    np.testing.assert_array_equal(r1["flat"], r3["flat"])
    _check_step(b, r2, what="after another shape")


# ---- the single-launch step against two launches ---------------------------

FUSED = [
    # (batch, Hq, Hkv, seq_lens, max_seq_len, hidden)
    (1, 4, 1, [256], 256, 512),
    (1, 32, 8, [2048], 2048, 4096),
    (1, 8, 8, [1], 1, 128),
    (2, 2, 1, [16, 17], 17, 1032),
    (2, 16, 2, [5, 100], 128, 256),
    (2, 8, 1, [1000, 257], 1024, 640),
]


@pytest.mark.parametrize("case", FUSED, ids=lambda c: "B%d_H%d_KV%d_Lmax%d_N%d" % (c[0], c[1], c[2], c[4], c[5]))
def test_single_launch_step_matches_the_oracle_and_two_launches(gpu, case):
    # (step_mode 1: the small single-launch step also where the tiny step would be the built-in)
    B, Hq, Hkv, sl, Lmax, hidden = case
    small = dict(step_mode=1)
    assert da.decode_attn_plan(da.make_shape(B, Hq, Hkv, Lmax, hidden, tiles=small)).fused == 1
    inp = workloads.custom_decode_inputs(B, Hq, Hkv, sl, max_seq_len=Lmax, hidden=hidden, seed=B * 1000 + Hq + hidden)
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    s, w = dev_i32(inp["seq_lens"]), dev_bf16(inp["o_weight"])
    ws = PoisonedWorkspace()
    flat = host_words(da.decode_attn_only(q, k, v, s, workspace=ws))
    outs = []
    for separate in (False, True, False, False):
        outs.append(host_words(da.decode_attn_fwd(q, k, v, s, w, workspace=ws, separate=separate,
                                                  tiles=None if separate else small)))
        _status_ok(ws, "single launch")
        _counter_block_is_clear(ws)
    _check_step(inp, {"flat": flat, "out": outs[0]}, what="single launch")
    _check_step(inp, {"flat": flat, "out": outs[1]}, what="two launches")
    # the single launch is deterministic across calls on one workspace
    np.testing.assert_array_equal(outs[0], outs[2])
    np.testing.assert_array_equal(outs[0], outs[3])


# ---- the projection alone ------------------------------------------------

@pytest.mark.parametrize("M", [1, 3, 8, 15, 16, 20, 33])
def test_oproj_integer_inputs_bit_exact(gpu, M):
    rng = np.random.default_rng(100 + M)
    K, N = 4096, 1024
    x = workloads.bf16_words_from_float(rng.integers(-1, 1, endpoint=True, size=(M, K)).astype(np.float32))
    w = workloads.bf16_words_from_float(rng.integers(-1, 1, endpoint=True, size=(K, N)).astype(np.float32))
    out = host_words(da.oproj_fwd(dev_bf16(x), dev_bf16(w)))
    ref, _ = oracle.oproj(x, w)
    np.testing.assert_array_equal(out, ref)


@pytest.mark.parametrize("M", [1, 4, 16, 17])
def test_oproj_identity_returns_input(gpu, M):
    rng = np.random.default_rng(200 + M)
    K = 512
    x = workloads.bf16_words_from_float(rng.standard_normal((M, K)).astype(np.float32))
    eye = workloads.bf16_words_from_float(np.eye(K, dtype=np.float32))
    out = host_words(da.oproj_fwd(dev_bf16(x), dev_bf16(eye)))
    np.testing.assert_array_equal(out, x)


@pytest.mark.parametrize("shape", [(1, 4096, 4096), (4, 8192, 8192), (16, 4096, 4096), (2, 384, 520), (24, 640, 72)])
def test_oproj_random(gpu, shape):
    M, K, N = shape
    rng = np.random.default_rng(M * 7 + N)
    x = workloads.bf16_words_from_float(rng.standard_normal((M, K)).astype(np.float32) * 0.05)
    w = workloads.bf16_words_from_float(rng.standard_normal((K, N)).astype(np.float32) * 0.02)
    out = host_words(da.oproj_fwd(dev_bf16(x), dev_bf16(w)))
    _, ref = oracle.oproj(x, w)
    assert_bf16_close(out, ref, "oproj %s" % (shape,))


# ---- tile overrides (the measured tile search runs through them) ---------

TILES = [
    dict(attn_workgroups=1), dict(attn_workgroups=7, attn_depth=2), dict(attn_workgroups=192, attn_depth=3),
    dict(attn_workgroups=1024), dict(attn_depth=2, proj_tile_n=64, proj_ksplit=1),
    dict(proj_tile_n=128, proj_ksplit=3), dict(proj_tile_n=256, proj_ksplit=64), dict(step_mode=2),
]


@pytest.mark.parametrize("tiles", TILES, ids=lambda t: "-".join("%s%d" % (k, v) for k, v in t.items()))
@pytest.mark.parametrize("B", [3, 17])
def test_tile_overrides_match_the_oracle(gpu, tiles, B):
    sl = [int(x) for x in np.random.default_rng(B).integers(1, 3000, size=B)]
    inp = workloads.custom_decode_inputs(B, 16, 4, sl, max_seq_len=3000, hidden=520, seed=300 + B)
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    s, w = dev_i32(inp["seq_lens"]), dev_bf16(inp["o_weight"])
    ws = PoisonedWorkspace()
    if B >= 16 and tiles.get("proj_tile_n", 128) != 128:
        # the GEMV-only tile widths serve batches below 16: the call is refused before any launch
        with pytest.raises(da.DecodeAttnError) as e:
            da.decode_attn_fwd(q, k, v, s, w, workspace=ws, tiles=tiles)
        assert e.value.status == da.DA_ERR_SHAPE
        return
    flat = host_words(da.decode_attn_only(q, k, v, s, workspace=ws, tiles=tiles))
    out = host_words(da.decode_attn_fwd(q, k, v, s, w, workspace=ws, tiles=tiles))
    _status_ok(ws, "tiles %s" % (tiles,))
    _counter_block_is_clear(ws)
    again = host_words(da.decode_attn_fwd(q, k, v, s, w, workspace=ws, tiles=tiles))
    np.testing.assert_array_equal(out, again)
    _check_step(inp, {"flat": flat, "out": out}, what="tiles %s" % (tiles,))



# ---- head_dim 256 (stream-K attention + separate projection) -------------

WIDE = [
    # (batch, Hq, Hkv, seq_lens, max_seq_len, hidden)
    (1, 4, 1, [1], 1, 256),
    (1, 8, 1, [33], 40, 512),
    (2, 16, 2, [700, 5], 700, 1024),
    (3, 8, 8, [129, 1, 2000], 2048, 264),
    (1, 32, 2, [4096], 4096, 2048),   # group 16
    (17, 4, 1, [64] * 17, 64, 256),   # the MFMA projection (17 rows)
]


@pytest.mark.parametrize("case", WIDE, ids=lambda c: "B%d_H%d_KV%d_Lmax%d_N%d" % (c[0], c[1], c[2], c[4], c[5]))
def test_head_dim_256_matches_the_oracle(gpu, case):
    B, Hq, Hkv, sl, Lmax, hidden = case
    inp = workloads.custom_decode_inputs(B, Hq, Hkv, sl, max_seq_len=Lmax, hidden=hidden, head_dim=256,
                                         seed=400 + B * 10 + Hq)
    res = _run_step(inp, debug=True)
    _check_step(inp, res, what="head_dim 256 %s" % (case,))
    att = oracle.attention(inp["q"], inp["k"], inp["v"], inp["seq_lens"], want_scores=True)
    for b, L in enumerate(sl):
        assert_scores_close(res["scores"][b, :, :L], att["scores"][b, :, :L], "head_dim 256 scores")
    np.testing.assert_allclose(res["lse"], att["lse"], rtol=1e-5, atol=1e-5)


def test_head_dim_256_single_key_is_bit_exact(gpu):
    inp = workloads.custom_decode_inputs(2, 8, 2, [1, 1], max_seq_len=5, hidden=256, head_dim=256, seed=41)
    res = _run_step(inp)
    for b in range(2):
        for qh in range(8):
            np.testing.assert_array_equal(res["flat"][b, qh * 256:(qh + 1) * 256], inp["v"][b, qh // 4, 0])


# ---- context (prefill) attention ------------------------------------------

def _prefill_case(B, T, Hq, Hkv, ctx, Lmax, seed):
    rng = np.random.default_rng(seed)
    q = workloads.bf16_words_from_float(rng.standard_normal((B, T, Hq, 128)).astype(np.float32))
    k = workloads.bf16_words_from_float(rng.standard_normal((B, Hkv, Lmax, 128)).astype(np.float32))
    v = workloads.bf16_words_from_float(rng.standard_normal((B, Hkv, Lmax, 128)).astype(np.float32))
    workloads.poison_padding(k, v, ctx)  # rows past each context are NaN: never read
    return q, k, v, np.asarray(ctx, dtype=np.int32)


PREFILL = [
    # (batch, tokens, Hq, Hkv, ctx_lens, max_seq_len)
    (1, 1, 4, 1, [5], 8),
    (1, 17, 8, 2, [17], 20),
    (2, 40, 32, 8, [100, 40], 128),
    (1, 64, 16, 1, [300], 300),
    (2, 5, 2, 2, [33, 7], 40),
    (3, 33, 24, 8, [1000, 500, 33], 1024),
    (1, 256, 32, 8, [2048], 2048),
    # small causal chunks (max_seq_len < 1.5 T, few row blocks): one row set per wave
    (2, 100, 8, 2, [120, 100], 128),   # ragged prefix 20 and 0
    (1, 300, 12, 4, [300], 310),       # 15 blocks of 64 rows, the last one partial
    (1, 33, 4, 4, [33], 33),           # G = 1, one block
]


@pytest.mark.parametrize("case", PREFILL, ids=lambda c: "B%d_T%d_H%d_KV%d_ctx%s" % (c[0], c[1], c[2], c[3],
                                                                                     "-".join(map(str, c[4]))))
def test_prefill_matches_the_oracle(gpu, case):
    B, T, Hq, Hkv, ctx, Lmax = case
    q, k, v, cl = _prefill_case(B, T, Hq, Hkv, ctx, Lmax, seed=500 + T + Hq)
    out = host_words(da.prefill_attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_i32(cl)))
    ref = oracle.prefill_attention(q, k, v, cl)
    assert_bf16_close(out, ref["ref"], "prefill %s" % (case,))


def test_prefill_first_token_without_prefix_is_bit_exact(gpu):
    q, k, v, cl = _prefill_case(2, 9, 8, 2, [9, 9], 16, seed=61)
    out = host_words(da.prefill_attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_i32(cl)))
    for b in range(2):
        for qh in range(8):
            np.testing.assert_array_equal(out[b, 0, qh * 128:(qh + 1) * 128], v[b, qh // 4, 0])


def test_prefill_of_one_token_matches_decode_attention(gpu):
    q, k, v, cl = _prefill_case(3, 1, 16, 4, [70, 1, 129], 130, seed=62)
    pre = host_words(da.prefill_attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_i32(cl)))
    dec = host_words(da.decode_attn_only(dev_bf16(q[:, 0]), dev_bf16(k), dev_bf16(v), dev_i32(cl)))
    # both within the bound of the same oracle; equal up to their different summation orders
    ref = oracle.attention(q[:, 0], k, v, cl)["ref"]
    assert_bf16_close(pre[:, 0], ref, "prefill T=1")
    assert_bf16_close(dec, ref, "decode")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("wl", workloads.PREFILL, ids=lambda w: w.name)
def test_prefill_benchmark_workloads(gpu, wl):
    # the benchmarked sizes: every output of every sequence against the oracle (the chunk's four
    # sequences take the oracle about a minute on the host's cores)
    inp = workloads.prefill_inputs(wl, poison=True)
    out = host_words(da.prefill_attn_fwd(dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"]),
                                         dev_i32(inp["ctx_lens"])))
    print("%s: oracle over %d sequence(s)" % (wl.name, wl.batch), flush=True)
    ref = oracle.prefill_attention(inp["q"], inp["k"], inp["v"], inp["ctx_lens"])["ref"]
    assert_bf16_close(out, ref, wl.name)


# ---- the single-launch step's bounded wait, forced to give up from the host ----

def test_single_launch_step_timeout_is_reported(gpu):
    # 8 kv heads of 8192 keys: the attention runs for several microseconds, while a projection
    # workgroup allowed a single poll checks its counters right after requesting its weights, so
    # it gives up. Every kernel still exits; the status call reports it, the output columns of a
    # workgroup that gave up are NaN, and after the counters are zero-filled the step is correct.
    B, Hq, Hkv, L, hidden = 1, 32, 8, 8192, 4096
    shape = da.make_shape(B, Hq, Hkv, L, hidden)
    assert da.decode_attn_plan(shape).fused == 1
    inp = workloads.custom_decode_inputs(B, Hq, Hkv, [L], max_seq_len=L, hidden=hidden, seed=71)
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    s, w = dev_i32(inp["seq_lens"]), dev_bf16(inp["o_weight"])
    ws = PoisonedWorkspace()
    flat = host_words(da.decode_attn_only(q, k, v, s, workspace=ws))
    assert da.decode_attn_step_status(ws) == da.DA_OK
    timed_out = False
    for _ in range(3):  # one try gives up in practice; a few guard against a lucky first poll
        out = host_words(da.decode_attn_fwd(q, k, v, s, w, workspace=ws, tiles=dict(step_wait_polls=1)))
        if da.decode_attn_step_status(ws) == da.DA_ERR_TIMEOUT:
            timed_out = True
            assert np.isnan(bf16_words_to_f64(out)).any(), "a workgroup gave up but no output is NaN"
            break
    assert timed_out, "a one-poll wait never gave up"
    ws.buf[:COUNTER_BLOCK].zero_()
    assert da.decode_attn_step_status(ws) == da.DA_OK
    out = host_words(da.decode_attn_fwd(q, k, v, s, w, workspace=ws))
    _status_ok(ws, "after the counters were zero-filled")
    _counter_block_is_clear(ws)
    _check_step(inp, {"flat": flat, "out": out}, what="after a timeout")


# ---- the tiny step: every workgroup computes the whole attention ----------------

TINY = [
    # (batch, Hq, Hkv, seq_lens, max_seq_len, hidden)
    (1, 4, 1, [256], 256, 512),          # the tiny workload's shape
    (2, 16, 2, [128, 5], 128, 256),      # two sequences per kv head, 256 KiB of K/V
    (1, 16, 1, [200], 200, 264),         # group 16; a last column tile half past N
    (2, 4, 1, [1, 250], 250, 512),       # a single key (its output is the value row) and a ragged tail
    (1, 8, 8, [33], 40, 1040),           # eight kv heads of one query head each; 65 column tiles on 4 XCDs
    (1, 4, 1, [64], 64, 8200),           # 513 column tiles: all eight XCDs, the last one past N
]


@pytest.mark.parametrize("case", TINY, ids=lambda c: "B%d_H%d_KV%d_Lmax%d_N%d" % (c[0], c[1], c[2], c[4], c[5]))
def test_tiny_step_matches_the_oracle(gpu, case):
    B, Hq, Hkv, sl, Lmax, hidden = case
    tiles = dict(step_mode=4)
    assert da.decode_attn_plan(da.make_shape(B, Hq, Hkv, Lmax, hidden, tiles=tiles)).fused == 3
    inp = workloads.custom_decode_inputs(B, Hq, Hkv, sl, max_seq_len=Lmax, hidden=hidden, seed=B * 31 + Hq + hidden)
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    s, w = dev_i32(inp["seq_lens"]), dev_bf16(inp["o_weight"])
    ws = PoisonedWorkspace()
    flat = host_words(da.decode_attn_only(q, k, v, s, workspace=ws))
    out = host_words(da.decode_attn_fwd(q, k, v, s, w, workspace=ws, tiles=tiles))
    _status_ok(ws, "tiny step")
    _check_step(inp, {"flat": flat, "out": out}, what="tiny step")
    again = host_words(da.decode_attn_fwd(q, k, v, s, w, workspace=ws, tiles=tiles))
    np.testing.assert_array_equal(out, again)


def test_tiny_step_single_key_projects_the_value_rows(gpu):
    # one key per sequence: the attention output is that key's value row exactly, so the step's
    # output is the oracle's projection of the value rows
    B, Hq, Hkv, hidden = 2, 8, 2, 256
    inp = workloads.custom_decode_inputs(B, Hq, Hkv, [1, 1], max_seq_len=3, hidden=hidden, seed=43)
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    s, w = dev_i32(inp["seq_lens"]), dev_bf16(inp["o_weight"])
    out = host_words(da.decode_attn_fwd(q, k, v, s, w, workspace=PoisonedWorkspace(), tiles=dict(step_mode=4)))
    flat = np.stack([np.concatenate([inp["v"][b, qh // (Hq // Hkv), 0] for qh in range(Hq)]) for b in range(B)])
    _, ref = oracle.oproj(flat, inp["o_weight"])
    assert_within_fp32_sum_bound(out, ref, flat, inp["o_weight"], "tiny step, one key")


# ---- the single-launch large step against two launches -----------------------

LARGE = [
    # (batch, Hq, Hkv, seq_lens, max_seq_len, hidden)
    (5, 32, 8, [3000, 17, 2048, 999, 64], 3000, 4096),
    (16, 32, 8, [1024 + 431 * i for i in range(16)], 8192, 4096),
    (6, 16, 2, [1, 33, 700, 129, 5000, 2], 5000, 264),      # sequences shorter than a stream-K range
    (32, 8, 1, [64 + 97 * i for i in range(32)], 3200, 512),   # two 16-row m-tiles, one kv head
    (4, 64, 8, [2000, 2001, 4095, 4096], 4096, 8192),          # group 8, 8 K-chunks of 1024 rows
    (3, 16, 2, [5, 37, 100], 128, 256),                         # small steps of more than two sequences
    (4, 8, 2, [255, 256, 257, 1000], 1024, 640),
    (4, 32, 8, [1000, 17, 600, 999], 1000, 4096),
]


@pytest.mark.parametrize("case", LARGE, ids=lambda c: "B%d_H%d_KV%d_Lmax%d_N%d" % (c[0], c[1], c[2], c[4], c[5]))
def test_single_launch_large_step_matches_the_oracle_and_two_launches(gpu, case):
    B, Hq, Hkv, sl, Lmax, hidden = case
    assert da.decode_attn_plan(da.make_shape(B, Hq, Hkv, Lmax, hidden)).fused == 2
    inp = workloads.custom_decode_inputs(B, Hq, Hkv, sl, max_seq_len=Lmax, hidden=hidden, seed=B * 100 + Hq + hidden)
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    s, w = dev_i32(inp["seq_lens"]), dev_bf16(inp["o_weight"])
    ws = PoisonedWorkspace()
    flat = host_words(da.decode_attn_only(q, k, v, s, workspace=ws))
    outs = []
    for separate in (False, True, False):
        outs.append(host_words(da.decode_attn_fwd(q, k, v, s, w, workspace=ws, separate=separate)))
        _status_ok(ws, "large single launch")
        _counter_block_is_clear(ws)
    _check_step(inp, {"flat": flat, "out": outs[0]}, what="large single launch")
    _check_step(inp, {"flat": flat, "out": outs[1]}, what="two launches")
    # one launch and two run the same kernels' arithmetic except where a sequence has more
    # pieces than one merge batch: two launches merge those weights first, so the forms
    # agree within the tolerance above; each form is bit-exact from call to call
    print("words that differ between one launch and two: %d" % int((outs[0] != outs[1]).sum()))
    np.testing.assert_array_equal(outs[0], outs[2])


@pytest.mark.parametrize("case", [(1, 32, 8, [2048], 2048, 4096), (2, 4, 1, [31, 700], 700, 512)],
                         ids=lambda c: "B%d_H%d_KV%d_Lmax%d_N%d" % (c[0], c[1], c[2], c[4], c[5]))
def test_large_step_chosen_for_a_small_shape(gpu, case):
    # step_mode 3 runs the large single-launch step where the built-in choice is the small one
    B, Hq, Hkv, sl, Lmax, hidden = case
    assert da.decode_attn_plan(da.make_shape(B, Hq, Hkv, Lmax, hidden)).fused == 1
    assert da.decode_attn_plan(da.make_shape(B, Hq, Hkv, Lmax, hidden, tiles=dict(step_mode=3))).fused == 2
    inp = workloads.custom_decode_inputs(B, Hq, Hkv, sl, max_seq_len=Lmax, hidden=hidden, seed=B * 7 + Hq)
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    s, w = dev_i32(inp["seq_lens"]), dev_bf16(inp["o_weight"])
    ws = PoisonedWorkspace()
    flat = host_words(da.decode_attn_only(q, k, v, s, workspace=ws))
    large = host_words(da.decode_attn_fwd(q, k, v, s, w, workspace=ws, tiles=dict(step_mode=3)))
    _status_ok(ws, "large single launch on a small shape")
    _counter_block_is_clear(ws)
    two = host_words(da.decode_attn_fwd(q, k, v, s, w, workspace=ws, separate=True))
    _check_step(inp, {"flat": flat, "out": large}, what="large single launch on a small shape")
    _check_step(inp, {"flat": flat, "out": two}, what="two launches")
    again = host_words(da.decode_attn_fwd(q, k, v, s, w, workspace=ws, tiles=dict(step_mode=3)))
    np.testing.assert_array_equal(large, again)


def test_single_launch_large_step_timeout_is_reported(gpu):
    # projection workgroups allowed one poll give up while the attention of 16 x 8192 keys still runs
    B, Hq, Hkv, L, hidden = 16, 32, 8, 8192, 4096
    assert da.decode_attn_plan(da.make_shape(B, Hq, Hkv, L, hidden)).fused == 2
    inp = workloads.custom_decode_inputs(B, Hq, Hkv, [L] * B, max_seq_len=L, hidden=hidden, seed=72)
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    s, w = dev_i32(inp["seq_lens"]), dev_bf16(inp["o_weight"])
    ws = PoisonedWorkspace()
    flat = host_words(da.decode_attn_only(q, k, v, s, workspace=ws))
    out = host_words(da.decode_attn_fwd(q, k, v, s, w, workspace=ws, tiles=dict(step_wait_polls=1)))
    assert da.decode_attn_step_status(ws) == da.DA_ERR_TIMEOUT
    assert np.isnan(bf16_words_to_f64(out)).any(), "a workgroup gave up but no output is NaN"
    ws.buf[:COUNTER_BLOCK].zero_()
    out = host_words(da.decode_attn_fwd(q, k, v, s, w, workspace=ws))
    _status_ok(ws, "after the counters were zero-filled")
    _counter_block_is_clear(ws)
    _check_step(inp, {"flat": flat, "out": out}, what="large step after a timeout")


def test_read_probe_reads_every_byte(gpu):
    # the measurement probe folds its share of the words with xor: every 16-byte unit is read once
    rng = np.random.default_rng(81)
    n16, W = 5000, 7
    words = rng.integers(0, 2 ** 32, size=(n16, 4), dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.zeros(W, dtype=torch.int32, device="cuda")
    rc = da.load_library().decode_attn_read_probe(src.data_ptr(), n16 * 16, sink.data_ptr(), W,
                                                  torch.cuda.current_stream().cuda_stream)
    assert rc == da.DA_OK
    got = sink.cpu().numpy().view(np.uint32)
    for w in range(W):
        b0 = (n16 * w // W) & ~63
        b1 = n16 if w + 1 == W else (n16 * (w + 1) // W) & ~63
        want = np.bitwise_xor.reduce(words[b0:b1].ravel()) if b1 > b0 else np.uint32(0)
        assert got[w] == want, w
