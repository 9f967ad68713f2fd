"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test checks the oracle against a closed form, an invariant of the
mathematics, a printed worked example of the pages (``tests/golden/``), an
independent library routine, or brute force on a tiny input. They are chosen so
that a plausible slip in the oracle -- a dropped term, a wrong sign, scale or
index, a transposed operand, double rounding -- fails at least one of them.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_fixture(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def bf16(x):
    return workloads.bf16_words_from_float(x)


def bw(x) -> int:
    """One bf16 word (as a Python int) for a float that bf16 holds exactly."""
    return int(np.asarray(bf16(x)).reshape(-1)[0])


def f64(words):
    """bf16 words -> float64 through torch (independent of the oracle's widening)."""
    t = torch.from_numpy(np.ascontiguousarray(words).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------

def test_bf16_all_words_round_trip():
    words = np.arange(65536, dtype=np.uint16)
    exp = (words >> 7) & 0xFF
    frac = words & 0x7F
    finite_or_inf = ~((exp == 0xFF) & (frac != 0))
    w = words[finite_or_inf]
    d = oracle.bf16_to_double(w)
    np.testing.assert_array_equal(d, f64(w))  # widening agrees with torch
    back = oracle.bf16_from_double(d)
    np.testing.assert_array_equal(back, w)  # every bf16 value rounds to itself


def test_bf16_rounding_matches_torch_on_float32_values():
    rng = np.random.default_rng(123)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(5000) * 1e-38).astype(np.float32),  # subnormal range
        np.clip(rng.standard_normal(5000) * 3e38, -3.3e38, 3.3e38).astype(np.float32),  # overflow edge
        # exact ties: a bf16 value plus half its last place
        (np.arange(1, 2000, dtype=np.float32) * np.float32(2.0 ** -7) + np.float32(2.0 ** -8) + 1).astype(np.float32),
    ])
    x = x[np.isfinite(x)]
    ours = oracle.bf16_from_double(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_bf16_rounds_from_double_without_double_rounding():
    # ties go to even
    assert oracle.bf16_from_double(1.0 + 2.0 ** -8) == 0x3F80
    assert oracle.bf16_from_double(1.0 + 3 * 2.0 ** -8) == 0x3F82
    # just above a tie, below float32 resolution: float32 would first round to
    # the tie and then to even (0x3F80); direct rounding must go up.
    assert oracle.bf16_from_double(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81
    assert oracle.bf16_from_double(-(1.0 + 2.0 ** -8 + 2.0 ** -40)) == 0xBF81
    # specials
    assert oracle.bf16_from_double(float("inf")) == 0x7F80
    assert oracle.bf16_from_double(-0.0) == 0x8000
    assert (oracle.bf16_from_double(float("nan")) & 0x7FFF) > 0x7F80
    assert oracle.bf16_from_double(3.5e38) == 0x7F80  # beyond max finite


def test_f16_round_trip_and_numpy_rounding():
    words = np.arange(65536, dtype=np.uint16)
    exp = (words >> 10) & 0x1F
    frac = words & 0x3FF
    w = words[~((exp == 0x1F) & (frac != 0))]
    d = oracle.f16_to_double(w)
    np.testing.assert_array_equal(d, w.view(np.float16).astype(np.float64))
    np.testing.assert_array_equal(oracle.f16_from_double(d), w)
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(20000) * 100, rng.standard_normal(5000) * 1e-6,
                        np.clip(rng.standard_normal(2000) * 7e4, -6.5e4, 6.5e4), np.arange(2040, 2070, 0.5),
                        np.array([65504.0, 65519.0, 65520.0, -65520.0, 70000.0])])
    with np.errstate(over="ignore"):  # 70000 overflows to inf on purpose
        expect = x.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(oracle.f16_from_double(x), expect)
    # integers above 2048 are spaced by 2: ties to even
    assert oracle.f16_from_double(2049.0) == np.float16(2048).view(np.uint16)
    assert oracle.f16_from_double(2051.0) == np.float16(2052).view(np.uint16)


# --------------------------------------------------------------------------
# dense fp16 GEMM
# --------------------------------------------------------------------------

def test_gemm_all_ones_golden_from_page():
    fx = {r[0]: r[1] for r in _read_fixture("basic_matmul_all_ones.txt")}
    m, n, k = int(fx["m"]), int(fx["n"]), int(fx["k"])
    a = np.ones((m, k), dtype=np.float16).view(np.uint16)
    b = np.ones((k, n), dtype=np.float16).view(np.uint16)
    c, ref = oracle.gemm_f16(a, b)
    assert c.shape == (m, n)
    assert np.all(ref == float(fx["c_value"]))
    assert np.all(c == int(fx["c_fp16_word"], 16))


def test_gemm_one_hot_and_permutation_catch_transposes():
    rng = np.random.default_rng(5)
    M, K, N = 6, 9, 7
    b = rng.integers(-1, 1, endpoint=True, size=(K, N)).astype(np.float16)
    a = np.zeros((M, K), dtype=np.float16)
    a[4, 2] = 1
    c, _ = oracle.gemm_f16(a.view(np.uint16), b.view(np.uint16))
    cf = c.view(np.float16).astype(np.float64)
    np.testing.assert_array_equal(cf[4], b[2].astype(np.float64))
    assert np.all(cf[np.arange(M) != 4] == 0)
    # right-multiplying by a permutation matrix permutes the columns of A
    A = rng.integers(-1, 1, endpoint=True, size=(M, K)).astype(np.float16)
    perm = rng.permutation(K)
    P = np.zeros((K, K), dtype=np.float16)
    P[np.arange(K), perm] = 1  # column perm[k] receives column k
    c, _ = oracle.gemm_f16(A.view(np.uint16), P.view(np.uint16))
    cf = c.view(np.float16).astype(np.float64)
    for kk in range(K):
        np.testing.assert_array_equal(cf[:, perm[kk]], A[:, kk].astype(np.float64))


def test_gemm_integer_brute_force_tiny():
    rng = np.random.default_rng(11)
    M, K, N = 5, 13, 4
    a = rng.integers(-1, 1, endpoint=True, size=(M, K))
    b = rng.integers(-1, 1, endpoint=True, size=(K, N))
    c, ref = oracle.gemm_f16(a.astype(np.float16).view(np.uint16), b.astype(np.float16).view(np.uint16))
    for i in range(M):
        for j in range(N):
            exact = 0
            for kk in range(K):
                exact += int(a[i, kk]) * int(b[kk, j])
            assert ref[i, j] == exact
            assert c[i, j] == np.float16(exact).view(np.uint16)


def test_gemm_config_values_are_exact_integers():
    g = workloads.gemm_inputs()
    c, ref = oracle.gemm_f16(g["a"][:32], g["b"])
    assert np.all(ref == np.round(ref))
    assert np.all(np.abs(ref) <= g["k"])
    np.testing.assert_array_equal(c.view(np.float16).astype(np.float64), ref)


# --------------------------------------------------------------------------
# attention (QK^T -> scaled softmax -> attn.V)
# --------------------------------------------------------------------------

def _zeros_inputs(B, Hq, Hkv, L, D=128):
    q = np.zeros((B, Hq, D), np.uint16)
    k = np.zeros((B, Hkv, L, D), np.uint16)
    v = np.zeros((B, Hkv, L, D), np.uint16)
    return q, k, v


def test_single_key_returns_that_value_row():
    inp = workloads.custom_decode_inputs(2, 8, 2, [1, 1], max_seq_len=5, seed=3)
    r = oracle.attention(inp["q"], inp["k"], inp["v"], inp["seq_lens"])
    G = 4
    for b in range(2):
        for qh in range(8):
            np.testing.assert_array_equal(r["flat"][b, qh * 128:(qh + 1) * 128], inp["v"][b, qh // G, 0])


def test_constant_value_rows_give_that_row():
    inp = workloads.custom_decode_inputs(1, 4, 1, [37], seed=4)
    row = inp["v"][0, 0, 0].copy()
    inp["v"][0, 0, :37] = row
    r = oracle.attention(inp["q"], inp["k"], inp["v"], inp["seq_lens"])
    for qh in range(4):
        np.testing.assert_array_equal(r["flat"][0, qh * 128:(qh + 1) * 128], row)


def test_zero_query_gives_uniform_weights_and_mean_of_values():
    inp = workloads.custom_decode_inputs(1, 2, 1, [11], seed=5)
    inp["q"][:] = 0
    r = oracle.attention(inp["q"], inp["k"], inp["v"], inp["seq_lens"], want_scores=True)
    np.testing.assert_allclose(r["probs"][0, :, :11], 1.0 / 11, rtol=1e-15)
    vals = f64(inp["v"][0, 0, :11])
    for d in range(128):
        exact = sum(Fraction(float(x)) for x in vals[:, d]) / 11
        for qh in range(2):
            assert abs(r["ref"][0, qh * 128 + d] - float(exact)) <= 1e-14


def test_two_keys_closed_form_pins_scale_and_sign():
    # q = all ones; K0 = 0 -> dot 0; K1 = ones on 16 dims -> dot 16.
    # s1 - s0 = 16 / sqrt(128) = sqrt(2); p1 = 1 / (1 + exp(-sqrt(2))).
    q, k, v = _zeros_inputs(1, 1, 1, 2)
    one, two_neg = bw(1.0), bw(-2.0)
    q[0, 0, :] = one
    k[0, 0, 1, :16] = one
    v[0, 0, 0, :] = one
    v[0, 0, 1, :] = two_neg
    r = oracle.attention(q, k, v, np.array([2], np.int32), want_scores=True)
    p1 = 1.0 / (1.0 + math.exp(-math.sqrt(2.0)))
    assert abs(r["probs"][0, 0, 1] - p1) < 1e-15
    assert abs(r["scores"][0, 0, 1] - math.sqrt(2.0)) < 1e-15
    assert r["scores"][0, 0, 0] == 0.0
    expect = (1 - p1) * 1.0 + p1 * (-2.0)
    np.testing.assert_allclose(r["ref"][0], expect, rtol=0, atol=1e-15)
    # explicit scale argument is honoured (scale 1: p1 = 1/(1+e^-16))
    r1 = oracle.attention(q, k, v, np.array([2], np.int32), scale=1.0, want_scores=True)
    assert abs(r1["probs"][0, 0, 1] - 1.0 / (1.0 + math.exp(-16.0))) < 1e-15


def test_weights_sum_to_one_and_match_lse():
    inp = workloads.custom_decode_inputs(2, 8, 4, [300, 17], seed=6)
    r = oracle.attention(inp["q"], inp["k"], inp["v"], inp["seq_lens"], want_scores=True)
    for b, L in enumerate([300, 17]):
        p = r["probs"][b, :, :L]
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        np.testing.assert_allclose(p, np.exp(r["scores"][b, :, :L] - r["lse"][b][:, None]), rtol=1e-12)
        assert np.all(np.isnan(r["scores"][b, :, L:]))  # nothing written beyond the sequence


def test_shift_of_all_scores_changes_nothing():
    inp = workloads.custom_decode_inputs(1, 4, 1, [50], seed=7)
    inp["k"][0, 0, :, 0] = bw(1.0)  # every key has 1 in dim 0
    base = inp["q"].copy()
    base[..., 0] = 0
    r0 = oracle.attention(base, inp["k"], inp["v"], inp["seq_lens"])
    shifted = base.copy()
    shifted[..., 0] = bw(3.0)  # adds 3/sqrt(128) to every score of every head
    r1 = oracle.attention(shifted, inp["k"], inp["v"], inp["seq_lens"])
    np.testing.assert_allclose(r1["ref"], r0["ref"], rtol=0, atol=1e-13)


def test_permuting_keys_with_values_changes_nothing():
    inp = workloads.custom_decode_inputs(1, 4, 2, [64], seed=8)
    perm = np.random.default_rng(0).permutation(64)
    k2, v2 = inp["k"].copy(), inp["v"].copy()
    k2[:, :, :64] = inp["k"][:, :, perm]
    v2[:, :, :64] = inp["v"][:, :, perm]
    r0 = oracle.attention(inp["q"], inp["k"], inp["v"], inp["seq_lens"])
    r1 = oracle.attention(inp["q"], k2, v2, inp["seq_lens"])
    np.testing.assert_allclose(r1["ref"], r0["ref"], rtol=0, atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv_heads():
    inp = workloads.custom_decode_inputs(2, 8, 2, [40, 23], seed=9)
    r_gqa = oracle.attention(inp["q"], inp["k"], inp["v"], inp["seq_lens"])
    k_rep = np.repeat(inp["k"], 4, axis=1)  # kv head h serves query heads 4h..4h+3
    v_rep = np.repeat(inp["v"], 4, axis=1)
    r_mha = oracle.attention(inp["q"], k_rep, v_rep, inp["seq_lens"])
    np.testing.assert_array_equal(r_gqa["ref"], r_mha["ref"])
    # and a different pairing (query head -> head % Hkv) gives a different answer
    k_tile = np.tile(inp["k"], (1, 4, 1, 1))
    v_tile = np.tile(inp["v"], (1, 4, 1, 1))
    r_wrong = oracle.attention(inp["q"], k_tile, v_tile, inp["seq_lens"])
    assert np.max(np.abs(r_wrong["ref"] - r_gqa["ref"])) > 1e-3


def test_matches_torch_float64_sdpa_with_repeated_kv():
    inp = workloads.custom_decode_inputs(2, 8, 2, [33, 70], seed=10)
    r = oracle.attention(inp["q"], inp["k"], inp["v"], inp["seq_lens"])
    for b, L in enumerate([33, 70]):
        q = torch.from_numpy(f64(inp["q"][b]))[:, None, :]                      # [Hq, 1, D]
        k = torch.from_numpy(np.repeat(f64(inp["k"][b, :, :L]), 4, axis=0))    # [Hq, L, D]
        v = torch.from_numpy(np.repeat(f64(inp["v"][b, :, :L]), 4, axis=0))
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v)          # [Hq, 1, D]
        np.testing.assert_allclose(r["ref"][b], o[:, 0, :].reshape(-1).numpy(), rtol=0, atol=1e-13)


def test_padding_rows_are_never_read():
    inp = workloads.custom_decode_inputs(3, 4, 2, [5, 64, 1], max_seq_len=80, seed=12, poison=True)
    r = oracle.attention(inp["q"], inp["k"], inp["v"], inp["seq_lens"])
    assert np.all(np.isfinite(r["ref"]))
    for b, L in enumerate([5, 64, 1]):
        rb = oracle.attention(inp["q"][b:b + 1], inp["k"][b:b + 1, :, :L].copy(), inp["v"][b:b + 1, :, :L].copy(),
                              np.array([L], np.int32))
        np.testing.assert_array_equal(rb["ref"][0], r["ref"][b])


def test_dominant_key_gives_its_value_row():
    q, k, v = _zeros_inputs(1, 1, 1, 9)
    q[0, 0, 0] = bw(8.0)
    k[0, 0, 6, 0] = bw(64.0)  # dot 512 -> score 45.25; every other score 0
    rng = np.random.default_rng(1)
    v[0, 0] = bf16(rng.standard_normal((9, 128)))
    r = oracle.attention(q, k, v, np.array([9], np.int32))
    # p6 = 1/(1+8 e^-45.25): o = v6 to within 1e-18 relative
    np.testing.assert_array_equal(r["flat"][0], v[0, 0, 6])
    np.testing.assert_allclose(r["ref"][0], f64(v[0, 0, 6]), rtol=1e-17, atol=1e-19)


def test_huge_scores_do_not_overflow():
    # the softmax must subtract the running maximum over *every* key: a last
    # key with score 65536/sqrt(128) ~ 5793 would overflow exp() otherwise.
    for pos in (0, 4, 8):
        q, k, v = _zeros_inputs(1, 1, 1, 9)
        q[0, 0, 0] = bw(256.0)
        k[0, 0, pos, 0] = bw(256.0)
        k[0, 0, (pos + 3) % 9, 0] = bw(128.0)  # runner-up at half the score: weight e^-2896
        v[0, 0] = bf16(np.random.default_rng(pos).standard_normal((9, 128)))
        r = oracle.attention(q, k, v, np.array([9], np.int32))
        assert np.all(np.isfinite(r["ref"]))
        np.testing.assert_array_equal(r["flat"][0], v[0, 0, pos])


def test_rejects_empty_sequences_and_bad_grouping():
    inp = workloads.custom_decode_inputs(1, 4, 2, [3], seed=13)
    with pytest.raises(oracle.OracleError):
        oracle.attention(inp["q"], inp["k"], inp["v"], np.array([0], np.int32))
    with pytest.raises(oracle.OracleError):
        oracle.attention(inp["q"], inp["k"], inp["v"], np.array([4], np.int32))  # beyond max_seq_len
    q3 = np.zeros((1, 3, 128), np.uint16)
    with pytest.raises(oracle.OracleError):
        oracle.attention(q3, inp["k"], inp["v"], inp["seq_lens"])  # 3 query heads over 2 kv heads


# --------------------------------------------------------------------------
# output projection and the whole step
# --------------------------------------------------------------------------

def test_oproj_identity_permutation_and_one_hot():
    rng = np.random.default_rng(14)
    K = 256
    x = bf16(rng.standard_normal((2, K)))
    eye = bf16(np.eye(K))
    out, ref = oracle.oproj(x, eye)
    np.testing.assert_array_equal(out, x)
    perm = rng.permutation(K)
    P = np.zeros((K, K), np.float32)
    P[np.arange(K), perm] = 1.0
    out, _ = oracle.oproj(x, bf16(P))
    np.testing.assert_array_equal(out[:, perm], x)
    W = bf16(rng.standard_normal((K, 48)))
    onehot = np.zeros((1, K), np.float32)
    onehot[0, 77] = 1.0
    out, _ = oracle.oproj(bf16(onehot), W)
    np.testing.assert_array_equal(out[0], W[77])


def test_oproj_all_ones_weight_sums_the_input():
    rng = np.random.default_rng(15)
    x = rng.integers(-1, 1, endpoint=True, size=(3, 512)).astype(np.float32)
    out, ref = oracle.oproj(bf16(x), bf16(np.ones((512, 10), np.float32)))
    for m in range(3):
        assert np.all(ref[m] == x[m].sum())


def test_decode_step_is_attention_then_projection_of_bf16_output():
    inp = workloads.custom_decode_inputs(2, 8, 2, [19, 7], hidden=64, seed=16)
    st = oracle.decode_step(inp["q"], inp["k"], inp["v"], inp["seq_lens"], inp["o_weight"])
    at = oracle.attention(inp["q"], inp["k"], inp["v"], inp["seq_lens"])
    np.testing.assert_array_equal(st["flat"], at["flat"])
    out, ref = oracle.oproj(at["flat"], inp["o_weight"])
    np.testing.assert_array_equal(st["out"], out)
    np.testing.assert_array_equal(st["out_ref"], ref)
    # head-major flatten: with W = identity the step returns the attention output
    inp2 = workloads.custom_decode_inputs(1, 2, 1, [5], hidden=256, seed=17)
    st2 = oracle.decode_step(inp2["q"], inp2["k"], inp2["v"], inp2["seq_lens"], bf16(np.eye(256)))
    np.testing.assert_array_equal(st2["out"], st2["flat"])
    v0 = oracle.attention(inp2["q"][:, :1], inp2["k"], inp2["v"], inp2["seq_lens"])["flat"]
    np.testing.assert_array_equal(st2["out"][0, :128], v0[0])  # head 0 occupies columns 0..127


def test_thread_count_does_not_change_results():
    inp = workloads.custom_decode_inputs(2, 8, 2, [100, 31], hidden=128, seed=18)
    a = oracle.decode_step(inp["q"], inp["k"], inp["v"], inp["seq_lens"], inp["o_weight"], nthreads=1)
    b = oracle.decode_step(inp["q"], inp["k"], inp["v"], inp["seq_lens"], inp["o_weight"], nthreads=7)
    np.testing.assert_array_equal(a["out_ref"], b["out_ref"])
    np.testing.assert_array_equal(a["attn_ref"], b["attn_ref"])


# ---- context (prefill) attention -----------------------------------------

def _prefill_inputs(B, T, Hq, Hkv, ctx, Lmax, D=128, seed=0):
    rng = np.random.default_rng(seed)
    q = workloads.bf16_words_from_float(rng.standard_normal((B, T, Hq, D)).astype(np.float32))
    k = workloads.bf16_words_from_float(rng.standard_normal((B, Hkv, Lmax, D)).astype(np.float32))
    v = workloads.bf16_words_from_float(rng.standard_normal((B, Hkv, Lmax, D)).astype(np.float32))
    return q, k, v, np.asarray(ctx, dtype=np.int32)


def test_prefill_of_one_token_is_the_decode_step():
    q, k, v, ctx = _prefill_inputs(2, 1, 8, 2, [37, 64], 64, seed=1)
    pre = oracle.prefill_attention(q, k, v, ctx)
    dec = oracle.attention(q[:, 0], k, v, ctx)
    np.testing.assert_array_equal(pre["out"][:, 0], dec["flat"])
    np.testing.assert_array_equal(pre["ref"][:, 0], dec["ref"])


def test_every_prefill_row_is_a_decode_step_over_its_prefix():
    # token t of sequence b sees exactly keys 0 .. ctx_b - T + t: the decode oracle on that prefix
    B, T, Hq, Hkv = 2, 5, 4, 2
    q, k, v, ctx = _prefill_inputs(B, T, Hq, Hkv, [9, 30], 32, seed=2)
    pre = oracle.prefill_attention(q, k, v, ctx)
    for t in range(T):
        lens = ctx - T + t + 1
        dec = oracle.attention(q[:, t], k, v, lens)
        np.testing.assert_array_equal(pre["ref"][:, t], dec["ref"])


def test_prefill_is_causal():
    B, T, Hq, Hkv = 1, 6, 4, 1
    q, k, v, ctx = _prefill_inputs(B, T, Hq, Hkv, [20], 24, seed=3)
    base = oracle.prefill_attention(q, k, v, ctx)["ref"]
    # a key/value past a token's position (and the cache rows past the context) never reach it
    for pos in (16, 19, 20, 23):
        k2, v2 = k.copy(), v.copy()
        k2[0, 0, pos] = workloads.bf16_words_from_float(np.full(128, 3.0, np.float32))
        v2[0, 0, pos] = workloads.bf16_words_from_float(np.full(128, 7.0, np.float32))
        got = oracle.prefill_attention(q, k2, v2, ctx)["ref"]
        first_seeing = pos - (20 - T)  # tokens t >= this index see position pos
        for t in range(T):
            if t < first_seeing:
                np.testing.assert_array_equal(got[0, t], base[0, t])
            else:
                assert np.abs(got[0, t] - base[0, t]).max() > 1e-3


def test_prefill_without_prefix_first_token_returns_its_value_row():
    q, k, v, ctx = _prefill_inputs(2, 4, 8, 2, [4, 4], 8, seed=4)
    out = oracle.prefill_attention(q, k, v, ctx)["out"]
    for b in range(2):
        for qh in range(8):
            np.testing.assert_array_equal(out[b, 0, qh * 128:(qh + 1) * 128], v[b, qh // 4, 0])


def test_prefill_ignores_the_order_of_the_prefix():
    q, k, v, ctx = _prefill_inputs(1, 3, 4, 1, [40], 40, seed=5)
    base = oracle.prefill_attention(q, k, v, ctx)["ref"]
    perm = np.random.default_rng(6).permutation(37)  # positions 0..36 are the prefix
    k2, v2 = k.copy(), v.copy()
    k2[0, 0, :37] = k[0, 0, perm]
    v2[0, 0, :37] = v[0, 0, perm]
    np.testing.assert_allclose(oracle.prefill_attention(q, k2, v2, ctx)["ref"], base, rtol=0, atol=1e-12)


def test_prefill_rejects_a_chunk_longer_than_the_context():
    q, k, v, _ = _prefill_inputs(1, 4, 4, 1, [4], 8)
    with pytest.raises(oracle.OracleError):
        oracle.prefill_attention(q, k, v, np.array([3], np.int32))
