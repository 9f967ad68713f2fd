"""CPU oracle of the decode-attention step, the output projection and the fp16 GEMM.

TEST INFRASTRUCTURE ONLY. This package wraps ``oracle.c`` (plain C, IEEE
double) with ctypes and numpy. Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import it; the HIP library and its
Python binding never do, and it never imports them.

All 16-bit tensors cross this boundary as ``numpy.uint16`` arrays holding the
raw bf16 / fp16 words.

What each function computes, and the pages it follows:

* ``attention`` -- the first two matmuls of one decode-attention forward and
  the vector ops between them ("PyPTO 开箱性能调优实战：Decode Attention 多
  Matmul 独立 TileShape 配置 F-16", section 代码对比 and the M/K/N table of
  section 三个 Matmul 的 Shape 特征分析): scaled scores q.K^T, softmax over the
  keys of the sequence, weights x V, rounded once to bf16.
* ``oproj`` -- the third matmul of that page, attn_output_flat x o_weight.
* ``decode_step`` -- the three in sequence, the projection reading the bf16
  attention output.
* ``prefill_attention`` -- context attention of a chunk of new tokens (the
  page "CCCL → Triton 方法论迁移", section 二, 2.1 prefix_prefill.py, names
  this context attention beside the decode attention without defining it; the
  plainest reading is taken: each token attends causally to the cached keys
  up to its own position, with the decode step's softmax). T = 1 is exactly
  ``attention``.
* ``gemm_f16`` -- the BasicMatmul example of the CANN msKPP page
  "自动调优流程 / Kernel级自动调优": C = A x B, fp16, row-major.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(closed forms, invariants, the page's all-ones golden and brute force on tiny
cases); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_u16p = ctypes.POINTER(ctypes.c_uint16)
_i32p = ctypes.POINTER(ctypes.c_int32)
_f64p = ctypes.POINTER(ctypes.c_double)


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (plain C11, -O2)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared", _SRC, "-o", tmp,
             "-lpthread", "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_bf16_to_double.restype = ctypes.c_double
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_double.restype = ctypes.c_double
    lib.oracle_f16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_from_double.restype = ctypes.c_uint16
    lib.oracle_bf16_from_double.argtypes = [ctypes.c_double]
    lib.oracle_f16_from_double.restype = ctypes.c_uint16
    lib.oracle_f16_from_double.argtypes = [ctypes.c_double]
    ci = ctypes.c_int
    lib.oracle_attention.restype = ci
    lib.oracle_attention.argtypes = [_u16p, _u16p, _u16p, _i32p, ci, ci, ci, ci, ci, ctypes.c_double,
                                     _f64p, _u16p, _f64p, _f64p, _f64p, ci]
    lib.oracle_oproj.restype = ci
    lib.oracle_oproj.argtypes = [_u16p, _u16p, ci, ci, ci, _f64p, _u16p, ci]
    lib.oracle_prefill_attention.restype = ci
    lib.oracle_prefill_attention.argtypes = [_u16p, _u16p, _u16p, _i32p, ci, ci, ci, ci, ci, ci, ctypes.c_double,
                                             _f64p, _u16p, ci]
    lib.oracle_gemm_f16.restype = ci
    lib.oracle_gemm_f16.argtypes = [_u16p, _u16p, ci, ci, ci, _f64p, _u16p, ci]
    lib.oracle_decode_step.restype = ci
    lib.oracle_decode_step.argtypes = [_u16p, _u16p, _u16p, _i32p, _u16p, ci, ci, ci, ci, ci, ci,
                                       ctypes.c_double, _f64p, _u16p, _f64p, _u16p, ci]
    _lib = lib
    return lib


class OracleError(RuntimeError):
    pass


MAX_THREADS = 16  # a fair share of a shared host


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, MAX_THREADS))


def _u16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("16-bit float tensors are passed as numpy.uint16 words, got %s" % a.dtype)
    return a


def _ptr(a, t):
    return None if a is None else a.ctypes.data_as(t)


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError("%s: oracle returned %d (invalid arguments)" % (what, rc))


def bf16_to_double(words) -> np.ndarray:
    lib = _load()
    w = np.asarray(words, dtype=np.uint16)
    return np.array([lib.oracle_bf16_to_double(int(x)) for x in w.ravel()], dtype=np.float64).reshape(w.shape)


def f16_to_double(words) -> np.ndarray:
    lib = _load()
    w = np.asarray(words, dtype=np.uint16)
    return np.array([lib.oracle_f16_to_double(int(x)) for x in w.ravel()], dtype=np.float64).reshape(w.shape)


def bf16_from_double(x) -> np.ndarray:
    lib = _load()
    a = np.asarray(x, dtype=np.float64)
    return np.array([lib.oracle_bf16_from_double(float(v)) for v in a.ravel()], dtype=np.uint16).reshape(a.shape)


def f16_from_double(x) -> np.ndarray:
    lib = _load()
    a = np.asarray(x, dtype=np.float64)
    return np.array([lib.oracle_f16_from_double(float(v)) for v in a.ravel()], dtype=np.uint16).reshape(a.shape)


def attention(q, k, v, seq_lens, scale=None, want_scores=False, nthreads=None):
    """q [B,Hq,D], k/v [B,Hkv,Lmax,D] (uint16 bf16 words), seq_lens [B] int32.

    Returns a dict with ``flat`` (uint16 [B, Hq*D]), ``ref`` (float64 [B, Hq*D],
    before rounding) and, if ``want_scores``, ``scores`` and ``probs``
    (float64 [B, Hq, Lmax], NaN beyond each sequence) and ``lse`` ([B, Hq]).
    """
    lib = _load()
    q, k, v = _u16(q), _u16(k), _u16(v)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    B, Hq, D = q.shape
    Bk, Hkv, Lmax, Dk = k.shape
    if Bk != B or Dk != D or v.shape != k.shape or sl.shape != (B,):
        raise OracleError("attention: inconsistent shapes")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    ref = np.empty((B, Hq * D), dtype=np.float64)
    flat = np.empty((B, Hq * D), dtype=np.uint16)
    scores = probs = lse = None
    if want_scores:
        scores = np.full((B, Hq, Lmax), np.nan, dtype=np.float64)
        probs = np.full((B, Hq, Lmax), np.nan, dtype=np.float64)
        lse = np.empty((B, Hq), dtype=np.float64)
    rc = lib.oracle_attention(_ptr(q, _u16p), _ptr(k, _u16p), _ptr(v, _u16p), _ptr(sl, _i32p), B, Hq, Hkv, D,
                              Lmax, float(scale), _ptr(ref, _f64p), _ptr(flat, _u16p), _ptr(scores, _f64p),
                              _ptr(probs, _f64p), _ptr(lse, _f64p), nthreads or default_threads())
    _check(rc, "attention")
    out = {"flat": flat, "ref": ref}
    if want_scores:
        out.update(scores=scores, probs=probs, lse=lse)
    return out


def prefill_attention(q, k, v, ctx_lens, scale=None, nthreads=None):
    """Context attention of a chunk: q [B,T,Hq,D], k/v [B,Hkv,Lmax,D] (uint16 bf16 words), ctx_lens [B]
    int32 (keys per sequence, the chunk's T tokens being the last T). Token t attends causally to keys
    0 .. ctx_lens[b]-T+t. Returns a dict with ``out`` (uint16 [B,T,Hq*D]) and ``ref`` (float64, unrounded).
    """
    lib = _load()
    q, k, v = _u16(q), _u16(k), _u16(v)
    cl = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    B, T, Hq, D = q.shape
    Bk, Hkv, Lmax, Dk = k.shape
    if Bk != B or Dk != D or v.shape != k.shape or cl.shape != (B,):
        raise OracleError("prefill_attention: inconsistent shapes")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    ref = np.empty((B, T, Hq * D), dtype=np.float64)
    out = np.empty((B, T, Hq * D), dtype=np.uint16)
    rc = lib.oracle_prefill_attention(_ptr(q, _u16p), _ptr(k, _u16p), _ptr(v, _u16p), _ptr(cl, _i32p), B, T, Hq,
                                      Hkv, D, Lmax, float(scale), _ptr(ref, _f64p), _ptr(out, _u16p),
                                      nthreads or default_threads())
    _check(rc, "prefill_attention")
    return {"out": out, "ref": ref}


def oproj(x, w, nthreads=None):
    """x [M,K], w [K,N] (uint16 bf16 words). Returns (out uint16 [M,N], ref float64 [M,N])."""
    lib = _load()
    x, w = _u16(x), _u16(w)
    M, K = x.shape
    K2, N = w.shape
    if K2 != K:
        raise OracleError("oproj: inconsistent shapes")
    ref = np.empty((M, N), dtype=np.float64)
    out = np.empty((M, N), dtype=np.uint16)
    rc = lib.oracle_oproj(_ptr(x, _u16p), _ptr(w, _u16p), M, K, N, _ptr(ref, _f64p), _ptr(out, _u16p),
                          nthreads or default_threads())
    _check(rc, "oproj")
    return out, ref


def gemm_f16(a, b, nthreads=None):
    """a [M,K], b [K,N] (uint16 fp16 words). Returns (C uint16 [M,N], ref float64 [M,N])."""
    lib = _load()
    a, b = _u16(a), _u16(b)
    M, K = a.shape
    K2, N = b.shape
    if K2 != K:
        raise OracleError("gemm_f16: inconsistent shapes")
    ref = np.empty((M, N), dtype=np.float64)
    out = np.empty((M, N), dtype=np.uint16)
    rc = lib.oracle_gemm_f16(_ptr(a, _u16p), _ptr(b, _u16p), M, N, K, _ptr(ref, _f64p), _ptr(out, _u16p),
                             nthreads or default_threads())
    _check(rc, "gemm_f16")
    return out, ref


def decode_step(q, k, v, seq_lens, o_weight, scale=None, nthreads=None):
    """The whole step. Returns a dict: flat, attn_ref, out (uint16 [B,N]), out_ref (float64 [B,N])."""
    lib = _load()
    q, k, v, w = _u16(q), _u16(k), _u16(v), _u16(o_weight)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    B, Hq, D = q.shape
    _, Hkv, Lmax, _ = k.shape
    Ko, N = w.shape
    if Ko != Hq * D or v.shape != k.shape or sl.shape != (B,):
        raise OracleError("decode_step: inconsistent shapes")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    attn_ref = np.empty((B, Hq * D), dtype=np.float64)
    flat = np.empty((B, Hq * D), dtype=np.uint16)
    out_ref = np.empty((B, N), dtype=np.float64)
    out = np.empty((B, N), dtype=np.uint16)
    rc = lib.oracle_decode_step(_ptr(q, _u16p), _ptr(k, _u16p), _ptr(v, _u16p), _ptr(sl, _i32p), _ptr(w, _u16p),
                                B, Hq, Hkv, D, Lmax, N, float(scale), _ptr(attn_ref, _f64p), _ptr(flat, _u16p),
                                _ptr(out_ref, _f64p), _ptr(out, _u16p), nthreads or default_threads())
    _check(rc, "decode_step")
    return {"flat": flat, "attn_ref": attn_ref, "out": out, "out_ref": out_ref}
