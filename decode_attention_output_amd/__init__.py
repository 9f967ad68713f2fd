"""Python binding of libdecode_attn.so (the gfx950 decode-attention library).

Argument marshalling only: every step of the decode path runs in the HIP
kernels behind the C ABI declared in ``include/decode_attn.h``. PyTorch
provides device memory and the stream; nothing here computes on its own, and
there is no fallback -- if the library is missing or fails to load, every call
raises.

The names mirror the C entry points: ``decode_attn_fwd``, ``decode_attn_only``,
``oproj_fwd``, ``gemm_f16``, ``decode_attn_workspace_size``,
``oproj_workspace_size``, ``decode_attn_plan``, ``decode_attn_status_str``,
``prefill_attn_fwd``, ``decode_attn_step_status``, ``decode_attn_fwd_noalloc``,
``decode_attn_read_probe`` (a plain streaming read, the measurement floor).

Before any call reaches the library, the torch wrappers check that the
tensors agree with each other (batch, heads, head_dim, cache length,
projection sizes, output and debug buffers): the C ABI sees only pointers,
so a mismatch would otherwise make the kernels run past an allocation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdecode_attn.so")

DA_OK = 0
DA_ERR_NULL = -1
DA_ERR_SHAPE = -2
DA_ERR_ALIGN = -3
DA_ERR_WORKSPACE = -4
DA_ERR_LAUNCH = -5
DA_ERR_TIMEOUT = -6
DA_HEAD_DIM = 128
DA_HEAD_DIM_WIDE = 256
DA_MAX_GROUP = 16
DA_FLAG_DEBUG_SCORES = 1
DA_FLAG_SEPARATE = 2

EXPORTED = (
    "decode_attn_workspace_size",
    "decode_attn_plan",
    "decode_attn_fwd",
    "decode_attn_only",
    "oproj_workspace_size",
    "oproj_fwd",
    "gemm_f16",
    "decode_attn_status_str",
    "prefill_attn_fwd",
    "decode_attn_step_status",
    "decode_attn_fwd_noalloc",
    "decode_attn_read_probe",
)


class DecodeAttnTiles(ctypes.Structure):
    """Tile override of one call (decode_attn_tiles_t); zero fields keep the built-in choice."""
    _fields_ = [(n, ctypes.c_int32) for n in ("attn_workgroups", "attn_depth", "proj_tile_n", "proj_ksplit",
                                              "step_mode", "step_wait_polls", "attn_seq_cost",
                                              "step_weight_delay")]


def make_tiles(tiles) -> Optional[DecodeAttnTiles]:
    """None, a DecodeAttnTiles or a dict of its fields -> DecodeAttnTiles or None."""
    if tiles is None or isinstance(tiles, DecodeAttnTiles):
        return tiles
    unknown = set(tiles) - {n for n, _ in DecodeAttnTiles._fields_}
    if unknown:
        raise ValueError("unknown tile fields: %s" % sorted(unknown))
    return DecodeAttnTiles(**{k: int(v) for k, v in tiles.items()})


class DecodeAttnShape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("flags", ctypes.c_uint32),
        ("debug_scores", ctypes.c_void_p),
        ("debug_lse", ctypes.c_void_p),
        ("tiles", ctypes.POINTER(DecodeAttnTiles)),
    ]


class MatmulPlan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("m", "k", "n", "tile_m", "tile_k", "tile_n", "split", "workgroups")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class DecodeAttnPlan(ctypes.Structure):
    _fields_ = [
        ("qk", MatmulPlan),
        ("pv", MatmulPlan),
        ("oproj", MatmulPlan),
        ("split_len", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("oproj_path", ctypes.c_int32),
        ("fused", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class PrefillAttnShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("batch", "num_tokens", "num_q_heads", "num_kv_heads", "head_dim",
                                              "max_seq_len")] + [("softmax_scale", ctypes.c_float)]


class DecodeAttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (what, status_str(status), status))


_lib = None


def load_library(path: str = LIB_PATH):
    """Load the built library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libdecode_attn.so not found at %s: build it first (python -c 'import "
                           "__graft_entry__ as g; g.build()' or python decode_attention_output_amd/build.py)"
                           % path)
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    shp = ctypes.POINTER(DecodeAttnShape)
    lib.decode_attn_workspace_size.restype = sz
    lib.decode_attn_workspace_size.argtypes = [shp]
    lib.decode_attn_plan.restype = ctypes.c_int
    lib.decode_attn_plan.argtypes = [shp, ctypes.POINTER(DecodeAttnPlan)]
    lib.decode_attn_fwd.restype = ctypes.c_int
    lib.decode_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, shp, vp]
    lib.decode_attn_only.restype = ctypes.c_int
    lib.decode_attn_only.argtypes = [vp, vp, vp, vp, vp, shp, vp]
    lib.oproj_workspace_size.restype = sz
    lib.oproj_workspace_size.argtypes = [i32, i32, i32]
    lib.oproj_fwd.restype = ctypes.c_int
    lib.oproj_fwd.argtypes = [vp, vp, vp, i32, i32, i32, vp, sz, vp]
    lib.gemm_f16.restype = ctypes.c_int
    lib.gemm_f16.argtypes = [vp, vp, vp, i32, i32, i32, vp]
    lib.prefill_attn_fwd.restype = ctypes.c_int
    lib.prefill_attn_fwd.argtypes = [vp, vp, vp, vp, vp, ctypes.POINTER(PrefillAttnShape), vp]
    lib.decode_attn_fwd_noalloc.restype = ctypes.c_int
    lib.decode_attn_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, shp, vp]
    lib.decode_attn_read_probe.restype = ctypes.c_int
    lib.decode_attn_read_probe.argtypes = [vp, sz, vp, i32, vp]
    lib.decode_attn_step_status.restype = ctypes.c_int
    lib.decode_attn_step_status.argtypes = [vp, sz, vp]
    lib.decode_attn_status_str.restype = ctypes.c_char_p
    lib.decode_attn_status_str.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load_library().decode_attn_status_str(int(status)).decode()


decode_attn_status_str = status_str


def make_shape(batch, num_q_heads, num_kv_heads, max_seq_len, hidden=0, head_dim=DA_HEAD_DIM, softmax_scale=0.0,
               workspace=None, workspace_bytes=0, flags=0, debug_scores=None, debug_lse=None,
               tiles=None) -> DecodeAttnShape:
    """The C shape struct; ``tiles`` (a dict or DecodeAttnTiles) is kept alive by the struct."""
    shape = DecodeAttnShape(int(batch), int(num_q_heads), int(num_kv_heads), int(head_dim), int(max_seq_len),
                            int(hidden), float(softmax_scale), workspace, int(workspace_bytes), int(flags),
                            debug_scores, debug_lse)
    t = make_tiles(tiles)
    if t is not None:
        shape._tiles = t
        shape.tiles = ctypes.pointer(t)
    return shape


def decode_attn_workspace_size(shape: DecodeAttnShape) -> int:
    return int(load_library().decode_attn_workspace_size(ctypes.byref(shape)))


def oproj_workspace_size(M: int, K: int, N: int) -> int:
    return int(load_library().oproj_workspace_size(int(M), int(K), int(N)))


def decode_attn_plan(shape: DecodeAttnShape) -> DecodeAttnPlan:
    plan = DecodeAttnPlan()
    rc = load_library().decode_attn_plan(ctypes.byref(shape), ctypes.byref(plan))
    if rc != DA_OK:
        raise DecodeAttnError(rc, "decode_attn_plan")
    return plan


# ---------------------------------------------------------------------------
# torch-facing wrappers (torch supplies device buffers and the stream)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream_handle(stream=None) -> Optional[int]:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check_dev(name, t, dtype):
    torch = _torch()
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.device.type != "cuda":
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return torch


def _dims(name, t, n):
    if t.dim() != n:
        raise ValueError("%s must have %d dimensions, got shape %s" % (name, n, tuple(t.shape)))
    return tuple(int(x) for x in t.shape)


def _want(name, t, shape):
    if tuple(int(x) for x in t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def _same_device(*named):
    devs = {(t.device.type, t.device.index) for _, t in named if t is not None}
    if len(devs) > 1:
        raise ValueError("tensors on different devices: %s" % ", ".join(
            "%s on %s" % (n, t.device) for n, t in named if t is not None))


def check_decode_tensors(q, k_cache, v_cache, seq_lens, o_weight=None, out=None, debug_scores=None,
                         debug_lse=None):
    """Shapes of one decode call's tensors against each other: q [B, Hq, D], K and V
    [B, Hkv, Lmax, D] alike, seq_lens [B], o_weight [Hq*D, hidden], out [B, hidden] (or
    [B, Hq*D] without o_weight), debug scores [B, Hq, Lmax] and lse [B, Hq] fp32.
    Raises ValueError / TypeError; returns (B, Hq, Hkv, D, Lmax, hidden or 0)."""
    B, Hq, D = _dims("q", q, 3)
    Bk, Hkv, Lmax, Dk = _dims("k_cache", k_cache, 4)
    if Bk != B or Dk != D:
        raise ValueError("k_cache %s does not match q %s (batch and head_dim)" % (tuple(k_cache.shape),
                                                                                 tuple(q.shape)))
    _want("v_cache", v_cache, (Bk, Hkv, Lmax, Dk))
    _want("seq_lens", seq_lens, (B,))
    hidden = 0
    if o_weight is not None:
        Ko, hidden = _dims("o_weight", o_weight, 2)
        if Ko != Hq * D:
            raise ValueError("o_weight has %d rows, the projection's K is num_q_heads * head_dim = %d" % (Ko, Hq * D))
    if out is not None:
        _want("out", out, (B, hidden if o_weight is not None else Hq * D))
    if (debug_scores is None) != (debug_lse is None):
        raise ValueError("debug_scores and debug_lse go together")
    if debug_scores is not None:
        _want("debug_scores", debug_scores, (B, Hq, Lmax))
        _want("debug_lse", debug_lse, (B, Hq))
        torch = _torch()
        for n, t in (("debug_scores", debug_scores), ("debug_lse", debug_lse)):
            _check_dev(n, t, torch.float32)
    torch = _torch()
    for n, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("o_weight", o_weight), ("out", out)):
        if t is not None:
            _check_dev(n, t, torch.bfloat16)
    _check_dev("seq_lens", seq_lens, torch.int32)
    _same_device(("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("seq_lens", seq_lens),
                 ("o_weight", o_weight), ("out", out), ("debug_scores", debug_scores), ("debug_lse", debug_lse))
    return B, Hq, Hkv, D, Lmax, hidden


def check_matmul_tensors(x, w, out=None, dtype=None):
    """x [M, K], w [K, N], out [M, N], all of one 16-bit dtype on one device."""
    M, K = _dims("x", x, 2)
    Kw, N = _dims("w", w, 2)
    if Kw != K:
        raise ValueError("w has %d rows, x has %d columns" % (Kw, K))
    if out is not None:
        _want("out", out, (M, N))
    torch = _torch()
    dtype = dtype or torch.bfloat16
    for n, t in (("x", x), ("w", w), ("out", out)):
        if t is not None:
            _check_dev(n, t, dtype)
    _same_device(("x", x), ("w", w), ("out", out))
    return M, K, N


def check_prefill_tensors(q, k_cache, v_cache, ctx_lens, out=None):
    """q [B, T, Hq, D], K and V [B, Hkv, Lmax, D], ctx_lens [B], out [B, T, Hq*D]."""
    B, T, Hq, D = _dims("q", q, 4)
    Bk, Hkv, Lmax, Dk = _dims("k_cache", k_cache, 4)
    if Bk != B or Dk != D:
        raise ValueError("k_cache %s does not match q %s (batch and head_dim)" % (tuple(k_cache.shape),
                                                                                 tuple(q.shape)))
    _want("v_cache", v_cache, (Bk, Hkv, Lmax, Dk))
    _want("ctx_lens", ctx_lens, (B,))
    if out is not None:
        _want("out", out, (B, T, Hq * D))
    torch = _torch()
    for n, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("out", out)):
        if t is not None:
            _check_dev(n, t, torch.bfloat16)
    _check_dev("ctx_lens", ctx_lens, torch.int32)
    _same_device(("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("ctx_lens", ctx_lens), ("out", out))
    return B, T, Hq, Hkv, D, Lmax


class Workspace:
    """Zero-filled device scratch reused across calls (grows on demand). The
    zero fill is enqueued on the stream of the call that needs it, so it is
    ordered before that call's kernels."""

    def __init__(self, device=None):
        self.device = device
        self.buf = None

    def get(self, nbytes: int, stream=None):
        torch = _torch()
        if nbytes == 0:
            return None
        if self.buf is None or self.buf.numel() < nbytes:
            s = stream if stream is not None else torch.cuda.current_stream(self.device)
            with torch.cuda.stream(s):
                self.buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=self.device or "cuda")
        return self.buf


def decode_attn_step_status(workspace, stream=None) -> int:
    """DA_OK, or DA_ERR_TIMEOUT if a single-launch step on this workspace gave up
    waiting since its counters were last zero-filled (waits for the stream).
    ``workspace=None`` asks about the no-allocation scratch of the current device."""
    if workspace is None:
        return int(load_library().decode_attn_step_status(None, 0, _stream_handle(stream)))
    buf = getattr(workspace, "buf", workspace)
    if buf is None:
        return DA_OK  # never used: no single-launch step ran on it
    return int(load_library().decode_attn_step_status(buf.data_ptr(), buf.numel(), _stream_handle(stream)))


def _ws_for(workspace, device, need, stream):
    return (workspace or Workspace(device)).get(need, stream)


def decode_attn_fwd(q, k_cache, v_cache, seq_lens, o_weight, out=None, workspace: Optional[Workspace] = None,
                    softmax_scale: float = 0.0, debug_scores=None, debug_lse=None, stream=None, separate=False,
                    tiles=None):
    """One decode step: returns out [B, hidden] bf16. ``separate`` asks for two
    launches (attention, projection) where the plan would use one; ``tiles``
    overrides the tile choice (decode_attn_tiles_t fields)."""
    B, Hq, Hkv, D, Lmax, hidden = check_decode_tensors(q, k_cache, v_cache, seq_lens, o_weight, out, debug_scores,
                                                       debug_lse)
    torch = _torch()
    if out is None:
        out = torch.empty((B, hidden), dtype=torch.bfloat16, device=q.device)
    flags = (DA_FLAG_DEBUG_SCORES if debug_scores is not None else 0) | (DA_FLAG_SEPARATE if separate else 0)
    shape = make_shape(B, Hq, Hkv, Lmax, hidden, D, softmax_scale, flags=flags, debug_scores=_ptr(debug_scores),
                       debug_lse=_ptr(debug_lse), tiles=tiles)
    need = decode_attn_workspace_size(shape)
    ws = _ws_for(workspace, q.device, need, stream)
    shape.workspace = _ptr(ws)
    shape.workspace_bytes = 0 if ws is None else ws.numel()
    rc = load_library().decode_attn_fwd(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seq_lens.data_ptr(),
                                        o_weight.data_ptr(), out.data_ptr(), ctypes.byref(shape),
                                        _stream_handle(stream))
    if rc != DA_OK:
        raise DecodeAttnError(rc, "decode_attn_fwd")
    return out


def decode_attn_fwd_noalloc(q, k_cache, v_cache, seq_lens, o_weight, out, softmax_scale: float = 0.0, stream=None,
                            separate=False, tiles=None):
    """decode_attn_fwd on the library's own scratch array: no workspace, and no
    allocation by the library; ``out`` [B, hidden] bf16 is the caller's."""
    B, Hq, Hkv, D, Lmax, hidden = check_decode_tensors(q, k_cache, v_cache, seq_lens, o_weight, out)
    if out is None:
        raise ValueError("decode_attn_fwd_noalloc writes into the caller's out tensor")
    shape = make_shape(B, Hq, Hkv, Lmax, hidden, D, softmax_scale, flags=DA_FLAG_SEPARATE if separate else 0,
                       tiles=tiles)
    rc = load_library().decode_attn_fwd_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                                seq_lens.data_ptr(), o_weight.data_ptr(), out.data_ptr(),
                                                ctypes.byref(shape), _stream_handle(stream))
    if rc != DA_OK:
        raise DecodeAttnError(rc, "decode_attn_fwd_noalloc")
    return out


def decode_attn_only(q, k_cache, v_cache, seq_lens, out=None, workspace: Optional[Workspace] = None,
                     softmax_scale: float = 0.0, debug_scores=None, debug_lse=None, stream=None, tiles=None):
    """Attention only: returns the bf16 [B, Hq*D] head-major attention output."""
    B, Hq, Hkv, D, Lmax, _ = check_decode_tensors(q, k_cache, v_cache, seq_lens, None, out, debug_scores,
                                                  debug_lse)
    torch = _torch()
    if out is None:
        out = torch.empty((B, Hq * D), dtype=torch.bfloat16, device=q.device)
    flags = DA_FLAG_DEBUG_SCORES if debug_scores is not None else 0
    shape = make_shape(B, Hq, Hkv, Lmax, 8, D, softmax_scale, flags=flags, debug_scores=_ptr(debug_scores),
                       debug_lse=_ptr(debug_lse), tiles=tiles)
    need = decode_attn_workspace_size(shape)
    ws = _ws_for(workspace, q.device, need, stream)
    shape.workspace = _ptr(ws)
    shape.workspace_bytes = 0 if ws is None else ws.numel()
    rc = load_library().decode_attn_only(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seq_lens.data_ptr(),
                                         out.data_ptr(), ctypes.byref(shape), _stream_handle(stream))
    if rc != DA_OK:
        raise DecodeAttnError(rc, "decode_attn_only")
    return out


def oproj_fwd(x, w, out=None, workspace: Optional[Workspace] = None, stream=None):
    """out [M, N] = x [M, K] @ w [K, N], bf16."""
    M, K, N = check_matmul_tensors(x, w, out)
    torch = _torch()
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    need = oproj_workspace_size(M, K, N)
    ws = _ws_for(workspace, x.device, need, stream)
    rc = load_library().oproj_fwd(x.data_ptr(), w.data_ptr(), out.data_ptr(), M, K, N, _ptr(ws),
                                  0 if ws is None else ws.numel(), _stream_handle(stream))
    if rc != DA_OK:
        raise DecodeAttnError(rc, "oproj_fwd")
    return out


def gemm_f16(a, b, c=None, stream=None):
    """C [M, N] = A [M, K] @ B [K, N], fp16."""
    torch = _torch()
    M, K, N = check_matmul_tensors(a, b, c, dtype=torch.float16)
    if c is None:
        c = torch.empty((M, N), dtype=torch.float16, device=a.device)
    rc = load_library().gemm_f16(a.data_ptr(), b.data_ptr(), c.data_ptr(), M, N, K, _stream_handle(stream))
    if rc != DA_OK:
        raise DecodeAttnError(rc, "gemm_f16")
    return c


def prefill_attn_fwd(q, k_cache, v_cache, ctx_lens, out=None, softmax_scale: float = 0.0, stream=None):
    """Context attention of a chunk: q [B, T, Hq, D] -> out [B, T, Hq*D] bf16 (token t attends causally
    to keys 0 .. ctx_lens[b] - T + t)."""
    B, T, Hq, Hkv, D, Lmax = check_prefill_tensors(q, k_cache, v_cache, ctx_lens, out)
    torch = _torch()
    if out is None:
        out = torch.empty((B, T, Hq * D), dtype=torch.bfloat16, device=q.device)
    shape = PrefillAttnShape(B, T, Hq, Hkv, D, Lmax, float(softmax_scale))
    rc = load_library().prefill_attn_fwd(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), ctx_lens.data_ptr(),
                                         out.data_ptr(), ctypes.byref(shape), _stream_handle(stream))
    if rc != DA_OK:
        raise DecodeAttnError(rc, "prefill_attn_fwd")
    return out


class PreparedCall:
    """One C-ABI call with its arguments marshalled in advance, so that each
    invocation costs a single ctypes call. Keeps every tensor it refers to
    alive. Invocations that share a workspace must stay ordered on one stream."""

    def __init__(self, fn, args, what, keep, result):
        self._fn, self._args, self._what, self._keep, self.result = fn, args, what, keep, result

    def __call__(self):
        rc = self._fn(*self._args)
        if rc != DA_OK:
            raise DecodeAttnError(rc, self._what)
        return self.result


def _prepare_shape(q, k_cache, hidden, softmax_scale, workspace, what, flags=0, tiles=None, stream=None):
    B, Hq, D = q.shape
    _, Hkv, Lmax, _ = k_cache.shape
    shape = make_shape(B, Hq, Hkv, Lmax, hidden, D, softmax_scale, flags=flags, tiles=tiles)
    need = decode_attn_workspace_size(shape)
    if need == 0:
        raise DecodeAttnError(DA_ERR_SHAPE, what)
    ws = _ws_for(workspace, q.device, need, stream)
    shape.workspace = _ptr(ws)
    shape.workspace_bytes = ws.numel()
    return shape, ws


def DecodeStep(q, k_cache, v_cache, seq_lens, o_weight, out=None, workspace: Optional[Workspace] = None,
               softmax_scale: float = 0.0, stream=None, separate=False, tiles=None) -> PreparedCall:
    """A prepared ``decode_attn_fwd``; calling it runs one decode step and returns ``out``."""
    B, _, _, _, _, hidden = check_decode_tensors(q, k_cache, v_cache, seq_lens, o_weight, out)
    torch = _torch()
    if out is None:
        out = torch.empty((B, hidden), dtype=torch.bfloat16, device=q.device)
    shape, ws = _prepare_shape(q, k_cache, hidden, softmax_scale, workspace, "decode_attn_fwd",
                               DA_FLAG_SEPARATE if separate else 0, tiles, stream)
    tensors = (q, k_cache, v_cache, seq_lens, o_weight, out)
    args = [ctypes.c_void_p(t.data_ptr()) for t in tensors] + [ctypes.byref(shape),
                                                              ctypes.c_void_p(_stream_handle(stream))]
    return PreparedCall(load_library().decode_attn_fwd, args, "decode_attn_fwd", (tensors, shape, ws), out)


def AttentionStep(q, k_cache, v_cache, seq_lens, out=None, workspace: Optional[Workspace] = None,
                  softmax_scale: float = 0.0, stream=None, tiles=None) -> PreparedCall:
    """A prepared ``decode_attn_only``; calling it returns the bf16 [B, Hq*D] attention output."""
    B, Hq, _, D, _, _ = check_decode_tensors(q, k_cache, v_cache, seq_lens, None, out)
    torch = _torch()
    if out is None:
        out = torch.empty((B, Hq * D), dtype=torch.bfloat16, device=q.device)
    shape, ws = _prepare_shape(q, k_cache, 8, softmax_scale, workspace, "decode_attn_only", tiles=tiles,
                               stream=stream)
    tensors = (q, k_cache, v_cache, seq_lens, out)
    args = [ctypes.c_void_p(t.data_ptr()) for t in tensors] + [ctypes.byref(shape),
                                                              ctypes.c_void_p(_stream_handle(stream))]
    return PreparedCall(load_library().decode_attn_only, args, "decode_attn_only", (tensors, shape, ws), out)


def OprojStep(x, w, out=None, workspace: Optional[Workspace] = None, stream=None) -> PreparedCall:
    """A prepared ``oproj_fwd``; calling it returns out = x @ w (bf16)."""
    M, K, N = check_matmul_tensors(x, w, out)
    torch = _torch()
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    need = oproj_workspace_size(M, K, N)
    ws = _ws_for(workspace, x.device, need, stream)
    args = [ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(w.data_ptr()), ctypes.c_void_p(out.data_ptr()),
            ctypes.c_int32(M), ctypes.c_int32(K), ctypes.c_int32(N), ctypes.c_void_p(_ptr(ws)),
            ctypes.c_size_t(0 if ws is None else ws.numel()), ctypes.c_void_p(_stream_handle(stream))]
    return PreparedCall(load_library().oproj_fwd, args, "oproj_fwd", ((x, w, out), ws), out)
