"""Seeded synthetic inputs for the decode-attention step and the fp16 GEMM check.

This module only draws numbers and lays them out; it holds none of the
arithmetic of the method. Both the CPU oracle (through the tests and the
benchmark) and the HIP library consume what it produces.

Every 16-bit tensor is returned as raw words in a ``numpy.uint16`` array.
Normal draws are made in float32 and converted to bf16 with torch's own
float32 -> bfloat16 conversion (round to nearest even).

The five named workloads are the shapes the method is measured on; no public
dataset or trained weights are involved, so nothing stands in for one.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

BF16_NAN = 0x7FC0


@dataclasses.dataclass(frozen=True)
class DecodeShape:
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    max_seq_len: int
    hidden: int

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def o_in(self) -> int:
        return self.num_q_heads * self.head_dim


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    shape: DecodeShape
    seed: int
    w_std: float = 0.02
    # seq_lens: fixed list, or drawn uniformly in [lo, hi] when ragged is set
    seq_len: Optional[int] = None
    ragged: Optional[tuple] = None


@dataclasses.dataclass(frozen=True)
class PrefillWorkload:
    """A chunk of ``tokens`` new tokens per sequence appended to a cache of
    ``ctx_len`` keys in all (the chunk being the last ``tokens`` of them)."""
    name: str
    batch: int
    tokens: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    ctx_len: int
    seed: int

    @property
    def max_seq_len(self) -> int:
        return self.ctx_len


@dataclasses.dataclass(frozen=True)
class GemmWorkload:
    name: str
    m: int
    n: int
    k: int
    seed: int


# The five workloads, in their canonical order (index = seed).
TINY = DecodeWorkload("tiny_b1_h4kv1_L256_o512", DecodeShape(1, 4, 1, 128, 256, 512), seed=0, seq_len=256)
PAGES = DecodeWorkload("decode_b1_h32kv8_L2048_o4096", DecodeShape(1, 32, 8, 128, 2048, 4096), seed=1,
                       seq_len=2048)
GEMM = GemmWorkload("gemm_f16_256x512x1024", 256, 512, 1024, seed=2)
BATCHED = DecodeWorkload("decode_b16_h32kv8_ragged1024-8192_o4096", DecodeShape(16, 32, 8, 128, 8192, 4096),
                         seed=3, ragged=(1024, 8192))
LONG = DecodeWorkload("decode_b4_h64kv8_L32768_o8192", DecodeShape(4, 64, 8, 128, 32768, 8192), seed=4,
                      seq_len=32768)

# head_dim 256 (not one of the five): a group of 8 query heads over 256-dim
# keys, 16384 cached keys per sequence, 128 MiB of KV and a 32 MiB projection.
WIDE = DecodeWorkload("decode_b4_h16kv2_d256_L16384_o4096", DecodeShape(4, 16, 2, 256, 16384, 4096), seed=5,
                      seq_len=16384)

# Context (prefill) attention of the same model shape (32 query / 8 KV heads,
# head_dim 128): a whole 2048-token prompt, and a 512-token chunk of each of 4
# sequences behind a 7680-key prefix.
PROMPT = PrefillWorkload("prefill_b1_t2048_h32kv8_ctx2048", 1, 2048, 32, 8, 128, 2048, seed=6)
CHUNK = PrefillWorkload("prefill_b4_t512_h32kv8_ctx8192", 4, 512, 32, 8, 128, 8192, seed=7)

# One GPU's share of the step when the decode workloads are spread over 8
# GPUs: a kv head per GPU with the projection split by its input rows (each GPU
# then adds its partial output into the others'), and an eighth of the batch.
# They are not benchmarked; the tile search weighs its built-in rules over them.
SHARE_PAGES_TP8 = DecodeWorkload("decode_b1_h4kv1_L2048_o4096", DecodeShape(1, 4, 1, 128, 2048, 4096), seed=8,
                                 seq_len=2048)
SHARE_LONG_TP8 = DecodeWorkload("decode_b4_h8kv1_L32768_o8192", DecodeShape(4, 8, 1, 128, 32768, 8192), seed=9,
                                seq_len=32768)
SHARE_BATCHED_DP8 = DecodeWorkload("decode_b2_h32kv8_ragged1024-8192_o4096", DecodeShape(2, 32, 8, 128, 8192, 4096),
                                   seed=10, ragged=(1024, 8192))
SHARES = [SHARE_PAGES_TP8, SHARE_LONG_TP8, SHARE_BATCHED_DP8]

ALL = [TINY, PAGES, GEMM, BATCHED, LONG, WIDE, PROMPT, CHUNK]
BY_NAME = {w.name: w for w in ALL + SHARES}
DECODE = [TINY, PAGES, BATCHED, LONG, WIDE]
RULE_SHAPES = [PAGES, BATCHED, LONG, WIDE] + SHARES
PREFILL = [PROMPT, CHUNK]


def _to_bf16_words(x: np.ndarray) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _normal_bf16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return _to_bf16_words(x)


def draw_seq_lens(wl: DecodeWorkload, rng: np.random.Generator) -> np.ndarray:
    B = wl.shape.batch
    if wl.ragged is not None:
        lo, hi = wl.ragged
        return rng.integers(lo, hi, endpoint=True, size=B).astype(np.int32)
    return np.full(B, wl.seq_len, dtype=np.int32)


def decode_inputs(wl: DecodeWorkload, poison: bool = False, with_weight: bool = True) -> dict:
    """Draw (seq_lens, q, k, v, o_weight) in that order from default_rng(seed).

    q ~ N(0,1) [B,Hq,D]; k, v ~ N(0,1) [B,Hkv,Lmax,D]; o_weight ~ N(0, w_std^2)
    [Hq*D, hidden]. With ``poison``, cache rows at or beyond each sequence's
    length hold bf16 NaN, so any read of them shows up in the output.
    """
    s = wl.shape
    rng = np.random.default_rng(wl.seed)
    seq_lens = draw_seq_lens(wl, rng)
    q = _normal_bf16(rng, (s.batch, s.num_q_heads, s.head_dim))
    k = _normal_bf16(rng, (s.batch, s.num_kv_heads, s.max_seq_len, s.head_dim))
    v = _normal_bf16(rng, (s.batch, s.num_kv_heads, s.max_seq_len, s.head_dim))
    w = _normal_bf16(rng, (s.o_in, s.hidden), wl.w_std) if with_weight else None
    if poison:
        poison_padding(k, v, seq_lens)
    return {"seq_lens": seq_lens, "q": q, "k": k, "v": v, "o_weight": w, "shape": s}


def poison_padding(k: np.ndarray, v: np.ndarray, seq_lens) -> None:
    for b, L in enumerate(np.asarray(seq_lens)):
        k[b, :, int(L):, :] = BF16_NAN
        v[b, :, int(L):, :] = BF16_NAN


def custom_decode_inputs(batch: int, num_q_heads: int, num_kv_heads: int, seq_lens: List[int],
                         max_seq_len: Optional[int] = None, hidden: int = 256, head_dim: int = 128,
                         seed: int = 0, w_std: float = 0.02, poison: bool = True) -> dict:
    """Same recipe as ``decode_inputs`` for an arbitrary shape (small parity cases)."""
    Lmax = max_seq_len if max_seq_len is not None else max(seq_lens)
    s = DecodeShape(batch, num_q_heads, num_kv_heads, head_dim, Lmax, hidden)
    rng = np.random.default_rng(seed)
    sl = np.asarray(seq_lens, dtype=np.int32)
    q = _normal_bf16(rng, (batch, num_q_heads, head_dim))
    k = _normal_bf16(rng, (batch, num_kv_heads, Lmax, head_dim))
    v = _normal_bf16(rng, (batch, num_kv_heads, Lmax, head_dim))
    w = _normal_bf16(rng, (s.o_in, hidden), w_std)
    if poison:
        poison_padding(k, v, sl)
    return {"seq_lens": sl, "q": q, "k": k, "v": v, "o_weight": w, "shape": s}


def prefill_inputs(wl: PrefillWorkload, poison: bool = True) -> dict:
    """Draw (q, k, v) in that order from default_rng(seed): q ~ N(0,1)
    [B,T,Hq,D], k, v ~ N(0,1) [B,Hkv,ctx_len,D]; every sequence holds ctx_len keys."""
    rng = np.random.default_rng(wl.seed)
    ctx = np.full(wl.batch, wl.ctx_len, dtype=np.int32)
    q = _normal_bf16(rng, (wl.batch, wl.tokens, wl.num_q_heads, wl.head_dim))
    k = _normal_bf16(rng, (wl.batch, wl.num_kv_heads, wl.max_seq_len, wl.head_dim))
    v = _normal_bf16(rng, (wl.batch, wl.num_kv_heads, wl.max_seq_len, wl.head_dim))
    if poison:
        poison_padding(k, v, ctx)
    return {"ctx_lens": ctx, "q": q, "k": k, "v": v}


def prefill_flops(tokens: int, num_q_heads: int, head_dim: int, ctx_lens) -> int:
    """Multiply-adds x 2 of a chunk's attention: every (token, query head) row
    of sequence b meets ctx_lens[b] - tokens + t + 1 keys, and each key costs
    head_dim products for its score and head_dim for its share of the output."""
    keys = sum(int(c) * tokens - tokens * (tokens - 1) // 2 for c in np.asarray(ctx_lens))
    return 4 * head_dim * num_q_heads * keys


def gemm_inputs(wl: GemmWorkload = GEMM, all_ones: bool = False) -> dict:
    """A [M,K], B [K,N] fp16 words with entries uniform in {-1, 0, 1} (or all ones)."""
    if all_ones:
        a = np.ones((wl.m, wl.k), dtype=np.float16)
        b = np.ones((wl.k, wl.n), dtype=np.float16)
    else:
        rng = np.random.default_rng(wl.seed)
        a = rng.integers(-1, 1, endpoint=True, size=(wl.m, wl.k)).astype(np.float16)
        b = rng.integers(-1, 1, endpoint=True, size=(wl.k, wl.n)).astype(np.float16)
    return {"a": a.view(np.uint16), "b": b.view(np.uint16), "m": wl.m, "n": wl.n, "k": wl.k}


def bf16_words_from_float(x) -> np.ndarray:
    """Exact-or-RNE float32 -> bf16 words (used to build small hand-made inputs)."""
    return _to_bf16_words(np.asarray(x, dtype=np.float32))


def algorithmic_bytes(shape: DecodeShape, seq_lens) -> int:
    """Bytes one decode step must move at minimum: q, the K and V rows each
    sequence attends to, the projection weight and the bf16 output."""
    D = shape.head_dim
    return (2 * shape.batch * shape.num_q_heads * D + 2 * 2 * shape.num_kv_heads * D * int(np.sum(seq_lens))
            + 2 * shape.o_in * shape.hidden + 2 * shape.batch * shape.hidden)
