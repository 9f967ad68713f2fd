// Device building blocks of GQA decode attention on gfx950, shared by the
// stream-K attention kernel and the single-launch decode-step kernel.
//
// What they compute is the first two matmuls of one decode-attention forward
// and the softmax between them ("PyPTO 开箱性能调优实战：Decode Attention 多
// Matmul 独立 TileShape 配置 F-16", section 代码对比): scores = q_grouped x
// k_cache^T in fp32, scaled softmax, attn_weights x v_cache.
//
// Per wavefront and per 32-key block:
//   QK^T  MFMA 16x16x32 bf16. A = the G query rows of the group (rows G..15
//         are zero: a tiny M never grows past one operand); B = K^T, loaded
//         straight from HBM in the operand layout, 16 bytes per lane.
//   softmax online in log2 units (scores times scale*log2 e), block max over
//         DPP rows, lazy rescale: the reference max moves only when a block
//         beats it by more than 8, so weights stay <= 2^8.
//   PV    fp32 on the vector ALUs (weights are not rounded to bf16); a lane
//         owns 8 dims of 8 keys, V loaded as whole 256-byte rows.
// Loads of block i+1 are issued before block i is computed (two register
// sets), so every wave keeps 16 KiB of K/V requests in flight.
#pragma once

#include "gfx950.hpp"

namespace da {

constexpr int kBlockKeys = 32;        // keys per block of the flattened key space
constexpr float kRescaleSlack = 8.f;   // log2 units
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kRowBytes = kHeadDim * 2;  // one K or V row

// ---- raw buffer resources: 32-bit offsets, loads beyond the range read 0 ----
constexpr int kRawBufferFlags = 0x00020000;  // dword 3 of a raw (untyped) buffer resource on gfx950
constexpr int kCachePolicySc1 = 16;          // device-scope coherence (sc1)
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRawBufferFlags);
}
__device__ __forceinline__ uint4 rsrc_ld16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ uint4 rsrc_ld16_coherent(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCachePolicySc1));
}
__device__ __forceinline__ uint2 rsrc_ld8_coherent(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kCachePolicySc1));
}
__device__ __forceinline__ float rsrc_ld4f_coherent(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kCachePolicySc1));
}
__device__ __forceinline__ void rsrc_st4f_coherent(rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, v), r, (int)off, 0, kCachePolicySc1);
}
__device__ __forceinline__ void rsrc_st16_coherent(rsrc_t r, uint32_t off, uint4 v) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, kCachePolicySc1);
}
__device__ __forceinline__ void rsrc_st8_coherent(rsrc_t r, uint32_t off, uint2 v) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, (int)off, 0, kCachePolicySc1);
}

// ---- per-wave running state ----
template <int GP>
struct AttnWave {
  float m_ref[4];  // row group grp: query grp*4 + r
  float l_acc[4];  // per-lane partial sum of weights (key column of this lane)
  float acc[GP][8];  // un-normalised output, dims col*8..+8, keys of row group grp

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      m_ref[r] = -INFINITY;
      l_acc[r] = 0.f;
    }
#pragma unroll
    for (int g = 0; g < GP; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
  }
};

// Keys one wave handles per step: KB = 32 (two 16-key MFMA tiles) or 16 (one
// tile, for large groups whose accumulators leave fewer registers free).
template <int KB>
struct KVTile {
  uint4 k[KB / 16][4];  // 16-key tiles, MFMA B layout
  uint4 v[KB / 4];      // keys grp + 4i, dims col*8..+8
};

// Everything a wave needs to know about the (batch, kv head) it works on.
struct AttnSeg {
  rsrc_t K, V;    // [L, 128] bf16 rows of this (batch, kv head); reads past L return 0
  int L;          // keys of the sequence
  int G;          // query heads of the group
  float scale_log2;
  float scale;
  float* dbg;     // scaled scores of query row 0 of the group, or null; row stride dbg_stride
  int dbg_stride;
};

__device__ __forceinline__ void load_query(uint4 (&qa)[4], const uint16_t* q_rows, int G, int col, int grp) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    qa[kk] = (col < G) ? ld16(q_rows + (size_t)col * kHeadDim + kk * 32 + grp * 8) : make_uint4(0, 0, 0, 0);
}

template <int KB>
__device__ __forceinline__ void load_kv(KVTile<KB>& t, const AttnSeg& sg, int key0, int col, int grp) {
#pragma unroll
  for (int tt = 0; tt < KB / 16; ++tt) {
    const uint32_t row = (uint32_t)(key0 + 16 * tt + col) * kRowBytes;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) t.k[tt][kk] = rsrc_ld16(sg.K, row + kk * 64 + grp * 16);
  }
#pragma unroll
  for (int i = 0; i < KB / 4; ++i) t.v[i] = rsrc_ld16(sg.V, (uint32_t)(key0 + grp + 4 * i) * kRowBytes + col * 16);
}

// One KB-key step starting at key0; keys >= end are masked out.
template <int GP, int KB>
__device__ __forceinline__ void attn_block(AttnWave<GP>& w, const KVTile<KB>& t, const uint4 (&qa)[4],
                                           const AttnSeg& sg, int key0, int end, float* sp, int col, int grp) {
  constexpr int NTL = KB / 16;
  f32x4_t sc[NTL];
#pragma unroll
  for (int tt = 0; tt < NTL; ++tt) {
    sc[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) sc[tt] = mfma_bf16(qa[kk], t.k[tt][kk], sc[tt]);
  }
  float s2[NTL][4];
#pragma unroll
  for (int tt = 0; tt < NTL; ++tt) {
    const int key = key0 + 16 * tt + col;
#pragma unroll
    for (int r = 0; r < 4; ++r) s2[tt][r] = (key < end) ? sc[tt][r] * sg.scale_log2 : -INFINITY;
  }
  if (sg.dbg) {
#pragma unroll
    for (int tt = 0; tt < NTL; ++tt) {
      const int key = key0 + 16 * tt + col;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = grp * 4 + r;
        if (row < sg.G && key < end) sg.dbg[(size_t)row * sg.dbg_stride + key] = sc[tt][r] * sg.scale;
      }
    }
  }

  float bm[4];
  bool need = false;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float mx = s2[0][r];
#pragma unroll
    for (int tt = 1; tt < NTL; ++tt) mx = fmaxf(mx, s2[tt][r]);
    bm[r] = row16_max(mx);
    need |= bm[r] > w.m_ref[r] + kRescaleSlack;
  }
  if (__builtin_amdgcn_ballot_w64(need) != 0) {
    float alpha[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float mn = fmaxf(w.m_ref[r], bm[r]);
      alpha[r] = exp2f(w.m_ref[r] - mn);
      w.m_ref[r] = mn;
      w.l_acc[r] *= alpha[r];
    }
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      const float a = readlane_f32(alpha[g & 3], (g >> 2) * 16);
#pragma unroll
      for (int e = 0; e < 8; ++e) w.acc[g][e] *= a;
    }
  }
  float pw[NTL][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
#pragma unroll
    for (int tt = 0; tt < NTL; ++tt) {
      // a masked key has weight 0 (also while the reference max is still -inf)
      pw[tt][r] = s2[tt][r] > -INFINITY ? exp2f(s2[tt][r] - w.m_ref[r]) : 0.f;
      w.l_acc[r] += pw[tt][r];
    }
  }

  // weights to LDS as [key][query] so that each PV lane reads its keys' rows
  if (grp * 4 < GP) {
#pragma unroll
    for (int tt = 0; tt < NTL; ++tt) {
      const int key = 16 * tt + col;
      if constexpr (GP >= 4) {
        *reinterpret_cast<float4*>(sp + key * GP + grp * 4) = make_float4(pw[tt][0], pw[tt][1], pw[tt][2], pw[tt][3]);
      } else {
#pragma unroll
        for (int r = 0; r < GP; ++r) sp[key * GP + r] = pw[tt][r];
      }
    }
  }
  wave_lds_fence();

#pragma unroll
  for (int i = 0; i < KB / 4; ++i) {
    const int key = grp + 4 * i;
    float vv[8];
    unpack_bf16x8(t.v[i], vv);
    float pg[GP];
    if constexpr (GP >= 4) {
#pragma unroll
      for (int g4 = 0; g4 < GP / 4; ++g4) {
        const float4 t4 = *reinterpret_cast<const float4*>(sp + key * GP + g4 * 4);
        pg[g4 * 4 + 0] = t4.x;
        pg[g4 * 4 + 1] = t4.y;
        pg[g4 * 4 + 2] = t4.z;
        pg[g4 * 4 + 3] = t4.w;
      }
    } else {
#pragma unroll
      for (int g = 0; g < GP; ++g) pg[g] = sp[key * GP + g];
    }
#pragma unroll
    for (int g = 0; g < GP; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) w.acc[g][e] = fmaf(pg[g], vv[e], w.acc[g][e]);
  }
  wave_lds_fence();
}

// The wave's steps first, first+step, ... (n of them, KB keys each). The loads
// of the next D-1 steps are in flight while a step is computed (D register
// sets, indexed statically through the unrolled inner loop).
template <int GP, int KB, int D>
__device__ __forceinline__ void attn_wave_steps(AttnWave<GP>& w, const uint4 (&qa)[4], const AttnSeg& sg, int first,
                                                int step, int n, int end, float* sp, int col, int grp) {
  if (n <= 0) return;
  KVTile<KB> t[D];
#pragma unroll
  for (int j = 0; j < D - 1; ++j)
    if (j < n) load_kv<KB>(t[j], sg, (first + j * step) * KB, col, grp);
  for (int i0 = 0; i0 < n; i0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int i = i0 + j;
      if (i < n) {
        if (i + D - 1 < n) load_kv<KB>(t[(j + D - 1) % D], sg, (first + (i + D - 1) * step) * KB, col, grp);
        attn_block<GP, KB>(w, t[j], qa, sg, (first + i * step) * KB, end, sp, col, grp);
      }
    }
  }
}

// Reduce the wave's state (row sums of l over the 16 key lanes, O over the 4
// key groups) and park it in LDS: so[g][128], sm[g], sl[g].
template <int GP>
__device__ __forceinline__ void attn_wave_to_lds(AttnWave<GP>& w, float (*so)[kHeadDim], float* sm, float* sl, int col,
                                                 int grp) {
#pragma unroll
  for (int r = 0; r < 4; ++r) w.l_acc[r] = row16_sum(w.l_acc[r]);
#pragma unroll
  for (int g = 0; g < GP; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      w.acc[g][e] += __shfl_xor(w.acc[g][e], 16);
      w.acc[g][e] += __shfl_xor(w.acc[g][e], 32);
    }
  if (grp == 0) {
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      *reinterpret_cast<float4*>(&so[g][col * 8]) = make_float4(w.acc[g][0], w.acc[g][1], w.acc[g][2], w.acc[g][3]);
      *reinterpret_cast<float4*>(&so[g][col * 8 + 4]) = make_float4(w.acc[g][4], w.acc[g][5], w.acc[g][6], w.acc[g][7]);
    }
  }
  if (col == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int g = grp * 4 + r;
      if (g < GP) {
        sm[g] = w.m_ref[r];
        sl[g] = w.l_acc[r];
      }
    }
  }
}

// Online merge of one (max, sum, 4 outputs) partial into a running one.
__device__ __forceinline__ void merge_partial(float& M, float& Ls, float (&O)[4], float m, float l, const float (&o)[4]) {
  if (m == -INFINITY) return;  // an empty partial
  if (m > M) {
    const float a = exp2f(M - m);
    Ls *= a;
#pragma unroll
    for (int e = 0; e < 4; ++e) O[e] *= a;
    M = m;
  }
  const float f = exp2f(m - M);
  Ls = fmaf(f, l, Ls);
#pragma unroll
  for (int e = 0; e < 4; ++e) O[e] = fmaf(f, o[e], O[e]);
}

}  // namespace da
