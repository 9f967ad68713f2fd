// Device building blocks of GQA decode attention on gfx950, shared by the
// stream-K attention kernel and the single-launch decode-step kernel.
//
// What they compute is the first two matmuls of one decode-attention forward
// and the softmax between them ("PyPTO 开箱性能调优实战：Decode Attention 多
// Matmul 独立 TileShape 配置 F-16", section 代码对比): scores = q_grouped x
// k_cache^T in fp32, scaled softmax, attn_weights x v_cache.
//
// Per wavefront and per 32-key step:
//   loads  K and V rows straight from HBM, 1 KiB per load instruction (four
//          whole 256-byte rows), the access pattern that streams fastest;
//          the tile is parked in the wave's own LDS stage (rows padded by 16
//          bytes, so that the operand reads below are free of bank conflicts)
//          and the registers take the loads of a later step at once.
//   S^T    = K x Q^T on MFMA 16x16x32 bf16: A = 16 keys read back from LDS in
//          the operand layout, B = the query group (columns G..15 zero). A lane
//          ends up with the 8 scores of one query for keys {4g..4g+3,
//          16+4g..16+4g+3} (g = lane / 16), which is exactly its share of the
//          A operand of the next product, so the weights never leave registers.
//   softmax online in log2 units (scores times scale*log2 e); the block max
//          meets across the four lane groups; lazy rescale: the reference max
//          moves only when a block beats it by more than 8, so weights <= 2^8.
//   PV     O = P x V on MFMA 16x16x32 bf16 with fp32 accumulation. P is split
//          into three bf16 terms (hi and mid by truncation, lo rounded), whose
//          sum is P within 2^-23 relative, about fp32's own rounding, so the
//          weights are not coarsened to bf16. V reaches the B layout through
//          the LDS transpose read: in each 16-lane group, lane i's element r
//          is element i%4 of the 8 bytes addressed by lane 4r + i/4.
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
__device__ __forceinline__ void rsrc_st16_coherent(rsrc_t r, uint32_t off, uint4 v) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, kCachePolicySc1);
}
__device__ __forceinline__ void rsrc_st8_coherent(rsrc_t r, uint32_t off, uint2 v) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, (int)off, 0, kCachePolicySc1);
}

// ---- per-wave running state ----
// The wave's 16 MFMA columns are query rows (G valid, the rest zero queries).
template <int HD>
struct AttnWaveT {
  float m_ref;        // reference max of query lane%16 (log2 units), equal in the 4 lane groups
  float l_acc;        // sum of this lane's weights of query lane%16
  f32x4_t o[HD / 16]; // O[query 4g + r][dim 16j + lane%16] in element r of o[j]

  __device__ __forceinline__ void reset() {
    m_ref = -INFINITY;
    l_acc = 0.f;
#pragma unroll
    for (int j = 0; j < HD / 16; ++j) o[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
};
using AttnWave = AttnWaveT<kHeadDim>;

constexpr int kStepKeys = 32;  // keys per wave step

// Sizes of one head_dim HD (128 or 256): a K or V row is 2*HD bytes; one load
// instruction of a wave reads 1 KiB, i.e. kRowsPerLoad whole rows, and a lane
// holds kLoads 16-byte pieces of a 32-key K (or V) tile: piece c is row
// kRowsPerLoad*c + lane/kLanesPerRow, bytes (lane%kLanesPerRow)*16. In LDS
// the K rows are padded by 16 bytes (the 16-byte operand reads of 16 rows by
// 16 lanes fall on distinct banks) and the V rows by 32 bytes (the
// transposing reads of 4 rows x 32 bytes by 16 lanes fall on distinct banks).
// Above head_dim 128 a wave takes its 32-key steps as two 16-key halves (a
// 16-row register set and stage), which keeps a lane's registers and a wave's
// LDS small enough for two workgroups per compute unit.
template <int HD>
struct Dims {
  static constexpr int kRowBytes = HD * 2;
  static constexpr int kLanesPerRow = kRowBytes / 16;
  static constexpr int kRowsPerLoad = kWave / kLanesPerRow;
  static constexpr int kLoads = kStepKeys / kRowsPerLoad;
  static constexpr bool kHalves = HD > 128;
  static constexpr int kStageKeys = kHalves ? kStepKeys / 2 : kStepKeys;  // keys in a wave's stage
  static constexpr int kStageRow = kRowBytes + 16;           // K row
  static constexpr int kStageTile = kStageKeys * kStageRow;  // the K tile; the V tile follows
  static constexpr int kStageRowV = kRowBytes + 32;          // V row
  static constexpr int kStageBytes = kStageTile + kStageKeys * kStageRowV;  // LDS of one wave
};
constexpr int kStageRow = Dims<kHeadDim>::kStageRow;
constexpr int kStageTile = Dims<kHeadDim>::kStageTile;
constexpr int kStageBytes = Dims<kHeadDim>::kStageBytes;

// One step's K and V as loaded (see Dims).
template <int HD>
struct KVTileT {
  uint4 k[Dims<HD>::kLoads], v[Dims<HD>::kLoads];
};
using KVTile = KVTileT<kHeadDim>;

// Everything a wave needs to know about the (batch, kv head) it works on.
struct AttnSeg {
  rsrc_t K, V;    // [L, head_dim] bf16 rows of this (batch, kv head); reads past L return 0
  int L;          // keys of the sequence
  int G;          // query heads of the group
  float scale_log2;
  float scale;
  float* dbg;     // scaled scores of the group's first query head, or null; row stride dbg_stride
  int dbg_stride;
};

// B operand of S^T = K x Q^T: lane (query col, group grp) holds dims
// kk*32 + grp*8 .. +8 of its query (zero for col >= G).
template <int HD = kHeadDim>
__device__ __forceinline__ void load_query(uint4 (&qa)[HD / 32], const uint16_t* q_rows, int G, int col, int grp) {
#pragma unroll
  for (int kk = 0; kk < HD / 32; ++kk)
    qa[kk] = (col < G) ? ld16(q_rows + (size_t)col * HD + kk * 32 + grp * 8) : make_uint4(0, 0, 0, 0);
}

template <int HD = kHeadDim>
__device__ __forceinline__ void load_kv(KVTileT<HD>& t, const AttnSeg& sg, int key0, int lane) {
  using Dm = Dims<HD>;
  const uint32_t off = (uint32_t)(key0 + lane / Dm::kLanesPerRow) * Dm::kRowBytes + (lane % Dm::kLanesPerRow) * 16;
#pragma unroll
  for (int c = 0; c < Dm::kLoads; ++c) t.k[c] = rsrc_ld16(sg.K, off + c * Dm::kRowsPerLoad * Dm::kRowBytes);
#pragma unroll
  for (int c = 0; c < Dm::kLoads; ++c) t.v[c] = rsrc_ld16(sg.V, off + c * Dm::kRowsPerLoad * Dm::kRowBytes);
}

template <int HD = kHeadDim>
__device__ __forceinline__ void stage_kv(char* stage, const KVTileT<HD>& t, int lane) {
  using Dm = Dims<HD>;
  char* p = stage + (lane / Dm::kLanesPerRow) * Dm::kStageRow + (lane % Dm::kLanesPerRow) * 16;
  char* pv = stage + Dm::kStageTile + (lane / Dm::kLanesPerRow) * Dm::kStageRowV + (lane % Dm::kLanesPerRow) * 16;
#pragma unroll
  for (int c = 0; c < Dm::kLoads; ++c) *reinterpret_cast<uint4*>(p + c * Dm::kRowsPerLoad * Dm::kStageRow) = t.k[c];
#pragma unroll
  for (int c = 0; c < Dm::kLoads; ++c) *reinterpret_cast<uint4*>(pv + c * Dm::kRowsPerLoad * Dm::kStageRowV) = t.v[c];
}

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

// LDS transpose read of four 16-bit elements (see the header comment).
__device__ __forceinline__ uint2 lds_read_tr16(const char* p) {
  const bf16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_bf16x4_t*)(__attribute__((address_space(3))) char*)(const_cast<char*>(p)));
  return __builtin_bit_cast(uint2, r);
}

typedef __attribute__((address_space(3))) char lds_char;

// Transposing LDS read of four 16-bit elements at an LDS address (offsets added
// to an LDS-space pointer fold into the instruction's offset field).
__device__ __forceinline__ uint2 lds_tr16_at(const lds_char* p) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)const_cast<lds_char*>(p)));
}

// bf16 pair of two floats whose low 16 bits are zero: the high halves.
__device__ __forceinline__ uint32_t pack_hi(float a, float b) {
  return (__builtin_bit_cast(uint32_t, a) >> 16) | (__builtin_bit_cast(uint32_t, b) & 0xffff0000u);
}
// Round a finite float to bf16 (nearest, ties to even), as a 32-bit pattern.
__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u;
}

// One 32-key step starting at key0, whose K/V tile is in the wave's stage;
// keys >= end are masked out.
template <int GP, int HD = kHeadDim>
__device__ __forceinline__ void attn_step(AttnWaveT<HD>& w, const char* stage, const uint4 (&qb)[HD / 32],
                                          const AttnSeg& sg, int key0, int end, int lane) {
  using Dm = Dims<HD>;
  const int i = lane & 15, g = lane >> 4;
  // ---- S^T = K x Q^T, two 16-key tiles ----
  f32x4_t sc[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    sc[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const char* kr = stage + (16 * tt + i) * Dm::kStageRow + g * 16;
#pragma unroll
    for (int kk = 0; kk < HD / 32; ++kk)
      sc[tt] = mfma_bf16(*reinterpret_cast<const uint4*>(kr + kk * 64), qb[kk], sc[tt]);
  }
  // lane (i, g) holds the scores of query i for keys 16tt + 4g + r
  float s2[2][4];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int r = 0; r < 4; ++r) s2[tt][r] = (key0 + 16 * tt + 4 * g + r < end) ? sc[tt][r] * sg.scale_log2 : -INFINITY;
  if (sg.dbg && i < sg.G) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = key0 + 16 * tt + 4 * g + r;
        if (key < end) sg.dbg[(size_t)i * sg.dbg_stride + key] = sc[tt][r] * sg.scale;
      }
  }

  // ---- online softmax with lazy rescale: the reference moves only when some
  // lane's own scores pass it by the slack; only then is the row max over the
  // four lanes of a row taken ----
  const float lmx = fmaxf(fmaxf(fmaxf(fmaxf(fmaxf(fmaxf(fmaxf(s2[0][0], s2[0][1]), s2[0][2]), s2[0][3]), s2[1][0]),
                                      s2[1][1]),
                                s2[1][2]),
                          s2[1][3]);
  if (__builtin_amdgcn_ballot_w64(lmx > w.m_ref + kRescaleSlack) != 0) {
    float mx = fmaxf(lmx, __shfl_xor(lmx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(w.m_ref, mx);
    const float alpha = w.m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(w.m_ref - mn);
    w.m_ref = mn;
    w.l_acc *= alpha;
    // accumulator row 4g + r belongs to query 4g + r, whose factor lane 4g + r holds
    float ar[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * g + r);
#pragma unroll
    for (int j = 0; j < HD / 16; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) w.o[j][r] *= ar[r];
  }
  float p[2][4];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      // a masked key has weight 0 (also while the reference max is still -inf)
      p[tt][r] = s2[tt][r] > -INFINITY ? __builtin_amdgcn_exp2f(s2[tt][r] - w.m_ref) : 0.f;
      w.l_acc += p[tt][r];
    }

  // ---- A operand of P x V: k index 8g + e is key 4g + e (e < 4), 16 + 4g + e - 4 ----
  // three bf16 terms per weight: hi and mid by truncation, lo rounded
  float hi[2][4], mid[2][4], lo[2][4];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      hi[tt][r] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, p[tt][r]) & 0xffff0000u);
      const float r1 = p[tt][r] - hi[tt][r];
      mid[tt][r] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, r1) & 0xffff0000u);
      lo[tt][r] = __builtin_bit_cast(float, bf16_bits_rne(r1 - mid[tt][r]));
    }
  auto pack = [](const float (&x)[2][4]) {
    return make_uint4(pack_hi(x[0][0], x[0][1]), pack_hi(x[0][2], x[0][3]), pack_hi(x[1][0], x[1][1]),
                      pack_hi(x[1][2], x[1][3]));
  };
  const uint4 a_hi = pack(hi), a_mid = pack(mid), a_lo = pack(lo);

  // ---- O += P x V, 16 dims per product, 128 dims at a time ----
  // one LDS address register per step; the empty asm keeps the compiler from
  // holding a register per read across the loop, so the offsets stay immediate
  uint32_t voff = Dm::kStageTile + (4 * g + (i >> 2)) * Dm::kStageRowV + (i & 3) * 8;
  asm volatile("" : "+v"(voff));
  const lds_char* vbase = (const lds_char*)stage + voff;
#pragma unroll
  for (int h0 = 0; h0 < HD / 16; h0 += 8) {
    const lds_char* vt = vbase + h0 * 32;
    uint4 vb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint2 v0 = lds_tr16_at(vt + j * 32);
      const uint2 v1 = lds_tr16_at(vt + 16 * Dm::kStageRowV + j * 32);
      vb[j] = make_uint4(v0.x, v0.y, v1.x, v1.y);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) w.o[h0 + j] = mfma_bf16(a_hi, vb[j], w.o[h0 + j]);
#pragma unroll
    for (int j = 0; j < 8; ++j) w.o[h0 + j] = mfma_bf16(a_mid, vb[j], w.o[h0 + j]);
#pragma unroll
    for (int j = 0; j < 8; ++j) w.o[h0 + j] = mfma_bf16(a_lo, vb[j], w.o[h0 + j]);
  }
}

// ---- head_dim above 128: 16-key half steps ----
template <int HD>
struct KVHalfT {
  uint4 k[Dims<HD>::kLoads / 2], v[Dims<HD>::kLoads / 2];  // 16 rows of K and of V
};

template <int HD>
__device__ __forceinline__ void load_half(KVHalfT<HD>& t, const AttnSeg& sg, int key0, int lane) {
  using Dm = Dims<HD>;
  const uint32_t off = (uint32_t)(key0 + lane / Dm::kLanesPerRow) * Dm::kRowBytes + (lane % Dm::kLanesPerRow) * 16;
#pragma unroll
  for (int c = 0; c < Dm::kLoads / 2; ++c) t.k[c] = rsrc_ld16(sg.K, off + c * Dm::kRowsPerLoad * Dm::kRowBytes);
#pragma unroll
  for (int c = 0; c < Dm::kLoads / 2; ++c) t.v[c] = rsrc_ld16(sg.V, off + c * Dm::kRowsPerLoad * Dm::kRowBytes);
}

template <int HD>
__device__ __forceinline__ void stage_half(char* stage, const KVHalfT<HD>& t, int lane) {
  using Dm = Dims<HD>;
  char* p = stage + (lane / Dm::kLanesPerRow) * Dm::kStageRow + (lane % Dm::kLanesPerRow) * 16;
  char* pv = stage + Dm::kStageTile + (lane / Dm::kLanesPerRow) * Dm::kStageRowV + (lane % Dm::kLanesPerRow) * 16;
#pragma unroll
  for (int c = 0; c < Dm::kLoads / 2; ++c) *reinterpret_cast<uint4*>(p + c * Dm::kRowsPerLoad * Dm::kStageRow) = t.k[c];
#pragma unroll
  for (int c = 0; c < Dm::kLoads / 2; ++c)
    *reinterpret_cast<uint4*>(pv + c * Dm::kRowsPerLoad * Dm::kStageRowV) = t.v[c];
}

// A 16-key half step starting at key0 on the 16-row K/V tile in the wave's
// stage (keys >= end masked out): the 32-key step with keys 16..31 absent (zero
// in both operands of P x V).
template <int GP, int HD>
__device__ __forceinline__ void attn_half_step(AttnWaveT<HD>& w, const char* stage, const uint4 (&qb)[HD / 32],
                                               const AttnSeg& sg, int key0, int end, int lane) {
  using Dm = Dims<HD>;
  const int i = lane & 15, g = lane >> 4;
  // ---- S^T = K x Q^T, one 16-key tile: lane (i, g) gets the scores of query i for keys 4g + r ----
  f32x4_t sc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const char* kr = stage + i * Dm::kStageRow + g * 16;
#pragma unroll
  for (int kk = 0; kk < HD / 32; ++kk) sc = mfma_bf16(*reinterpret_cast<const uint4*>(kr + kk * 64), qb[kk], sc);
  float s2[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) s2[r] = (key0 + 4 * g + r < end) ? sc[r] * sg.scale_log2 : -INFINITY;
  if (sg.dbg && i < sg.G) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = key0 + 4 * g + r;
      if (key < end) sg.dbg[(size_t)i * sg.dbg_stride + key] = sc[r] * sg.scale;
    }
  }
  // ---- online softmax with lazy rescale (as in the 32-key step) ----
  const float lmx = fmaxf(fmaxf(fmaxf(s2[0], s2[1]), s2[2]), s2[3]);
  if (__builtin_amdgcn_ballot_w64(lmx > w.m_ref + kRescaleSlack) != 0) {
    float mx = fmaxf(lmx, __shfl_xor(lmx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(w.m_ref, mx);
    const float alpha = w.m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(w.m_ref - mn);
    w.m_ref = mn;
    w.l_acc *= alpha;
    float ar[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * g + r);
#pragma unroll
    for (int j = 0; j < HD / 16; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) w.o[j][r] *= ar[r];
  }
  float p[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    p[r] = s2[r] > -INFINITY ? __builtin_amdgcn_exp2f(s2[r] - w.m_ref) : 0.f;
    w.l_acc += p[r];
  }
  // three bf16 terms per weight; k index 8g + e is key 4g + e for e < 4, absent above
  float hi[4], mid[4], lo[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    hi[r] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, p[r]) & 0xffff0000u);
    const float r1 = p[r] - hi[r];
    mid[r] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, r1) & 0xffff0000u);
    lo[r] = __builtin_bit_cast(float, bf16_bits_rne(r1 - mid[r]));
  }
  const uint4 a_hi = make_uint4(pack_hi(hi[0], hi[1]), pack_hi(hi[2], hi[3]), 0u, 0u);
  const uint4 a_mid = make_uint4(pack_hi(mid[0], mid[1]), pack_hi(mid[2], mid[3]), 0u, 0u);
  const uint4 a_lo = make_uint4(pack_hi(lo[0], lo[1]), pack_hi(lo[2], lo[3]), 0u, 0u);
  // ---- O += P x V over the 16 rows, 16 dims per product ----
  uint32_t voff = Dm::kStageTile + (4 * g + (i >> 2)) * Dm::kStageRowV + (i & 3) * 8;
  asm volatile("" : "+v"(voff));
  const lds_char* vbase = (const lds_char*)stage + voff;
#pragma unroll
  for (int h0 = 0; h0 < HD / 16; h0 += 8) {
    const lds_char* vt = vbase + h0 * 32;
    uint4 vb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint2 v0 = lds_tr16_at(vt + j * 32);
      vb[j] = make_uint4(v0.x, v0.y, 0u, 0u);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) w.o[h0 + j] = mfma_bf16(a_hi, vb[j], w.o[h0 + j]);
#pragma unroll
    for (int j = 0; j < 8; ++j) w.o[h0 + j] = mfma_bf16(a_mid, vb[j], w.o[h0 + j]);
#pragma unroll
    for (int j = 0; j < 8; ++j) w.o[h0 + j] = mfma_bf16(a_lo, vb[j], w.o[h0 + j]);
  }
}

// The wave's steps first, first+step, ... (n of them, 32 keys each). D
// register sets: a set is parked in LDS as its step begins and at once takes
// the loads of the step D later, so D steps are in flight during a step.
template <int GP, int D, int HD = kHeadDim>
__device__ __forceinline__ void attn_wave_steps(AttnWaveT<HD>& w, const uint4 (&qb)[HD / 32], const AttnSeg& sg,
                                                int first, int step, int n, int end, char* stage, int lane) {
  if (n <= 0) return;
  if constexpr (Dims<HD>::kHalves) {
    // 2n half steps; one 16-row register set parked as its half begins
    static_assert(D == 1, "one step in flight");
    auto hkey = [&](int u) { return (first + (u >> 1) * step) * kStepKeys + (u & 1) * (kStepKeys / 2); };
    KVHalfT<HD> t;
    load_half<HD>(t, sg, hkey(0), lane);
    for (int u = 0; u < 2 * n; ++u) {
      wave_lds_fence();  // the previous half's LDS reads come first
      stage_half<HD>(stage, t, lane);
      if (u + 1 < 2 * n) load_half<HD>(t, sg, hkey(u + 1), lane);
      wave_lds_fence();
      attn_half_step<GP, HD>(w, stage, qb, sg, hkey(u), end, lane);
    }
    wave_lds_fence();
    return;
  }
  KVTileT<HD> t[D];
#pragma unroll
  for (int j = 0; j < D; ++j)
    if (j < n) load_kv<HD>(t[j], sg, (first + j * step) * kStepKeys, lane);
  for (int i0 = 0; i0 < n; i0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int i = i0 + j;
      if (i < n) {
        wave_lds_fence();  // the previous step's LDS reads come first
        stage_kv<HD>(stage, t[j], lane);
        if (i + D < n) load_kv<HD>(t[j], sg, (first + (i + D) * step) * kStepKeys, lane);
        wave_lds_fence();
        attn_step<GP, HD>(w, stage, qb, sg, (first + i * step) * kStepKeys, end, lane);
      }
    }
  }
  wave_lds_fence();
}

// The same with one register set, the first tile already loaded (through
// resources that may reach past `end`): rows of it at or past `end` are
// zeroed before use, so that whatever the cache holds there (NaN padding
// included) never meets a weight.
template <int GP>
__device__ __forceinline__ void attn_wave_steps_preloaded(AttnWave& w, KVTile& t, const uint4 (&qb)[4],
                                                          const AttnSeg& sg, int first, int step, int n, int end,
                                                          char* stage, int lane) {
  if (n <= 0) return;
#pragma unroll
  for (int c = 0; c < 8; ++c)
    if (first * kStepKeys + 4 * c + (lane >> 4) >= end) {
      t.k[c] = make_uint4(0, 0, 0, 0);
      t.v[c] = make_uint4(0, 0, 0, 0);
    }
  for (int i = 0; i < n; ++i) {
    wave_lds_fence();  // the previous step's LDS reads come first
    stage_kv(stage, t, lane);
    if (i + 1 < n) load_kv(t, sg, (first + (i + 1) * step) * kStepKeys, lane);
    wave_lds_fence();
    attn_step<GP>(w, stage, qb, sg, (first + i * step) * kStepKeys, end, lane);
  }
  wave_lds_fence();
}

// Park the wave's state in LDS: so[g][128], sm[g], sl[g] for g < GP. These
// may overlap the wave's own stage (its last reads are complete).
template <int GP, int HD = kHeadDim>
__device__ __forceinline__ void attn_wave_to_lds(AttnWaveT<HD>& w, float (*so)[HD], float* sm, float* sl, int lane) {
  const int i = lane & 15, g = lane >> 4;
  float l = w.l_acc;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  wave_lds_fence();
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int q = 4 * g + r;
    if (q < GP) {
#pragma unroll
      for (int j = 0; j < HD / 16; ++j) so[q][16 * j + i] = w.o[j][r];
    }
  }
  if (g == 0 && i < GP) {
    sm[i] = w.m_ref;
    sl[i] = l;
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
