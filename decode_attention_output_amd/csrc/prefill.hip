// Context (prefill) attention of a chunk of new tokens on gfx950.
//
// The F-16 page ("PyPTO 开箱性能调优实战：Decode Attention 多 Matmul 独立
// TileShape 配置 F-16") names a context-attention kernel next to the decode one
// without defining it; the reading taken here: sequence b holds ctx_lens[b]
// cached keys, the last T of which are the chunk's own tokens, and token t
// attends causally to keys 0 .. ctx_lens[b] - T + t with the decode step's
// scaled softmax (T = 1 is the decode attention).
//
// Many query rows share every key, so this is a real MFMA contraction. A
// workgroup owns 4 * 16 * kRowSets query rows of one (batch, kv head) -- row r
// is token r / G, query head r % G of the group -- and each wave kRowSets sets
// of 16 rows, every set one 16-column B operand of S^T = K x Q^T: each K and V
// operand read from LDS feeds kRowSets products. The four waves share each
// 32-key K/V tile: the workgroup loads it cooperatively (whole rows, 1 KiB per
// load instruction) and stores it into one of three LDS stages a tile ahead of
// the waves, which compute the scores of the next tile while they turn the
// current tile's scores into weights (online softmax with a lazy rescale, each
// lane masking the keys past its own row's position) and multiply them into
// O. A wave skips the tiles past the last key of its rows; the workgroup stops
// loading at the last key of its last row; the workgroups of the longest rows
// (the end of the chunk) start first.
//
// The weights enter P x V as two bf16 terms (truncated high part, then the
// rounded rest): together they carry 16 significant bits, a relative error of at
// most 2^-17 per weight, which is the accuracy its fp32 score itself has after
// the 128-term dot product; the decode kernels keep three (fp32-exact weights)
// because there the matrix cores are idle anyway.
#include "attn_core.hpp"
#include "kernels.hpp"

namespace da {

namespace {

constexpr int kPrefillWaves = 4;
constexpr int kPrefillThreads = kPrefillWaves * kWave;
constexpr int kRowSets = 2;                                // 16-row sets per wave
constexpr int kPrefillRows = kPrefillWaves * 16 * kRowSets;  // query rows per workgroup
constexpr int kPrefillStages = 3;                          // K/V stages shared by the waves
// A stage holds a 32-key K tile and V tile. K rows are read 16 bytes a lane,
// 16 rows per 16 lanes: a 272-byte row stride puts the rows on distinct banks.
// V rows are read by transposing 8-byte reads, 4 rows x 32 bytes per 16
// lanes: a 288-byte stride spreads those rows over the banks.
constexpr int kKRow = kRowBytes + 16;
constexpr int kVRow = kRowBytes + 32;
constexpr int kKTileBytes = kStepKeys * kKRow;
constexpr int kPStageBytes = kKTileBytes + kStepKeys * kVRow;
constexpr int kPrefillLds = kPrefillStages * kPStageBytes;

typedef __attribute__((address_space(3))) char lds_char;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;

// Transposing LDS read of four 16-bit elements at an LDS address.
__device__ __forceinline__ uint2 lds_tr16_at(const lds_char* p) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)const_cast<lds_char*>(p)));
}

template <int RS>
struct PrefillWave {
  f32x4_t o[RS][8];  // set s: O[row 4g + r][dim 16j + lane%16] in element r of o[s][j]
  float m_ref[RS];   // reference max (log2 units) of row lane%16 of each set
  float l_acc[RS];   // this lane's share of that row's weight sum
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// The three parts of a wave's 32-key step on a K/V tile, for RS row sets.
//
// Scores: S^T = K x Q^T; lane (i, g) gets the scores of row i for keys
// 16tt + 4g + r of the tile in sc[s][tt][r].
template <int RS>
__device__ __forceinline__ void prefill_scores(f32x4_t (&sc)[RS][2], const lds_char* stage, const uint4 (&qb)[RS][4],
                                               int lane) {
  const int i = lane & 15, g = lane >> 4;
#pragma unroll
  for (int s = 0; s < RS; ++s)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) sc[s][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const lds_char* kr = stage + (16 * tt + i) * kKRow + g * 16;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const uint4 a = __builtin_bit_cast(uint4, *reinterpret_cast<const lds_u32x4*>(kr + kk * 64));
#pragma unroll
      for (int s = 0; s < RS; ++s) sc[s][tt] = mfma_bf16(a, qb[s][kk], sc[s][tt]);
    }
  }
}

// Reference: with MASK, key k of the tile is dropped (score -inf) for row
// lane%16 of set s unless k < end[s] (tiles that cross the causal diagonal).
// The reference max moves only when some lane's own scores pass it by the
// slack; only then is the row max over the four lanes of a row taken and the
// accumulators rescaled. Every row has key 0, so its first tile gives it a
// finite reference.
template <int RS, bool MASK>
__device__ __forceinline__ void prefill_reference(PrefillWave<RS>& w, const f32x4_t (&sc)[RS][2],
                                                  float (&x)[RS][2][4], int key0, const int (&end)[RS],
                                                  float scale_log2, int lane) {
  const int g = lane >> 4;
#pragma unroll
  for (int s = 0; s < RS; ++s) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        x[s][tt][r] = (!MASK || key0 + 16 * tt + 4 * g + r < end[s]) ? sc[s][tt][r] : -INFINITY;
    // a chain of three-input maxima
    const float lm = fmaxf(fmaxf(fmaxf(fmaxf(fmaxf(fmaxf(fmaxf(x[s][0][0], x[s][0][1]), x[s][0][2]), x[s][0][3]),
                                             x[s][1][0]), x[s][1][1]), x[s][1][2]), x[s][1][3]);
    if (__builtin_amdgcn_ballot_w64(lm * scale_log2 > w.m_ref[s] + kRescaleSlack) != 0) {
      float mx = fmaxf(lm, __shfl_xor(lm, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32)) * scale_log2;
      const float mn = fmaxf(w.m_ref[s], mx);
      const float alpha = __builtin_amdgcn_exp2f(w.m_ref[s] - mn);  // 0 while the reference is -inf
      w.m_ref[s] = mn;
      w.l_acc[s] *= alpha;
      float ar[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * g + r);
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) w.o[s][j][r] *= ar[r];
    }
  }
}

// Weights: p = 2^(x * scale_log2 - reference), summed into the row's weight
// sum and written as two bf16 terms of the P x V A operand (k index 8g + e is
// key 4g + e for e < 4, then 16 + 4g + e - 4).
template <int RS>
__device__ __forceinline__ void prefill_weights(PrefillWave<RS>& w, const float (&x)[RS][2][4], uint4 (&pa)[RS][2],
                                                float scale_log2) {
#pragma unroll
  for (int s = 0; s < RS; ++s) {
    const float neg_m = -w.m_ref[s];
    float p[2][4], rest[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // a dropped key: exp2(-inf) = 0
        p[tt][r] = __builtin_amdgcn_exp2f(fmaf(x[s][tt][r], scale_log2, neg_m));
        w.l_acc[s] += p[tt][r];
        rest[tt][r] = p[tt][r] - __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, p[tt][r]) & 0xffff0000u);
      }
    auto lo2 = [](float a, float b) {
      return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));  // round to nearest even
    };
    pa[s][0] = make_uint4(pack_hi(p[0][0], p[0][1]), pack_hi(p[0][2], p[0][3]), pack_hi(p[1][0], p[1][1]),
                          pack_hi(p[1][2], p[1][3]));
    pa[s][1] = make_uint4(lo2(rest[0][0], rest[0][1]), lo2(rest[0][2], rest[0][3]), lo2(rest[1][0], rest[1][1]),
                          lo2(rest[1][2], rest[1][3]));
  }
}

// O += P x V, 16 dims per product; each V operand serves every set and term.
// The wave runs the products at raised priority: when both waves of a SIMD
// are ready to issue, the products go first and the other wave's vector work
// fills the cycles the matrix core leaves to the vector unit.
template <int RS>
__device__ __forceinline__ void prefill_pv(PrefillWave<RS>& w, const uint4 (&pa)[RS][2], const lds_char* stage,
                                           int lane) {
  __builtin_amdgcn_s_setprio(1);
  const int i = lane & 15, g = lane >> 4;
  // one address register per step; the empty asm keeps the compiler from
  // hoisting a register per (j, half) out of the tile loop, so the offsets
  // below stay immediate fields of the reads
  uint32_t va = (uint32_t)(uintptr_t)(stage + kKTileBytes + (4 * g + (i >> 2)) * kVRow + (i & 3) * 8);
  asm volatile("" : "+v"(va));
  const lds_char* vt = (const lds_char*)(uintptr_t)va;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint2 v0 = lds_tr16_at(vt + j * 32);
    const uint2 v1 = lds_tr16_at(vt + 16 * kVRow + j * 32);
    const uint4 vb = make_uint4(v0.x, v0.y, v1.x, v1.y);
#pragma unroll
    for (int s = 0; s < RS; ++s)
#pragma unroll
      for (int e = 0; e < 2; ++e) w.o[s][j] = mfma_bf16(pa[s][e], vb, w.o[s][j]);
  }
  __builtin_amdgcn_s_setprio(0);
}

__global__ __launch_bounds__(kPrefillThreads, 2) void prefill_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) char smem[kPrefillLds];
  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
  const int i = lane & 15, grp = lane >> 4;
  const int R = p.T * p.G;                        // query rows of one (batch, kv head)
  const int blocks = (R + kPrefillRows - 1) / kPrefillRows;
  const int nseq = p.B * p.Hkv;
  // the last blocks of every sequence (longest rows) first; consecutive
  // workgroups take different sequences
  const int blk = blocks - 1 - (int)(blockIdx.x / nseq);
  const int seq = blockIdx.x % nseq;              // (batch, kv head)
  const int b = seq / p.Hkv, h = seq % p.Hkv;
  const int ctx = min(max(p.ctx_lens[b], 0), p.Lmax);
  const int base = ctx - p.T;                     // position of the chunk's first token

  // ---- this wave's rows: the queries (B operands) and the number of keys each row sees ----
  const int r0 = blk * kPrefillRows + wave * 16 * kRowSets;
  uint4 qb[kRowSets][4];
  int end[kRowSets];
#pragma unroll
  for (int s = 0; s < kRowSets; ++s) {
    const int rr = r0 + 16 * s + i;
    const bool ok = rr < R;
    const int tok = rr / p.G, gq = rr % p.G;
    const uint16_t* qrow = p.q + (((size_t)b * p.T + tok) * p.Hq + (size_t)h * p.G + gq) * kHeadDim;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qb[s][kk] = ok ? ld16(qrow + kk * 32 + grp * 8) : make_uint4(0, 0, 0, 0);
    end[s] = ok ? base + tok + 1 : 1;             // keys 0 .. end-1 (a row past the end: key 0, not stored)
  }
  // keys of the wave's first and last rows, and of the workgroup's last row
  const int wave_first_keys = r0 < R ? base + r0 / p.G + 1 : 0;
  const int wave_keys = r0 < R ? base + min(r0 + 16 * kRowSets - 1, R - 1) / p.G + 1 : 0;
  const int blk_keys = base + min(blk * kPrefillRows + kPrefillRows - 1, R - 1) / p.G + 1;
  const int ntiles = (blk_keys + kStepKeys - 1) / kStepKeys;

  const size_t kv_off = (size_t)seq * p.Lmax * kHeadDim;
  const rsrc_t K = make_rsrc(p.k + kv_off, (uint32_t)ctx * kRowBytes);  // rows past the context read as 0
  const rsrc_t V = make_rsrc(p.v + kv_off, (uint32_t)ctx * kRowBytes);

  // ---- the shared K/V tiles: thread t loads rows t/16 and 16 + t/16, bytes (t%16)*16 ----
  uint4 kr[2], vr[2];
  auto load_tile = [&](int tile) {
    const uint32_t off = (uint32_t)(tile * kStepKeys + t / 16) * kRowBytes + (t % 16) * 16;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      kr[j] = rsrc_ld16(K, off + j * 16 * kRowBytes);
      vr[j] = rsrc_ld16(V, off + j * 16 * kRowBytes);
    }
  };
  auto store_tile = [&](lds_char* stage) {
    lds_char* qk = stage + (t / 16) * kKRow + (t % 16) * 16;
    lds_char* qv = stage + kKTileBytes + (t / 16) * kVRow + (t % 16) * 16;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      *reinterpret_cast<lds_u32x4*>(qk + j * 16 * kKRow) = __builtin_bit_cast(u32x4_t, kr[j]);
      *reinterpret_cast<lds_u32x4*>(qv + j * 16 * kVRow) = __builtin_bit_cast(u32x4_t, vr[j]);
    }
  };

  PrefillWave<kRowSets> aw;
#pragma unroll
  for (int s = 0; s < kRowSets; ++s) {
#pragma unroll
    for (int j = 0; j < 8; ++j) aw.o[s][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    aw.m_ref[s] = -INFINITY;
    aw.l_acc[s] = 0.f;
  }
  // Tile t sits in stage t % 3. In iteration t the wave applies the softmax of
  // tile t and multiplies it into O while its scores for tile t + 1 are
  // computed (independent work for the matrix cores during the vector part);
  // before the barrier the workgroup stores tile t + 1, after it loads tile
  // t + 2 into registers. A stage is rewritten two barriers after its last read.
  const int my_tiles = (wave_keys + kStepKeys - 1) / kStepKeys;  // tiles this wave multiplies
  const int full_tiles = wave_first_keys / kStepKeys;            // ... without a masked key
  lds_char* const lds = (lds_char*)smem;
  auto stage_of = [&](int tile) { return lds + (tile % kPrefillStages) * kPStageBytes; };
  f32x4_t sc[kRowSets][2];
  if (ntiles > 0) {
    load_tile(0);
    store_tile(stage_of(0));
  }
  if (ntiles > 1) load_tile(1);
  __syncthreads();
  if (my_tiles > 0) prefill_scores<kRowSets>(sc, stage_of(0), qb, lane);
  for (int tile = 0; tile < ntiles; ++tile) {
    if (tile + 1 < ntiles) store_tile(stage_of(tile + 1));
    __syncthreads();
    if (tile + 2 < ntiles) load_tile(tile + 2);
    if (tile >= my_tiles) continue;
    const int key0 = tile * kStepKeys;
    const bool next = tile + 1 < my_tiles;
    float x[kRowSets][2][4];
    uint4 pa[kRowSets][2];
    if (tile < full_tiles && next) {
      prefill_reference<kRowSets, false>(aw, sc, x, key0, end, p.scale_log2, lane);
      prefill_scores<kRowSets>(sc, stage_of(tile + 1), qb, lane);
      prefill_weights<kRowSets>(aw, x, pa, p.scale_log2);
      prefill_pv<kRowSets>(aw, pa, stage_of(tile), lane);
    } else {
      if (tile < full_tiles)
        prefill_reference<kRowSets, false>(aw, sc, x, key0, end, p.scale_log2, lane);
      else
        prefill_reference<kRowSets, true>(aw, sc, x, key0, end, p.scale_log2, lane);
      prefill_weights<kRowSets>(aw, x, pa, p.scale_log2);
      prefill_pv<kRowSets>(aw, pa, stage_of(tile), lane);
      if (next) prefill_scores<kRowSets>(sc, stage_of(tile + 1), qb, lane);
    }
  }

  // ---- normalise and store: element r of o[s][j] is row 16s + 4*grp + r, dim 16j + i ----
#pragma unroll
  for (int s = 0; s < kRowSets; ++s) {
    float l = aw.l_acc[s];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);  // lane i (every group) holds the weight sum of its set's row i
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int q = 4 * grp + r;
      const int row = r0 + 16 * s + q;
      const float inv = 1.f / __shfl(l, q);
      if (row >= R) continue;
      uint16_t* orow = p.out + (((size_t)b * p.T + row / p.G) * p.Hq + (size_t)h * p.G + row % p.G) * kHeadDim;
#pragma unroll
      for (int j = 0; j < 8; ++j) orow[16 * j + i] = f32_to_bf16_rne(aw.o[s][j][r] * inv);
    }
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, hipStream_t s) {
  const int blocks = (p.T * p.G + kPrefillRows - 1) / kPrefillRows;
  prefill_kernel<<<dim3(p.B * p.Hkv * blocks), dim3(kPrefillThreads), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace da
