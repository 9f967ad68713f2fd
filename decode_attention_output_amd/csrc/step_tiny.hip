// The whole decode step in one launch for tiny steps, with no hand-over
// between workgroups: attention and output projection of "PyPTO 开箱性能调优
// 实战：Decode Attention 多 Matmul 独立 TileShape 配置 F-16" (section 代码对比:
// the three matmul calls of one forward).
//
// When every sequence's K/V cache is a few hundred KiB at most, each
// projection workgroup computes the whole attention itself (the repeated K/V
// reads are served by L2) instead of waiting for attention workgroups: every
// cross-workgroup hand-over costs a device-coherent store, an atomic and a
// load, about a microsecond each, which is most of such a step. A workgroup
// owns kTinyCols output columns over all of K (placement: see kTinyXcds):
//  1. it requests its weight tile at once (thread t holds rows t, t + 256, ...,
//     32 bytes each), so the weight streams while the attention runs;
//  2. for every (batch, kv head) sequence, its four waves take interleaved
//     32-key steps (attn_core.hpp), merge in LDS, and the attention output is
//     rounded to bf16 and kept in LDS;
//  3. every thread multiplies its rows, and the 256 partial sums of each output
//     meet in LDS in a fixed order (deterministic); the result is rounded to bf16.
#include "attn_core.hpp"
#include "kernels.hpp"

namespace da {

namespace {

// Workgroup i of a launch runs on XCD i % 8, and the XCDs begin a launch one
// after another (the last ~2-4 us after the first). The column tiles therefore
// go to the first kTinyXcds XCDs, more only where they would not fit one per
// compute unit; the other workgroups exit at once. Measured on the 4/1-head,
// 256-key, 512-column step: 2 XCDs 8.1-8.2 us, 1 XCD or all 8 8.3 us.
constexpr int kTinyXcds = 2;
constexpr int kCusPerXcd = 32;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kRowsPerThread = kTinyMaxK / kThreads;
constexpr int kOuts = kTinyMaxBatch * kTinyCols;      // outputs of a workgroup
constexpr int kRedGroups = kThreads / kOuts;            // first-level sums per output
constexpr int kStagesLds = kWaves * kStageBytes;
static_assert(kThreads * kOuts * 4 <= kStagesLds, "the partial sums fit the stages");
static_assert(kThreads % kOuts == 0, "whole groups of partial sums");

template <int GP>
__global__ __launch_bounds__(kThreads, 1) void decode_step_tiny_kernel(StepTinyParams p) {
  __shared__ __attribute__((aligned(16))) char s_stage[kStagesLds];
  __shared__ float s_flat[kTinyMaxBatch][kTinyMaxK];  // the bf16-rounded attention output
  __shared__ float s_red2[kRedGroups][kOuts];
  constexpr int kWaveOut = GP * kHeadDim * 4;
  static_assert(kWaveOut + 2 * GP * 4 <= kStageBytes, "a wave's output fits its stage");
  auto s_o = [&](int w) { return reinterpret_cast<float (*)[kHeadDim]>(s_stage + w * kStageBytes); };
  auto s_m = [&](int w) { return reinterpret_cast<float*>(s_stage + w * kStageBytes + kWaveOut); };
  auto s_l = [&](int w) { return reinterpret_cast<float*>(s_stage + w * kStageBytes + kWaveOut + GP * 4); };
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  const int col = lane & 15, grp = lane >> 4;
  const int B = p.B, G = p.G, K = p.Hq * kHeadDim;
  // column tiles xcd * per_xcd + slot: consecutive ones share an XCD's L2
  const int xcd = (int)blockIdx.x % kXcds, slot = (int)blockIdx.x / kXcds;
  if (xcd >= p.xcds) return;
  const int n0 = (xcd * p.per_xcd + slot) * kTinyCols;
  if (n0 >= p.N) return;
  DA_TRACE(0);

  // ---- 1. the weight tile: rows t + 256 i, columns n0 .. n0+15 (two 16-byte loads a row) ----
  const uint32_t rowb = (uint32_t)p.N * 2;
  const rsrc_t wr = make_rsrc(p.w + n0, (uint32_t)((size_t)K * rowb - (size_t)n0 * 2));
  uint4 wv[kRowsPerThread][2];
#pragma unroll
  for (int i = 0; i < kRowsPerThread; ++i) {
    const int k = t + kThreads * i;
    const uint32_t off = k < K ? (uint32_t)k * rowb : 0xffffffffu - 63u;  // past the range: reads 0
    wv[i][0] = rsrc_ld16(wr, off);
    wv[i][1] = rsrc_ld16(wr, off + 16);
  }

  // ---- 2. the attention of every sequence, rounded to bf16, into LDS ----
  // (requesting the first sequence's first step before its length is known, as
  // the small single launch does, measured 0.9 us slower here: the extra
  // register set moves the step loop's values into AGPRs)
  for (int seq = 0; seq < B * p.Hkv; ++seq) {
    const int b = seq / p.Hkv, h = seq % p.Hkv;
    const int L = uniform(min(max(p.seq_lens[b], 0), p.Lmax));
    AttnSeg sg;
    const size_t kv_off = ((size_t)b * p.Hkv + h) * p.Lmax * kHeadDim;
    sg.K = make_rsrc(p.k + kv_off, (uint32_t)L * kRowBytes);
    sg.V = make_rsrc(p.v + kv_off, (uint32_t)L * kRowBytes);
    sg.L = L;
    sg.G = G;
    sg.scale_log2 = p.scale_log2;
    sg.scale = 0.f;
    sg.dbg = nullptr;
    sg.dbg_stride = 0;
    uint4 qa[kHeadDim / 32];
    load_query<kHeadDim>(qa, p.q + ((size_t)b * p.Hq + (size_t)h * G) * kHeadDim, G, col, grp);
    AttnWaveT<kHeadDim> aw;
    aw.reset();
    const int nstep = (L + kStepKeys - 1) / kStepKeys;
    const int n = nstep > wave ? (nstep - wave + kWaves - 1) / kWaves : 0;
    attn_wave_steps<GP, 1, kHeadDim>(aw, qa, sg, wave, kWaves, n, L, s_stage + wave * kStageBytes, lane);
    attn_wave_to_lds<GP, kHeadDim>(aw, s_o(wave), s_m(wave), s_l(wave), lane);
    __syncthreads();
    for (int idx = t; idx < G * kHeadDim; idx += kThreads) {
      const int g = idx / kHeadDim, d = idx % kHeadDim;
      float M = s_m(0)[g];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m(w)[g]);
      float Ls = 0.f, O = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = exp2f(s_m(w)[g] - M);
        Ls = fmaf(f, s_l(w)[g], Ls);
        O = fmaf(f, s_o(w)[g][d], O);
      }
      s_flat[b][(h * G + g) * kHeadDim + d] = bf16_lo(f32_to_bf16_rne(O / Ls));
    }
    __syncthreads();  // the stages are reused by the next sequence
  }
  DA_TRACE(2);

  // ---- 3. the projection: partial sums of this thread's rows, then a fixed-order reduction ----
  float (*s_red)[kOuts] = reinterpret_cast<float (*)[kOuts]>(s_stage);  // [thread][b * 16 + c]
  for (int b = 0; b < kTinyMaxBatch; ++b) {
    float acc[kTinyCols];
#pragma unroll
    for (int c = 0; c < kTinyCols; ++c) acc[c] = 0.f;
    if (b < B) {
#pragma unroll
      for (int i = 0; i < kRowsPerThread; ++i) {
        const int k = t + kThreads * i;
        if (k < K) {
          const float x = s_flat[b][k];
          float wf[8];
          unpack_bf16x8(wv[i][0], wf);
#pragma unroll
          for (int c = 0; c < 8; ++c) acc[c] = fmaf(x, wf[c], acc[c]);
          unpack_bf16x8(wv[i][1], wf);
#pragma unroll
          for (int c = 0; c < 8; ++c) acc[8 + c] = fmaf(x, wf[c], acc[8 + c]);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < kTinyCols; ++c) s_red[t][b * kTinyCols + c] = acc[c];
  }
  __syncthreads();
  {
    // first level: output j = t % kOuts, threads s * 32 .. s * 32 + 31 of group s = t / kOuts
    const int j = t % kOuts, s = t / kOuts;
    constexpr int kPer = kThreads / kRedGroups;
    float v = 0.f;
#pragma unroll 8
    for (int u = 0; u < kPer; ++u) v += s_red[s * kPer + u][j];
    s_red2[s][j] = v;
  }
  __syncthreads();
  if (t < kOuts) {
    const int b = t / kTinyCols, c = t % kTinyCols;
    float v = 0.f;
#pragma unroll
    for (int s = 0; s < kRedGroups; ++s) v += s_red2[s][t];
    if (b < B && n0 + c < p.N) p.out[(size_t)b * p.N + n0 + c] = f32_to_bf16_rne(v);
  }
  DA_TRACE(6);
}

}  // namespace

hipError_t launch_decode_step_tiny(const StepTinyParams& prm, int gpad, hipStream_t s) {
  // the fewest leading XCDs that hold the column tiles one per compute unit
  StepTinyParams p = prm;
  const int tiles = (p.N + kTinyCols - 1) / kTinyCols;
  p.xcds = kTinyXcds;
  while (p.xcds < kXcds && (tiles + p.xcds - 1) / p.xcds > kCusPerXcd) p.xcds *= 2;
  p.per_xcd = (tiles + p.xcds - 1) / p.xcds;
  const dim3 grid(kXcds * p.per_xcd), block(kThreads);
  switch (gpad) {
    case 1: decode_step_tiny_kernel<1><<<grid, block, 0, s>>>(p); break;
    case 2: decode_step_tiny_kernel<2><<<grid, block, 0, s>>>(p); break;
    case 4: decode_step_tiny_kernel<4><<<grid, block, 0, s>>>(p); break;
    case 8: decode_step_tiny_kernel<8><<<grid, block, 0, s>>>(p); break;
    case 16: decode_step_tiny_kernel<16><<<grid, block, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace da
