// Output projection (the third matmul of one decode-attention forward in
// "PyPTO 开箱性能调优实战：Decode Attention 多 Matmul 独立 TileShape 配置
// F-16", section 代码对比: attn_output_flat x o_weight -> bf16) and the dense
// MFMA GEMM used for M >= 16 and for the fp16 BasicMatmul check of the CANN
// msKPP page "自动调优流程 / Kernel级自动调优".
//
// M < 16 (a handful of decode tokens) is a skinny GEMV: every weight byte is
// used M times, far below the MFMA ridge, so it runs on the vector ALUs.
// A workgroup owns a tile of up to 512 output columns (1 KiB of each weight
// row, read by one wave in one instruction) times a K-chunk of rows; every
// lane keeps 8 rows of 16 bytes in flight. Partial sums of the K-chunks meet
// in the workspace through device-coherent stores, and the last workgroup of
// a column tile to arrive adds them in a fixed order (deterministic).
//
// M >= 16 is a real dense contraction and runs on MFMA 16x16x32: the weight
// tile is transposed through LDS into the operand layout (B needs 8
// consecutive k per lane, the weight is row-major in n), the activation
// fragment is read straight from global memory.
#include "gfx950.hpp"
#include "kernels.hpp"

namespace da {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;  // weight rows per lane in flight per pass

// Workgroup tile of the GEMV: TC output columns (TC/8 lanes of 16 bytes per
// weight row, so a wave reads 1 KiB of contiguous rows when TC = 512) times a
// K-chunk of rows; MB activation rows are held per lane.
template <int MB, int TC>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvParams p) {
  constexpr int LPR = TC / 8;             // lanes per weight row
  constexpr int RPP = kThreads / LPR;     // rows per pass of the workgroup
  constexpr int RPW = kWave / LPR > 0 ? kWave / LPR : 1;  // row lanes inside one wave
  extern __shared__ float s_x[];          // [kchunk][MB] activations of this K-chunk, fp32
  __shared__ float s_red[kThreads / kWave][MB][TC];

  const int tile = blockIdx.x, ks = blockIdx.y;
  const int n0 = tile * TC;
  const int k0 = ks * p.kchunk;
  const int kn = min(p.kchunk, p.K - k0);
  const int t = threadIdx.x;
  const int cg = t % LPR;  // 8-column group inside the tile
  const int rr = t / LPR;  // row lane
  const int n = n0 + cg * 8;
  const bool col_ok = n < p.N;

  for (int idx = t; idx < MB * kn; idx += kThreads) {
    const int m = idx / kn, kk = idx % kn;
    const uint16_t xw = (m < p.M) ? p.x[(size_t)m * p.K + k0 + kk] : (uint16_t)0;
    s_x[kk * MB + m] = __builtin_bit_cast(float, (uint32_t)xw << 16);
  }
  __syncthreads();

  float acc[MB][8];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[m][e] = 0.f;

  const uint16_t* __restrict__ wbase = p.w + (size_t)k0 * p.N + n;
  for (int base = 0; base < kn; base += RPP * kUnroll) {
    uint4 wv[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int kk = base + rr + RPP * u;
      wv[u] = (col_ok && kk < kn) ? ld16(wbase + (size_t)kk * p.N) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int kk = base + rr + RPP * u;
      if (kk < kn) {
        float wf[8];
        unpack_bf16x8(wv[u], wf);
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          const float xm = s_x[kk * MB + m];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[m][e] = fmaf(xm, wf[e], acc[m][e]);
        }
      }
    }
  }

  // reduce the row lanes of a wave (lanes l, l^LPR, l^2LPR, ...), then the waves
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = acc[m][e];
#pragma unroll
      for (int x = LPR; x < kWave; x <<= 1) v += __shfl_xor(v, x);
      acc[m][e] = v;
    }
  const int wave = t / kWave, lane = t % kWave;
  if (lane < LPR) {
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int e = 0; e < 8; ++e) s_red[wave][m][lane * 8 + e] = acc[m][e];
  }
  (void)RPW;
  __syncthreads();

  const int M = p.M;
  float* part = p.part;
  for (int idx = t; idx < M * TC; idx += kThreads) {
    const int m = idx / TC, c = idx % TC;
    if (n0 + c >= p.N) continue;
    const float v = s_red[0][m][c] + s_red[1][m][c] + s_red[2][m][c] + s_red[3][m][c];
    if (p.ksplit == 1)
      p.out[(size_t)m * p.N + n0 + c] = f32_to_bf16_rne(v);
    else
      store_coherent(&part[((size_t)ks * M + m) * p.N + n0 + c], v);
  }
  if (p.ksplit == 1) return;
  if (!arrive_last_coherent(&p.counters[tile], (uint32_t)p.ksplit)) return;
  for (int idx = t; idx < M * TC; idx += kThreads) {
    const int m = idx / TC, c = idx % TC;
    if (n0 + c >= p.N) continue;
    float v = 0.f;
    for (int s = 0; s < p.ksplit; ++s) v += load_coherent(&part[((size_t)s * M + m) * p.N + n0 + c]);
    p.out[(size_t)m * p.N + n0 + c] = f32_to_bf16_rne(v);
  }
}

// ---- MFMA GEMM: 16 x 64 output tile, K staged 128 rows at a time ----
constexpr int kStrip = 64;
constexpr int kKStep = 128;
constexpr int kBtPitch = kKStep + 8;  // bf16 elements per transposed row (pad vs bank conflicts)

template <bool F16>
__device__ __forceinline__ uint16_t to_out(float v) {
  if constexpr (F16) {
    return __builtin_bit_cast(uint16_t, (_Float16)v);
  } else {
    return f32_to_bf16_rne(v);
  }
}

template <bool F16>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmParams p) {
  __shared__ uint16_t s_bt[kStrip][kBtPitch];  // B tile transposed: [n][k]

  const int nt = blockIdx.x, mt = blockIdx.y, ks = blockIdx.z;
  const int n0 = nt * kStrip, m0 = mt * 16;
  const int k0 = ks * p.kchunk;
  const int kn = min(p.kchunk, p.K - k0);
  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
  const int col = lane & 15, grp = lane >> 4;
  const int arow = m0 + col;
  const bool arow_ok = arow < p.M;
  const int bcg = t & 7;   // 8-column group this lane loads
  const int brow = t >> 3; // first of the 4 rows this lane loads
  const bool bcol_ok = n0 + bcg * 8 < p.N;

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int kb = 0; kb < kn; kb += kKStep) {
    const int rows = min(kKStep, kn - kb);
    uint4 bv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = brow + 32 * j;
      bv[j] = (bcol_ok && r < rows) ? ld16(p.b + (size_t)(k0 + kb + r) * p.N + n0 + bcg * 8) : make_uint4(0, 0, 0, 0);
    }
    __syncthreads();  // previous tile fully consumed
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = brow + 32 * j;
      const uint32_t w4[4] = {bv[j].x, bv[j].y, bv[j].z, bv[j].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s_bt[bcg * 8 + 2 * e][r] = (uint16_t)(w4[e] & 0xffffu);
        s_bt[bcg * 8 + 2 * e + 1][r] = (uint16_t)(w4[e] >> 16);
      }
    }
    __syncthreads();
    for (int sub = 0; sub < rows; sub += 32) {
      const int k = k0 + kb + sub + grp * 8;
      const uint4 a = arow_ok ? ld16(p.a + (size_t)arow * p.K + k) : make_uint4(0, 0, 0, 0);
      const uint4 bb = *reinterpret_cast<const uint4*>(&s_bt[wave * 16 + col][sub + grp * 8]);
      if constexpr (F16)
        acc = mfma_f16(a, bb, acc);
      else
        acc = mfma_bf16(a, bb, acc);
    }
  }

  // lane holds C[m0 + grp*4 + r][n0 + wave*16 + col]
  const int cn = n0 + wave * 16 + col;
  const bool cn_ok = cn < p.N;
  if (p.ksplit == 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + grp * 4 + r;
      if (m < p.M && cn_ok) p.c[(size_t)m * p.N + cn] = to_out<F16>(acc[r]);
    }
    return;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = m0 + grp * 4 + r;
    if (m < p.M && cn_ok) store_coherent(&p.part[((size_t)ks * p.M + m) * p.N + cn], acc[r]);
  }
  const int tile = mt * gridDim.x + nt;
  if (!arrive_last_coherent(&p.counters[tile], (uint32_t)p.ksplit)) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = m0 + grp * 4 + r;
    if (m < p.M && cn_ok) {
      float v = 0.f;
      for (int s = 0; s < p.ksplit; ++s) v += load_coherent(&p.part[((size_t)s * p.M + m) * p.N + cn]);
      p.c[(size_t)m * p.N + cn] = to_out<F16>(v);
    }
  }
}

}  // namespace

template <int MB, int TC>
hipError_t launch_gemv_tc(const GemvParams& p, hipStream_t s) {
  const dim3 grid((p.N + TC - 1) / TC, p.ksplit), block(kThreads);
  const size_t shm = (size_t)p.kchunk * MB * sizeof(float);
  gemv_kernel<MB, TC><<<grid, block, shm, s>>>(p);
  return hipGetLastError();
}

template <int MB>
hipError_t launch_gemv_mb(const GemvParams& p, hipStream_t s) {
  switch (p.tile_n) {
    case 64: return launch_gemv_tc<MB, 64>(p, s);
    case 128: return launch_gemv_tc<MB, 128>(p, s);
    case 256: if constexpr (MB <= 8) return launch_gemv_tc<MB, 256>(p, s); else return hipErrorInvalidValue;
    case 512: if constexpr (MB <= 4) return launch_gemv_tc<MB, 512>(p, s); else return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemv(const GemvParams& p, int mpad, hipStream_t s) {
  switch (mpad) {
    case 1: return launch_gemv_mb<1>(p, s);
    case 2: return launch_gemv_mb<2>(p, s);
    case 4: return launch_gemv_mb<4>(p, s);
    case 8: return launch_gemv_mb<8>(p, s);
    case 16: return launch_gemv_mb<16>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_bf16(const GemmParams& p, hipStream_t s) {
  const dim3 grid((p.N + kStrip - 1) / kStrip, (p.M + 15) / 16, p.ksplit);
  gemm_kernel<false><<<grid, dim3(kThreads), 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_gemm_f16(const GemmParams& p, hipStream_t s) {
  const dim3 grid((p.N + kStrip - 1) / kStrip, (p.M + 15) / 16, p.ksplit);
  gemm_kernel<true><<<grid, dim3(kThreads), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace da
