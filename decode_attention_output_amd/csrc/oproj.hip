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
#include "gemv_core.hpp"

namespace da {

namespace {

constexpr int kThreads = 256;

// GEMV workgroup: one work item of gemv_core.hpp per workgroup.
template <int MB, int TC>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvParams p) {
  extern __shared__ float s_x[];  // [kchunk][MB]
  __shared__ __attribute__((aligned(16))) char s_fin[gemv_finish_lds<MB, TC>()];
  gemv_item<MB, TC, false>(p, blockIdx.x, blockIdx.y, s_x, s_fin, [] {});
}

// ---- MFMA GEMM: 16 x 64 output tile, K staged 128 rows at a time ----
//
// The MFMA operands need 8 consecutive k per lane, while the weight is
// row-major in n: each 128-row step of the weight tile is stored in LDS as
// loaded ([k][n], 16-byte writes) and read back transposed, eight 16-bit reads
// per lane per operand. The activation step is staged in LDS as [m][k] and
// read with one 16-byte read per operand. The global loads of step s+1 are in
// flight while step s is multiplied.
constexpr int kStrip = 64;
constexpr int kKStep = 128;
constexpr int kBPitch = kStrip + 8;  // bf16 per weight row in LDS
constexpr int kAPitch = kKStep + 8;  // bf16 per activation row in LDS

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
  __shared__ __attribute__((aligned(16))) uint16_t s_b[kKStep][kBPitch];
  __shared__ __attribute__((aligned(16))) uint16_t s_a[16][kAPitch];
  __shared__ float4 s_fin[kThreads];

  const int nt = blockIdx.x, mt = blockIdx.y, ks = blockIdx.z;
  const int n0 = nt * kStrip, m0 = mt * 16;
  const int k0 = ks * p.kchunk;
  const int kn = min(p.kchunk, p.K - k0);
  const int nsteps = (kn + kKStep - 1) / kKStep;
  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
  const int col = lane & 15, grp = lane >> 4;
  const int bcg = t & 7;    // 8-column group this lane loads
  const int brow = t >> 3;  // first of the 4 weight rows this lane loads
  const bool bcol_ok = n0 + bcg * 8 < p.N;
  const int am = t >> 4, ak = (t & 15) * 8;  // activation element this lane loads
  const bool arow_ok = m0 + am < p.M;

  uint4 bv[4], av;
  auto load_step = [&](int st) {
    const int kb = st * kKStep;
    const int rows = min(kKStep, kn - kb);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = brow + 32 * j;
      bv[j] = (bcol_ok && r < rows) ? ld16(p.b + (size_t)(k0 + kb + r) * p.N + n0 + bcg * 8) : make_uint4(0, 0, 0, 0);
    }
    av = (arow_ok && ak < rows) ? ld16(p.a + (size_t)(m0 + am) * p.K + k0 + kb + ak) : make_uint4(0, 0, 0, 0);
  };

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  load_step(0);
  for (int st = 0; st < nsteps; ++st) {
    __syncthreads();  // the previous step is no longer read
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<uint4*>(&s_b[brow + 32 * j][bcg * 8]) = bv[j];
    *reinterpret_cast<uint4*>(&s_a[am][ak]) = av;
    __syncthreads();
    if (st + 1 < nsteps) load_step(st + 1);
    const int rows = min(kKStep, kn - st * kKStep);
    for (int sub = 0; sub < rows; sub += 32) {
      const uint4 a = *reinterpret_cast<const uint4*>(&s_a[col][sub + grp * 8]);
      uint32_t bw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = s_b[sub + grp * 8 + 2 * j][wave * 16 + col];
        const uint32_t hi = s_b[sub + grp * 8 + 2 * j + 1][wave * 16 + col];
        bw[j] = lo | (hi << 16);
      }
      const uint4 bb = make_uint4(bw[0], bw[1], bw[2], bw[3]);
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
  const rsrc_t part = make_rsrc(p.part, p.part_bytes);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = m0 + grp * 4 + r;
    if (m < p.M && cn_ok) rsrc_st4f_coherent(part, (uint32_t)((((size_t)ks * p.M + m) * p.N + cn) * 4), acc[r]);
  }
  const int tile = mt * gridDim.x + nt;
  if (!arrive_last_coherent(&p.counters[tile], (uint32_t)p.ksplit)) return;
  // the last K-chunk adds every chunk's partial; lane (r, n) of the tile, splits in 8-wide batches
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < p.ksplit; s0 += 8) {
    float pv[8][4];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = min(m0 + grp * 4 + r, p.M - 1);
        const int sidx = min(s0 + u, p.ksplit - 1);
        pv[u][r] = rsrc_ld4f_coherent(part, (uint32_t)((((size_t)sidx * p.M + m) * p.N + min(cn, p.N - 1)) * 4));
      }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (s0 + u < p.ksplit)
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] += pv[u][r];
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = m0 + grp * 4 + r;
    if (m < p.M && cn_ok) p.c[(size_t)m * p.N + cn] = to_out<F16>(v[r]);
  }
  (void)s_fin;
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
