// Output projection (the third matmul of one decode-attention forward in
// "PyPTO 开箱性能调优实战：Decode Attention 多 Matmul 独立 TileShape 配置
// F-16", section 代码对比: attn_output_flat x o_weight -> bf16) and the fp16
// BasicMatmul check of the CANN msKPP page "自动调优流程 / Kernel级自动调优".
//
// Both run on the MFMA GEMM below whenever K is a multiple of 32, at every M:
// a projection of a few tokens is far below the MFMA ridge, so the weight
// stream sets its pace, and the GEMM's whole-row-block loads stream it faster
// than the GEMV (measured at M = 1, 2, 4 and 8). The weight tile is
// transposed through LDS into the MFMA operand layout (B needs 8 consecutive
// k per lane, the weight is row-major in n); the activation fragment is read
// straight from global memory.
//
// The VALU GEMV (M < 16) serves a K that is not a multiple of 32 and the
// column-tile widths only it has. A workgroup owns a tile of up to 512 output
// columns (1 KiB of each weight row, read by one wave in one instruction)
// times a K-chunk of rows; every lane keeps 8 rows of 16 bytes in flight.
//
// In both, the partial sums of the K-chunks meet in the workspace through
// device-coherent stores, and the last workgroup of an output tile to arrive
// adds them in a fixed order (deterministic). A product with too few
// 128-column tiles to fill the chip (the fp16 check) runs on 16 x 32 tiles
// over all of K instead, which needs no workspace.
#include "gemm_core.hpp"
#include "gemv_core.hpp"

namespace da {

namespace {

constexpr int kThreads = 256;

// GEMV workgroup: one work item of gemv_core.hpp per workgroup.
template <int MB, int TC>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvParams p) {
  extern __shared__ float s_x[];  // [kchunk][MB]
  __shared__ __attribute__((aligned(16))) char s_fin[gemv_finish_lds<MB, TC>()];
  gemv_item<MB, TC>(p, blockIdx.x, blockIdx.y, s_x, s_fin);
}

// ---- MFMA GEMM: one gemm_core.hpp item per workgroup ----
template <bool F16, int MT, int D>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) char smem[kGemmLds];
  DA_TRACE(14);
  gemm_item<F16, MT, D, false>(p, blockIdx.x, blockIdx.y, blockIdx.z, gridDim.x, smem, nullptr);
}

// ---- narrow-tile MFMA GEMM: every workgroup a 16 x NC tile of C over all of K ----
// For a product whose 128-column tiles would leave most of the chip idle (the
// fp16 check: 256 x 512 outputs are 64 such tiles), a workgroup owns NC
// columns of 16 rows instead, and no K-split is needed, so nothing meets in a
// workspace. Its NW waves take interleaved 32-row K-steps and request up to
// kNarrowDepth of them at once (on the fp16 check, 8 waves of 4 steps: 6.2 us
// a launch from HBM against 6.9 with 4 waves of 8 and 9.4 with 128-column
// tiles; 16-column tiles read A twice as often and take 8.5). A step's B rows (2 NC bytes each) are parked
// in the wave's LDS stage (rows padded by 16 bytes) and read back with the
// transposing LDS read: lane (i, g) of a 16-lane group receives rows
// 4g..4g+3 and 16+4g..16+4g+3 of column 16j+i for product j, and its A
// fragment holds the same k of row i, read straight from global memory. The
// waves' sums meet in LDS in wave order.
constexpr int kNarrowDepth = 4;
constexpr int kNarrowWaves = 8;
constexpr int kNarrowCols = 32;

template <bool F16, int NW, int NC>
__global__ __launch_bounds__(NW * kWave) void gemm_narrow_kernel(GemmParams p) {
  constexpr int kRow = NC * 2 + 16;        // LDS stage row
  constexpr int kLanesPerRow = NC * 2 / 16;
  constexpr int kRowsPerLoad = kWave / kLanesPerRow;
  constexpr int kLoads = kGemmRows / kRowsPerLoad;  // B load instructions per step
  constexpr int NT = NW * kWave;
  constexpr int kOut = 16 * NC > NT ? 16 * NC / NT : 1;  // consecutive outputs per thread in the final sum
  static_assert(kOut == 1 || kOut == 2 || kOut == 4, "1, 2 or 4 outputs per thread");
  __shared__ __attribute__((aligned(16))) char s_stage[NW][kGemmRows * kRow];
  __shared__ float s_red[NW][16][NC];
  const int n0 = blockIdx.x * NC, m0 = blockIdx.y * 16;
  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
  const int i = lane & 15, g = lane >> 4;
  char* const stage = s_stage[wave];
  DA_TRACE(14);

  // B from column n0 on (reads past the end return 0; columns past N are never stored)
  const uint32_t rowb = (uint32_t)p.N * 2;
  const rsrc_t wr = make_rsrc(p.b + n0, (uint32_t)((size_t)p.K * rowb - (size_t)n0 * 2));
  const uint32_t woff = (uint32_t)(lane / kLanesPerRow) * rowb + (lane % kLanesPerRow) * 16;
  const int m = m0 + i;
  const rsrc_t xr = make_rsrc(p.a, (uint32_t)min((size_t)p.M * p.K * 2, (size_t)0xffffffffu));
  const uint32_t xoff = (uint32_t)(((size_t)min(m, p.M - 1) * p.K + 4 * g) * 2);
  const bool xok = m < p.M;

  const int nsteps = p.K / kGemmRows;
  const int nst = nsteps > wave ? (nsteps - wave + NW - 1) / NW : 0;
  f32x4_t acc[NC / 16];
#pragma unroll
  for (int jj = 0; jj < NC / 16; ++jj) acc[jj] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const char* bt = stage + (4 * g + (i >> 2)) * kRow + (i & 3) * 8;
  char* const wp = stage + (lane / kLanesPerRow) * kRow + (lane % kLanesPerRow) * 16;
  for (int s0 = 0; s0 < nst; s0 += kNarrowDepth) {
    uint4 wt[kNarrowDepth][kLoads];
    uint2 xa[kNarrowDepth][2];
#pragma unroll
    for (int j = 0; j < kNarrowDepth; ++j) {
      if (s0 + j < nst) {
        const uint32_t r0 = (uint32_t)(wave + NW * (s0 + j)) * kGemmRows;
#pragma unroll
        for (int c = 0; c < kLoads; ++c) wt[j][c] = rsrc_ld16(wr, (r0 + c * kRowsPerLoad) * rowb + woff);
        xa[j][0] = xok ? __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(xr, (int)(xoff + r0 * 2), 0, 0))
                       : make_uint2(0, 0);
        xa[j][1] = xok ? __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                                                       xr, (int)(xoff + (r0 + 16) * 2), 0, 0))
                       : make_uint2(0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < kNarrowDepth; ++j) {
      if (s0 + j < nst) {
        wave_lds_fence();  // the previous step's LDS reads come first
#pragma unroll
        for (int c = 0; c < kLoads; ++c) *reinterpret_cast<uint4*>(wp + c * kRowsPerLoad * kRow) = wt[j][c];
        wave_lds_fence();
        if (s0 + j == 0) DA_TRACE(1);
        const uint4 a = make_uint4(xa[j][0].x, xa[j][0].y, xa[j][1].x, xa[j][1].y);
#pragma unroll
        for (int jj = 0; jj < NC / 16; ++jj) {
          const uint2 v0 = lds_read_tr16(bt + jj * 32);
          const uint2 v1 = lds_read_tr16(bt + 16 * kRow + jj * 32);
          acc[jj] = mfma16<F16>(a, make_uint4(v0.x, v0.y, v1.x, v1.y), acc[jj]);
        }
      }
    }
  }
  DA_TRACE(2);
  // lane holds C[4g + r][16jj + i]; the waves' sums in wave order
#pragma unroll
  for (int jj = 0; jj < NC / 16; ++jj)
#pragma unroll
    for (int r = 0; r < 4; ++r) s_red[wave][4 * g + r][16 * jj + i] = acc[jj][r];
  __syncthreads();
  DA_TRACE(3);
  if (t >= 16 * NC / kOut) return;
  const int row = t / (NC / kOut), col = (t % (NC / kOut)) * kOut;
  float v[kOut];
#pragma unroll
  for (int e = 0; e < kOut; ++e) {
    v[e] = s_red[0][row][col + e];
#pragma unroll
    for (int w = 1; w < NW; ++w) v[e] += s_red[w][row][col + e];
  }
  if (m0 + row < p.M && n0 + col < p.N) {
    uint16_t* dst = p.c + (size_t)(m0 + row) * p.N + n0 + col;
    if constexpr (kOut == 1) {
      *dst = to_out<F16>(v[0]);
    } else if constexpr (kOut == 2) {
      *reinterpret_cast<uint32_t*>(dst) = (uint32_t)to_out<F16>(v[0]) | ((uint32_t)to_out<F16>(v[1]) << 16);
    } else {
      // N is a multiple of 16 and col of 4: the four outputs are all in C or all past N
      *reinterpret_cast<uint2*>(dst) = make_uint2((uint32_t)to_out<F16>(v[0]) | ((uint32_t)to_out<F16>(v[1]) << 16),
                                                  (uint32_t)to_out<F16>(v[2]) | ((uint32_t)to_out<F16>(v[3]) << 16));
    }
  }
  DA_TRACE(6);
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

template <bool F16, int MT>
static hipError_t launch_gemm_mt(const GemmParams& p, hipStream_t s) {
  const dim3 grid((p.N + kGemmCols - 1) / kGemmCols, (p.M + 16 * MT - 1) / (16 * MT), p.ksplit);
  static_assert(kThreads == kGemmThreads, "one GEMM item per 256-thread workgroup");
  gemm_kernel<F16, MT, kGemmDepth><<<grid, dim3(kThreads), 0, s>>>(p);
  return hipGetLastError();
}

template <bool F16>
static hipError_t launch_gemm(const GemmParams& p, hipStream_t s) {
  switch (p.mtiles) {
    case 1: return launch_gemm_mt<F16, 1>(p, s);
    case 2: return launch_gemm_mt<F16, 2>(p, s);
    case 4: return launch_gemm_mt<F16, 4>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_bf16(const GemmParams& p, hipStream_t s) { return launch_gemm<false>(p, s); }
hipError_t launch_gemm_f16(const GemmParams& p, hipStream_t s) { return launch_gemm<true>(p, s); }

hipError_t launch_gemm_narrow_f16(const GemmParams& p, hipStream_t s) {
  const dim3 grid((p.N + kNarrowCols - 1) / kNarrowCols, (p.M + 15) / 16);
  gemm_narrow_kernel<true, kNarrowWaves, kNarrowCols><<<grid, dim3(kNarrowWaves * kWave), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace da
