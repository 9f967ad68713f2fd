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
// adds them in a fixed order (deterministic).
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

}  // namespace da
