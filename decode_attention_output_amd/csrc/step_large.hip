// The whole decode step in one launch for large steps (many sequences or long
// ones): attention and output projection of "PyPTO 开箱性能调优实战：Decode
// Attention 多 Matmul 独立 TileShape 配置 F-16" (section 代码对比: the three
// matmul calls of one forward).
//
// The grid holds the stream-K attention workgroups first (attn_streamk.hpp,
// each counting its finished sequences in their kv head's ready counter), then
// one workgroup per MFMA GEMM item of the projection (gemm_core.hpp), K-chunk
// by K-chunk. Workgroups are dispatched in index order, so every attention
// workgroup is running or done before a projection workgroup starts; a
// projection workgroup requests the weight rows of its first steps at once,
// then waits (bounded) for the kv heads of its K-chunk and reads the attention
// output with device-coherent loads. Compared with two launches, the weight
// stream starts while the attention's last pieces merge, and the projection's
// start-up (dispatch, first loads) overlaps the attention's tail.
#include "attn_streamk.hpp"
#include "gemm_core.hpp"

namespace da {

namespace {

constexpr int kThreads = 256;
constexpr int kLds = attn_streamk_lds<kAttnWaves, kHeadDim>() > kGemmLds ? attn_streamk_lds<kAttnWaves, kHeadDim>()
                                                                         : kGemmLds;

template <int GP, int MT>
__global__ __launch_bounds__(kThreads, 2) void decode_step_large_kernel(StepLargeParams p) {
  __shared__ __attribute__((aligned(16))) char smem[kLds];
  DA_TRACE(14);
  if ((int)blockIdx.x < p.attn.num_workgroups) {
    attn_streamk_body<GP, kAttnWaves, 1, kHeadDim, true>(p.attn, blockIdx.x, p.attn.num_workgroups, smem);
    return;
  }
  const int r = (int)blockIdx.x - p.attn.num_workgroups;
  const int nt = r % p.ntiles, rest = r / p.ntiles;
  const int mg = rest % p.mgroups, ks = rest / p.mgroups;
  GemmWait w = p.wait;
  w.waiter = r;
  // (two m-tiles keep the plain depth: four steps of both would not fit the registers)
  gemm_item<false, MT, MT == 1 ? kGemmDepthWait : kGemmDepth, true>(p.gemm, nt, mg, ks, p.ntiles, smem, &w);
}

template <int GP>
hipError_t launch_gp(const StepLargeParams& p, hipStream_t s) {
  const dim3 grid(p.attn.num_workgroups + p.ntiles * p.mgroups * p.gemm.ksplit), block(kThreads);
  switch (p.gemm.mtiles) {
    case 1: decode_step_large_kernel<GP, 1><<<grid, block, 0, s>>>(p); break;
    case 2: decode_step_large_kernel<GP, 2><<<grid, block, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_step_large(const StepLargeParams& p, int gpad, hipStream_t s) {
  switch (gpad) {
    case 1: return launch_gp<1>(p, s);
    case 2: return launch_gp<2>(p, s);
    case 4: return launch_gp<4>(p, s);
    case 8: return launch_gp<8>(p, s);
    case 16: return launch_gp<16>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace da
