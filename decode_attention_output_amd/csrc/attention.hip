// Stream-K GQA decode attention for gfx950: the first two matmuls of one
// decode-attention forward and the softmax between them ("PyPTO 开箱性能调优实战：
// Decode Attention 多 Matmul 独立 TileShape 配置 F-16", section 代码对比) for every
// (batch, kv head) of a step in a single launch. The work split and the merge
// are described in attn_streamk.hpp, the per-wave steps in attn_core.hpp.
#include "attn_streamk.hpp"

namespace da {

namespace {

// One step in flight per wave: two workgroups fit a compute unit (head_dim 256
// takes its steps in 16-key halves for that); deeper pipelines use one
// workgroup per compute unit and its AGPRs.
template <int GP, int NW, int D, int HD>
__global__ __launch_bounds__(NW* kWave, D == 1 ? 2 : 1) void attn_streamk_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) char smem[attn_streamk_lds<NW, HD>()];
  DA_TRACE(14);
  attn_streamk_body<GP, NW, D, HD>(p, blockIdx.x, gridDim.x, smem);
}

}  // namespace

template <int GP, int D, int HD>
static hipError_t launch_variant(const AttnParams& p, hipStream_t s) {
  attn_streamk_kernel<GP, kAttnWaves, D, HD><<<dim3(p.num_workgroups), dim3(kAttnWaves * kWave), 0, s>>>(p);
  return hipGetLastError();
}

// Pipeline depth (32-key steps in flight per wave while one is computed): 1 by
// default (the registers of a step drain to LDS as it begins), 2..3 selectable
// at head_dim 128; head_dim 256 runs one step in flight.
template <int GP>
static hipError_t launch_gp(const AttnParams& p, hipStream_t s) {
  if (p.head_dim == 256) return p.step_variant <= 1 ? launch_variant<GP, 1, 256>(p, s) : hipErrorInvalidValue;
  if (p.head_dim != 128) return hipErrorInvalidValue;
  switch (p.step_variant) {
    case 0: return launch_variant<GP, 1, 128>(p, s);
    case 1: return launch_variant<GP, 1, 128>(p, s);
    case 2: return launch_variant<GP, 2, 128>(p, s);
    case 3: return launch_variant<GP, 3, 128>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attention(const AttnParams& p, int gpad, hipStream_t s) {
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
