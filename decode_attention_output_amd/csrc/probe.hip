// A plain streaming read, used to measure what the memory system delivers for
// a given number of bytes: the floor that a decode step of the same size is
// compared against (the profiler-backed verification the MT-S page asks for in
// section 5, 性能验证).
//
// Workgroup w of W reads its contiguous 1/W share in 1 KiB blocks -- 64 lanes
// x 16 bytes per load instruction, the pattern the attention kernels stream
// K/V rows with -- eight loads in flight per lane, folds the words with xor and
// writes one word to sink[w] so that no load is dead.
#include "attn_core.hpp"
#include "kernels.hpp"

namespace da {

namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 8;

__global__ __launch_bounds__(kThreads) void read_probe_kernel(const uint4* src, uint64_t n16, uint32_t* sink) {
  const uint64_t W = gridDim.x, w = blockIdx.x;
  const uint64_t b0 = (n16 * w / W) & ~(uint64_t)63, b1 = w + 1 == W ? n16 : (n16 * (w + 1) / W) & ~(uint64_t)63;
  uint32_t acc = 0;
  for (uint64_t base = b0 + threadIdx.x; base < b1; base += (uint64_t)kThreads * kInFlight) {
    uint4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const uint64_t i = base + (uint64_t)u * kThreads;
      v[u] = i < b1 ? src[i] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // fold the wave, then one word per workgroup
  for (int x = 1; x < kWave; x <<= 1) acc ^= __shfl_xor(acc, x);
  __shared__ uint32_t s_acc[kThreads / kWave];
  if ((threadIdx.x & (kWave - 1)) == 0) s_acc[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0;
    for (int i = 0; i < kThreads / kWave; ++i) a ^= s_acc[i];
    sink[w] = a;
  }
}

}  // namespace

hipError_t launch_read_probe(const void* src, uint64_t bytes, uint32_t* sink, int workgroups, hipStream_t s) {
  read_probe_kernel<<<dim3(workgroups), dim3(kThreads), 0, s>>>((const uint4*)src, bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace da
