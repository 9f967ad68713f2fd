// gfx950 (MI355X, CDNA4) target constants and device helpers shared by the
// kernels of this library. Nothing here is specific to one kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace da {

// ---- target facts (checked against hipGetDeviceProperties in the tests) ----
constexpr int kWave = 64;              // wavefront width
constexpr int kHeadDim = 128;          // head_dim of the single-launch step and the context attention

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ---- 16-bit float words ----------------------------------------------------

// bf16 is the top half of a binary32 word: widening is a shift.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// binary32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN;
// values beyond the largest bf16 become infinity.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Unpack 8 bf16 (one 16-byte load) into fp32.
__device__ __forceinline__ void unpack_bf16x8(const uint4& v, float* f) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// ---- MFMA 16x16x32 (bf16 / fp16 in, fp32 accumulate) ------------------------
//
// Lane layout (verified on the device): lane l supplies A[row l%16][k (l/16)*8
// .. +8] and B[k (l/16)*8 .. +8][col l%16]; it receives C[row (l/16)*4 + r]
// [col l%16] in element r of the f32x4 result.
__device__ __forceinline__ f32x4_t mfma_bf16(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_f16(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                0, 0, 0);
}

// A value that is the same in every lane, moved to a scalar register.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Orders LDS traffic of one wavefront (a compiler barrier; LDS requests of a
// wave are served in issue order).
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---- cross-workgroup communication inside one kernel ----------------------
//
// The eight XCDs of an MI355X each have their own L2, which is not coherent
// with the others for ordinary stores. Data handed from one workgroup to
// another therefore goes through device-scope (sc1) stores and loads, which
// are made coherent at device level, instead of ordinary stores followed by a
// device-wide fence (that fence writes back and invalidates the whole L2).
// Wait until every store this thread issued has been acknowledged.
__device__ __forceinline__ void wait_stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Arrival counter of a group of `expected` workgroups: returns true (in every
// thread) in the one workgroup that arrives last, after each workgroup's
// coherent stores are complete. The last workgroup resets the counter, so it
// is zero again for the next use.
__device__ __forceinline__ bool arrive_last_coherent(uint32_t* counter, uint32_t expected) {
  __shared__ uint32_t s_last;
  wait_stores_done();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t last = (prev == expected - 1) ? 1u : 0u;
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last;
  }
  __syncthreads();
  const bool last = s_last != 0;
  asm volatile("" ::: "memory");
  return last;
}

// 16-byte global load.
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

}  // namespace da
