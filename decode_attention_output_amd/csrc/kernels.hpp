// Kernel parameter blocks and host launchers (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace da {

// Every workspace starts with a block of arrival counters that are zero
// between calls; the scratch data of a call follows it.
constexpr size_t kCounterBlockBytes = 65536;
constexpr int kMaxCounters = (int)(kCounterBlockBytes / sizeof(uint32_t));

constexpr int kMaxAttnBatch = 1024;  // batch limit of the attention kernels
constexpr int kAttnWaves = 4;        // wavefronts per stream-K attention workgroup

// Stream-K attention over all (batch, kv head) sequences of one step.
struct AttnParams {
  const uint16_t* q;        // bf16 [B, Hq, 128]
  const uint16_t* k;        // bf16 [B, Hkv, Lmax, 128]
  const uint16_t* v;        // bf16 [B, Hkv, Lmax, 128]
  const int32_t* seq_lens;  // [B]
  uint16_t* flat;           // bf16 [B, Hq*128] head-major attention output
  float* part_o;            // fp32 [slots, G, 128] un-normalised partial outputs
  float* part_ml;           // fp32 [slots, G, 2]   (max in log2 units, weight sum)
  uint32_t part_o_bytes, part_ml_bytes;
  uint32_t* counters;       // [B * Hkv] arrival counters, zero between calls
  float* dbg_scores;        // optional fp32 [B, Hq, Lmax]
  float* dbg_lse;           // optional fp32 [B, Hq]
  int B, Hq, Hkv, G, Lmax;
  int num_workgroups;       // stream-K workgroups; slots = num_workgroups + B * Hkv
  float scale;       // softmax scale (natural units)
  float scale_log2;  // scale * log2(e)
};

// out[M, N] = x[M, K] @ w[K, N], M < 16, on the vector ALUs, split over K.
struct GemvParams {
  const uint16_t* x;  // bf16 [M, K]
  const uint16_t* w;  // bf16 [K, N]
  uint16_t* out;      // bf16 [M, N]
  float* part;        // fp32 [ksplit, M, N] (ksplit > 1)
  uint32_t part_bytes;
  uint32_t* counters; // [ceil(N / 64)] arrival counters (ksplit > 1)
  int M, K, N;
  int kchunk, ksplit;
  int tile_n;         // output columns per workgroup (64)
};

// C[M, N] = A[M, K] @ B[K, N] on MFMA, 16 x 64 output tile per workgroup.
struct GemmParams {
  const uint16_t* a;  // [M, K]
  const uint16_t* b;  // [K, N]
  uint16_t* c;        // [M, N]
  float* part;        // fp32 [ksplit, M, N] (ksplit > 1)
  uint32_t part_bytes;
  uint32_t* counters; // [ceil(M/16) * N/64] arrival counters (ksplit > 1)
  int M, K, N;
  int kchunk, ksplit;
};

hipError_t launch_attention(const AttnParams& p, int gpad, hipStream_t s);
hipError_t launch_gemv(const GemvParams& p, int mpad, hipStream_t s);
hipError_t launch_gemm_bf16(const GemmParams& p, hipStream_t s);
hipError_t launch_gemm_f16(const GemmParams& p, hipStream_t s);

}  // namespace da
