// Kernel parameter blocks and host launchers (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

// Timeline hook: thread 0 of a workgroup may record a timestamp at numbered
// points of the kernels. It expands to nothing unless a build defines it.
#ifndef DA_TRACE
#define DA_TRACE(point) ((void)0)
#endif

namespace da {

// Every workspace starts with a block of arrival counters that are zero
// between calls; the scratch data of a call follows it.
constexpr size_t kCounterBlockBytes = 65536;
constexpr int kMaxCounters = (int)(kCounterBlockBytes / sizeof(uint32_t));

constexpr int kMaxAttnBatch = 1024;  // batch limit of the attention kernels
constexpr int kAttnWaves = 4;        // wavefronts per stream-K attention workgroup

// Stream-K attention over all (batch, kv head) sequences of one step.
struct AttnParams {
  const uint16_t* q;        // bf16 [B, Hq, D]
  const uint16_t* k;        // bf16 [B, Hkv, Lmax, D]
  const uint16_t* v;        // bf16 [B, Hkv, Lmax, D]
  const int32_t* seq_lens;  // [B]
  uint16_t* flat;           // bf16 [B, Hq*D] head-major attention output
  float* part_o;            // fp32 [slots, G, D] un-normalised partial outputs
  float* part_ml;           // fp32 [slots, G, 2]   (max in log2 units, weight sum)
  uint32_t part_o_bytes, part_ml_bytes;
  uint32_t* counters;       // [B * Hkv] arrival counters, zero between calls
  uint32_t* head_ready;     // single-launch large step: finished sequences per kv head (kStepReplicas copies)
  float* dbg_scores;        // optional fp32 [B, Hq, Lmax]
  float* dbg_lse;           // optional fp32 [B, Hq]
  int B, Hq, Hkv, G, Lmax;
  int head_dim;             // 128 or 256
  int num_workgroups;       // stream-K workgroups; slots = num_workgroups + B * Hkv
  int step_variant;         // 32-key steps in flight per wave: 0 = default (1), else 1..3
  int seq_cost;             // virtual 32-key blocks a workgroup is charged for starting a sequence
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

// C[M, N] = A[M, K] @ B[K, N] on MFMA, a (16 * mtiles) x 128 output tile per
// workgroup; K and kchunk are multiples of 32, N of 8.
struct GemmParams {
  const uint16_t* a;  // [M, K]
  const uint16_t* b;  // [K, N]
  uint16_t* c;        // [M, N]
  float* part;        // fp32 [ksplit, M, N] (ksplit > 1)
  uint32_t part_bytes;
  uint32_t* counters; // [ceil(M / (16 * mtiles)) * ceil(N / 128)] arrival counters (ksplit > 1)
  int M, K, N;
  int kchunk, ksplit;
  int mtiles;         // 16-row m-tiles per workgroup: 1, 2 or 4
};
constexpr int kGemmTileN = 128;   // output columns per GEMM workgroup
constexpr int kGemmDepth = 2;     // 32-row steps per wave in flight while one is multiplied
constexpr int kGemmDepthWait = 4;  // the same in the single-launch large step, whose items request
                                   // that many steps before they wait for the attention

hipError_t launch_attention(const AttnParams& p, int gpad, hipStream_t s);
// The single-launch decode step for small steps (a few tokens, a few
// thousand cached keys): attention workgroups, one per fixed piece of every
// (batch, kv head) sequence, followed in the same grid by projection
// workgroups that wait for the pieces of the kv heads they need, merge them
// and multiply.
// Counters of the single-launch steps that many workgroups poll or update sit
// one per 128-byte line (accesses to one line are serialised), and every kv
// head's ready counter is kept kStepReplicas times, so that each copy has only
// a few pollers: ready[(head * kStepReplicas + copy) * kCounterStride].
constexpr int kCounterStride = 32;
constexpr int kStepReplicas = 4;

// Fixed slots of the counter block used by the single-launch step.
constexpr int kStepCounterBase = kMaxCounters - 64;  // pass_top, error, then pass_sub[32] at +32
constexpr int kStepErrorWord = kStepCounterBase + 1;  // the error word, read back by decode_attn_step_status
constexpr uint32_t kStepWaitPolls = 1u << 20;         // default bound of a projection workgroup's wait

// Hand-over from the attention to the projection workgroups of a
// single-launch step (step_sync.hpp): per-kv-head ready counters, kept
// kStepReplicas times one per line, and the count of workgroups past their wait.
struct ReadySync {
  uint32_t* ready;      // [heads * kStepReplicas] copies, kCounterStride words apart
  uint32_t* pass_sub;   // [32] workgroups past their wait, by index mod 32
  uint32_t* pass_top;   // groups of pass_sub that are complete
  uint32_t* error;      // set to 1 when a wait gave up
  int heads;            // kv heads
  uint32_t target;      // a head is ready when its counter reaches this
  uint32_t wait_polls;  // polls of one counter before giving up (>= 1)
  int waiters;          // workgroups that wait
};

// What a GEMM item of the single-launch large step waits for: the ready
// counters of the kv heads whose query heads (head_dim rows of K each, `group`
// query heads per kv head) make up its K-chunk; `waiter` is its index among the
// waiting workgroups.
struct GemmWait {
  ReadySync sync;
  int head_dim, group;
  int waiter;
};

constexpr int kXcds = 8;  // XCDs of an MI355X; workgroup i of a launch runs on XCD i % kXcds

struct StepParams {
  const uint16_t* q;        // bf16 [B, Hq, 128]
  const uint16_t* k;        // bf16 [B, Hkv, Lmax, 128]
  const uint16_t* v;        // bf16 [B, Hkv, Lmax, 128]
  const int32_t* seq_lens;  // [B]
  const uint16_t* w;        // bf16 [Hq*128, N]
  uint16_t* out;            // bf16 [B, N]
  float* part_o;            // fp32 [B*Hkv*pieces, G, 128] un-normalised piece outputs
  float* part_ml;           // fp32 [B*Hkv*pieces, G, 2]   (max in log2 units, weight sum)
  float* proj_part;         // fp32 [chunks, B, N] (chunks > 1)
  uint32_t part_o_bytes, part_ml_bytes, proj_part_bytes;
  uint32_t* proj_cnt;       // arrival counters of the K-chunks per column tile (chunks > 1), one per line
  ReadySync sync;           // stored pieces per kv head, the projection's wait and its pass count
  int B, Hq, Hkv, G, Lmax, N;
  int piece_keys, pieces;   // keys per piece (a multiple of 128), pieces per sequence
  int attn_wgs;             // B * Hkv * pieces
  int tiles, chunks;        // projection: column tiles x K-chunks (whole query heads)
  uint32_t weight_delay;    // 100 MHz ticks between a projection workgroup's start and its weight requests
  float scale_log2;         // softmax scale * log2(e)
};

// The single-launch step for tiny steps: every workgroup computes the whole
// attention itself (its K/V are a few hundred KiB at most) and then kTinyCols
// output columns of the projection over all of K; no workspace, no hand-over.
struct StepTinyParams {
  const uint16_t* q;        // bf16 [B, Hq, 128]
  const uint16_t* k;        // bf16 [B, Hkv, Lmax, 128]
  const uint16_t* v;        // bf16 [B, Hkv, Lmax, 128]
  const int32_t* seq_lens;  // [B]
  const uint16_t* w;        // bf16 [Hq*128, N]
  uint16_t* out;            // bf16 [B, N]
  int B, Hq, Hkv, G, Lmax, N;
  float scale_log2;         // softmax scale * log2(e)
  int xcds, per_xcd;        // set by the launch: column tiles on the first xcds XCDs, per_xcd each
};
constexpr int kTinyCols = 16;                    // output columns per workgroup
constexpr int kTinyMaxK = 2048;                  // Hq * 128 at most
constexpr int kTinyMaxBatch = 2;
constexpr size_t kTinyMaxKvBytes = 256u << 10;   // K and V bytes of the whole step at most
hipError_t launch_decode_step_tiny(const StepTinyParams& p, int gpad, hipStream_t s);

// The single-launch large step: stream-K attention workgroups, then one
// workgroup per MFMA GEMM item (ntiles column tiles x mgroups row groups x
// gemm.ksplit K-chunks, K-chunk major).
struct StepLargeParams {
  AttnParams attn;
  GemmParams gemm;
  GemmWait wait;
  int ntiles, mgroups;
};
hipError_t launch_decode_step_large(const StepLargeParams& p, int gpad, hipStream_t s);

// Shapes the single-launch step is built for: query group (padded), batch rows
// (padded) and tile_n output columns per projection workgroup, whose K-chunk
// is then 32 rows per lane: 16384 / tile_n rows.
bool decode_step_supported(int gpad, int mpad, int tile_n);
int decode_step_chunk(int tile_n);
hipError_t launch_decode_step(const StepParams& p, int gpad, int mpad, int tile_n, hipStream_t s);

// Context (prefill) attention of a chunk of T tokens per sequence, head_dim 128.
struct PrefillParams {
  const uint16_t* q;        // bf16 [B, T, Hq, 128]
  const uint16_t* k;        // bf16 [B, Hkv, Lmax, 128]
  const uint16_t* v;        // bf16 [B, Hkv, Lmax, 128]
  const int32_t* ctx_lens;  // [B] keys per sequence, the chunk being the last T
  uint16_t* out;            // bf16 [B, T, Hq*128]
  int B, T, Hq, Hkv, G, Lmax;
  float scale_log2;         // softmax scale * log2(e)
};
hipError_t launch_prefill(const PrefillParams& p, hipStream_t s);

// A plain streaming read of `bytes` (a multiple of 16) by `workgroups` workgroups; one word per workgroup to sink.
hipError_t launch_read_probe(const void* src, uint64_t bytes, uint32_t* sink, int workgroups, hipStream_t s);

hipError_t launch_gemv(const GemvParams& p, int mpad, hipStream_t s);
hipError_t launch_gemm_bf16(const GemmParams& p, hipStream_t s);
hipError_t launch_gemm_f16(const GemmParams& p, hipStream_t s);
// 16 x 32 output tiles over all of K, 512 threads (no workspace): for products whose 128-column tiles
// would not fill the chip; M and N multiples of 16, K a multiple of 32.
hipError_t launch_gemm_narrow_f16(const GemmParams& p, hipStream_t s);
constexpr int kGemmNarrowBelow = 256;  // 128-column tiles below which the narrow tiles are used

}  // namespace da
