/*
 * decode_attn.h -- C ABI of the MI355X (gfx950) decode-attention library.
 *
 * One grouped-query decode-attention step followed by the output projection,
 * as in "PyPTO 开箱性能调优实战：Decode Attention 多 Matmul 独立 TileShape
 * 配置 F-16" (section 代码对比; shapes in the table of section 三个 Matmul 的
 * Shape 特征分析):
 *
 *   scores[g, j] = (q[b, h*G+g, :] . K[b, h, j, :]) * softmax_scale   fp32
 *   p[g, :]      = softmax over j < seq_lens[b] of scores[g, :]
 *   o[b, h*G+g]  = sum_j p[g, j] * V[b, h, j, :]                      -> bf16
 *   out[b, :]    = flat(o)[b, :] @ o_weight                            -> bf16
 *
 * with G = num_q_heads / num_kv_heads, flat(o) head-major (column qh*D + d)
 * and o_weight [num_q_heads*head_dim, hidden] row-major (no transpose).
 *
 * Conventions shared by every entry point:
 *  - Pointers named *_dev are device pointers (hipMalloc or equivalent). The
 *    caller owns every buffer; the library never allocates or frees memory
 *    and keeps no pointer after it returns.
 *  - 16-bit tensors are raw bf16 (or fp16 where stated) words, densely packed
 *    in the row-major layout given, every base address 16-byte aligned.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is only enqueued; the outputs are valid once the stream has
 *    reached that point. Nothing blocks the host.
 *  - Every argument check happens before any HIP call, so a non-zero status
 *    means nothing was enqueued (except DA_ERR_LAUNCH, reported after a
 *    launch failed).
 *  - Calls that share a workspace must be ordered (same stream or
 *    synchronised); calls with distinct workspaces may run concurrently.
 */
#ifndef DECODE_ATTN_H
#define DECODE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------- */
#define DA_OK 0
#define DA_ERR_NULL (-1)      /* a required pointer is NULL                          */
#define DA_ERR_SHAPE (-2)     /* unsupported or inconsistent sizes                    */
#define DA_ERR_ALIGN (-3)     /* a base address is not 16-byte aligned                */
#define DA_ERR_WORKSPACE (-4) /* workspace missing or smaller than required          */
#define DA_ERR_LAUNCH (-5)    /* a kernel launch failed (hipGetLastError after it)   */
#define DA_ERR_TIMEOUT (-6)   /* decode_attn_step_status: a single-launch step stopped
                                 waiting for its attention pieces (see there)        */

/* head_dim: 128 (every path) or DA_HEAD_DIM_WIDE (stream-K attention and the
 * separate projection; the single-launch step is built for 128 only). */
#define DA_HEAD_DIM 128
#define DA_HEAD_DIM_WIDE 256
/* Largest query-head group (num_q_heads / num_kv_heads). */
#define DA_MAX_GROUP 16

/* flags */
#define DA_FLAG_DEBUG_SCORES 1u /* also write debug_scores / debug_lse (test use) */
#define DA_FLAG_SEPARATE 2u     /* decode_attn_fwd: attention and projection as two
                                   launches even where the plan would fuse them */

/*
 * Optional override of the tile choice for one call, for measured tile
 * searches (the per-matmul sweep of the F-16 page, section 迭代过程). A zero
 * field keeps the built-in choice; a value outside its range makes the call
 * return DA_ERR_SHAPE.
 *
 *  attn_workgroups  stream-K attention workgroups, 1..1024 (capped at the
 *                   number of 32-key blocks of the longest possible step); in
 *                   the single-launch step, the attention workgroups aimed at
 *                   (every sequence is cut into the same number of pieces)
 *  attn_depth       32-key steps each attention wave has in flight while it
 *                   computes one, 1..3 (1 only at head_dim 256)
 *  proj_tile_n      output columns per projection workgroup: 64, 128, 256 or
 *                   512. 128 is the MFMA GEMM's tile (the built-in projection
 *                   of the two-launch step at every batch); 64, 256 and 512
 *                   select the VALU GEMV instead, for B < 16 only, with
 *                   tile_n * B <= 2048 after B is rounded up to a power of two.
 *                   The single-launch step takes 128, 256 or 512 for its own
 *                   projection and falls back to two launches if the shape
 *                   does not fit that tile
 *  proj_ksplit      K-chunks the projection is cut into, >= 1 (rounded so that
 *                   every chunk is a whole number of the kernel's row batches)
 *  step_mode        0 built-in, 1 one launch where the single-launch step
 *                   supports the shape (never the tiny one), 2 two launches
 *                   (as DA_FLAG_SEPARATE), 3 the large single-launch step where
 *                   it supports the shape (never the small one), 4 the tiny
 *                   step where it supports the shape
 *  step_wait_polls  bound of the single-launch steps' waits, in polls of a
 *                   counter, 1..2^24 (built-in 2^20, a fraction of a second);
 *                   a workgroup that reaches it gives up (decode_attn_step_status)
 *  attn_seq_cost    stream-K attention: 32-key blocks of work a workgroup is
 *                   charged for each sequence it starts, 1..256 (built-in 6),
 *                   so that workgroups whose range crosses sequence boundaries
 *                   get fewer keys
 *  step_weight_delay small single-launch step: time between a projection
 *                   workgroup's start and its weight requests, in 10 ns ticks,
 *                   0..1000 (built-in 0), so that the attention's K/V requests
 *                   are served ahead of the weight
 */
typedef struct {
  int32_t attn_workgroups;
  int32_t attn_depth;
  int32_t proj_tile_n;
  int32_t proj_ksplit;
  int32_t step_mode;
  int32_t step_wait_polls;
  int32_t attn_seq_cost;
  int32_t step_weight_delay;
} decode_attn_tiles_t;

/*
 * Shape and per-call options of one decode step. All sizes in elements.
 *
 *  batch          B >= 1
 *  num_q_heads    Hq >= 1, a multiple of num_kv_heads, Hq/Hkv <= DA_MAX_GROUP
 *  num_kv_heads   Hkv >= 1
 *  head_dim       D: DA_HEAD_DIM (128) or DA_HEAD_DIM_WIDE (256)
 *  max_seq_len    Lmax >= 1: rows per (batch, kv head) in the K/V caches
 *  hidden         N >= 1, output features of the projection (its K is Hq*D);
 *                 unused by decode_attn_only
 *  softmax_scale  multiplier of q.k; 0 selects 1/sqrt(head_dim)
 *  workspace      device scratch of at least decode_attn_workspace_size()
 *                 bytes, 256-byte aligned. It must be zero-filled before its
 *                 first use; every completed call leaves it ready for the
 *                 next one (its counters return to zero).
 *  workspace_bytes size of that buffer
 *  flags          DA_FLAG_* bits
 *  debug_scores   with DA_FLAG_DEBUG_SCORES: device fp32 [B, Hq, Lmax]; entry
 *                 [b, qh, j] receives the scaled score of key j for j <
 *                 seq_lens[b]; other entries are left untouched
 *  debug_lse      with DA_FLAG_DEBUG_SCORES: device fp32 [B, Hq], natural log
 *                 of sum_j exp(score_j)
 *  tiles          host pointer to a tile override, or NULL for the built-in
 *                 choice (the measured tile table's row for this exact shape
 *                 if it has one, else the built-in rules); read during the
 *                 call only. The workspace size depends on it.
 */
typedef struct {
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t max_seq_len;
  int32_t hidden;
  float softmax_scale;
  void* workspace;
  size_t workspace_bytes;
  uint32_t flags;
  float* debug_scores;
  float* debug_lse;
  const decode_attn_tiles_t* tiles;
} decode_attn_shape_t;

/*
 * Tiles chosen for one shape: one entry per matmul of the step, each sized to
 * its own M/K/N rather than one shared setting (the per-matmul tile lesson of
 * the F-16 page, sections 核心原则 and 迭代过程). Filled by decode_attn_plan.
 */
typedef struct {
  int32_t m, k, n;     /* the matmul's own M, K, N (per kv head / per step)           */
  int32_t tile_m;      /* rows of M one wave holds (a 16-row MFMA operand, G valid)  */
  int32_t tile_k;      /* K extent staged per step                                    */
  int32_t tile_n;      /* N extent one workgroup owns                                 */
  int32_t split;       /* number of independent slices along the reduced axis        */
  int32_t workgroups;  /* workgroups launched for this matmul                          */
} decode_attn_matmul_plan_t;

typedef struct {
  decode_attn_matmul_plan_t qk;     /* q_grouped x k_cache^T: M=G, K=D, N=keys       */
  decode_attn_matmul_plan_t pv;     /* attn_weights x v_cache: M=G, K=keys, N=D      */
  decode_attn_matmul_plan_t oproj;  /* attn_output_flat x o_weight: M=B, K=Hq*D, N   */
  int32_t split_len;    /* keys per attention workgroup (flash-decoding split)       */
  int32_t num_splits;   /* ceil(max_seq_len / split_len)                              */
  int32_t oproj_path;   /* 0: VALU GEMV, 1: MFMA GEMM (two-launch projection)        */
  int32_t fused;        /* 1: decode_attn_fwd runs the step as one launch (small
                           steps, B <= 2): projection workgroups stream their weight
                           tile while the attention runs, then wait for it;
                           2: one launch for larger steps (head_dim 128, B <= 32):
                           the stream-K attention workgroups, then the MFMA
                           projection's items, each of which requests its first
                           weight rows and waits for the kv heads of its K-chunk;
                           3: one launch for tiny steps (head_dim 128, B <= 2,
                           Hq*128 <= 2048, at most 256 KiB of K and V): every
                           workgroup computes the whole attention itself and 16
                           output columns over all of K; no workspace is used;
                           0: two launches                                         */
  size_t workspace_bytes;
} decode_attn_plan_t;

/* Bytes of workspace decode_attn_fwd / decode_attn_only need for `shape`
 * (workspace fields ignored); 0 if the shape is invalid. */
size_t decode_attn_workspace_size(const decode_attn_shape_t* shape);

/* Host-only: fill `plan` with the tile choice for `shape`. No HIP call. */
int decode_attn_plan(const decode_attn_shape_t* shape, decode_attn_plan_t* plan);

/*
 * The whole step.
 *  q_dev         bf16 [B, Hq, D]
 *  k_cache_dev   bf16 [B, Hkv, Lmax, D]   (rows >= seq_lens[b] are never read)
 *  v_cache_dev   bf16 [B, Hkv, Lmax, D]
 *  seq_lens_dev  int32 [B], each in [1, Lmax] (precondition, not checked on
 *                the device; a value outside it gives undefined results)
 *  o_weight_dev  bf16 [Hq*D, hidden]
 *  out_dev       bf16 [B, hidden]
 * Returns DA_OK or a DA_ERR_* code.
 */
int decode_attn_fwd(const void* q_dev, const void* k_cache_dev, const void* v_cache_dev,
                    const int32_t* seq_lens_dev, const void* o_weight_dev, void* out_dev,
                    const decode_attn_shape_t* shape, void* stream);

/*
 * Status of the single-launch steps run on a workspace since its counter block
 * was last zero-filled. In that launch (decode_attn_plan's `fused`), the
 * projection workgroups wait for the attention pieces of their kv heads, and
 * each wait is bounded (decode_attn_tiles_t.step_wait_polls). One that gives up
 * sets an error word in the workspace's counter block, writes NaN to its
 * output columns and leaves the counters dirty. This call waits for `stream`
 * (a hipStream_t as void*, NULL = the default stream) to drain, reads that word
 * and returns:
 *   DA_OK           no wait gave up;
 *   DA_ERR_TIMEOUT  some wait gave up: the outputs of those calls are invalid
 *                   (NaN), and the first 64 KiB of the workspace must be
 *                   zero-filled again before its next use;
 *   DA_ERR_WORKSPACE (under 64 KiB) or DA_ERR_ALIGN (not 256-byte aligned)
 *                   before any HIP call, or DA_ERR_LAUNCH if the copy or the
 *                   synchronisation fails.
 * A NULL workspace names the scratch array of decode_attn_fwd_noalloc on the
 * current device; after a timeout there, this call zero-fills its counters.
 * It blocks the host, so it cannot be captured into a graph. Two-launch steps
 * never wait and never set the word.
 */
int decode_attn_step_status(const void* workspace, size_t workspace_bytes, void* stream);

/*
 * decode_attn_fwd for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same step, whose workspace is the library's own scratch array of
 * DA_NOALLOC_SCRATCH_BYTES per device instead of shape->workspace (the
 * workspace fields are ignored). It calls no allocating routine; the first
 * call on a device looks up that device's array and enqueues a zero fill of
 * its counters on `stream`. Arguments, layouts and checks are those of
 * decode_attn_fwd, plus DA_ERR_WORKSPACE (before any HIP call) when the shape
 * needs more scratch than the array holds. Every call on one device shares
 * that array and leaves it ready for the next one, so calls that overlap on
 * one device (different streams, no ordering between them) race and give
 * wrong results. decode_attn_step_status(NULL, 0, stream) reports this
 * path's single-launch timeouts and then zero-fills the array's counters.
 */
#define DA_NOALLOC_SCRATCH_BYTES (16u << 20)
int decode_attn_fwd_noalloc(const void* q_dev, const void* k_cache_dev, const void* v_cache_dev,
                            const int32_t* seq_lens_dev, const void* o_weight_dev, void* out_dev,
                            const decode_attn_shape_t* shape, void* stream);

/* The first two matmuls and the softmax only: attn_out_dev receives the
 * bf16 [B, Hq*D] head-major attention output (attn_output_flat). */
int decode_attn_only(const void* q_dev, const void* k_cache_dev, const void* v_cache_dev,
                     const int32_t* seq_lens_dev, void* attn_out_dev, const decode_attn_shape_t* shape,
                     void* stream);

/* Bytes of workspace oproj_fwd needs for an [M,K] x [K,N] product. */
size_t oproj_workspace_size(int32_t M, int32_t K, int32_t N);

/*
 * The output projection alone (the third matmul of the F-16 page):
 * out[M,N] = x[M,K] @ w[K,N]; bf16 in, fp32 accumulation, bf16 out (round to
 * nearest even). It runs an MFMA GEMM (K a multiple of 32 for every M) or,
 * for M < 16 with K a multiple of 8 only, a VALU GEMV. `workspace`
 * (>= oproj_workspace_size bytes, zero-filled before first use, may be NULL
 * when that size is 0) holds split-K partial sums and counters.
 */
int oproj_fwd(const void* x_dev, const void* w_dev, void* out_dev, int32_t M, int32_t K, int32_t N,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Dense GEMM of the CANN msKPP BasicMatmul example ("自动调优流程 / Kernel级
 * 自动调优"): C[M,N] = A[M,K] @ B[K,N], all fp16 row-major, fp32 accumulation,
 * fp16 out (round to nearest even). M, N multiples of 16; K a multiple of 32;
 * K * N * 2 < 4 GiB (DA_ERR_SHAPE otherwise).
 */
int gemm_f16(const void* a_dev, const void* b_dev, void* c_dev, int32_t M, int32_t N, int32_t K, void* stream);

/*
 * Context (prefill) attention of a chunk of new tokens. The page "CCCL →
 * Triton 方法论迁移" (section 二, 2.1 prefix_prefill.py) names this context
 * attention beside the decode attention and gives only its tile knobs; read
 * plainly: sequence b holds ctx_lens[b] cached keys, the last num_tokens of
 * which are the chunk's own tokens (already written to the caches), and token t
 * attends causally to keys 0 .. ctx_lens[b] - num_tokens + t with the decode
 * step's scaled softmax (num_tokens = 1 is decode_attn_only).
 *
 *  q_dev         bf16 [B, T, Hq, D] (T = num_tokens, token-major)
 *  k_cache_dev   bf16 [B, Hkv, Lmax, D]
 *  v_cache_dev   bf16 [B, Hkv, Lmax, D]
 *  ctx_lens_dev  int32 [B], each in [T, Lmax] (precondition, not checked on the
 *                device: the kernel clamps it to [0, Lmax] and reads no cache
 *                row at or past it, but a token left with no key gets an
 *                unspecified output)
 *  out_dev       bf16 [B, T, Hq*D], head-major within a token as in decode
 * head_dim 128 only, Hq a multiple of Hkv with Hq/Hkv <= DA_MAX_GROUP,
 * 1 <= T <= Lmax, Lmax*D*2 < 4 GiB; softmax_scale 0 selects 1/sqrt(head_dim).
 * Tensors: 16-byte aligned device pointers (ctx_lens 4-byte), owned by the
 * caller; the library allocates nothing, needs no workspace and keeps no
 * pointer after the call. The work is enqueued on `stream` (a hipStream_t,
 * NULL = the default stream); outputs are valid once the caller synchronises.
 * Returns DA_OK, DA_ERR_NULL, DA_ERR_ALIGN or DA_ERR_SHAPE before any HIP
 * call, or DA_ERR_LAUNCH if the launch fails.
 */
typedef struct {
  int32_t batch;
  int32_t num_tokens;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t max_seq_len;
  float softmax_scale;
} prefill_attn_shape_t;

int prefill_attn_fwd(const void* q_dev, const void* k_cache_dev, const void* v_cache_dev,
                     const int32_t* ctx_lens_dev, void* out_dev, const prefill_attn_shape_t* shape,
                     void* stream);

/*
 * Measurement aid, not part of the step: a plain streaming read of `bytes`
 * (a multiple of 16) from src_dev by `workgroups` 256-thread workgroups, each
 * reading its contiguous share in 1 KiB blocks (the attention's K/V load
 * pattern); sink_dev receives one uint32 per workgroup. Timing it on a decode
 * step's algorithmic bytes gives the floor a step of that size is compared
 * with, as the profiler-backed verification of the MT-S page (section 5,
 * 性能验证) asks. Returns DA_ERR_NULL / DA_ERR_ALIGN / DA_ERR_SHAPE before any
 * HIP call, DA_ERR_LAUNCH if the launch fails; work is enqueued on `stream`.
 */
int decode_attn_read_probe(const void* src_dev, size_t bytes, uint32_t* sink_dev, int32_t workgroups, void* stream);

/* Static text for a status code. */
const char* decode_attn_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* DECODE_ATTN_H */
