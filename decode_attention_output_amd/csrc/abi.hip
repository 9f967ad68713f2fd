// C ABI of the library: argument checks, per-matmul tile selection, workspace
// layout and the launch sequence of one decode step.
//
// Tile selection follows the per-matmul lesson of "PyPTO 开箱性能调优实战：
// Decode Attention 多 Matmul 独立 TileShape 配置 F-16" (sections 核心原则 and
// 迭代过程): every matmul of the step gets a tile sized to its own M/K/N --
// a tiny M (the query group, the batch) is never padded past one 16-row
// operand, a short axis (head_dim 128) is not split, and a long axis (the
// keys, the projection's K and N) is cut into many large slices so that the
// 256 compute units each receive several workgroups.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/decode_attn.h"
#include "gfx950.hpp"
#include "kernels.hpp"

namespace {

using da::kHeadDim;

// Stream-K attention workgroups: 176 (22 per XCD), about two thirds of the
// compute units. Chosen by the geometric mean of the step time over the
// ragged 16-sequence, 4 x 32768-key and head_dim 256 steps and one-GPU shares
// of them (112..256 tried): the projection workgroups of the single-launch
// step then find free compute units to start their weight stream early, which
// gains 2-4 % over 192 on the long steps; 128 and fewer leave HBM idle.
constexpr int kAttnWorkgroups = 176;
constexpr int kMaxAttnWorkgroups = 1024;    // largest stream-K grid a tile override may ask for
constexpr int kAttnBlockKeys = 32;          // keys per wave step
// Virtual 32-key blocks a stream-K workgroup is charged for starting a
// sequence (finishing a piece and restarting take about as long as streaming
// this many blocks; measured per workgroup on the ragged 16-sequence batch).
constexpr int kAttnSeqCost = 6;
constexpr int kMaxAttnSeqCost = 256;
constexpr int kTargetProjWorkgroups = 512;   // GEMV: two per compute unit
constexpr int kTargetGemmWorkgroups = 256;   // MFMA GEMM: one per compute unit (measured best of 64..1024)
constexpr int kGemvUnroll = 8;               // weight rows per lane in flight
constexpr int kGemmKStep = 128;
constexpr size_t kAlign = 256;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }
int pow2_at_least(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}
bool misaligned(const void* p, size_t a) { return ((uintptr_t)p % a) != 0; }

// ---- the measured tile table (tile_table.inc, written by autotune.py) ----
struct TileEntry {
  int32_t B, Hq, Hkv, D, Lmax, N;
  decode_attn_tiles_t tiles;
};
constexpr TileEntry kTileTable[] = {
#define TILE_ENTRY(b, hq, hkv, d, lmax, n, w, dp, tn, ks, mode, cost, delay) \
  {b, hq, hkv, d, lmax, n, {w, dp, tn, ks, mode, 0, cost, delay}},
#include "tile_table.inc"
#undef TILE_ENTRY
    {0, 0, 0, 0, 0, 0, {0, 0, 0, 0, 0, 0, 0, 0}},  // end of the table
};

// The shape a call runs with: the caller's, plus the table's tiles for its
// exact shape when the caller brings no override. An attention-only call has
// no projection, so its hidden size is not compared (the row's attention
// tiles apply).
decode_attn_shape_t effective_shape(const decode_attn_shape_t* s, bool with_proj = true) {
  decode_attn_shape_t e = *s;
  if (e.tiles) return e;
  for (const TileEntry& t : kTileTable)
    if (t.B == e.batch && t.Hq == e.num_q_heads && t.Hkv == e.num_kv_heads && t.D == e.head_dim &&
        t.Lmax == e.max_seq_len && (!with_proj || t.N == e.hidden) && t.B > 0) {
      e.tiles = &t.tiles;
      break;
    }
  return e;
}

// Ranges of a tile override (decode_attn_tiles_t); no override is always fine.
bool tiles_ok(const decode_attn_shape_t* s) {
  const decode_attn_tiles_t* t = s->tiles;
  if (!t) return true;
  if (t->attn_workgroups < 0 || t->attn_workgroups > kMaxAttnWorkgroups) return false;
  if (t->attn_depth < 0 || t->attn_depth > 3) return false;
  if (t->proj_ksplit < 0 || t->step_mode < 0 || t->step_mode > 4) return false;
  if (t->step_wait_polls < 0 || t->step_wait_polls > (1 << 24)) return false;
  if (t->attn_seq_cost < 0 || t->attn_seq_cost > kMaxAttnSeqCost) return false;
  if (t->step_weight_delay < 0 || t->step_weight_delay > 1000) return false;
  if (const int tn = t->proj_tile_n) {
    if (tn != 64 && tn != 128 && tn != 256 && tn != 512) return false;
    // 128 is the MFMA GEMM's tile; the other widths ask for the GEMV (batch < 16)
    if (tn != da::kGemmTileN && (s->batch >= 16 || pow2_at_least(s->batch) * tn > 2048)) return false;
  }
  return true;
}

bool shape_ok(const decode_attn_shape_t* s, bool need_hidden) {
  if (s->batch < 1 || s->num_q_heads < 1 || s->num_kv_heads < 1 || s->max_seq_len < 1) return false;
  if (s->head_dim != 128 && s->head_dim != 256) return false;
  if (s->head_dim != 128 && s->tiles && s->tiles->attn_depth > 1) return false;
  if (s->num_q_heads % s->num_kv_heads != 0) return false;
  if (s->num_q_heads / s->num_kv_heads > DA_MAX_GROUP) return false;
  if (need_hidden && (s->hidden < 1 || s->hidden % 8 != 0)) return false;
  if (s->batch > da::kMaxAttnBatch) return false;
  if ((size_t)s->max_seq_len * s->head_dim * 2 >= (1ull << 32)) return false;  // one sequence's K rows < 4 GiB
  // element counts must stay addressable
  const double kv = (double)s->batch * s->num_kv_heads * s->max_seq_len * s->head_dim;
  if (kv > 9.0e15) return false;
  return tiles_ok(s);
}

// ---- projection tiles (shared by decode_attn_fwd and oproj_fwd) ----
struct ProjPlan {
  int path;  // 0 GEMV, 1 MFMA
  int mpad;  // GEMV: rows held per lane (power of two >= M); GEMM: rows per workgroup
  int mtiles;  // GEMM: 16-row m-tiles per workgroup
  int tile_n;  // output columns per workgroup
  int kchunk, ksplit;
  int tiles;  // output tiles (counters)
  size_t part_bytes;
};

// A zero request keeps the built-in choice (tile_n and ksplit come from a
// tile override, already range-checked by tiles_ok).
ProjPlan plan_proj(int M, int K, int N, int tile_n_req = 0, int ksplit_req = 0) {
  ProjPlan pp{};
  // The MFMA GEMM streams the weight in 1 KiB row blocks per load instruction
  // and was measured faster than the GEMV at every batch (1, 2, 4, 8; 2-9 %
  // per step); the GEMV serves a K that is not a multiple of 32 and a tile
  // width only it has (64, 256 or 512 columns, batch < 16).
  const bool gemv = M < 16 && (K % 32 != 0 || (tile_n_req != 0 && tile_n_req != da::kGemmTileN));
  if (gemv) {
    // GEMV: column tiles of up to 256 columns (512 bytes of each weight row
    // per workgroup) and a K-chunk sized so that about kTargetProjWorkgroups
    // workgroups stream the weight; every lane keeps 8 rows in flight.
    pp.path = 0;
    pp.mpad = pow2_at_least(M);
    // widest tile (up to 256 columns) that still leaves 32 column tiles
    int tc = 256;
    while (tc > 64 && (N / tc < 32 || pp.mpad * tc > 2048)) tc /= 2;
    if (tile_n_req) tc = tile_n_req;
    pp.tile_n = tc;
    pp.tiles = ceil_div(N, tc);
    const int gran = (2048 / tc) * kGemvUnroll;  // rows of one batch of the workgroup
    int ksplit = std::max(1, kTargetProjWorkgroups / pp.tiles);
    if (ksplit_req) ksplit = ksplit_req;
    ksplit = std::min(ksplit, std::max(1, ceil_div(K, gran)));
    int kchunk = (int)align_up((size_t)ceil_div(K, ksplit), gran);
    // activations of a chunk + the reduction buffers fit 64 KiB of LDS
    const int max_chunk = (65536 - 4096 - 16 * pp.mpad * tc) / (4 * pp.mpad);
    kchunk = std::min(kchunk, std::max(gran, max_chunk / gran * gran));
    pp.kchunk = kchunk;
    pp.ksplit = ceil_div(K, kchunk);
  } else {
    // MFMA GEMM: 128-column tiles of 16, 32 or 64 activation rows, K-chunks
    // of whole 128-row steps (32 rows per wave)
    pp.path = 1;
    pp.mtiles = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    pp.mpad = 16 * pp.mtiles;
    pp.tile_n = da::kGemmTileN;
    pp.tiles = ceil_div(N, da::kGemmTileN) * ceil_div(M, pp.mpad);
    int ksplit = std::max(1, kTargetGemmWorkgroups / pp.tiles);
    if (ksplit_req) ksplit = ksplit_req;
    ksplit = std::min(ksplit, std::max(1, ceil_div(K, kGemmKStep)));
    pp.kchunk = (int)align_up((size_t)ceil_div(K, ksplit), kGemmKStep);
    pp.ksplit = ceil_div(K, pp.kchunk);
  }
  if (pp.ksplit > 1) pp.part_bytes = align_up((size_t)pp.ksplit * M * N * sizeof(float), kAlign);
  return pp;
}

// The kernels address the K-chunk partials, and a GEMM workgroup its weight
// chunk, with 32-bit offsets.
bool proj_fits(const ProjPlan& pp, int N) {
  if (pp.part_bytes > 0xffffffffull) return false;
  if (pp.path == 1 && (size_t)pp.kchunk * N * 2 > 0xffffffffull) return false;
  return pp.tiles <= da::kMaxCounters;
}

// ---- attention: stream-K over the keys of all sequences ----
struct AttnPlan {
  int gpad;
  int seq_cost;    // virtual blocks charged per sequence start
  int depth;       // 32-key steps in flight per wave while one is computed
  int workgroups;  // stream-K workgroups
  int keys_per_wg; // upper bound of the keys one workgroup streams
  size_t slots;
  size_t part_o_bytes, part_ml_bytes;
};

AttnPlan plan_attn(const decode_attn_shape_t* s) {
  AttnPlan ap{};
  const int G = s->num_q_heads / s->num_kv_heads;
  ap.gpad = pow2_at_least(G);
  const long pairs = (long)s->batch * s->num_kv_heads;
  const long blocks_max = pairs * ceil_div(s->max_seq_len, kAttnBlockKeys);
  // about four blocks (128 keys) per workgroup at least: short problems are
  // latency bound and gain nothing from more, smaller pieces
  ap.workgroups = (int)std::max<long>(1, std::min<long>(kAttnWorkgroups, blocks_max / 4));
  ap.depth = 1;
  ap.seq_cost = kAttnSeqCost;
  if (const decode_attn_tiles_t* t = s->tiles) {
    if (t->attn_workgroups) ap.workgroups = (int)std::max<long>(1, std::min<long>(t->attn_workgroups, blocks_max));
    if (t->attn_depth) ap.depth = t->attn_depth;
    if (t->attn_seq_cost) ap.seq_cost = t->attn_seq_cost;
  }
  ap.keys_per_wg = ceil_div(blocks_max, ap.workgroups) * kAttnBlockKeys;
  ap.slots = (size_t)ap.workgroups + (size_t)pairs;
  ap.part_o_bytes = align_up(ap.slots * G * s->head_dim * sizeof(float), kAlign);
  ap.part_ml_bytes = align_up(ap.slots * G * 2 * sizeof(float), kAlign);
  return ap;
}

// ---- the single-launch step for small steps (decode_step.hip) ----
// Used when the whole step is a few dozen MiB or less: the fixed cost of
// every dependent trip through memory then outweighs the streaming time.
constexpr size_t kStepMaxKvBytes = 64ull << 20;
constexpr size_t kStepMaxWeightBytes = 64ull << 20;
constexpr int kStepMaxBatch = 2;          // projection rows held per lane (four spill registers)
constexpr int kStepResident = 512;        // workgroups resident at once: two 256-thread ones per CU
constexpr int kStepAttnTarget = 192;      // attention workgroups aimed at (5 % faster than 128 on two
                                          // ragged sequences of 8 kv heads; shorter steps have fewer pieces)
constexpr int kStepMaxAttn = 384;         // at most, leaving room for the projection
constexpr int kPieceGrain = 128;          // keys of a piece: a multiple of 4 waves x 32 keys
struct StepPlan {
  bool ok;
  int gpad, mpad;
  int pieces, piece_keys, attn_wgs;
  int tile_n, chunk, tiles, chunks;
  size_t part_o_bytes, part_ml_bytes, proj_part_bytes;
};

StepPlan plan_step(const decode_attn_shape_t* s) {
  StepPlan sp{};
  const int B = s->batch, Hkv = s->num_kv_heads, G = s->num_q_heads / s->num_kv_heads;
  const int K = s->num_q_heads * kHeadDim, N = s->hidden;
  // (head_dim 128 only: the step's projection works in whole 128-dim query heads)
  if (B > kStepMaxBatch || (s->flags & DA_FLAG_DEBUG_SCORES) || s->head_dim != kHeadDim) return sp;
  if ((size_t)B * Hkv * s->max_seq_len * kHeadDim * 4 > kStepMaxKvBytes) return sp;
  if ((size_t)K * N * 2 > kStepMaxWeightBytes) return sp;
  sp.gpad = pow2_at_least(G);
  sp.mpad = pow2_at_least(B);
  const int seqs = B * Hkv;
  const int grains = ceil_div(s->max_seq_len, kPieceGrain);
  const decode_attn_tiles_t* t = s->tiles;
  const int attn_target = t && t->attn_workgroups ? t->attn_workgroups : kStepAttnTarget;
  int pieces = std::min(grains, std::max(1, ceil_div(attn_target, seqs)));
  sp.piece_keys = kPieceGrain * ceil_div(grains, pieces);
  sp.pieces = ceil_div(s->max_seq_len, sp.piece_keys);
  sp.attn_wgs = seqs * sp.pieces;
  if (sp.attn_wgs > kStepMaxAttn) return sp;
  // projection: a tile of tile_n columns x a K-chunk of 16384 / tile_n rows per
  // workgroup, the first that fits in the order 256, 512, 128. With 256
  // columns each weight row is read in 512-byte segments, which stream faster
  // than 1 KiB ones (measured: 18.0 against 18.4 us for the 32/8-head,
  // 2048-key, 4096-hidden step).
  int best = 0;
  for (int tc : {256, 512, 128}) {
    if (best) break;
    if (t && t->proj_tile_n && t->proj_tile_n != tc) continue;
    const int kc = da::decode_step_chunk(tc), nh = kc / kHeadDim;
    if (K % kc != 0 || (nh % G != 0 && G % nh != 0)) continue;
    if (!da::decode_step_supported(sp.gpad, sp.mpad, tc)) continue;
    const int tiles = ceil_div(N, tc), chunks = K / kc;
    const int wgs = tiles * chunks;
    if (sp.attn_wgs + wgs > kStepResident) continue;
    best = wgs;
    sp.tile_n = tc;
    sp.chunk = kc;
    sp.tiles = tiles;
    sp.chunks = chunks;
  }
  if (best == 0) return sp;
  sp.part_o_bytes = align_up((size_t)sp.attn_wgs * G * kHeadDim * sizeof(float), kAlign);
  sp.part_ml_bytes = align_up((size_t)sp.attn_wgs * G * 2 * sizeof(float), kAlign);
  sp.proj_part_bytes = sp.chunks > 1 ? align_up((size_t)sp.chunks * B * N * sizeof(float), kAlign) : 0;
  // counters, one per line: ready copies per kv head, K-chunks per column tile
  sp.ok = (Hkv * da::kStepReplicas + sp.tiles) * da::kCounterStride <= da::kStepCounterBase;
  return sp;
}

struct Layout {
  AttnPlan attn;
  ProjPlan proj;
  StepPlan step;
  size_t off_part_o, off_part_ml, off_flat, off_proj_part, total;
  int attn_counter0, proj_counter0, ready_counter0;
  bool fits;
  bool fused;  // decode_attn_fwd runs the single-launch step
  bool large;  // decode_attn_fwd runs the single-launch large step (stream-K attention + MFMA GEMM items)
  bool tiny;   // decode_attn_fwd runs the tiny step (every workgroup computes the whole attention)
};

// Workspace: [arrival counters][attention partials][attention output][projection partials]
// for two launches; the single-launch step lays [piece partials][projection
// partials] over the same bytes after the counters. Both are reserved, so the
// size does not depend on the flags.
Layout layout_for(const decode_attn_shape_t* s, bool with_proj) {
  Layout L{};
  L.attn = plan_attn(s);
  size_t off = da::kCounterBlockBytes;
  L.off_part_o = off;
  off += L.attn.part_o_bytes;
  L.off_part_ml = off;
  off += L.attn.part_ml_bytes;
  L.attn_counter0 = 0;
  int counters = s->batch * s->num_kv_heads;
  L.fused = false;
  if (with_proj) {
    const decode_attn_tiles_t* t = s->tiles;
    L.proj = plan_proj(s->batch, s->num_q_heads * s->head_dim, s->hidden, t ? t->proj_tile_n : 0,
                       t ? t->proj_ksplit : 0);
    L.off_flat = off;
    off += align_up((size_t)s->batch * s->num_q_heads * s->head_dim * sizeof(uint16_t), kAlign);
    L.off_proj_part = off;
    off += L.proj.part_bytes;
    L.proj_counter0 = counters;
    counters += L.proj.tiles;
    L.step = plan_step(s);
    const bool one_launch = !(s->flags & DA_FLAG_SEPARATE) && !(t && t->step_mode == 2);
    if (L.step.ok) {
      const size_t step_total =
          da::kCounterBlockBytes + L.step.part_o_bytes + L.step.part_ml_bytes + L.step.proj_part_bytes;
      off = std::max(off, step_total);
      L.fused = one_launch && !(t && t->step_mode == 3);
    }
    // the large single-launch step: the two-launch layout plus per-kv-head ready counters
    L.ready_counter0 = (int)align_up((size_t)counters, da::kCounterStride);
    const int ready_end = L.ready_counter0 + s->num_kv_heads * da::kStepReplicas * da::kCounterStride;
    // (its attention keeps one 32-key step in flight per wave: a deeper pipeline runs in two launches)
    L.large = one_launch && !L.fused && L.proj.path == 1 && L.proj.mtiles <= 2 && s->head_dim == kHeadDim &&
              L.attn.depth <= 1 &&
              !(s->flags & DA_FLAG_DEBUG_SCORES) && ready_end <= da::kStepCounterBase;
    // the tiny step: K/V small enough for every workgroup to compute the whole attention
    const size_t kv_bytes = (size_t)s->batch * s->num_kv_heads * s->max_seq_len * s->head_dim * 2 * 2;
    const int mode = t ? t->step_mode : 0;
    L.tiny = one_launch && (mode == 0 || mode == 4) && s->head_dim == kHeadDim && s->batch <= da::kTinyMaxBatch &&
             s->num_q_heads * s->head_dim <= da::kTinyMaxK && kv_bytes <= da::kTinyMaxKvBytes &&
             !(s->flags & DA_FLAG_DEBUG_SCORES);
    if (L.tiny) L.fused = L.large = false;
  }
  L.total = off;
  L.fits = counters <= da::kStepCounterBase && L.attn.part_o_bytes < (1ull << 32) &&
           (!with_proj || proj_fits(L.proj, s->hidden));
  return L;
}

int check_attn_ptrs(const void* q, const void* k, const void* v, const int32_t* sl, const void* out) {
  if (!q || !k || !v || !sl || !out) return DA_ERR_NULL;
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(out, 16) || misaligned(sl, 4))
    return DA_ERR_ALIGN;
  return DA_OK;
}

int check_workspace(const decode_attn_shape_t* s, size_t need) {
  if (need == 0) return DA_OK;
  if (!s->workspace || s->workspace_bytes < need) return DA_ERR_WORKSPACE;
  if (misaligned(s->workspace, kAlign)) return DA_ERR_ALIGN;
  return DA_OK;
}

int check_debug(const decode_attn_shape_t* s) {
  if (!(s->flags & DA_FLAG_DEBUG_SCORES)) return DA_OK;
  if (!s->debug_scores || !s->debug_lse) return DA_ERR_NULL;
  if (misaligned(s->debug_scores, 4) || misaligned(s->debug_lse, 4)) return DA_ERR_ALIGN;
  return DA_OK;
}

da::AttnParams attn_params(const void* q, const void* k, const void* v, const int32_t* sl, void* flat,
                           const decode_attn_shape_t* s, const Layout& L) {
  da::AttnParams p{};
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.seq_lens = sl;
  p.flat = (uint16_t*)flat;
  char* ws = (char*)s->workspace;
  p.part_o = (float*)(ws + L.off_part_o);
  p.part_ml = (float*)(ws + L.off_part_ml);
  p.part_o_bytes = (uint32_t)L.attn.part_o_bytes;
  p.part_ml_bytes = (uint32_t)L.attn.part_ml_bytes;
  p.counters = (uint32_t*)ws + L.attn_counter0;
  const bool dbg = (s->flags & DA_FLAG_DEBUG_SCORES) != 0;
  p.dbg_scores = dbg ? s->debug_scores : nullptr;
  p.dbg_lse = dbg ? s->debug_lse : nullptr;
  p.B = s->batch;
  p.Hq = s->num_q_heads;
  p.Hkv = s->num_kv_heads;
  p.G = s->num_q_heads / s->num_kv_heads;
  p.Lmax = s->max_seq_len;
  p.head_dim = s->head_dim;
  p.num_workgroups = L.attn.workgroups;
  p.step_variant = L.attn.depth;
  p.seq_cost = L.attn.seq_cost;
  p.head_ready = nullptr;
  const float scale = s->softmax_scale != 0.f ? s->softmax_scale : 1.0f / sqrtf((float)s->head_dim);
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  return p;
}

int run_attention(const da::AttnParams& p, const Layout& L, hipStream_t st) {
  return da::launch_attention(p, L.attn.gpad, st) == hipSuccess ? DA_OK : DA_ERR_LAUNCH;
}

da::GemvParams gemv_params(const ProjPlan& pp, const void* x, const void* w, void* out, int M, int K, int N,
                           char* part, char* cnt) {
  da::GemvParams g{};
  g.x = (const uint16_t*)x;
  g.w = (const uint16_t*)w;
  g.out = (uint16_t*)out;
  g.part = (float*)part;
  g.counters = (uint32_t*)cnt;
  g.M = M;
  g.K = K;
  g.N = N;
  g.kchunk = pp.kchunk;
  g.ksplit = pp.ksplit;
  g.tile_n = pp.tile_n;
  g.part_bytes = (uint32_t)std::min<size_t>(pp.part_bytes, 0xffffffffu);
  return g;
}

int run_proj(const ProjPlan& pp, const void* x, const void* w, void* out, int M, int K, int N, char* part,
             char* cnt, hipStream_t st) {
  if (pp.path == 0) {
    const da::GemvParams g = gemv_params(pp, x, w, out, M, K, N, part, cnt);
    return da::launch_gemv(g, pp.mpad, st) == hipSuccess ? DA_OK : DA_ERR_LAUNCH;
  }
  da::GemmParams g{};
  g.a = (const uint16_t*)x;
  g.b = (const uint16_t*)w;
  g.c = (uint16_t*)out;
  g.part = (float*)part;
  g.counters = (uint32_t*)cnt;
  g.M = M;
  g.K = K;
  g.N = N;
  g.kchunk = pp.kchunk;
  g.ksplit = pp.ksplit;
  g.mtiles = pp.mtiles;
  g.part_bytes = (uint32_t)std::min<size_t>(pp.part_bytes, 0xffffffffu);
  return da::launch_gemm_bf16(g, st) == hipSuccess ? DA_OK : DA_ERR_LAUNCH;
}

int run_step(const void* q, const void* k, const void* v, const int32_t* sl, const void* w, void* out,
             const decode_attn_shape_t* s, const Layout& L, hipStream_t st) {
  const StepPlan& sp = L.step;
  char* ws = (char*)s->workspace;
  uint32_t* cnt = (uint32_t*)ws;
  da::StepParams p{};
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.seq_lens = sl;
  p.w = (const uint16_t*)w;
  p.out = (uint16_t*)out;
  char* data = ws + da::kCounterBlockBytes;
  p.part_o = (float*)data;
  p.part_ml = (float*)(data + sp.part_o_bytes);
  p.proj_part = (float*)(data + sp.part_o_bytes + sp.part_ml_bytes);
  p.part_o_bytes = (uint32_t)sp.part_o_bytes;
  p.part_ml_bytes = (uint32_t)sp.part_ml_bytes;
  p.proj_part_bytes = (uint32_t)sp.proj_part_bytes;
  da::ReadySync& r = p.sync;
  r.ready = cnt;
  r.pass_top = cnt + da::kStepCounterBase;
  r.error = cnt + da::kStepErrorWord;
  r.pass_sub = cnt + da::kStepCounterBase + 32;
  r.heads = s->num_kv_heads;
  r.target = (uint32_t)(s->batch * sp.pieces);  // pieces of every sequence of the kv head
  r.wait_polls = s->tiles && s->tiles->step_wait_polls ? (uint32_t)s->tiles->step_wait_polls : da::kStepWaitPolls;
  r.waiters = sp.tiles * sp.chunks;
  p.proj_cnt = r.ready + s->num_kv_heads * da::kStepReplicas * da::kCounterStride;
  p.B = s->batch;
  p.Hq = s->num_q_heads;
  p.Hkv = s->num_kv_heads;
  p.G = s->num_q_heads / s->num_kv_heads;
  p.Lmax = s->max_seq_len;
  p.N = s->hidden;
  p.piece_keys = sp.piece_keys;
  p.pieces = sp.pieces;
  p.attn_wgs = sp.attn_wgs;
  p.tiles = sp.tiles;
  p.chunks = sp.chunks;
  p.weight_delay = s->tiles ? (uint32_t)s->tiles->step_weight_delay : 0u;
  const float scale = s->softmax_scale != 0.f ? s->softmax_scale : 1.0f / sqrtf((float)kHeadDim);
  p.scale_log2 = scale * 1.4426950408889634f;
  return da::launch_decode_step(p, sp.gpad, sp.mpad, sp.tile_n, st) == hipSuccess ? DA_OK : DA_ERR_LAUNCH;
}

// The tiny step: no workspace, no waits.
int run_step_tiny(const void* q, const void* k, const void* v, const int32_t* sl, const void* w, void* out,
                  const decode_attn_shape_t* s, hipStream_t st) {
  da::StepTinyParams p{};
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.seq_lens = sl;
  p.w = (const uint16_t*)w;
  p.out = (uint16_t*)out;
  p.B = s->batch;
  p.Hq = s->num_q_heads;
  p.Hkv = s->num_kv_heads;
  p.G = s->num_q_heads / s->num_kv_heads;
  p.Lmax = s->max_seq_len;
  p.N = s->hidden;
  const float scale = s->softmax_scale != 0.f ? s->softmax_scale : 1.0f / sqrtf((float)kHeadDim);
  p.scale_log2 = scale * 1.4426950408889634f;
  return da::launch_decode_step_tiny(p, pow2_at_least(p.G), st) == hipSuccess ? DA_OK : DA_ERR_LAUNCH;
}

// The single-launch large step: stream-K attention workgroups and the MFMA
// GEMM items of the projection in one grid.
int run_step_large(const da::AttnParams& attn, const void* w, void* out, const decode_attn_shape_t* s,
                   const Layout& L, hipStream_t st) {
  const ProjPlan& pp = L.proj;
  char* ws = (char*)s->workspace;
  uint32_t* cnt = (uint32_t*)ws;
  da::StepLargeParams p{};
  p.attn = attn;
  p.attn.head_ready = cnt + L.ready_counter0;
  da::GemmParams& g = p.gemm;
  g.a = (const uint16_t*)(ws + L.off_flat);
  g.b = (const uint16_t*)w;
  g.c = (uint16_t*)out;
  g.part = (float*)(ws + L.off_proj_part);
  g.counters = cnt + L.proj_counter0;
  g.M = s->batch;
  g.K = s->num_q_heads * s->head_dim;
  g.N = s->hidden;
  g.kchunk = pp.kchunk;
  g.ksplit = pp.ksplit;
  g.mtiles = pp.mtiles;
  g.part_bytes = (uint32_t)std::min<size_t>(pp.part_bytes, 0xffffffffu);
  p.ntiles = ceil_div(s->hidden, da::kGemmTileN);
  p.mgroups = ceil_div(s->batch, pp.mpad);
  da::ReadySync& r = p.wait.sync;
  r.ready = cnt + L.ready_counter0;
  r.pass_top = cnt + da::kStepCounterBase;
  r.error = cnt + da::kStepErrorWord;
  r.pass_sub = cnt + da::kStepCounterBase + 32;
  r.heads = s->num_kv_heads;
  r.target = (uint32_t)s->batch;
  r.wait_polls = s->tiles && s->tiles->step_wait_polls ? (uint32_t)s->tiles->step_wait_polls : da::kStepWaitPolls;
  r.waiters = p.ntiles * p.mgroups * pp.ksplit;
  p.wait.head_dim = s->head_dim;
  p.wait.group = s->num_q_heads / s->num_kv_heads;
  return da::launch_decode_step_large(p, L.attn.gpad, st) == hipSuccess ? DA_OK : DA_ERR_LAUNCH;
}

// ---- the no-allocation entry point's scratch: one array per device ----
//
// decode_attn_fwd_noalloc takes its workspace from this array instead of the
// caller. Host code never uses the array's name as an address (on the host it
// is only a stand-in for the symbol): every kernel argument, fill and copy
// uses the device address hipGetSymbolAddress returns, looked up once per
// device with that device current.
constexpr size_t kScratchBytes = (size_t)DA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__global__ void zero_counter_block(uint32_t* words) { words[blockIdx.x * blockDim.x + threadIdx.x] = 0u; }

struct ScratchSlot {
  void* ptr;           // device address of `scratch` on this device
  bool needs_clear;    // its counter block is to be zero-filled before the next call
};
ScratchSlot g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

}  // namespace

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

// The scratch address of the current device (*dev); the first call on a
// device looks it up. *clear tells whether its counter block must be
// zero-filled first (mark_cleared once that is enqueued).
int scratch_of_current_device(void** ptr, bool* clear, int* dev) {
  *dev = -1;
  if (hipGetDevice(dev) != hipSuccess || *dev < 0 || *dev >= kMaxDevices) return DA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ScratchSlot& slot = g_scratch[*dev];
  if (!slot.ptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DA_ERR_LAUNCH;
    slot.ptr = p;
    slot.needs_clear = true;
  }
  *ptr = slot.ptr;
  *clear = slot.needs_clear;
  return DA_OK;
}

void mark_cleared(int dev) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  g_scratch[dev].needs_clear = false;
}

// Zero-fill a workspace's counter block on `st` with a kernel (no memset node
// ends up in a graph that captures the call).
int clear_counter_block(void* ws, hipStream_t st) {
  constexpr int kWords = (int)(da::kCounterBlockBytes / sizeof(uint32_t));
  zero_counter_block<<<dim3(kWords / 256), dim3(256), 0, st>>>((uint32_t*)ws);
  return hipGetLastError() == hipSuccess ? DA_OK : DA_ERR_LAUNCH;
}

// decode_attn_fwd, with the caller's workspace or (noalloc) the scratch array.
int fwd_impl(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens, const void* o_weight,
             void* out, const decode_attn_shape_t* shape_in, void* stream, bool noalloc) {
  if (!shape_in) return DA_ERR_NULL;
  decode_attn_shape_t eff = effective_shape(shape_in);
  const decode_attn_shape_t* shape = &eff;
  int rc = check_attn_ptrs(q, k_cache, v_cache, seq_lens, out);
  if (rc) return rc;
  if (!o_weight) return DA_ERR_NULL;
  if (misaligned(o_weight, 16)) return DA_ERR_ALIGN;
  if (!shape_ok(shape, true)) return DA_ERR_SHAPE;
  const Layout L = layout_for(shape, true);
  if (!L.fits) return DA_ERR_SHAPE;
  hipStream_t st = (hipStream_t)stream;
  if (noalloc) {
    if (L.total > kScratchBytes) return DA_ERR_WORKSPACE;
    if ((rc = check_debug(shape))) return rc;
    void* ptr = nullptr;
    bool clear = false;
    int dev = -1;
    if ((rc = scratch_of_current_device(&ptr, &clear, &dev))) return rc;
    if (clear) {
      if ((rc = clear_counter_block(ptr, st))) return rc;
      mark_cleared(dev);
    }
    eff.workspace = ptr;
    eff.workspace_bytes = kScratchBytes;
  } else {
    if ((rc = check_workspace(shape, L.total))) return rc;
    if ((rc = check_debug(shape))) return rc;
  }
  char* ws = (char*)shape->workspace;
  void* flat = ws + L.off_flat;
  const da::AttnParams p = attn_params(q, k_cache, v_cache, seq_lens, flat, shape, L);
  if (L.tiny) return run_step_tiny(q, k_cache, v_cache, seq_lens, o_weight, out, shape, st);
  if (L.fused) return run_step(q, k_cache, v_cache, seq_lens, o_weight, out, shape, L, st);
  if (L.large) return run_step_large(p, o_weight, out, shape, L, st);
  if ((rc = run_attention(p, L, st))) return rc;
  return run_proj(L.proj, flat, o_weight, out, shape->batch, shape->num_q_heads * shape->head_dim, shape->hidden,
                  ws + L.off_proj_part, (char*)((uint32_t*)ws + L.proj_counter0), st);
}

}  // namespace

extern "C" {

size_t decode_attn_workspace_size(const decode_attn_shape_t* shape_in) {
  if (!shape_in) return 0;
  const decode_attn_shape_t eff = effective_shape(shape_in);
  const decode_attn_shape_t* shape = &eff;
  if (!shape_ok(shape, true)) return 0;
  const Layout L = layout_for(shape, true);
  if (!L.fits) return 0;
  // enough for decode_attn_only too, whose table lookup ignores the hidden size
  const decode_attn_shape_t eff_attn = effective_shape(shape_in, false);
  const Layout La = layout_for(&eff_attn, false);
  return std::max(L.total, La.fits ? La.total : (size_t)0);
}

int decode_attn_plan(const decode_attn_shape_t* shape_in, decode_attn_plan_t* plan) {
  if (!shape_in || !plan) return DA_ERR_NULL;
  const decode_attn_shape_t eff = effective_shape(shape_in);
  const decode_attn_shape_t* shape = &eff;
  if (!shape_ok(shape, true)) return DA_ERR_SHAPE;
  const Layout L = layout_for(shape, true);
  if (!L.fits) return DA_ERR_SHAPE;
  const int G = shape->num_q_heads / shape->num_kv_heads;
  const int D = shape->head_dim;
  const int Ko = shape->num_q_heads * D;
  memset(plan, 0, sizeof *plan);
  if (L.tiny) {
    // one launch, every workgroup the whole attention (one piece per sequence) and 16 columns over all of K
    const int wgs = ceil_div(shape->hidden, da::kTinyCols);
    plan->qk = {G, kHeadDim, shape->max_seq_len, 16, kHeadDim, kAttnBlockKeys, 1, wgs};
    plan->pv = {G, shape->max_seq_len, kHeadDim, 16, kAttnBlockKeys, kHeadDim, 1, wgs};
    plan->oproj = {shape->batch, Ko, shape->hidden, shape->batch, Ko, da::kTinyCols, 1, wgs};
    plan->split_len = shape->max_seq_len;
    plan->num_splits = 1;
    plan->oproj_path = 0;
    plan->fused = 3;
    plan->workspace_bytes = L.total;
    return DA_OK;
  }
  if (L.fused) {
    // one launch: a fixed number of pieces per sequence, projection tiles of whole kv heads
    const StepPlan& sp = L.step;
    const int wgs = sp.attn_wgs;
    plan->qk = {G, kHeadDim, shape->max_seq_len, 16, kHeadDim, kAttnBlockKeys, sp.pieces, wgs};
    plan->pv = {G, shape->max_seq_len, kHeadDim, 16, kAttnBlockKeys, kHeadDim, sp.pieces, wgs};
    plan->oproj = {shape->batch, Ko, shape->hidden, sp.mpad, sp.chunk, sp.tile_n, sp.chunks, sp.tiles * sp.chunks};
    plan->split_len = sp.piece_keys;
    plan->num_splits = sp.pieces;
    plan->oproj_path = 0;
    plan->fused = 1;
    plan->workspace_bytes = L.total;
    return DA_OK;
  }
  const int wgs = L.attn.workgroups;
  // QK^T per kv head: M = G, K = head_dim (whole), N = keys (32 per wave step)
  plan->qk = {G, D, shape->max_seq_len, 16, D, kAttnBlockKeys, wgs, wgs};
  // attn x V per kv head: M = G, K = keys (32 per wave step), N = head_dim (whole)
  plan->pv = {G, shape->max_seq_len, D, 16, kAttnBlockKeys, D, wgs, wgs};
  plan->oproj = {shape->batch, Ko, shape->hidden, L.proj.mpad, L.proj.kchunk, L.proj.tile_n, L.proj.ksplit,
                 L.proj.tiles * L.proj.ksplit};
  plan->split_len = L.attn.keys_per_wg;
  plan->num_splits = wgs;
  plan->oproj_path = L.proj.path;
  plan->fused = L.large ? 2 : 0;
  plan->workspace_bytes = L.total;
  return DA_OK;
}

int decode_attn_fwd(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                    const void* o_weight, void* out, const decode_attn_shape_t* shape_in, void* stream) {
  return fwd_impl(q, k_cache, v_cache, seq_lens, o_weight, out, shape_in, stream, false);
}

int decode_attn_fwd_noalloc(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                            const void* o_weight, void* out, const decode_attn_shape_t* shape, void* stream) {
  return fwd_impl(q, k_cache, v_cache, seq_lens, o_weight, out, shape, stream, true);
}

int decode_attn_only(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                     void* attn_out, const decode_attn_shape_t* shape_in, void* stream) {
  if (!shape_in) return DA_ERR_NULL;
  const decode_attn_shape_t eff = effective_shape(shape_in, false);
  const decode_attn_shape_t* shape = &eff;
  int rc = check_attn_ptrs(q, k_cache, v_cache, seq_lens, attn_out);
  if (rc) return rc;
  if (!shape_ok(shape, false)) return DA_ERR_SHAPE;
  const Layout L = layout_for(shape, false);
  if (!L.fits) return DA_ERR_SHAPE;
  if ((rc = check_workspace(shape, L.total))) return rc;
  if ((rc = check_debug(shape))) return rc;
  const da::AttnParams p = attn_params(q, k_cache, v_cache, seq_lens, attn_out, shape, L);
  return run_attention(p, L, (hipStream_t)stream);
}

size_t oproj_workspace_size(int32_t M, int32_t K, int32_t N) {
  if (M < 1 || K < 1 || N < 1) return 0;
  const ProjPlan pp = plan_proj(M, K, N);
  if (!proj_fits(pp, N)) return 0;
  return pp.ksplit > 1 ? da::kCounterBlockBytes + pp.part_bytes : 0;
}

int oproj_fwd(const void* x, const void* w, void* out, int32_t M, int32_t K, int32_t N, void* workspace,
              size_t workspace_bytes, void* stream) {
  if (!x || !w || !out) return DA_ERR_NULL;
  if (misaligned(x, 16) || misaligned(w, 16) || misaligned(out, 16)) return DA_ERR_ALIGN;
  if (M < 1 || K < 1 || N < 1 || N % 8 != 0) return DA_ERR_SHAPE;
  if (M >= 16 && K % 32 != 0) return DA_ERR_SHAPE;
  if (M < 16 && K % 8 != 0) return DA_ERR_SHAPE;
  const ProjPlan pp = plan_proj(M, K, N);
  if (!proj_fits(pp, N)) return DA_ERR_SHAPE;
  const size_t need = oproj_workspace_size(M, K, N);
  if (need) {
    if (!workspace || workspace_bytes < need) return DA_ERR_WORKSPACE;
    if (misaligned(workspace, kAlign)) return DA_ERR_ALIGN;
  }
  char* ws = (char*)workspace;
  return run_proj(pp, x, w, out, M, K, N, ws ? ws + da::kCounterBlockBytes : nullptr, ws, (hipStream_t)stream);
}

int gemm_f16(const void* a, const void* b, void* c, int32_t M, int32_t N, int32_t K, void* stream) {
  if (!a || !b || !c) return DA_ERR_NULL;
  if (misaligned(a, 16) || misaligned(b, 16) || misaligned(c, 16)) return DA_ERR_ALIGN;
  if (M < 1 || N < 1 || K < 1 || M % 16 != 0 || N % 16 != 0 || K % 32 != 0) return DA_ERR_SHAPE;
  if ((size_t)K * N * 2 > 0xffffffffull) return DA_ERR_SHAPE;
  da::GemmParams g{};
  g.a = (const uint16_t*)a;
  g.b = (const uint16_t*)b;
  g.c = (uint16_t*)c;
  g.M = M;
  g.K = K;
  g.N = N;
  g.kchunk = K;
  g.ksplit = 1;
  g.mtiles = 1;
  // too few 128-column tiles to fill the chip: 16 x 32 tiles over all of K
  const bool narrow = (long)ceil_div(N, da::kGemmTileN) * (M / 16) < da::kGemmNarrowBelow;
  const hipError_t e = narrow ? da::launch_gemm_narrow_f16(g, (hipStream_t)stream)
                              : da::launch_gemm_f16(g, (hipStream_t)stream);
  return e == hipSuccess ? DA_OK : DA_ERR_LAUNCH;
}

int prefill_attn_fwd(const void* q, const void* k_cache, const void* v_cache, const int32_t* ctx_lens, void* out,
                     const prefill_attn_shape_t* s, void* stream) {
  if (!s || !q || !k_cache || !v_cache || !ctx_lens || !out) return DA_ERR_NULL;
  if (misaligned(q, 16) || misaligned(k_cache, 16) || misaligned(v_cache, 16) || misaligned(out, 16) ||
      misaligned(ctx_lens, 4))
    return DA_ERR_ALIGN;
  if (s->batch < 1 || s->num_tokens < 1 || s->num_q_heads < 1 || s->num_kv_heads < 1 || s->max_seq_len < 1)
    return DA_ERR_SHAPE;
  if (s->head_dim != kHeadDim || s->num_q_heads % s->num_kv_heads != 0) return DA_ERR_SHAPE;
  if (s->num_q_heads / s->num_kv_heads > DA_MAX_GROUP || s->num_tokens > s->max_seq_len) return DA_ERR_SHAPE;
  if ((size_t)s->max_seq_len * kHeadDim * 2 >= (1ull << 32)) return DA_ERR_SHAPE;
  const double rows = (double)s->batch * s->num_kv_heads * s->num_tokens * (s->num_q_heads / s->num_kv_heads);
  if (rows / 64 > 2.0e9 || (double)s->batch * s->num_tokens * s->num_q_heads * kHeadDim > 9.0e15)
    return DA_ERR_SHAPE;
  da::PrefillParams p{};
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k_cache;
  p.v = (const uint16_t*)v_cache;
  p.ctx_lens = ctx_lens;
  p.out = (uint16_t*)out;
  p.B = s->batch;
  p.T = s->num_tokens;
  p.Hq = s->num_q_heads;
  p.Hkv = s->num_kv_heads;
  p.G = s->num_q_heads / s->num_kv_heads;
  p.Lmax = s->max_seq_len;
  const float scale = s->softmax_scale != 0.f ? s->softmax_scale : 1.0f / sqrtf((float)kHeadDim);
  p.scale_log2 = scale * 1.4426950408889634f;
  return da::launch_prefill(p, (hipStream_t)stream) == hipSuccess ? DA_OK : DA_ERR_LAUNCH;
}

int decode_attn_read_probe(const void* src, size_t bytes, uint32_t* sink, int32_t workgroups, void* stream) {
  if (!src || !sink) return DA_ERR_NULL;
  if (misaligned(src, 16) || misaligned(sink, 4)) return DA_ERR_ALIGN;
  if (bytes == 0 || bytes % 16 != 0 || workgroups < 1 || workgroups > 65536) return DA_ERR_SHAPE;
  return da::launch_read_probe(src, bytes, sink, workgroups, (hipStream_t)stream) == hipSuccess ? DA_OK
                                                                                               : DA_ERR_LAUNCH;
}

int decode_attn_step_status(const void* workspace, size_t workspace_bytes, void* stream) {
  const bool own = workspace == nullptr;  // the no-allocation scratch of the current device
  if (!own) {
    if (workspace_bytes < da::kCounterBlockBytes) return DA_ERR_WORKSPACE;
    if (misaligned(workspace, kAlign)) return DA_ERR_ALIGN;
  }
  hipStream_t st = (hipStream_t)stream;
  if (own) {
    void* ptr = nullptr;
    bool clear = false;
    int dev = -1;
    const int rc = scratch_of_current_device(&ptr, &clear, &dev);
    if (rc) return rc;
    if (clear) return DA_OK;  // no call has run on it yet
    workspace = ptr;
  }
  uint32_t word = 0;
  const uint32_t* src = (const uint32_t*)workspace + da::kStepErrorWord;
  if (hipMemcpyAsync(&word, src, sizeof word, hipMemcpyDeviceToHost, st) != hipSuccess) return DA_ERR_LAUNCH;
  if (hipStreamSynchronize(st) != hipSuccess) return DA_ERR_LAUNCH;
  if (word == 0) return DA_OK;
  if (own) {
    // the caller cannot reach the scratch: its counter block is zero-filled here
    if (clear_counter_block(const_cast<void*>(workspace), st) != DA_OK) return DA_ERR_LAUNCH;
    if (hipStreamSynchronize(st) != hipSuccess) return DA_ERR_LAUNCH;
  }
  return DA_ERR_TIMEOUT;
}

const char* decode_attn_status_str(int status) {
  switch (status) {
    case DA_OK: return "ok";
    case DA_ERR_NULL: return "a required pointer is NULL";
    case DA_ERR_SHAPE: return "unsupported or inconsistent shape";
    case DA_ERR_ALIGN: return "misaligned pointer (16-byte tensors, 256-byte workspace)";
    case DA_ERR_WORKSPACE: return "workspace missing or too small";
    case DA_ERR_LAUNCH: return "kernel launch failed";
    case DA_ERR_TIMEOUT: return "a single-launch step stopped waiting for its attention (outputs invalid; "
                                "zero-fill the workspace counters again)";
    default: return "unknown status";
  }
}

}  // extern "C"
