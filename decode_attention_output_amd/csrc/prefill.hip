// Context (prefill) attention of a chunk of new tokens on gfx950.
//
// The F-16 page ("PyPTO 开箱性能调优实战：Decode Attention 多 Matmul 独立
// TileShape 配置 F-16") names a context-attention kernel next to the decode one
// without defining it; the reading taken here: sequence b holds ctx_lens[b]
// cached keys, the last T of which are the chunk's own tokens, and token t
// attends causally to keys 0 .. ctx_lens[b] - T + t with the decode step's
// scaled softmax (T = 1 is the decode attention).
//
// Many query rows share every key, so this is a real MFMA contraction. A
// workgroup owns 64 query rows of one (batch, kv head) -- row r is token
// r / G, query head r % G of the group -- 16 per wave, which is exactly the
// B operand (16 columns) of the decode step's S^T = K x Q^T product. The four
// waves share each 32-key K/V tile: the workgroup loads it cooperatively
// (1 KiB per load instruction, whole rows) into one of two LDS stages while
// the waves compute the previous tile with the per-wave step of attn_core.hpp
// (online softmax, P x V with fp32-exact weights), each lane masking the keys
// past its own row's position. A wave stops computing once every key of its
// rows is done; the workgroup stops loading at the last key of its last row.
#include "attn_core.hpp"
#include "kernels.hpp"

namespace da {

namespace {

constexpr int kPrefillWaves = 4;
constexpr int kPrefillThreads = kPrefillWaves * kWave;
constexpr int kPrefillRows = kPrefillWaves * 16;  // query rows per workgroup
constexpr int kPrefillLds = 2 * kStageBytes;      // two K/V stages shared by the waves

__global__ __launch_bounds__(kPrefillThreads, 2) void prefill_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) char smem[kPrefillLds];
  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
  const int i = lane & 15, grp = lane >> 4;
  const int R = p.T * p.G;                        // query rows of one (batch, kv head)
  const int blocks = (R + kPrefillRows - 1) / kPrefillRows;
  const int blk = blockIdx.x % blocks;
  const int seq = blockIdx.x / blocks;            // (batch, kv head)
  const int b = seq / p.Hkv, h = seq % p.Hkv;
  const int ctx = min(max(p.ctx_lens[b], 0), p.Lmax);
  const int base = ctx - p.T;                     // position of the chunk's first token

  // ---- this wave's 16 rows: the query (B operand) and the number of keys each row sees ----
  const int r0 = blk * kPrefillRows + wave * 16;
  const int rr = r0 + i;                          // the row of this lane's column
  const int tok = rr / p.G, gq = rr % p.G;
  const bool row_ok = rr < R;
  uint4 qb[4];
  const uint16_t* qrow = p.q + (((size_t)b * p.T + tok) * p.Hq + (size_t)h * p.G + gq) * kHeadDim;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) qb[kk] = row_ok ? ld16(qrow + kk * 32 + grp * 8) : make_uint4(0, 0, 0, 0);
  const int end = row_ok ? base + tok + 1 : 0;    // keys 0 .. end-1
  // keys of the wave's last row and of the workgroup's last row
  const int wave_last = min(r0 + 15, R - 1), blk_last = min(blk * kPrefillRows + kPrefillRows - 1, R - 1);
  const int wave_keys = r0 < R ? base + wave_last / p.G + 1 : 0;
  const int blk_keys = base + blk_last / p.G + 1;
  const int ntiles = (blk_keys + kStepKeys - 1) / kStepKeys;

  AttnSeg sg;
  const size_t kv_off = (size_t)seq * p.Lmax * kHeadDim;
  sg.K = make_rsrc(p.k + kv_off, (uint32_t)ctx * kRowBytes);  // rows past the context read as 0
  sg.V = make_rsrc(p.v + kv_off, (uint32_t)ctx * kRowBytes);
  sg.L = ctx;
  sg.G = p.G;
  sg.scale_log2 = p.scale_log2;
  sg.scale = 0.f;
  sg.dbg = nullptr;
  sg.dbg_stride = 0;

  // ---- the shared K/V tiles: thread t loads rows t/16 and 16 + t/16, bytes (t%16)*16 ----
  uint4 kr[2], vr[2];
  auto load_tile = [&](int tile) {
    const uint32_t off = (uint32_t)(tile * kStepKeys + t / 16) * kRowBytes + (t % 16) * 16;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      kr[j] = rsrc_ld16(sg.K, off + j * 16 * kRowBytes);
      vr[j] = rsrc_ld16(sg.V, off + j * 16 * kRowBytes);
    }
  };
  auto store_tile = [&](char* stage) {
    char* q = stage + (t / 16) * kStageRow + (t % 16) * 16;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      *reinterpret_cast<uint4*>(q + j * 16 * kStageRow) = kr[j];
      *reinterpret_cast<uint4*>(q + kStageTile + j * 16 * kStageRow) = vr[j];
    }
  };

  AttnWave aw;
  aw.reset();
  if (ntiles > 0) load_tile(0);
  for (int tile = 0; tile < ntiles; ++tile) {
    char* stage = smem + (tile & 1) * kStageBytes;
    // the stage was last read two tiles ago, before the previous barrier
    store_tile(stage);
    __syncthreads();
    if (tile + 1 < ntiles) load_tile(tile + 1);
    if (tile * kStepKeys < wave_keys) attn_step<16>(aw, stage, qb, sg, tile * kStepKeys, end, lane);
  }

  // ---- normalise and store: element r of o[j] is row 4*grp + r, dim 16j + i ----
  float l = aw.l_acc;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);  // lane i (every group) holds the weight sum of its column's row
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int q = 4 * grp + r;
    const int row = r0 + q;
    const float inv = 1.f / __shfl(l, q);
    if (row >= R) continue;
    uint16_t* orow = p.out + (((size_t)b * p.T + row / p.G) * p.Hq + (size_t)h * p.G + row % p.G) * kHeadDim;
#pragma unroll
    for (int j = 0; j < 8; ++j) orow[16 * j + i] = f32_to_bf16_rne(aw.o[j][r] * inv);
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, hipStream_t s) {
  const int blocks = (p.T * p.G + kPrefillRows - 1) / kPrefillRows;
  prefill_kernel<<<dim3(p.B * p.Hkv * blocks), dim3(kPrefillThreads), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace da
