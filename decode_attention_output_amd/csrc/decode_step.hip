// The whole decode step in one launch, for steps small enough that the fixed
// cost of each dependent trip through memory dominates (a few tokens, a few
// thousand cached keys): attention and output projection of "PyPTO 开箱性能调优
// 实战：Decode Attention 多 Matmul 独立 TileShape 配置 F-16" (section 代码对比:
// the three matmul calls of one forward).
//
// The grid holds two kinds of 256-thread workgroups, all resident at once:
//  - blockIdx < attn_wgs: attention. Every (batch, kv head) sequence is cut
//    into `pieces` fixed pieces of piece_keys keys (the last ones may be short
//    or empty); a workgroup computes one piece for the G query heads of the
//    group, stores its un-normalised output, running max and weight sum
//    through device-coherent stores, and counts the piece in its kv head's
//    ready counter (step_sync.hpp).
//  - the rest: projection. A workgroup owns TC output columns of one K-chunk
//    of the weight, the rows of whole kv heads. It first issues the loads of
//    its whole weight tile (held in registers), so the weight streams from
//    HBM while the attention runs; then it waits until every piece of its kv
//    heads is counted, merges those pieces itself (the same online merge in
//    the same piece order everywhere, so all column tiles see the same bf16
//    attention output), multiplies, and the K-chunks of a column tile meet in
//    the workspace like the split-K GEMV.
// The attention output thus never makes a separate round trip through
// memory, and no workgroup waits for heads it does not use.
// Workgroups are dispatched in index order, so every attention workgroup is
// running before a projection workgroup waits; the waits are bounded (a
// workgroup that gives up sets the error word and writes NaN), and the last
// projection workgroup past its wait returns the ready counters to zero.
#include "attn_core.hpp"
#include "gemv_core.hpp"
#include "step_sync.hpp"

namespace da {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMergeLoads = 8;             // pieces whose loads are in flight together in the merge
constexpr int kRowsPerLane = 32;           // weight rows a projection lane holds (16 bytes each)
constexpr uint32_t kNoLoad = 0x80000000u;  // buffer offset past every range: the load returns 0, no request

// ---- attention: piece `a` = (sequence a / pieces, piece a % pieces) ----
// `smem` holds one K/V stage per wave; a wave's output later reuses its stage.
constexpr int kAttnLds = kWaves * kStageBytes;

template <int GP>
__device__ __forceinline__ void piece_attention(const StepParams& p, int a, char* smem) {
  constexpr int kWaveOut = GP * kHeadDim * 4;
  static_assert(kWaveOut + 2 * GP * 4 <= kStageBytes, "a wave's output fits its stage");
  auto s_o = [&](int w) { return reinterpret_cast<float (*)[kHeadDim]>(smem + w * kStageBytes); };
  auto s_m = [&](int w) { return reinterpret_cast<float*>(smem + w * kStageBytes + kWaveOut); };
  auto s_l = [&](int w) { return reinterpret_cast<float*>(smem + w * kStageBytes + kWaveOut + GP * 4); };
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  const int col = lane & 15, grp = lane >> 4;
  const int seq = a / p.pieces, piece = a % p.pieces;
  const int b = seq / p.Hkv, h = seq % p.Hkv;
  DA_TRACE(0);

  // the wave's first 32-key step is requested before the sequence length is
  // known, through resources bounded by the cache's rows (always inside the
  // allocation); rows past the length are zeroed once it is known
  const size_t kv_off = (size_t)seq * p.Lmax * kHeadDim;
  const int k0 = piece * p.piece_keys;
  const int first = k0 / kStepKeys + wave;
  KVTile t0;
  if (first * kStepKeys < min(k0 + p.piece_keys, p.Lmax)) {
    AttnSeg cap;
    cap.K = make_rsrc(p.k + kv_off, (uint32_t)p.Lmax * kRowBytes);
    cap.V = make_rsrc(p.v + kv_off, (uint32_t)p.Lmax * kRowBytes);
    load_kv(t0, cap, first * kStepKeys, lane);
  }
  uint4 qa[4];
  load_query(qa, p.q + ((size_t)b * p.Hq + (size_t)h * p.G) * kHeadDim, p.G, col, grp);
  const int L = min(max(p.seq_lens[b], 0), p.Lmax);
  const int k1 = min(k0 + p.piece_keys, L);
  DA_TRACE(1);

  AttnSeg sg;
  sg.K = make_rsrc(p.k + kv_off, (uint32_t)L * kRowBytes);
  sg.V = make_rsrc(p.v + kv_off, (uint32_t)L * kRowBytes);
  sg.L = L;
  sg.G = p.G;
  sg.scale_log2 = p.scale_log2;
  sg.scale = 0.f;
  sg.dbg = nullptr;
  sg.dbg_stride = 0;
  AttnWave aw;
  aw.reset();
  // the piece's 32-key steps, interleaved over the waves
  const int nstep = k1 > k0 ? (k1 - k0 + kStepKeys - 1) / kStepKeys : 0;
  const int n = nstep > wave ? (nstep - wave + kWaves - 1) / kWaves : 0;
  attn_wave_steps_preloaded<GP>(aw, t0, qa, sg, first, kWaves, n, L, smem + wave * kStageBytes, lane);
  attn_wave_to_lds<GP>(aw, s_o(wave), s_m(wave), s_l(wave), lane);
  __syncthreads();
  DA_TRACE(2);

  // merge the waves into the piece's partial (an empty piece keeps max -inf)
  const rsrc_t po = make_rsrc(p.part_o, p.part_o_bytes);
  const rsrc_t pml = make_rsrc(p.part_ml, p.part_ml_bytes);
  for (int idx = t; idx < p.G * 32; idx += kThreads) {
    const int g = idx >> 5, d4 = idx & 31;
    float M = s_m(0)[g];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m(w)[g]);
    float Ls = 0.f, O[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = s_m(w)[g] == -INFINITY ? 0.f : exp2f(s_m(w)[g] - M);
      Ls = fmaf(f, s_l(w)[g], Ls);
      const float4 o4 = *reinterpret_cast<const float4*>(&s_o(w)[g][d4 * 4]);
      O[0] = fmaf(f, o4.x, O[0]);
      O[1] = fmaf(f, o4.y, O[1]);
      O[2] = fmaf(f, o4.z, O[2]);
      O[3] = fmaf(f, o4.w, O[3]);
    }
    const uint32_t slot = (uint32_t)a * p.G + g;
    rsrc_st16_coherent(po, (slot * kHeadDim + d4 * 4) * 4,
                       make_uint4(__builtin_bit_cast(uint32_t, O[0]), __builtin_bit_cast(uint32_t, O[1]),
                                  __builtin_bit_cast(uint32_t, O[2]), __builtin_bit_cast(uint32_t, O[3])));
    if (d4 == 0)
      rsrc_st8_coherent(pml, slot * 8, make_uint2(__builtin_bit_cast(uint32_t, M), __builtin_bit_cast(uint32_t, Ls)));
  }
  wait_stores_done();
  __syncthreads();
  if (t < kStepReplicas)
    __hip_atomic_fetch_add(&p.sync.ready[(h * kStepReplicas + t) * kCounterStride], 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  DA_TRACE(3);
}

// ---- projection: column tile r % tiles of K-chunk r / tiles ----
template <int MB, int TC>
__device__ __forceinline__ void projection(const StepParams& p, int r, char* smem) {
  constexpr int LPR = TC / 8;             // lanes per weight row (16 bytes each)
  constexpr int RPP = kThreads / LPR;     // rows per pass of the workgroup
  constexpr int UR = kRowsPerLane;
  constexpr int KC = UR * RPP;            // rows of the K-chunk
  constexpr int NH = KC / kHeadDim;       // query heads of the chunk
  static_assert(NH >= 1, "chunk of whole query heads");
  constexpr int kFinOff = (KC * MB + 6 * kThreads) * 4;
  static_assert(kFinOff + gemv_finish_lds<MB, TC>() <= kAttnLds, "projection scratch fits the kernel's LDS");
  float* const s_x = reinterpret_cast<float*>(smem);  // [row of the chunk][MB] attention output, fp32 of bf16
  float* const s_cm = s_x + KC * MB;
  float* const s_cl = s_cm + kThreads;
  float4* const s_co = reinterpret_cast<float4*>(s_cl + kThreads);
  const int t = threadIdx.x;
  const int tile = r % p.tiles, chunk = r / p.tiles;
  const int n = tile * TC + (t % LPR) * 8;
  const int rr = t / LPR;
  DA_TRACE(8);

  // the whole weight tile of this workgroup, requested at once and held in
  // registers, so that it streams while the attention runs. Loads return in
  // order, so the wave that polls below (wave 0) waits only for its own rows.
  uint4 wv[UR];
  const uint16_t* wrow = p.w + (size_t)(chunk * KC + rr) * p.N + n;
  if (p.weight_delay) {
    // requested weight_delay ticks (100 MHz) after the workgroup starts, so that the
    // attention's K/V requests, issued first, are not queued behind the weight
    const uint64_t t0 = wall_clock64();
    while (wall_clock64() - t0 < p.weight_delay) __builtin_amdgcn_s_sleep(4);
  }
#pragma unroll
  for (int u = 0; u < UR; ++u) wv[u] = n < p.N ? ld16(wrow + (size_t)u * RPP * p.N) : make_uint4(0, 0, 0, 0);

  // wait until every piece of the chunk's kv heads (all batch rows) is stored;
  // a workgroup that gives up writes NaN, so that the failure cannot pass for a
  // result (step_sync.hpp)
  // The count of workgroups past their wait is settled after the multiply, so
  // that its atomics' round trips overlap the merge.
  __shared__ uint32_t s_flag;
  uint32_t prev_pass = 0;
  const int qh0 = chunk * NH;
  if (t == 0) {
    s_flag = ready_wait(p.sync, qh0 / p.G, (qh0 + NH - 1) / p.G, r % kStepReplicas) ? 0u : 1u;
    prev_pass = ready_pass_sub(p.sync, r);
  }
  __syncthreads();
  const bool gave_up = s_flag != 0;
  DA_TRACE(9);

  // merge the pieces of the chunk's heads: (batch row, head, 4 dims) per lane,
  // the pieces split into nph interleaved phases that are combined in order
  const rsrc_t po = make_rsrc(p.part_o, p.part_o_bytes);
  const rsrc_t pml = make_rsrc(p.part_ml, p.part_ml_bytes);
  const int groups = p.B * NH * 32;
  for (int base = 0; base < groups; base += kThreads) {
    const int cnt = min(groups - base, kThreads);
    const int nph = kThreads / cnt;
    const int pr = base + t % cnt, ph = t / cnt;
    const int m = pr / (NH * 32), hl = (pr / 32) % NH, d4 = pr % 32;
    const int qh = qh0 + hl;
    const int slot0 = (m * p.Hkv + qh / p.G) * p.pieces;
    const int g = qh % p.G;
    float M = -INFINITY, Ls = 0.f, O[4] = {0.f, 0.f, 0.f, 0.f};
    if (ph < nph) {
      for (int j0 = ph; j0 < p.pieces; j0 += kMergeLoads * nph) {
        uint2 ml[kMergeLoads];
        uint4 ov[kMergeLoads];
#pragma unroll
        for (int u = 0; u < kMergeLoads; ++u) {
          const bool ok = j0 + u * nph < p.pieces;
          const uint32_t sl = (uint32_t)(slot0 + j0 + u * nph) * p.G + g;
          ml[u] = rsrc_ld8_coherent(pml, ok ? sl * 8 : kNoLoad);
          ov[u] = rsrc_ld16_coherent(po, ok ? (sl * kHeadDim + d4 * 4) * 4 : kNoLoad);
        }
#pragma unroll
        for (int u = 0; u < kMergeLoads; ++u) {
          if (j0 + u * nph < p.pieces) {
            const float o[4] = {__builtin_bit_cast(float, ov[u].x), __builtin_bit_cast(float, ov[u].y),
                                __builtin_bit_cast(float, ov[u].z), __builtin_bit_cast(float, ov[u].w)};
            merge_partial(M, Ls, O, __builtin_bit_cast(float, ml[u].x), __builtin_bit_cast(float, ml[u].y), o);
          }
        }
      }
    }
    s_cm[t] = M;
    s_cl[t] = Ls;
    s_co[t] = make_float4(O[0], O[1], O[2], O[3]);
    __syncthreads();
    if (t < cnt) {
      float Mf = -INFINITY, Lf = 0.f, Of[4] = {0.f, 0.f, 0.f, 0.f};
      for (int q2 = 0; q2 < nph; ++q2) {
        const float4 o4 = s_co[t + q2 * cnt];
        const float o[4] = {o4.x, o4.y, o4.z, o4.w};
        merge_partial(Mf, Lf, Of, s_cm[t + q2 * cnt], s_cl[t + q2 * cnt], o);
      }
      // the attention output is bf16: round once, multiply in fp32
      const float inv = 1.f / Lf;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        s_x[(hl * kHeadDim + d4 * 4 + e) * MB + m] =
            __builtin_bit_cast(float, (uint32_t)f32_to_bf16_rne(Of[e] * inv) << 16);
    }
    __syncthreads();
  }
  DA_TRACE(10);

  float acc[MB][8];
#pragma unroll
  for (int mm = 0; mm < MB; ++mm)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[mm][e] = 0.f;
#pragma unroll
  for (int u0 = 0; u0 < UR; u0 += 8) {
    float xr[8][MB];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int mm = 0; mm < MB; ++mm) xr[u][mm] = s_x[(rr + RPP * (u0 + u)) * MB + mm];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      float wf[8];
      unpack_bf16x8(wv[u0 + u], wf);
#pragma unroll
      for (int mm = 0; mm < MB; ++mm)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[mm][e] = fmaf(xr[u][mm], wf[e], acc[mm][e]);
    }
  }
  DA_TRACE(11);
  // the last workgroup past its wait returns the ready counters to zero
  __syncthreads();  // every thread has read s_flag
  if (t == 0) s_flag = ready_pass_last(p.sync, r, prev_pass) ? 1u : 0u;
  __syncthreads();
  ready_clear(p.sync, s_flag != 0);
  if (gave_up) {
#pragma unroll
    for (int mm = 0; mm < MB; ++mm)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[mm][e] = __builtin_nanf("");
  }

  GemvParams g{};
  g.out = p.out;
  g.part = p.proj_part;
  g.part_bytes = p.proj_part_bytes;
  g.M = p.B;
  g.K = p.Hq * kHeadDim;
  g.N = p.N;
  g.kchunk = KC;
  g.ksplit = p.chunks;
  g.tile_n = TC;
  gemv_finish<MB, TC>(g, acc, tile, chunk, &p.proj_cnt[tile * kCounterStride], smem + kFinOff);
  DA_TRACE(12);
}

template <int GP, int MB, int TC>
__global__ __launch_bounds__(kThreads, 2) void decode_step_kernel(StepParams p) {
  __shared__ __attribute__((aligned(16))) char smem[kAttnLds];
  DA_TRACE(14);
  if ((int)blockIdx.x < p.attn_wgs) {
    piece_attention<GP>(p, (int)blockIdx.x, smem);
    return;
  }
  projection<MB, TC>(p, (int)blockIdx.x - p.attn_wgs, smem);
}

template <int GP, int MB, int TC>
hipError_t launch_step(const StepParams& p, hipStream_t s) {
  decode_step_kernel<GP, MB, TC><<<dim3(p.attn_wgs + p.tiles * p.chunks), dim3(kThreads), 0, s>>>(p);
  return hipGetLastError();
}

template <int GP, int MB>
hipError_t launch_step_mb(const StepParams& p, int tile_n, hipStream_t s) {
  switch (tile_n) {
    case 128: return launch_step<GP, MB, 128>(p, s);
    case 256: return launch_step<GP, MB, 256>(p, s);
    case 512: return launch_step<GP, MB, 512>(p, s);
    default: return hipErrorInvalidValue;
  }
}

template <int GP>
hipError_t launch_step_gp(const StepParams& p, int mpad, int tile_n, hipStream_t s) {
  switch (mpad) {
    case 1: return launch_step_mb<GP, 1>(p, tile_n, s);
    case 2: return launch_step_mb<GP, 2>(p, tile_n, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool decode_step_supported(int gpad, int mpad, int tile_n) {
  const bool g_ok = gpad == 1 || gpad == 2 || gpad == 4 || gpad == 8;
  const bool m_ok = mpad == 1 || mpad == 2;
  const bool t_ok = tile_n == 128 || tile_n == 256 || tile_n == 512;
  return g_ok && m_ok && t_ok;
}

int decode_step_chunk(int tile_n) { return kRowsPerLane * kThreads / (tile_n / 8); }

hipError_t launch_decode_step(const StepParams& p, int gpad, int mpad, int tile_n, hipStream_t s) {
  switch (gpad) {
    case 1: return launch_step_gp<1>(p, mpad, tile_n, s);
    case 2: return launch_step_gp<2>(p, mpad, tile_n, s);
    case 4: return launch_step_gp<4>(p, mpad, tile_n, s);
    case 8: return launch_step_gp<8>(p, mpad, tile_n, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace da
