// The stream-K attention of one workgroup.
//
// The keys of all (batch, kv head) sequences are laid end to end as 32-key
// blocks: sequence (b, h) owns ceil(L_b / 32) consecutive blocks, b-major. In
// front of every sequence sit `seq_cost` virtual blocks that hold no keys: a
// workgroup pays for each sequence it starts (finishing a piece, storing its
// partial, requesting the next piece's first tile) about as much time as it
// takes to stream a few blocks, so counting that cost in the split keeps the
// workgroups that cross sequence boundaries from finishing last. The T
// virtual blocks are cut into W equal contiguous ranges, one per workgroup,
// so ragged and uniform batches alike give every workgroup the same amount of
// work. A workgroup walks its range sequence by sequence; its waves take
// interleaved steps of the piece it is on (attn_core.hpp). A piece that is a
// whole sequence is normalised and written as bf16 at once; otherwise its
// un-normalised partial (O, running max, weight sum) goes to a workspace slot
// through device-coherent stores, and the last workgroup to finish a piece of
// that sequence (an arrival counter per sequence tells it) merges all of its
// pieces and writes the bf16 output.
//
// In the single-launch large step (kSignal), the bf16 output is written with
// device-coherent stores and every finished sequence is counted in its kv
// head's ready counter, which the projection workgroups of the same grid wait
// for.
#pragma once

#include "attn_core.hpp"
#include "kernels.hpp"

namespace da {

constexpr int kMergeBatch = 8;   // partials whose loads are in flight together in the merge
constexpr int kWideLoads = 16;   // output loads in flight per thread in the merge of many partials

// Block range [bound(i), bound(i+1)) of workgroup i of W over T blocks, and the
// workgroup that owns block x. With T < W the first T workgroups take one
// block each and the rest none.
__device__ __forceinline__ long range_bound(long i, long T, long W) { return T >= W ? (i * T) / W : (i < T ? i : T); }
__device__ __forceinline__ long range_owner(long x, long T, long W) { return T >= W ? ((x + 1) * W - 1) / T : x; }

// LDS of attn_streamk_body: sequence table, then one K/V stage per wave (the
// same bytes later hold the waves' outputs and the merge scratch; each use is
// separated from the next by a barrier).
constexpr int kAttnTableBytes = ((2 * kMaxAttnBatch + 1) * 4 + 15) / 16 * 16;
template <int NW, int HD>
constexpr int attn_streamk_lds() {
  return kAttnTableBytes + NW * Dims<HD>::kStageBytes;
}

// One workgroup's share of the stream-K attention: workgroup `wg` of `W`,
// head_dim HD; `smem` is attn_streamk_lds<NW, HD>() bytes of LDS, 16-byte aligned.
template <int GP, int NW, int D, int HD, bool kSignal = false>
__device__ __forceinline__ void attn_streamk_body(const AttnParams& p, long wg, long W, char* smem) {
  constexpr int NT = NW * kWave;
  constexpr int kStageBytes = Dims<HD>::kStageBytes;
  constexpr int kRowBytes = Dims<HD>::kRowBytes;
  constexpr int D4 = HD / 4;                // groups of 4 dims of one head
  constexpr int kWaveOut = GP * HD * 4;     // a wave's un-normalised output in its stage
  static_assert(kWaveOut + 2 * GP * 4 <= kStageBytes, "a wave's output fits its stage");
  static_assert(NT * 24 <= kStageBytes && NT * 4 <= kStageBytes, "merge scratch fits one stage");
  static_assert(NT * 24 + 2 * GP * 4 <= NW * kStageBytes, "wide-merge scratch fits the stages");
  int* const s_pre = reinterpret_cast<int*>(smem);  // virtual blocks of the sequences before batch b (per kv head)
  int* const s_len = s_pre + kMaxAttnBatch + 1;
  char* const s_stage = smem + kAttnTableBytes;
  int* const s_scan = reinterpret_cast<int*>(s_stage);
  float* const s_cm = reinterpret_cast<float*>(s_stage);
  float* const s_cl = s_cm + NT;
  float4* const s_co = reinterpret_cast<float4*>(s_cl + NT);
  auto s_o = [&](int w) { return reinterpret_cast<float (*)[HD]>(s_stage + w * kStageBytes); };
  auto s_m = [&](int w) { return reinterpret_cast<float*>(s_stage + w * kStageBytes + kWaveOut); };
  auto s_l = [&](int w) { return reinterpret_cast<float*>(s_stage + w * kStageBytes + kWaveOut + GP * 4); };

  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  const int col = lane & 15, grp = lane >> 4;
  const int B = p.B, Hkv = p.Hkv, G = p.G;
  const int cost = p.seq_cost;
  DA_TRACE(0);

  // ---- virtual blocks per sequence and their prefix sums (one scan per workgroup) ----
  const int per = (B + NT - 1) / NT;
  int local = 0;
  for (int j = 0; j < per; ++j) {
    const int b = t * per + j;
    if (b < B) {
      const int L = min(max(p.seq_lens[b], 0), p.Lmax);
      s_len[b] = L;
      local += (L + kBlockKeys - 1) / kBlockKeys + cost;
    }
  }
  // inclusive scan of the threads' sums: within each wave by shuffles, then the wave totals
  int inc = local;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(inc, off);
    if (lane >= off) inc += y;
  }
  if (lane == kWave - 1) s_scan[wave] = inc;
  __syncthreads();
  for (int w = 0; w < wave; ++w) inc += s_scan[w];
  {
    int run = inc - local;
    for (int j = 0; j < per; ++j) {
      const int b = t * per + j;
      if (b < B) {
        s_pre[b] = run;
        run += (s_len[b] + kBlockKeys - 1) / kBlockKeys + cost;
      }
    }
    if (t == NT - 1) s_pre[B] = inc;
  }
  __syncthreads();

  DA_TRACE(1);
  // Values read from LDS are per-lane to the compiler; those that are the same
  // in every lane are made wave-uniform, so that the buffer descriptors built
  // from them live in scalar registers (a per-lane descriptor would make every
  // load a loop over the distinct values).
  const long T = (long)Hkv * uniform(s_pre[B]);
  long x = range_bound(wg, T, W);
  const long xe = range_bound(wg + 1, T, W);
  const rsrc_t part_o = make_rsrc(p.part_o, p.part_o_bytes);
  const rsrc_t part_ml = make_rsrc(p.part_ml, p.part_ml_bytes);
  const rsrc_t flat_r = make_rsrc(p.flat, (uint32_t)min((size_t)p.B * p.Hq * HD * 2, (size_t)0xffffffffu));
  // the bf16 output of 4 dims (device-coherent when a projection in the same grid reads it)
  auto store4 = [&](int b, int qh, int d4, const float (&o)[4], float inv) {
    const uint32_t w01 = (uint32_t)f32_to_bf16_rne(o[0] * inv) | ((uint32_t)f32_to_bf16_rne(o[1] * inv) << 16);
    const uint32_t w23 = (uint32_t)f32_to_bf16_rne(o[2] * inv) | ((uint32_t)f32_to_bf16_rne(o[3] * inv) << 16);
    const size_t e = ((size_t)b * p.Hq + qh) * HD + d4 * 4;
    if constexpr (kSignal)
      rsrc_st8_coherent(flat_r, (uint32_t)(e * 2), make_uint2(w01, w23));
    else
      *reinterpret_cast<uint2*>(p.flat + e) = make_uint2(w01, w23);
  };
  // a sequence's output is complete: count it in its kv head's ready counter
  auto signal_ready = [&](int h) {
    if constexpr (kSignal) {
      wait_stores_done();
      __syncthreads();
      if (t < kStepReplicas)
        __hip_atomic_fetch_add(&p.head_ready[(h * kStepReplicas + t) * kCounterStride], 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
  };

  // ---- the sequence whose virtual blocks hold position y, and this range's piece of it ----
  struct Piece {
    int b, h, seg, L, nb;
    int lb0, lb1;     // real blocks [lb0, lb1) of the sequence (empty if lb0 >= lb1)
    long rs, se;      // the sequence's first real block and end block (virtual positions)
    bool whole;
  };
  auto piece_at = [&](long y) {
    Piece pc;
    int lo = 0, hi = B;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if ((long)Hkv * uniform(s_pre[mid]) <= y) lo = mid; else hi = mid;
    }
    pc.b = lo;
    const int pre_b = uniform(s_pre[pc.b]);
    const int vb = uniform(s_pre[pc.b + 1]) - pre_b;
    const long seg0 = (long)Hkv * pre_b;
    pc.h = (int)((y - seg0) / vb);
    const long vs = seg0 + (long)pc.h * vb;
    pc.rs = vs + cost;
    pc.se = vs + vb;
    pc.nb = vb - cost;
    pc.lb0 = (int)(max(y, pc.rs) - pc.rs);
    pc.lb1 = (int)(min(xe, pc.se) - pc.rs);
    pc.whole = (pc.lb0 == 0 && pc.lb1 == pc.nb);
    pc.seg = pc.b * Hkv + pc.h;
    pc.L = uniform(s_len[pc.b]);
    return pc;
  };
  auto seg_of = [&](const Piece& pc) {
    AttnSeg sg;
    const size_t kv_off = (size_t)pc.seg * p.Lmax * HD;
    sg.K = make_rsrc(p.k + kv_off, (uint32_t)pc.L * kRowBytes);
    sg.V = make_rsrc(p.v + kv_off, (uint32_t)pc.L * kRowBytes);
    sg.L = pc.L;
    sg.G = G;
    sg.scale_log2 = p.scale_log2;
    sg.scale = p.scale;
    sg.dbg = p.dbg_scores ? p.dbg_scores + ((size_t)pc.b * p.Hq + (size_t)pc.h * G) * p.Lmax : nullptr;
    sg.dbg_stride = p.Lmax;
    return sg;
  };
  auto query_of = [&](uint4 (&qa)[HD / 32], const Piece& pc) {
    load_query<HD>(qa, p.q + ((size_t)pc.b * p.Hq + (size_t)pc.h * G) * HD, G, col, grp);
  };
  // this wave's 32-key steps of a piece: the piece's keys [lb0*32, min(lb1*32, L)),
  // interleaved over the waves; every step holds at least one key of the sequence
  auto wave_steps = [&](const Piece& pc) {
    const int nstep = (min(pc.lb1 * kBlockKeys, pc.L) - pc.lb0 * kBlockKeys + kStepKeys - 1) / kStepKeys;
    return nstep > wave ? (nstep - wave + NW - 1) / NW : 0;
  };

  // ---- the merge of more partials than one batch holds ----
  // Every partial's running max and weight sum are read first (one per lane,
  // a segment of lanes per query that reduces them with shuffles) and turned
  // into per-query weights in LDS, so that the output loads of all
  // partials can be requested together: two memory trips where batches of
  // kMergeBatch take one trip each. The outputs are then added in partial
  // order, each scaled by its weight (deterministic).
  constexpr int kPairsPerThread = (GP * D4 + NT - 1) / NT;
  constexpr int kWideBatch = kWideLoads / kPairsPerThread;
  static_assert(kWideBatch >= 1, "at least one partial per batch");
  auto merge_wide = [&](int b, int h, int slot0, int P) {
    float* const w_f = s_cm;  // [P][G]: the partials' maxima, then their weights
    float* const w_l = s_cl;  // [P][G]: the partials' weight sums
    float* const w_M = reinterpret_cast<float*>(s_co + NT);  // [G]
    float* const w_L = w_M + GP;                              // [G]
    const int npairs = G * D4;
    const int cnt = min(npairs, NT), nph = NT / cnt;  // threads per (query, 4 dims) pair
    const int c = t % cnt, ph = t / cnt;
    // this thread's partials: ph, ph + nph, ... (none if ph >= nph)
    const int njp = ph < nph ? (P - ph + nph - 1) / nph : 0;
    const uint32_t no_load = (uint32_t)p.part_o_bytes;  // beyond the range: reads 0
    uint4 ov[kWideBatch][kPairsPerThread];
    auto load_batch = [&](int jb) {
#pragma unroll
      for (int u = 0; u < kWideBatch; ++u)
#pragma unroll
        for (int pp = 0; pp < kPairsPerThread; ++pp) {
          const int pr = c + pp * cnt, jj = jb + u;
          const int g = pr / D4, d4 = pr % D4;
          const uint32_t off = (jj < njp && pr < npairs)
                                   ? ((uint32_t)((slot0 + ph + jj * nph) * G + g) * HD + d4 * 4) * 4
                                   : no_load;
          ov[u][pp] = rsrc_ld16_coherent(part_o, off);
        }
    };
    // query g's partials in a segment of kSeg lanes (lane j of it: partial j) when they
    // fit, so that each maximum and weight sum is a few shuffles; else one thread per query
    constexpr int kSeg = NT / GP < kWave ? NT / GP : kWave;
    const bool in_seg = P <= kSeg;  // uniform
    const int sg = t / kSeg, sj = t % kSeg;
    const bool mine = in_seg ? (sg < G && sj < P) : t < P * G;
    uint2 ml = make_uint2(0u, 0u);
    if (mine) ml = rsrc_ld8_coherent(part_ml, (uint32_t)(in_seg ? (slot0 + sj) * G + sg : slot0 * G + t) * 8);
    load_batch(0);
    if (in_seg) {
      const float m = mine ? __builtin_bit_cast(float, ml.x) : -INFINITY;
      float M = m;
#pragma unroll
      for (int off = kSeg / 2; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
      const float f = m == -INFINITY ? 0.f : exp2f(m - M);  // an empty partial weighs nothing
      float Ls = f * (mine ? __builtin_bit_cast(float, ml.y) : 0.f);
#pragma unroll
      for (int off = kSeg / 2; off >= 1; off >>= 1) Ls += __shfl_xor(Ls, off);
      if (mine) w_f[sj * G + sg] = f;
      if (sg < G && sj == 0) {
        w_M[sg] = M;
        w_L[sg] = Ls;
      }
    } else {
      if (mine) {
        w_f[t] = __builtin_bit_cast(float, ml.x);
        w_l[t] = __builtin_bit_cast(float, ml.y);
      }
      __syncthreads();
      if (t < G) {
        float M = -INFINITY;
#pragma unroll 8
        for (int j = 0; j < P; ++j) M = fmaxf(M, w_f[j * G + t]);
        float Ls = 0.f;
#pragma unroll 8
        for (int j = 0; j < P; ++j) {
          const float m = w_f[j * G + t];
          const float f = m == -INFINITY ? 0.f : exp2f(m - M);
          Ls = fmaf(f, w_l[j * G + t], Ls);
          w_f[j * G + t] = f;
        }
        w_M[t] = M;
        w_L[t] = Ls;
      }
    }
    __syncthreads();
    DA_TRACE(5);
    float acc[kPairsPerThread][4];
#pragma unroll
    for (int pp = 0; pp < kPairsPerThread; ++pp)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[pp][e] = 0.f;
    for (int jb = 0; jb < njp; jb += kWideBatch) {
      if (jb > 0) load_batch(jb);
#pragma unroll
      for (int u = 0; u < kWideBatch; ++u)
#pragma unroll
        for (int pp = 0; pp < kPairsPerThread; ++pp) {
          const int pr = c + pp * cnt, jj = jb + u;
          if (jj < njp && pr < npairs) {
            const float f = w_f[(ph + jj * nph) * G + pr / D4];
            acc[pp][0] = fmaf(f, __builtin_bit_cast(float, ov[u][pp].x), acc[pp][0]);
            acc[pp][1] = fmaf(f, __builtin_bit_cast(float, ov[u][pp].y), acc[pp][1]);
            acc[pp][2] = fmaf(f, __builtin_bit_cast(float, ov[u][pp].z), acc[pp][2]);
            acc[pp][3] = fmaf(f, __builtin_bit_cast(float, ov[u][pp].w), acc[pp][3]);
          }
        }
    }
    DA_TRACE(7);
    auto write_pair = [&](int pr, const float (&o)[4]) {
      const int g = pr / D4, d4 = pr % D4;
      const int qh = h * G + g;
      store4(b, qh, d4, o, 1.f / w_L[g]);
      if (p.dbg_lse && d4 == 0) p.dbg_lse[(size_t)b * p.Hq + qh] = (w_M[g] + log2f(w_L[g])) * kLn2;
    };
    if (nph == 1) {
#pragma unroll
      for (int pp = 0; pp < kPairsPerThread; ++pp)
        if (c + pp * cnt < npairs) write_pair(c + pp * cnt, acc[pp]);
    } else {
      // fewer pairs than threads: one pair per thread, the threads of a pair add up in order
      s_co[t] = make_float4(acc[0][0], acc[0][1], acc[0][2], acc[0][3]);
      __syncthreads();
      if (t < cnt) {
        float o[4] = {0.f, 0.f, 0.f, 0.f};
        for (int q2 = 0; q2 < nph; ++q2) {
          const float4 v = s_co[t + q2 * cnt];
          o[0] += v.x; o[1] += v.y; o[2] += v.z; o[3] += v.w;
        }
        write_pair(t, o);
      }
    }
  };

  // Merges of many partials wait until the range is done: only the first and
  // the last piece of a range can be partial, and the last arriver of a
  // sequence is nearly always at the end of its range. After the range the
  // registers that the piece loop keeps are free for the merge's loads.
  uint32_t wide_pending = 0;  // bit 0: the range's first piece waits for its merge, bit 1: its last piece

  // ---- the end of a piece: merge the waves, then write the sequence's output or store a partial ----
  auto finish_piece = [&](const Piece& pc, AttnWaveT<HD>& aw, bool first_of_range) {
    const int b = pc.b, h = pc.h, seg = pc.seg;
    attn_wave_to_lds<GP, HD>(aw, s_o(wave), s_m(wave), s_l(wave), lane);
    __syncthreads();
    DA_TRACE(2);
    const int slot = seg + (int)wg;
    for (int idx = t; idx < G * D4; idx += NT) {
      const int g = idx / D4, d4 = idx % D4;
      float M = s_m(0)[g];
#pragma unroll
      for (int w = 1; w < NW; ++w) M = fmaxf(M, s_m(w)[g]);
      float Ls = 0.f, O[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = exp2f(s_m(w)[g] - M);
        Ls = fmaf(f, s_l(w)[g], Ls);
        const float4 o4 = *reinterpret_cast<const float4*>(&s_o(w)[g][d4 * 4]);
        O[0] = fmaf(f, o4.x, O[0]);
        O[1] = fmaf(f, o4.y, O[1]);
        O[2] = fmaf(f, o4.z, O[2]);
        O[3] = fmaf(f, o4.w, O[3]);
      }
      const int qh = h * G + g;
      if (pc.whole) {
        store4(b, qh, d4, O, 1.f / Ls);
        if (p.dbg_lse && d4 == 0) p.dbg_lse[(size_t)b * p.Hq + qh] = (M + log2f(Ls)) * kLn2;
      } else {
        const uint32_t so = ((uint32_t)(slot * G + g) * HD + d4 * 4) * 4;
        rsrc_st16_coherent(part_o, so, make_uint4(__builtin_bit_cast(uint32_t, O[0]), __builtin_bit_cast(uint32_t, O[1]),
                                                  __builtin_bit_cast(uint32_t, O[2]), __builtin_bit_cast(uint32_t, O[3])));
        if (d4 == 0)
          rsrc_st8_coherent(part_ml, (uint32_t)(slot * G + g) * 8,
                            make_uint2(__builtin_bit_cast(uint32_t, M), __builtin_bit_cast(uint32_t, Ls)));
      }
    }

    if (pc.whole) {
      signal_ready(h);
    } else {
      // (the barrier inside arrive_last_coherent also ends the reads of the waves' outputs,
      // whose bytes the merge scratch reuses)
      const long first = range_owner(pc.rs, T, W), last = range_owner(pc.se - 1, T, W);
      const int P = (int)(last - first + 1);
      const bool last_piece = arrive_last_coherent(&p.counters[seg], (uint32_t)P);
      DA_TRACE(3);
      if (last_piece) {
        // ---- the last piece merges the P partials at slots seg+first .. seg+last ----
        const int slot0 = seg + (int)first;
        const int npairs = G * D4;
        if (!kSignal && P > kMergeBatch && P * G <= NT) {
          wide_pending |= first_of_range ? 1u : 2u;
        } else {
          for (int base = 0; base < npairs; base += NT) {
            const int cnt = min(npairs - base, NT);
            const int nph = NT / cnt;
            const int pr = base + t % cnt, ph = t / cnt;
            float M = -INFINITY, Ls = 0.f, O[4] = {0.f, 0.f, 0.f, 0.f};
            if (ph < nph) {
              const int g = pr / D4, d4 = pr % D4;
              for (int j0 = ph; j0 < P; j0 += kMergeBatch * nph) {
                uint2 ml[kMergeBatch];
                uint4 ov[kMergeBatch];
#pragma unroll
                for (int u = 0; u < kMergeBatch; ++u) {
                  const int j = j0 + u * nph;
                  const uint32_t sl = (uint32_t)((slot0 + min(j, P - 1)) * G + g);
                  ml[u] = rsrc_ld8_coherent(part_ml, sl * 8);
                  ov[u] = rsrc_ld16_coherent(part_o, (sl * HD + d4 * 4) * 4);
                }
#pragma unroll
                for (int u = 0; u < kMergeBatch; ++u) {
                  if (j0 + u * nph < P) {
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
              const int g = pr / D4, d4 = pr % D4;
              const int qh = h * G + g;
              store4(b, qh, d4, Of, 1.f / Lf);
              if (p.dbg_lse && d4 == 0) p.dbg_lse[(size_t)b * p.Hq + qh] = (Mf + log2f(Lf)) * kLn2;
            }
            __syncthreads();
          }
          signal_ready(h);
        }
        DA_TRACE(4);
      }
    }
    __syncthreads();  // LDS is reused by the next piece
  };

  const long x0 = x;
  while (x < xe) {
    const Piece pc = piece_at(x);
    if (pc.lb0 < pc.lb1) {
      const AttnSeg sg = seg_of(pc);
      uint4 qa[HD / 32];
      query_of(qa, pc);
      AttnWaveT<HD> aw;
      aw.reset();
      attn_wave_steps<GP, D, HD>(aw, qa, sg, pc.lb0 + wave, NW, wave_steps(pc), pc.L, s_stage + wave * kStageBytes,
                                 lane);
      finish_piece(pc, aw, x == x0);
    }
    x = min(xe, pc.se);
  }
  // the merges that waited: a partial piece is the range's first one or holds its last block
#pragma unroll 1
  for (int k = 0; k < 2; ++k) {
    if (!(wide_pending & (1u << k))) continue;
    const Piece pc = piece_at(k == 0 ? x0 : xe - 1);
    const long first = range_owner(pc.rs, T, W), last = range_owner(pc.se - 1, T, W);
    merge_wide(pc.b, pc.h, pc.seg + (int)first, (int)(last - first + 1));
    signal_ready(pc.h);
    __syncthreads();  // the merge scratch is reused
  }
  DA_TRACE(6);
}

}  // namespace da
