// GEMV building blocks shared by the projection kernel and the single-launch
// decode step: out[M, N] = x[M, K] @ w[K, N] for M < 16 on the vector ALUs.
#pragma once

#include "attn_core.hpp"
#include "kernels.hpp"

namespace da {

constexpr int kGemvThreads = 256;

// The end of a GEMV workgroup: reduce the per-lane sums of a TC-column tile
// (row lanes of a wave by shuffles, the 4 waves in LDS), then write bf16 when
// the K axis is not split, or store the fp32 partial through device-coherent
// stores; the last K-chunk of the tile to arrive adds all partials in chunk
// order (deterministic) and writes bf16. `counter` is the tile's arrival counter;
// `smem` is gemv_finish_lds<MB, TC>() bytes of LDS, 16-byte aligned, that no
// other thread of the workgroup touches meanwhile.
template <int MB, int TC>
constexpr int gemv_finish_lds() {
  return (kGemvThreads / kWave) * MB * TC * 4 + kGemvThreads * 16;
}

template <int MB, int TC>
__device__ __forceinline__ void gemv_finish(const GemvParams& p, float (&acc)[MB][8], int tile, int ks,
                                            uint32_t* counter, char* smem) {
  constexpr int kStrip = TC;
  constexpr int kLanesPerRow = TC / 8;
  auto s_red = reinterpret_cast<float (*)[MB][kStrip]>(smem);  // [wave][MB][kStrip]
  float4* const s_fin = reinterpret_cast<float4*>(smem + (kGemvThreads / kWave) * MB * kStrip * 4);
  const int t = threadIdx.x;
  const int n0 = tile * kStrip;
  // reduce the row lanes of a wave (lanes l, l^LPR, l^2LPR, ...), then the 4 waves
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = acc[m][e];
#pragma unroll
      for (int x = kLanesPerRow; x < kWave; x <<= 1) v += __shfl_xor(v, x);
      acc[m][e] = v;
    }
  const int wave = t / kWave, lane = t % kWave;
  if (lane < kLanesPerRow) {
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      *reinterpret_cast<float4*>(&s_red[wave][m][lane * 8]) = make_float4(acc[m][0], acc[m][1], acc[m][2], acc[m][3]);
      *reinterpret_cast<float4*>(&s_red[wave][m][lane * 8 + 4]) =
          make_float4(acc[m][4], acc[m][5], acc[m][6], acc[m][7]);
    }
  }
  __syncthreads();

  // 16 groups of 4 columns per activation row
  const int M = p.M;
  const int npairs = M * (kStrip / 4);
  const rsrc_t part = make_rsrc(p.part, p.part_bytes);
  for (int pr = t; pr < npairs; pr += kGemvThreads) {
    const int m = pr / (kStrip / 4), c4 = pr % (kStrip / 4);
    float4 v = *reinterpret_cast<const float4*>(&s_red[0][m][c4 * 4]);
#pragma unroll
    for (int w = 1; w < kGemvThreads / kWave; ++w) {
      const float4 o = *reinterpret_cast<const float4*>(&s_red[w][m][c4 * 4]);
      v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
    }
    const int col = n0 + c4 * 4;
    if (col >= p.N) continue;
    if (p.ksplit == 1) {
      const uint32_t w01 = (uint32_t)f32_to_bf16_rne(v.x) | ((uint32_t)f32_to_bf16_rne(v.y) << 16);
      const uint32_t w23 = (uint32_t)f32_to_bf16_rne(v.z) | ((uint32_t)f32_to_bf16_rne(v.w) << 16);
      *reinterpret_cast<uint2*>(p.out + (size_t)m * p.N + col) = make_uint2(w01, w23);
    } else {
      rsrc_st16_coherent(part, (uint32_t)((((size_t)ks * M + m) * p.N + col) * 4),
                         make_uint4(__builtin_bit_cast(uint32_t, v.x), __builtin_bit_cast(uint32_t, v.y),
                                    __builtin_bit_cast(uint32_t, v.z), __builtin_bit_cast(uint32_t, v.w)));
    }
  }
  if (p.ksplit == 1) return;
  if (!arrive_last_coherent(counter, (uint32_t)p.ksplit)) return;
  DA_TRACE(13);

  // last K-chunk of the strip: add the partials of all chunks, in chunk order per phase
  for (int base = 0; base < npairs; base += kGemvThreads) {
    const int cnt = min(npairs - base, kGemvThreads);
    const int nph = kGemvThreads / cnt;
    const int pr = base + t % cnt, ph = t / cnt;
    const int m = pr / (kStrip / 4), c4 = pr % (kStrip / 4);
    const int col = n0 + c4 * 4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (ph < nph && col < p.N) {
      for (int s0 = ph; s0 < p.ksplit; s0 += 16 * nph) {
        uint4 pv[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int sidx = min(s0 + u * nph, p.ksplit - 1);
          pv[u] = rsrc_ld16_coherent(part, (uint32_t)((((size_t)sidx * M + m) * p.N + col) * 4));
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          if (s0 + u * nph < p.ksplit) {
            v.x += __builtin_bit_cast(float, pv[u].x);
            v.y += __builtin_bit_cast(float, pv[u].y);
            v.z += __builtin_bit_cast(float, pv[u].z);
            v.w += __builtin_bit_cast(float, pv[u].w);
          }
        }
      }
    }
    s_fin[t] = v;
    __syncthreads();
    if (t < cnt && col < p.N) {
      float4 f = s_fin[t];
      for (int q2 = 1; q2 < nph; ++q2) {
        const float4 o = s_fin[t + q2 * cnt];
        f.x += o.x; f.y += o.y; f.z += o.z; f.w += o.w;
      }
      const uint32_t w01 = (uint32_t)f32_to_bf16_rne(f.x) | ((uint32_t)f32_to_bf16_rne(f.y) << 16);
      const uint32_t w23 = (uint32_t)f32_to_bf16_rne(f.z) | ((uint32_t)f32_to_bf16_rne(f.w) << 16);
      *reinterpret_cast<uint2*>(p.out + (size_t)m * p.N + col) = make_uint2(w01, w23);
    }
    __syncthreads();
  }
}


// One GEMV work item: a TC-column tile of the weight (TC*2 bytes of every row)
// times a K-chunk of rows. Lane t streams 16-byte pieces of rows rr, rr+RPP,
// ... (rr = t/(TC/8)) of column group t%(TC/8), a batch of kGemvUnroll rows at
// a time. The activation chunk (a few KiB) is requested first, then the first
// two weight batches, so that the activations arrive ahead of the weight
// stream (loads of one wave complete in order) and two batches are in flight
// while the activations are staged in LDS as fp32 (`s_x`: kchunk * MB floats).
// After that one batch is multiplied while the next is in flight.
constexpr int kGemvUnroll = 8;
constexpr int kGemvXRegs = 8;  // activation loads (8 bytes) a lane holds before the weight requests

template <int MB, int TC>
__device__ __forceinline__ void gemv_item(const GemvParams& p, int tile, int ks, float* s_x, char* fin_smem) {
  constexpr int kLanesPerRow = TC / 8;
  constexpr int kRowLanes = kGemvThreads / kLanesPerRow;
  const int n0 = tile * TC;
  const int k0 = ks * p.kchunk;
  const int kn = min(p.kchunk, p.K - k0);
  const int t = threadIdx.x;
  const int cg = t % kLanesPerRow, rr = t / kLanesPerRow;
  const int n = n0 + cg * 8;
  const bool col_ok = n < p.N;
  const uint16_t* __restrict__ wbase = p.w + (size_t)k0 * p.N + n;
  const int nbatch = (kn + kRowLanes * kGemvUnroll - 1) / (kRowLanes * kGemvUnroll);

  auto load_batch = [&](uint4 (&wv)[kGemvUnroll], int bt) {
#pragma unroll
    for (int u = 0; u < kGemvUnroll; ++u) {
      const int kk = bt * kRowLanes * kGemvUnroll + rr + kRowLanes * u;
      wv[u] = (col_ok && kk < kn) ? ld16(wbase + (size_t)kk * p.N) : make_uint4(0, 0, 0, 0);
    }
  };
  float acc[MB][8];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[m][e] = 0.f;
  auto use_batch = [&](const uint4 (&wv)[kGemvUnroll], int bt) {
#pragma unroll
    for (int u = 0; u < kGemvUnroll; ++u) {
      const int kk = bt * kRowLanes * kGemvUnroll + rr + kRowLanes * u;
      if (kk < kn) {
        float wf[8];
        unpack_bf16x8(wv[u], wf);
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          const float xm = s_x[kk * MB + m];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[m][e] = fmaf(xm, wf[e], acc[m][e]);
        }
      }
    }
  };

  // activations in groups of 4 (K and the chunk are multiples of 8): element idx
  // of the chunk is row m = idx / (kn/4), columns 4*(idx % (kn/4)) .. +4
  const rsrc_t xr = make_rsrc(p.x, (uint32_t)min((size_t)p.M * p.K * 2, (size_t)0x7fffffff));
  const int nx = MB * (kn / 4);
  auto x_load = [&](int idx) {
    const int m = idx / (kn / 4), k4 = idx % (kn / 4);
    if (idx >= nx || m >= p.M) return make_uint2(0, 0);
    const uint32_t off = (uint32_t)(((size_t)m * p.K + k0 + 4 * k4) * 2);
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(xr, (int)off, 0, 0));
  };
  auto x_store = [&](int idx, uint2 v) {
    if (idx >= nx) return;
    const int m = idx / (kn / 4), k4 = idx % (kn / 4);
    s_x[(4 * k4 + 0) * MB + m] = bf16_lo(v.x);
    s_x[(4 * k4 + 1) * MB + m] = bf16_hi(v.x);
    s_x[(4 * k4 + 2) * MB + m] = bf16_lo(v.y);
    s_x[(4 * k4 + 3) * MB + m] = bf16_hi(v.y);
  };
  uint2 xv[kGemvXRegs];
#pragma unroll
  for (int j = 0; j < kGemvXRegs; ++j) xv[j] = x_load(t + j * kGemvThreads);

  uint4 wa[kGemvUnroll], wb[kGemvUnroll];
  load_batch(wa, 0);
  if (nbatch > 1) load_batch(wb, 1);
#pragma unroll
  for (int j = 0; j < kGemvXRegs; ++j) x_store(t + j * kGemvThreads, xv[j]);
  for (int idx = t + kGemvXRegs * kGemvThreads; idx < nx; idx += kGemvThreads) x_store(idx, x_load(idx));
  __syncthreads();
  for (int bt = 0; bt < nbatch; bt += 2) {
    use_batch(wa, bt);
    if (bt + 2 < nbatch) load_batch(wa, bt + 2);
    if (bt + 1 >= nbatch) break;
    use_batch(wb, bt + 1);
    if (bt + 3 < nbatch) load_batch(wb, bt + 3);
  }
  gemv_finish<MB, TC>(p, acc, tile, ks, &p.counters[tile], fin_smem);
}

}  // namespace da
