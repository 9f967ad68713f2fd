// MFMA GEMM work item: a (16 x MT) x 128 output tile of C = A x B over one
// K-chunk, weight rows streamed whole. Used by the projection kernel, the
// fp16 GEMM check and the single-launch large decode step.
//
// A workgroup owns 128 output columns (256 bytes of every weight row) of 16*MT
// activation rows and a K-chunk of weight rows. Its four waves take
// interleaved 32-row steps of the chunk. A step is loaded as whole 256-byte
// row segments, four rows (1 KiB) per load instruction -- the pattern that
// streams fastest -- parked in the wave's LDS stage (rows padded by 16 bytes)
// and read back with the transposing LDS read into the MFMA B layout: lane
// (i, g) of a 16-lane group g receives rows 4g..4g+3 and 16+4g..16+4g+3 of
// column 16j+i for product j. The A operand (the activations, a few KiB that
// stay in L2) is read straight from global memory in the same k order. D
// steps per wave are in flight while one is multiplied. The four waves' sums
// meet in LDS; K-chunk partials meet in the workspace, where the last chunk of
// a tile to arrive adds them in chunk order (deterministic).
//
// With a ReadySync (the single-launch step), the item first requests the
// weight rows of its first D steps -- they do not depend on the attention --
// then waits until the kv heads whose query heads make up its K-chunk are
// finished, and reads the activations (the attention output, written by other
// workgroups of the same grid) with device-coherent loads.
#pragma once

#include "attn_core.hpp"
#include "kernels.hpp"
#include "step_sync.hpp"

namespace da {

constexpr int kGemmThreads = 256;
constexpr int kGemmCols = 128;     // output columns per workgroup
constexpr int kGemmRows = 32;      // weight rows per wave step
constexpr int kGemmWaves = kGemmThreads / kWave;
constexpr int kGemmStage = kGemmRows * kStageRow;  // one wave's LDS stage
// LDS: the waves' stages, later the waves' sums of one m-tile
constexpr int kGemmLds = kGemmWaves * kGemmStage > kGemmWaves * 16 * kGemmCols * 4 ? kGemmWaves * kGemmStage
                                                                                  : kGemmWaves * 16 * kGemmCols * 4;

template <bool F16>
__device__ __forceinline__ uint16_t to_out(float v) {
  if constexpr (F16) {
    return __builtin_bit_cast(uint16_t, (_Float16)v);
  } else {
    return f32_to_bf16_rne(v);
  }
}

template <bool F16>
__device__ __forceinline__ f32x4_t mfma16(const uint4& a, const uint4& b, f32x4_t c) {
  if constexpr (F16)
    return mfma_f16(a, b, c);
  else
    return mfma_bf16(a, b, c);
}

// Output tile (nt, mg) of K-chunk ks; `smem` is kGemmLds bytes, 16-byte aligned.
template <bool F16, int MT, int D, bool kWait>
__device__ __forceinline__ void gemm_item(const GemmParams& p, int nt, int mg, int ks, int ntiles, char* smem,
                                          const GemmWait* wt_sync) {
  const int n0 = nt * kGemmCols, m0 = mg * 16 * MT;
  const int k0 = ks * p.kchunk;
  const int kn = min(p.kchunk, p.K - k0);  // a multiple of 32
  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
  const int i = lane & 15, g = lane >> 4;
  char* const stage = smem + wave * kGemmStage;

  // the weight rows [k0, k0 + kn) from column n0 on; reads past the end return 0
  const uint32_t rowb = (uint32_t)p.N * 2;
  const rsrc_t wr = make_rsrc(p.b + (size_t)k0 * p.N + n0, (uint32_t)((size_t)kn * rowb - (size_t)n0 * 2));
  const uint32_t woff = (uint32_t)(lane >> 4) * rowb + (lane & 15) * 16;
  // activation rows of this lane (A operand row i of every m-tile); rows past M read as zero
  const rsrc_t xr = make_rsrc(p.a, (uint32_t)min((size_t)p.M * p.K * 2, (size_t)0xffffffffu));
  uint32_t xoff[MT];
  bool xok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = m0 + 16 * mt + i;
    xok[mt] = m < p.M;
    xoff[mt] = (uint32_t)(((size_t)min(m, p.M - 1) * p.K + k0 + 4 * g) * 2);
  }

  const int nsteps = kn / kGemmRows;
  const int nst = nsteps > wave ? (nsteps - wave + kGemmWaves - 1) / kGemmWaves : 0;
  uint4 wt[D][8];
  uint2 xa[D][MT][2];
  auto load_w = [&](int j, int st) {
    const int r0 = (wave + kGemmWaves * st) * kGemmRows;
#pragma unroll
    for (int c = 0; c < 8; ++c) wt[j][c] = rsrc_ld16(wr, (uint32_t)(r0 + 4 * c) * rowb + woff);
  };
  auto load_x = [&](int j, int st) {
    const int r0 = (wave + kGemmWaves * st) * kGemmRows;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if constexpr (kWait) {
        xa[j][mt][0] = xok[mt] ? rsrc_ld8_coherent(xr, xoff[mt] + r0 * 2) : make_uint2(0, 0);
        xa[j][mt][1] = xok[mt] ? rsrc_ld8_coherent(xr, xoff[mt] + (r0 + 16) * 2) : make_uint2(0, 0);
      } else {
        xa[j][mt][0] = xok[mt] ? __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                                                               xr, (int)(xoff[mt] + r0 * 2), 0, 0))
                               : make_uint2(0, 0);
        xa[j][mt][1] = xok[mt] ? __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                                                               xr, (int)(xoff[mt] + (r0 + 16) * 2), 0, 0))
                               : make_uint2(0, 0);
      }
    }
  };
  f32x4_t acc[MT][8];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[mt][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int j = 0; j < D; ++j)
    if (j < nst) load_w(j, j);
  bool gave_up = false;
  uint32_t prev_pass = 0;  // thread 0: its group's count before this workgroup passed its wait
  __shared__ uint32_t s_flag;
  if constexpr (kWait) {
    // wait for the attention output of the kv heads this K-chunk reads; the
    // count of workgroups past their wait is settled at the end (pass_tail)
    const GemmWait& ws = *wt_sync;
    const int qh_rows = ws.head_dim;
    const int h0 = (k0 / qh_rows) / ws.group, h1 = ((k0 + kn - 1) / qh_rows) / ws.group;
    if (t == 0) {
      s_flag = ready_wait(ws.sync, h0, h1, nt % kStepReplicas) ? 0u : 1u;
      prev_pass = ready_pass_sub(ws.sync, ws.waiter);
    }
    __syncthreads();
    gave_up = s_flag != 0;
  }
  // the last workgroup past its wait returns the ready counters to zero
  auto pass_tail = [&]() {
    if constexpr (kWait) {
      __syncthreads();  // s_flag is read by every thread above
      if (t == 0) s_flag = ready_pass_last(wt_sync->sync, wt_sync->waiter, prev_pass) ? 1u : 0u;
      __syncthreads();
      ready_clear(wt_sync->sync, s_flag != 0);
    }
  };
#pragma unroll
  for (int j = 0; j < D; ++j)
    if (j < nst) load_x(j, j);
  DA_TRACE(9);

  const char* bt = stage + (4 * g + (i >> 2)) * kStageRow + (i & 3) * 8;
  for (int s0 = 0; s0 < nst; s0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int st = s0 + j;
      if (st < nst) {
        wave_lds_fence();  // the previous step's LDS reads come first
        char* wp = stage + (lane >> 4) * kStageRow + (lane & 15) * 16;
#pragma unroll
        for (int c = 0; c < 8; ++c) *reinterpret_cast<uint4*>(wp + c * 4 * kStageRow) = wt[j][c];
        uint4 a[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) a[mt] = make_uint4(xa[j][mt][0].x, xa[j][mt][0].y, xa[j][mt][1].x, xa[j][mt][1].y);
        if (st + D < nst) {
          load_w(j, st + D);
          load_x(j, st + D);
        }
        wave_lds_fence();
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const uint2 v0 = lds_read_tr16(bt + jj * 32);
          const uint2 v1 = lds_read_tr16(bt + 16 * kStageRow + jj * 32);
          const uint4 b = make_uint4(v0.x, v0.y, v1.x, v1.y);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[mt][jj] = mfma16<F16>(a[mt], b, acc[mt][jj]);
        }
      }
    }
  }
  wave_lds_fence();
  DA_TRACE(10);

  // ---- the four waves' sums, one m-tile at a time; lane holds C[4g + r][16jj + i] ----
  float (*s_red)[16][kGemmCols] = reinterpret_cast<float (*)[16][kGemmCols]>(smem);  // [wave][row][col]
  const rsrc_t part = make_rsrc(p.part, p.part_bytes);
  const int col4 = (t & 31) * 4;  // 4 output columns of this thread
  const int rowq = t >> 5;         // rows rowq and rowq + 8 of the m-tile
  const int cn = n0 + col4;
  float res[MT][2][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    __syncthreads();  // the stages (and the previous m-tile's sums) are no longer read
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
#pragma unroll
      for (int r = 0; r < 4; ++r) s_red[wave][4 * g + r][16 * jj + i] = acc[mt][jj][r];
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = rowq + 8 * h;
      float4 v = *reinterpret_cast<const float4*>(&s_red[0][row][col4]);
#pragma unroll
      for (int w = 1; w < kGemmWaves; ++w) {
        const float4 o = *reinterpret_cast<const float4*>(&s_red[w][row][col4]);
        v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
      }
      // a wait that gave up leaves the tile NaN, so that the failure cannot pass for a result
      if (gave_up) v = make_float4(__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""));
      res[mt][h][0] = v.x; res[mt][h][1] = v.y; res[mt][h][2] = v.z; res[mt][h][3] = v.w;
    }
  }
  auto store_out = [&](int m, const float (&v)[4]) {
    const uint32_t w01 = (uint32_t)to_out<F16>(v[0]) | ((uint32_t)to_out<F16>(v[1]) << 16);
    const uint32_t w23 = (uint32_t)to_out<F16>(v[2]) | ((uint32_t)to_out<F16>(v[3]) << 16);
    *reinterpret_cast<uint2*>(p.c + (size_t)m * p.N + cn) = make_uint2(w01, w23);
  };
  if (p.ksplit == 1) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int m = m0 + 16 * mt + rowq + 8 * h;
        if (m < p.M && cn < p.N) store_out(m, res[mt][h]);
      }
    pass_tail();
    return;
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int m = m0 + 16 * mt + rowq + 8 * h;
      if (m < p.M && cn < p.N)
        rsrc_st16_coherent(part, (uint32_t)((((size_t)ks * p.M + m) * p.N + cn) * 4),
                           make_uint4(__builtin_bit_cast(uint32_t, res[mt][h][0]), __builtin_bit_cast(uint32_t, res[mt][h][1]),
                                      __builtin_bit_cast(uint32_t, res[mt][h][2]), __builtin_bit_cast(uint32_t, res[mt][h][3])));
    }
  const int tile = mg * ntiles + nt;
  if (!arrive_last_coherent(&p.counters[tile], (uint32_t)p.ksplit)) {
    pass_tail();
    return;
  }
  DA_TRACE(11);
  // the last K-chunk adds every chunk's partial in chunk order, 8 chunks in flight
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int m = m0 + 16 * mt + rowq + 8 * h;
      if (m >= p.M || cn >= p.N) continue;
      float v[4] = {0.f, 0.f, 0.f, 0.f};
      for (int s0 = 0; s0 < p.ksplit; s0 += 8) {
        uint4 pv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int sidx = min(s0 + u, p.ksplit - 1);
          pv[u] = rsrc_ld16_coherent(part, (uint32_t)((((size_t)sidx * p.M + m) * p.N + cn) * 4));
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (s0 + u < p.ksplit) {
            v[0] += __builtin_bit_cast(float, pv[u].x);
            v[1] += __builtin_bit_cast(float, pv[u].y);
            v[2] += __builtin_bit_cast(float, pv[u].z);
            v[3] += __builtin_bit_cast(float, pv[u].w);
          }
      }
      store_out(m, v);
    }
  DA_TRACE(12);
  pass_tail();
}

}  // namespace da
