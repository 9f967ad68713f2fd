// Output projection (the third matmul of one decode-attention forward in
// "PyPTO 开箱性能调优实战：Decode Attention 多 Matmul 独立 TileShape 配置
// F-16", section 代码对比: attn_output_flat x o_weight -> bf16) and the fp16
// BasicMatmul check of the CANN msKPP page "自动调优流程 / Kernel级自动调优".
//
// Both run on the MFMA GEMM below whenever K is a multiple of 32, at every M:
// a projection of a few tokens is far below the MFMA ridge, so the weight
// stream sets its pace, and the GEMM's whole-row-block loads stream it faster
// than the GEMV (measured at M = 1, 2, 4 and 8). The weight tile is
// transposed through LDS into the MFMA operand layout (B needs 8 consecutive
// k per lane, the weight is row-major in n); the activation fragment is read
// straight from global memory.
//
// The VALU GEMV (M < 16) serves a K that is not a multiple of 32 and the
// column-tile widths only it has. A workgroup owns a tile of up to 512 output
// columns (1 KiB of each weight row, read by one wave in one instruction)
// times a K-chunk of rows; every lane keeps 8 rows of 16 bytes in flight.
//
// In both, the partial sums of the K-chunks meet in the workspace through
// device-coherent stores, and the last workgroup of an output tile to arrive
// adds them in a fixed order (deterministic).
#include "gemv_core.hpp"

namespace da {

namespace {

constexpr int kThreads = 256;

// GEMV workgroup: one work item of gemv_core.hpp per workgroup.
template <int MB, int TC>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvParams p) {
  extern __shared__ float s_x[];  // [kchunk][MB]
  __shared__ __attribute__((aligned(16))) char s_fin[gemv_finish_lds<MB, TC>()];
  gemv_item<MB, TC>(p, blockIdx.x, blockIdx.y, s_x, s_fin);
}

// ---- MFMA GEMM: (16 x MT) x 128 output tile, weight rows streamed whole ----
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
// meet in LDS; K-chunk partials meet in the workspace as in the GEMV.
constexpr int kGemmCols = 128;     // output columns per workgroup
constexpr int kGemmRows = 32;      // weight rows per wave step
constexpr int kGemmWaves = kThreads / kWave;
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

template <bool F16, int MT, int D>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) char smem[kGemmLds];
  const int nt = blockIdx.x, mg = blockIdx.y, ks = blockIdx.z;
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
  const uint16_t* xrow[MT];
  bool xok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = m0 + 16 * mt + i;
    xok[mt] = m < p.M;
    xrow[mt] = p.a + (size_t)min(m, p.M - 1) * p.K + k0 + 4 * g;
  }

  const int nsteps = kn / kGemmRows;
  const int nst = nsteps > wave ? (nsteps - wave + kGemmWaves - 1) / kGemmWaves : 0;
  uint4 wt[D][8];
  uint2 xa[D][MT][2];
  auto load = [&](int j, int st) {
    const int r0 = (wave + kGemmWaves * st) * kGemmRows;
#pragma unroll
    for (int c = 0; c < 8; ++c) wt[j][c] = rsrc_ld16(wr, (uint32_t)(r0 + 4 * c) * rowb + woff);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      xa[j][mt][0] = xok[mt] ? *reinterpret_cast<const uint2*>(xrow[mt] + r0) : make_uint2(0, 0);
      xa[j][mt][1] = xok[mt] ? *reinterpret_cast<const uint2*>(xrow[mt] + r0 + 16) : make_uint2(0, 0);
    }
  };
  f32x4_t acc[MT][8];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[mt][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int j = 0; j < D; ++j)
    if (j < nst) load(j, j);
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
        if (st + D < nst) load(j, st + D);
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
  const int tile = mg * gridDim.x + nt;
  if (!arrive_last_coherent(&p.counters[tile], (uint32_t)p.ksplit)) return;
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
}

}  // namespace

template <int MB, int TC>
hipError_t launch_gemv_tc(const GemvParams& p, hipStream_t s) {
  const dim3 grid((p.N + TC - 1) / TC, p.ksplit), block(kThreads);
  const size_t shm = (size_t)p.kchunk * MB * sizeof(float);
  gemv_kernel<MB, TC><<<grid, block, shm, s>>>(p);
  return hipGetLastError();
}

template <int MB>
hipError_t launch_gemv_mb(const GemvParams& p, hipStream_t s) {
  switch (p.tile_n) {
    case 64: return launch_gemv_tc<MB, 64>(p, s);
    case 128: return launch_gemv_tc<MB, 128>(p, s);
    case 256: if constexpr (MB <= 8) return launch_gemv_tc<MB, 256>(p, s); else return hipErrorInvalidValue;
    case 512: if constexpr (MB <= 4) return launch_gemv_tc<MB, 512>(p, s); else return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemv(const GemvParams& p, int mpad, hipStream_t s) {
  switch (mpad) {
    case 1: return launch_gemv_mb<1>(p, s);
    case 2: return launch_gemv_mb<2>(p, s);
    case 4: return launch_gemv_mb<4>(p, s);
    case 8: return launch_gemv_mb<8>(p, s);
    case 16: return launch_gemv_mb<16>(p, s);
    default: return hipErrorInvalidValue;
  }
}

template <bool F16, int MT>
static hipError_t launch_gemm_mt(const GemmParams& p, hipStream_t s) {
  const dim3 grid((p.N + kGemmCols - 1) / kGemmCols, (p.M + 16 * MT - 1) / (16 * MT), p.ksplit);
  gemm_kernel<F16, MT, kGemmDepth><<<grid, dim3(kThreads), 0, s>>>(p);
  return hipGetLastError();
}

template <bool F16>
static hipError_t launch_gemm(const GemmParams& p, hipStream_t s) {
  switch (p.mtiles) {
    case 1: return launch_gemm_mt<F16, 1>(p, s);
    case 2: return launch_gemm_mt<F16, 2>(p, s);
    case 4: return launch_gemm_mt<F16, 4>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_bf16(const GemmParams& p, hipStream_t s) { return launch_gemm<false>(p, s); }
hipError_t launch_gemm_f16(const GemmParams& p, hipStream_t s) { return launch_gemm<true>(p, s); }

}  // namespace da
