// Projection GEMMs of the selected rows: C[M][N] = A[M][K] . B[N][K]^T (weights stored
// [out][in]). CacheBlend ("Selective Recompute Without Skipping"): the Q/K/V, O and MLP
// projections run on the gathered selected rows only.
//
// bf16 path: MFMA v_mfma_f32_16x16x32_bf16 (gfx950), fp32 accumulation. Block tile 128x128x64,
// 256 threads = 2x2 waves of 64x64 (4x4 MFMA tiles each). Global -> registers -> LDS with a
// 16-byte-chunk XOR swizzle (chunk c of row r lives at c ^ (r & 7)), double-buffered LDS, one
// barrier per K step. Epilogues: fp32 store, residual add with row gather/scatter, fused SwiGLU
// (the block's 128 B rows are 64 gate + 64 up rows of the same 64 output columns, arranged so
// every lane holds matching gate and up values), and split-K partials.
//
// fp32 path: a plain LDS-tiled FMA GEMM (64x64x16), used for fp32 models.
#include "common.h"
#include "kernels.h"

namespace cf {

// Tile configuration: BM x BN block tile, WGM x WGN waves (each a (BM/WGM) x (BN/WGN) wave tile
// of 16x16 MFMA tiles), BK = 64, PF = 1 or 2 K steps of global loads in flight (register sets).
template <int BM_, int BN_, int WGM_, int WGN_, int PF_, int MINB_, int SWZ_ = 0>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_, PF = PF_, MINB = MINB_;
  // LDS swizzle of the 16-byte chunks of a 128-byte tile row: chunk c of row r is stored at
  // c ^ (r & 7) (SWZ 0) or c ^ ((r >> 1) & 7) (SWZ 1, rows paired across the two bank halves)
  static constexpr int SWZ = SWZ_;
  __device__ static __forceinline__ int swz(int r) { return SWZ ? ((r >> 1) & 7) : (r & 7); }
  static constexpr int BK = 64;
  static constexpr int THREADS = WGM * WGN * WAVE;
  static constexpr int TM = BM / WGM, TN = BN / WGN;  // wave tile
  static constexpr int FM = TM / 16, FN = TN / 16;    // MFMA tiles per wave
  static constexpr int ROWS_PER_PASS = THREADS / 8;   // 8 threads (16 B each) per 128-byte row
  static constexpr int AP = BM / ROWS_PER_PASS, BP = BN / ROWS_PER_PASS;
  static_assert(BM % ROWS_PER_PASS == 0 && BN % ROWS_PER_PASS == 0, "tile rows must split evenly");
  static_assert(TM % 16 == 0 && TN % 32 == 0, "wave tile must be a multiple of 16 x 32");
};

// Weight row feeding tile row r of column tile n_tile. SwiGLU tiles interleave gate and up rows:
// wave column wn owns tile rows [wn*TN, (wn+1)*TN), the first half gate rows and the second half
// the up rows of the same TN/2 output columns.
template <class C>
__device__ __forceinline__ const bf16* b_row_ptr(const GemmArgs& a, int n_tile, int r) {
  if (a.epi == EPI_SWIGLU) {
    const int part = r / C::TN, within = r % C::TN, h = C::TN / 2;
    const int c0 = n_tile * (C::BN / 2) + part * h;
    const int row = min(within < h ? c0 + within : c0 + within - h, a.N - 1);
    return (const bf16*)(within < h ? a.B[0] : a.B[1]) + (int64_t)row * a.K;
  }
  const int col = min(n_tile * C::BN + r, a.N - 1);
  if (col < a.nb0) return (const bf16*)a.B[0] + (int64_t)col * a.K;
  if (col < a.nb1) return (const bf16*)a.B[1] + (int64_t)(col - a.nb0) * a.K;
  return (const bf16*)a.B[2] + (int64_t)(col - a.nb1) * a.K;
}

template <class C>
__device__ __forceinline__ int n_tiles_of(const GemmArgs& a) {
  return a.epi == EPI_SWIGLU ? (a.N + C::BN / 2 - 1) / (C::BN / 2) : (a.N + C::BN - 1) / C::BN;
}

template <class C>
__global__ __launch_bounds__(C::THREADS, C::MINB) void gemm_bf16_kernel(GemmArgs a) {
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, AP = C::AP, BP = C::BP, FM = C::FM, FN = C::FN;
  __shared__ __attribute__((aligned(16))) bf16 As[2][BM * BK];
  __shared__ __attribute__((aligned(16))) bf16 Bs[2][BN * BK];
  // logical tile: M fastest, so the M tiles that share a weight tile are neighbours (same XCD)
  const int m_tiles = (a.M + BM - 1) / BM;
  const int n_tiles = n_tiles_of<C>(a);
  const int t = xcd_tile(blockIdx.x, m_tiles * n_tiles * a.splits);
  const int m_tile = t % m_tiles, n_tile = (t / m_tiles) % n_tiles, split = t / (m_tiles * n_tiles);
  const int m0 = m_tile * BM;
  const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE;
  const int wm = wave / C::WGN, wn = wave % C::WGN;

  const int kps = ((a.K + a.splits - 1) / a.splits + BK - 1) / BK * BK;
  const int k_begin = split * kps;
  const int k_end = min(a.K, k_begin + kps);
  const int nk = k_end > k_begin ? (k_end - k_begin + BK - 1) / BK : 0;

  // per-thread load slots: tile row p * ROWS_PER_PASS + tid / 8, 16-byte chunk tid % 8
  const int lc = tid % 8, lr = tid / 8;
  const bf16* arow[AP];
  const bf16* brow[BP];
#pragma unroll
  for (int p = 0; p < AP; ++p) arow[p] = (const bf16*)a.A + (int64_t)min(m0 + p * C::ROWS_PER_PASS + lr, a.M - 1) * a.lda;
#pragma unroll
  for (int p = 0; p < BP; ++p) brow[p] = b_row_ptr<C>(a, n_tile, p * C::ROWS_PER_PASS + lr);

  uint4 ra0[AP], rb0[BP], ra1[AP], rb1[BP];
  auto gload = [&](uint4* ra, uint4* rb, int step) {
    const int k = k_begin + step * BK + lc * 8;
    const bool ok = k < k_end;
#pragma unroll
    for (int p = 0; p < AP; ++p) ra[p] = ok ? *reinterpret_cast<const uint4*>(arow[p] + k) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int p = 0; p < BP; ++p) rb[p] = ok ? *reinterpret_cast<const uint4*>(brow[p] + k) : make_uint4(0, 0, 0, 0);
  };
  auto sstore = [&](const uint4* ra, const uint4* rb, int buf) {
#pragma unroll
    for (int p = 0; p < AP; ++p) {
      const int r = p * C::ROWS_PER_PASS + lr;
      *reinterpret_cast<uint4*>(&As[buf][r * BK + ((lc ^ C::swz(r)) * 8)]) = ra[p];
    }
#pragma unroll
    for (int p = 0; p < BP; ++p) {
      const int r = p * C::ROWS_PER_PASS + lr;
      *reinterpret_cast<uint4*>(&Bs[buf][r * BK + ((lc ^ C::swz(r)) * 8)]) = rb[p];
    }
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int cur) {
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      const int ch = kk * 4 + lane / 16;
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm * C::TM + i * 16 + (lane % 16);
        af[i] = *reinterpret_cast<const bf16x8*>(&As[cur][r * BK + ((ch ^ C::swz(r)) * 8)]);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = wn * C::TN + j * 16 + (lane % 16);
        bfr[j] = *reinterpret_cast<const bf16x8*>(&Bs[cur][r * BK + ((ch ^ C::swz(r)) * 8)]);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };

  if constexpr (C::PF == 1) {
    if (nk > 0) {
      gload(ra0, rb0, 0);
      sstore(ra0, rb0, 0);
    }
    __syncthreads();
    for (int it = 0; it < nk; ++it) {
      if (it + 1 < nk) gload(ra0, rb0, it + 1);
      compute(it & 1);
      if (it + 1 < nk) sstore(ra0, rb0, (it + 1) & 1);
      __syncthreads();
    }
  } else {
    // two K steps of loads in flight: step s lives in register set s % 2 from its load (two
    // iterations ahead) until it is stored to LDS at the end of the preceding iteration
    if (nk > 0) gload(ra0, rb0, 0);
    if (nk > 1) gload(ra1, rb1, 1);
    if (nk > 0) sstore(ra0, rb0, 0);
    __syncthreads();
    auto body = [&](int it, uint4* la, uint4* lb, const uint4* sa, const uint4* sb) {
      if (it + 2 < nk) gload(la, lb, it + 2);
      compute(it & 1);
      if (it + 1 < nk) sstore(sa, sb, (it + 1) & 1);
      __syncthreads();
    };
    for (int it = 0; it < nk; it += 2) {
      body(it, ra0, rb0, ra1, rb1);
      if (it + 1 < nk) body(it + 1, ra1, rb1, ra0, rb0);
    }
  }

  // epilogue: acc[i][j][r] = C[m0 + wm*TM + i*16 + 4*(lane/16) + r][tile col wn*TN + j*16 + lane%16]
  const int lrow = 4 * (lane / 16), lcol = lane % 16;
  if (a.epi == EPI_SWIGLU) {
    bf16* act = (bf16*)a.act;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * C::TM + i * 16 + lrow + r;
        if (m >= a.M) continue;
#pragma unroll
        for (int j = 0; j < FN / 2; ++j) {
          const int col = n_tile * (BN / 2) + wn * (C::TN / 2) + j * 16 + lcol;
          if (col >= a.N) continue;
          const float g = acc[i][j][r], u = acc[i][j + FN / 2][r];
          act[(int64_t)m * a.ld_act + col] = (bf16)(g / (1.0f + expf(-g)) * u);
        }
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + wm * C::TM + i * 16 + lrow + r;
      if (m >= a.M) continue;
      int64_t orow = m, rrow = m;
      if (a.epi == EPI_RESID) {
        orow = a.out_rows ? clampi(a.out_rows[m], 0, a.L - 1) : m;
        rrow = a.resid_rows ? clampi(a.resid_rows[m], 0, a.L - 1) : m;
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = n_tile * BN + wn * C::TN + j * 16 + lcol;
        if (col >= a.N) continue;
        const float v = acc[i][j][r];
        if (a.epi == EPI_F32)
          a.C[(int64_t)m * a.ldc + col] = v;
        else if (a.epi == EPI_PARTIAL)
          a.C[((int64_t)split * a.M + m) * a.ldc + col] = v;
        else
          a.out[orow * a.N + col] = a.resid[rrow * a.N + col] + v;
      }
    }
}

template <class C>
hipError_t launch_gemm_cfg(const GemmArgs& a, hipStream_t st) {
  const int tiles = ((a.M + C::BM - 1) / C::BM) *
                    (a.epi == EPI_SWIGLU ? (a.N + C::BN / 2 - 1) / (C::BN / 2) : (a.N + C::BN - 1) / C::BN) * a.splits;
  hipLaunchKernelGGL(gemm_bf16_kernel<C>, dim3(tiles), dim3(C::THREADS), 0, st, a);
  return hipGetLastError();
}

using GemmSmall = TileCfg<128, 128, 2, 2, 2, 2>;  // 2 blocks per CU
using GemmBig = TileCfg<256, 256, 4, 4, 1, 1>;    // 16 waves, 1 block per CU

// ----------------------------------------------------------------------------- fp32 path
__device__ __forceinline__ const float* b_row_ptr_f32(const GemmArgs& a, int col) {
  col = min(col, a.N - 1);
  if (col < a.nb0) return (const float*)a.B[0] + (int64_t)col * a.K;
  if (col < a.nb1) return (const float*)a.B[1] + (int64_t)(col - a.nb0) * a.K;
  return (const float*)a.B[2] + (int64_t)(col - a.nb1) * a.K;
}

__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a) {
  constexpr int T = 64, TK = 16;
  __shared__ float As[TK][T + 4];
  __shared__ float Bs[TK][T + 4];
  const int n0 = blockIdx.x * T, m0 = blockIdx.y * T;
  const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < a.K; k0 += TK) {
    for (int e = tid; e < T * TK; e += 256) {
      const int r = e / TK, kk = e % TK, k = k0 + kk;
      const int m = min(m0 + r, a.M - 1);
      As[kk][r] = k < a.K ? ((const float*)a.A)[(int64_t)m * a.lda + k] : 0.f;
      Bs[kk][r] = k < a.K ? b_row_ptr_f32(a, n0 + r)[k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += av[i] * bv[j];
    }
    __syncthreads();
  }
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= a.M) continue;
    int64_t orow = m, rrow = m;
    if (a.epi == EPI_RESID) {
      orow = a.out_rows ? clampi(a.out_rows[m], 0, a.L - 1) : m;
      rrow = a.resid_rows ? clampi(a.resid_rows[m], 0, a.L - 1) : m;
    }
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (col >= a.N) continue;
      if (a.epi == EPI_F32)
        a.C[(int64_t)m * a.ldc + col] = acc[i][j];
      else
        a.out[orow * a.N + col] = a.resid[rrow * a.N + col] + acc[i][j];
    }
  }
}

GemmPlan gemm_plan(Dt dt, int M, int N, int K, bool swiglu, bool allow_split, int n_cu) {
  GemmPlan best{GEMM_SMALL, 1};
  if (dt != BF16) return best;
  // relative time of one configuration: rounds of resident blocks x work of one block /
  // per-block rate (GemmBig runs one block per CU at 1.28x the per-CU rate of two GemmSmall
  // blocks, measured on the projection shapes); ties go to fewer splits
  double best_cost = 1e300;
  const int cols = swiglu ? 2 * N : N;
  for (int c = 0; c < 2; ++c) {
    const int bm = c ? GemmBig::BM : GemmSmall::BM, bn = c ? GemmBig::BN : GemmSmall::BN;
    const int per_cu = c ? 1 : 2;
    const double rate = c ? 1.28 : 1.0;
    const long tiles = (long)((M + bm - 1) / bm) * ((cols + bn - 1) / bn);
    for (int sp = 1; sp <= (allow_split ? 4 : 1); ++sp) {
      if (sp > 1 && K / sp < 512) break;
      const long slots = (long)n_cu * per_cu;
      const long rounds = (tiles * sp + slots - 1) / slots;
      const double cost = rounds * (double)bm * bn * ((double)K / sp) * per_cu / rate * (1.0 + 0.02 * (sp - 1));
      if (cost < best_cost * 0.999) {
        best_cost = cost;
        best = GemmPlan{c, sp};
      }
    }
  }
  return best;
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  if (a.dt == BF16) {
    return a.cfg == GEMM_BIG ? launch_gemm_cfg<GemmBig>(a, st) : launch_gemm_cfg<GemmSmall>(a, st);
  } else {
    dim3 grid((a.N + 63) / 64, (a.M + 63) / 64, 1);
    hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace cf
