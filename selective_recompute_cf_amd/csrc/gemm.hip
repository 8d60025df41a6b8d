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

constexpr int BM = 128, BN = 128, BK = 64;

__device__ __forceinline__ const bf16* b_row_ptr(const GemmArgs& a, int n_tile, int r) {
  if (a.epi == EPI_SWIGLU) {
    const int part = r / 64, within = r % 64;
    const int c0 = n_tile * 64 + part * 32;
    const int row = min((within < 32 ? c0 + within : c0 + within - 32), a.N - 1);
    return (const bf16*)(within < 32 ? a.B[0] : a.B[1]) + (int64_t)row * a.K;
  }
  const int col = min(n_tile * BN + r, a.N - 1);
  if (col < a.nb0) return (const bf16*)a.B[0] + (int64_t)col * a.K;
  if (col < a.nb1) return (const bf16*)a.B[1] + (int64_t)(col - a.nb0) * a.K;
  return (const bf16*)a.B[2] + (int64_t)(col - a.nb1) * a.K;
}

__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 As[2][BM * BK];
  __shared__ __attribute__((aligned(16))) bf16 Bs[2][BN * BK];
  // logical tile: M fastest, so the M tiles that share a weight tile are neighbours (same XCD)
  const int m_tiles = (a.M + BM - 1) / BM;
  const int n_tiles = a.epi == EPI_SWIGLU ? (a.N + 63) / 64 : (a.N + BN - 1) / BN;
  const int t = xcd_tile(blockIdx.x, m_tiles * n_tiles * a.splits);
  const int m_tile = t % m_tiles, n_tile = (t / m_tiles) % n_tiles, split = t / (m_tiles * n_tiles);
  const int m0 = m_tile * BM;
  const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE;
  const int wm = wave / 2, wn = wave % 2;

  const int kps = ((a.K + a.splits - 1) / a.splits + BK - 1) / BK * BK;
  const int k_begin = split * kps;
  const int k_end = min(a.K, k_begin + kps);
  const int nk = k_end > k_begin ? (k_end - k_begin + BK - 1) / BK : 0;

  // per-thread load slots: tile row p*32 + tid/8, 16-byte chunk tid%8
  const int lc = tid % 8;
  const bf16* arow[4];
  const bf16* brow[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int r = p * 32 + tid / 8;
    arow[p] = (const bf16*)a.A + (int64_t)min(m0 + r, a.M - 1) * a.lda;
    brow[p] = b_row_ptr(a, n_tile, r);
  }
  uint4 ra[4], rb[4];
  auto gload = [&](int k0) {
    const int k = k0 + lc * 8;
    const bool ok = k < k_end;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      if (ok) {
        ra[p] = *reinterpret_cast<const uint4*>(arow[p] + k);
        rb[p] = *reinterpret_cast<const uint4*>(brow[p] + k);
      } else {
        ra[p] = make_uint4(0, 0, 0, 0);
        rb[p] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = p * 32 + tid / 8;
      const int off = r * BK + ((lc ^ (r & 7)) * 8);
      *reinterpret_cast<uint4*>(&As[buf][off]) = ra[p];
      *reinterpret_cast<uint4*>(&Bs[buf][off]) = rb[p];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (nk > 0) {
    gload(k_begin);
    sstore(0);
  }
  __syncthreads();
  for (int it = 0; it < nk; ++it) {
    const int cur = it & 1;
    if (it + 1 < nk) gload(k_begin + (it + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      const int ch = kk * 4 + lane / 16;
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm * 64 + i * 16 + (lane % 16);
        af[i] = *reinterpret_cast<const bf16x8*>(&As[cur][r * BK + ((ch ^ (r & 7)) * 8)]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = wn * 64 + j * 16 + (lane % 16);
        bfr[j] = *reinterpret_cast<const bf16x8*>(&Bs[cur][r * BK + ((ch ^ (r & 7)) * 8)]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (it + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // epilogue: acc[i][j][r] = C[m0 + wm*64 + i*16 + 4*(lane/16) + r][tile col wn*64 + j*16 + lane%16]
  const int lrow = 4 * (lane / 16), lcol = lane % 16;
  if (a.epi == EPI_SWIGLU) {
    bf16* act = (bf16*)a.act;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * 64 + i * 16 + lrow + r;
        if (m >= a.M) continue;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = n_tile * 64 + wn * 32 + j * 16 + lcol;
          if (col >= a.N) continue;
          const float g = acc[i][j][r], u = acc[i][j + 2][r];
          act[(int64_t)m * a.ld_act + col] = (bf16)(g / (1.0f + expf(-g)) * u);
        }
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + wm * 64 + i * 16 + lrow + r;
      if (m >= a.M) continue;
      int64_t orow = m, rrow = m;
      if (a.epi == EPI_RESID) {
        orow = a.out_rows ? clampi(a.out_rows[m], 0, a.L - 1) : m;
        rrow = a.resid_rows ? clampi(a.resid_rows[m], 0, a.L - 1) : m;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n_tile * BN + wn * 64 + j * 16 + lcol;
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

int gemm_splits(Dt dt, int M, int N, int K, int epi, int n_cu) {
  if (dt != BF16 || epi != EPI_RESID) return 1;
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  int s = 1;
  while (s < 4 && tiles * s * 2 <= 2 * n_cu && K / (s * 2) >= 1024) s *= 2;
  return s;
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  if (a.dt == BF16) {
    const int ncols = a.epi == EPI_SWIGLU ? (a.N + 63) / 64 : (a.N + BN - 1) / BN;
    dim3 grid(ncols * ((a.M + BM - 1) / BM) * a.splits);
    hipLaunchKernelGGL(gemm_bf16_kernel, grid, dim3(256), 0, st, a);
  } else {
    dim3 grid((a.N + 63) / 64, (a.M + 63) / 64, 1);
    hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace cf
