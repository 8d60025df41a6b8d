// Projection GEMMs of the selected rows: C[M][N] = A[M][K] . B[N][K]^T (weights stored
// [out][in]). CacheBlend ("Selective Recompute Without Skipping"): the Q/K/V, O and MLP
// projections run on the gathered selected rows only.
//
// bf16 path: MFMA v_mfma_f32_16x16x32_bf16 (gfx950), fp32 accumulation, BK = 64. The main kernel
// (gemm_bf16_dtl) streams A and B tiles straight from global memory into a ring of LDS stages
// (direct-to-LDS loads, no register staging), block tiles {128, 96, 64} x 256 with 8 waves; the
// register-staged kernel (gemm_bf16_kernel, 128x128) covers K % 64 != 0. Both keep tiles in LDS
// with a 16-byte-chunk XOR swizzle (chunk c of row r lives at c ^ (r & 7)). Epilogues: fp32
// store, residual add with row gather/scatter, fused SwiGLU (a block's B rows are gate and up
// rows of the same output columns, arranged so every lane holds matching gate and up values),
// and split-K partials.
//
// fp32 path: a plain LDS-tiled FMA GEMM (64x64x16), used for fp32 models.
#include <type_traits>
#include <utility>

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
  static constexpr int MT = 16;                       // MFMA tile edge (v_mfma_f32_16x16x32_bf16)
  static constexpr int FM = TM / 16, FN = TN / 16;    // MFMA tiles per wave
  typedef f32x4 Acc;
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

// Accumulator element e of MFMA tile (i, j) sits at wave-tile row i*MT + acc_row(e, lane), column
// j*MT + lane % MT: for the 16x16 tiles rows 4*(lane/16) + e (e < 4); for the 32x32 tiles rows
// 8*(e/4) + 4*(lane/32) + e%4 (e < 16).
template <int MT>
__device__ __forceinline__ int acc_row(int e, int lane) {
  return MT == 16 ? 4 * (lane / 16) + e : 8 * (e / 4) + 4 * (lane / 32) + (e % 4);
}

template <class C>
__device__ __forceinline__ void epilogue(const GemmArgs& a, typename C::Acc (&acc)[C::FM][C::FN], int m0, int n_tile,
                                         int split, int wm, int wn, int lane) {
  constexpr int BN = C::BN, FM = C::FM, FN = C::FN, MT = C::MT, NE = MT * MT / WAVE;
  static_assert(FN % 2 == 0, "SwiGLU pairs gate and up tiles within a wave");
  const int lcol = lane % MT;
  if (a.epi == EPI_SWIGLU) {
    bf16* act = (bf16*)a.act;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const int m = m0 + wm * C::TM + i * MT + acc_row<MT>(e, lane);
        if (m >= a.M) continue;
#pragma unroll
        for (int j = 0; j < FN / 2; ++j) {
          const int col = n_tile * (BN / 2) + wn * (C::TN / 2) + j * MT + lcol;
          if (col >= a.N) continue;
          const float g = acc[i][j][e], u = acc[i][j + FN / 2][e];
          act[(int64_t)m * a.ld_act + col] = (bf16)(g / (1.0f + expf(-g)) * u);
        }
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const int m = m0 + wm * C::TM + i * MT + acc_row<MT>(e, lane);
      if (m >= a.M) continue;
      int64_t orow = m, rrow = m;
      if (a.epi == EPI_RESID) {
        orow = a.out_rows ? clampi(a.out_rows[m], 0, a.L - 1) : m;
        rrow = a.resid_rows ? clampi(a.resid_rows[m], 0, a.L - 1) : m;
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = n_tile * BN + wn * C::TN + j * MT + lcol;
        if (col >= a.N) continue;
        const float v = acc[i][j][e];
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

  // Global loads are unconditional (a per-lane predicate would turn each into an exec-masked
  // branch, and the wait-count insertion then drains every load before the next LDS store,
  // collapsing the prefetch depth): the column is clamped into the row (K >= 8, K % 8 == 0) and
  // chunks past the step's K range are zeroed when they are stored to LDS. A register set is
  // one vector value (AP + BP 16-byte chunks), passed by value so it never leaves registers.
  typedef uint32_t RVec __attribute__((ext_vector_type(4 * (AP + BP))));
  auto gload = [&](int step) __attribute__((always_inline)) {
    const int k = min(k_begin + step * BK + lc * 8, a.K - 8);
    RVec r;
#pragma unroll
    for (int p = 0; p < AP + BP; ++p) {
      const uint4 x = *reinterpret_cast<const uint4*>((p < AP ? arow[p] : brow[p - AP]) + k);
      r[4 * p] = x.x, r[4 * p + 1] = x.y, r[4 * p + 2] = x.z, r[4 * p + 3] = x.w;
    }
    return r;
  };
  auto sstore = [&](RVec r, int buf, int step) __attribute__((always_inline)) {
    const bool full = k_begin + (step + 1) * BK <= k_end;  // uniform: the whole step is in range
    const bool ok = full || k_begin + step * BK + lc * 8 < k_end;
#pragma unroll
    for (int p = 0; p < AP + BP; ++p) {
      const int row = (p < AP ? p : p - AP) * C::ROWS_PER_PASS + lr;
      bf16* dst = (p < AP ? As[buf] : Bs[buf]) + row * BK + ((lc ^ C::swz(row)) * 8);
      *reinterpret_cast<uint4*>(dst) = ok ? make_uint4(r[4 * p], r[4 * p + 1], r[4 * p + 2], r[4 * p + 3])
                                          : make_uint4(0, 0, 0, 0);
    }
  };

  typename C::Acc acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = typename C::Acc{};

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

  // The loads inside the loop are branch-free too (a branch around them makes the wait counts
  // conservative at the join): past the last step they re-load the last step, which is never
  // stored again.
  const int last = max(nk - 1, 0);
  if constexpr (C::PF == 1) {
    RVec r0 = gload(0);
    sstore(r0, 0, 0);
    __syncthreads();
    for (int it = 0; it < nk; ++it) {
      r0 = gload(min(it + 1, last));
      compute(it & 1);
      if (it + 1 < nk) sstore(r0, (it + 1) & 1, it + 1);
      __syncthreads();
    }
  } else {
    // two K steps of loads in flight: step s is loaded into set s % 2 two steps ahead and stored
    // to LDS buffer s % 2 at the end of step s - 1
    RVec r0 = gload(0), r1 = gload(min(1, last));
    sstore(r0, 0, 0);
    __syncthreads();
    int it = 0;
    for (; it + 1 < nk; it += 2) {
      r0 = gload(min(it + 2, last));
      compute(0);
      sstore(r1, 1, it + 1);
      __syncthreads();
      r1 = gload(min(it + 3, last));
      compute(1);
      if (it + 2 < nk) sstore(r0, 0, it + 2);
      __syncthreads();
    }
    if (it < nk) compute(0);  // odd step count: the last step sits in buffer 0
  }

  epilogue<C>(a, acc, m0, n_tile, split, wm, wn, lane);
}

// ----------------------------------------------------------------------------- direct-to-LDS
// Ring of S LDS stages filled by direct global->LDS 16-byte loads (global_load_lds_dwordx4: lane
// l of a wave writes bytes [16 l, 16 l + 16) after the wave-uniform LDS base), so the K steps in
// flight cost no registers and no LDS store instructions. One wave instruction fills 1 KB: 8 tile
// rows of 128 bytes (BK = 64) or 16 rows of 64 bytes (BK = 32). The XOR swizzle is applied on the
// global side: the lane that lands in chunk slot c' of row r fetches global chunk c' ^ swz(r).
// Requires K % BK == 0.
// Each K step has two halves of BK/2 (one or two MFMA k sub-steps each). Per K step s:
//   [S > 2: load step s + S - 1 into the stage of step s - 1] | read half 1 of step s | MFMAs half 0
//   wait for this wave's loads of step s + 1 and its own LDS reads | barrier
//   [S = 2: load step s + 2 into the stage of step s] | read half 0 of step s + 1 | MFMAs half 1
// The barrier publishes step s + 1 (every wave waited for its own loads of it) and retires all
// reads of step s's stage before any wave issues the load that overwrites it.
template <int BM_, int BN_, int WGM_, int WGN_, int S_, int MINB_, int MT_ = 32, int BK_ = 64>
struct DtlCfg {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_, S = S_, MINB = MINB_, SWZ = 0, BK = BK_;
  static constexpr int W = WGM * WGN, THREADS = W * WAVE;
  static constexpr int TM = BM / WGM, TN = BN / WGN;
  // MFMA shape: MT = 32 (v_mfma_f32_32x32x16_bf16, k 16 per instruction) or 16
  // (v_mfma_f32_16x16x32_bf16, k 32 per instruction)
  static constexpr int MT = MT_, KI = MT == 32 ? 16 : 32;
  static constexpr int HK = BK / 2, NSUB = HK / KI;  // k per half step; MFMA k sub-steps per half
  static constexpr int CH = BK / 8;                  // 16-byte chunks per LDS row
  static constexpr int RG = 512 / BK;                // rows per 1 KB load group
  static constexpr int FM = TM / MT, FN = TN / MT;
  typedef typename std::conditional<MT == 32, f32x16, f32x4>::type Acc;
  static constexpr int G = (BM + BN) / RG;         // load groups per K step
  static constexpr int NL = (G + W - 1) / W;       // load instructions per wave per K step
  static constexpr int STAGE = (BM + BN) * BK;     // bf16 elements per stage
  static_assert(MT == 16 || MT == 32, "MFMA tile edge");
  static_assert(BK == 64 || BK == 32, "K step");
  static_assert(NSUB >= 1, "a half step holds at least one MFMA k sub-step");
  static_assert(TM % MT == 0 && TN % MT == 0, "wave tile must be a multiple of the MFMA tile");
  static_assert(BM % RG == 0 && BN % RG == 0 && NL * W - G <= W, "whole load groups");
  static_assert(S >= 2 && (S - 1) * NL <= 63, "in-flight loads must fit the vmcnt counter");
  // Conflict-free fragment reads: 8 or 16 consecutive lanes read consecutive rows at one logical
  // chunk. 128-byte rows: r & 7 gives 8 consecutive rows 8 distinct chunks. 64-byte rows: rows
  // r, r + 2, r + 4, r + 6 (same half of a 128-byte bank line) and r, r + 4, r + 8, r + 12 (same
  // quarter of a 256-byte line) each get 4 distinct chunks.
  __device__ static __forceinline__ int swz(int r) { return BK == 64 ? (r & 7) : (((r >> 1) ^ (r >> 3)) & 3); }
};

// s_waitcnt immediate (gfx9 encoding): vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]
#define CF_WAITCNT(vm, lgkm) ((((vm) & 15) | (((vm) >> 4) << 14)) | 0x70 | (((lgkm) & 15) << 8))

// Scheduling pattern for NF LDS reads among NM MFMAs: read q is followed by MFMAs
// [NM*q/NF, NM*(q+1)/NF) (the builtin needs constant arguments, hence the fold over q).
template <int NM, int NF, int ID, int... Q>
__device__ __forceinline__ void sched_interleave(std::integer_sequence<int, Q...>) {
  ((__builtin_amdgcn_sched_group_barrier(0x100, 1, ID),
    __builtin_amdgcn_sched_group_barrier(0x008, NM * (Q + 1) / NF - NM * Q / NF, ID)),
   ...);
}

template <class C>
__global__ __launch_bounds__(C::THREADS, C::MINB) void gemm_bf16_dtl(GemmArgs a) {
  constexpr int BM = C::BM, BK = C::BK, FM = C::FM, FN = C::FN, S = C::S, NL = C::NL, W = C::W;
  __shared__ __attribute__((aligned(1024))) bf16 smem[S * C::STAGE];  // stage: BM A rows, then BN B rows
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
  const int nk = k_end > k_begin ? (k_end - k_begin) / BK : 0;

  // load q of this wave covers combined tile rows [g*RG, (g + 1)*RG), g = q*W + wave (A rows
  // first, then B rows). When the groups do not split evenly over the waves, a wave's surplus slot
  // repeats its previous group (same bytes to the same place), so every wave issues NL loads per
  // step and the wait counts hold for all of them.
  auto group = [&](int q) { const int g = q * W + wave; return g < C::G ? g : g - W; };
  const bf16* src[NL];
#pragma unroll
  for (int q = 0; q < NL; ++q) {
    const int row = group(q) * C::RG + lane / C::CH;
    const int r = row < BM ? row : row - BM;
    const int c = (lane % C::CH) ^ C::swz(r);
    const bf16* base = row < BM ? (const bf16*)a.A + (int64_t)min(m0 + r, a.M - 1) * a.lda : b_row_ptr<C>(a, n_tile, r);
    src[q] = base + k_begin + c * 8;
  }
  // The load is issued from inline assembly: with the compiler builtin, the wait-count pass
  // treats the pending LDS write as unordered and drains every outstanding LDS read before the
  // next MFMA, which serialises the fragment reads with the matrix cores. The pass does not see
  // these loads, so the waits for them are explicit (CF_WAITCNT below); its own vmcnt waits stay
  // correct because vector-memory loads retire in order. M0 is written only here, right before
  // each load (the compiler reserves M0 and does not use it in this kernel).
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) bf16*)smem;
  auto issue = [&](int step) __attribute__((always_inline)) {
    const int stage = step % S;
#pragma unroll
    for (int q = 0; q < NL; ++q) {
      const uint32_t dst = __builtin_amdgcn_readfirstlane(lds0 + 2u * (uint32_t)(stage * C::STAGE + group(q) * C::RG * BK));
      asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src[q] + step * BK), "s"(dst) : "memory", "m0");
    }
  };

  // operands of one half step: NSUB sub-steps x (FM A + FN B) fragments of 8 bf16 per lane
  constexpr int NSUB = C::NSUB, MT = C::MT, NF = NSUB * (FM + FN);
  typedef uint32_t FVec __attribute__((ext_vector_type(4 * NF)));
  typedef uint32_t U4 __attribute__((ext_vector_type(4)));
  auto fread = [&](int stage, int kk) __attribute__((always_inline)) {
    const bf16* st = smem + stage * C::STAGE;
    FVec f;
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      const int ch = kk * (C::HK / 8) + sub * (C::KI / 8) + lane / MT;
#pragma unroll
      for (int q = 0; q < FM + FN; ++q) {
        const int r = q < FM ? wm * C::TM + q * MT + (lane % MT) : BM + wn * C::TN + (q - FM) * MT + (lane % MT);
        const int rr = q < FM ? r : r - BM;
        const U4 x = *reinterpret_cast<const U4*>(st + r * BK + ((ch ^ C::swz(rr)) * 8));
        const int o = 4 * (sub * (FM + FN) + q);
        f[o] = x[0], f[o + 1] = x[1], f[o + 2] = x[2], f[o + 3] = x[3];
      }
    }
    return f;
  };
  typename C::Acc acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = typename C::Acc{};
  auto fmma = [&](FVec f) __attribute__((always_inline)) {
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int oa = 4 * (sub * (FM + FN) + i), ob = 4 * (sub * (FM + FN) + FM + j);
          const U4 av = {f[oa], f[oa + 1], f[oa + 2], f[oa + 3]};
          const U4 bv = {f[ob], f[ob + 1], f[ob + 2], f[ob + 3]};
          if constexpr (MT == 32)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                               __builtin_bit_cast(bf16x8, bv), acc[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                               __builtin_bit_cast(bf16x8, bv), acc[i][j], 0, 0, 0);
        }
  };
  // a raw barrier: no fence, so the compiler adds no drain of the in-flight LDS loads; the
  // empty asm statements keep LDS accesses from moving across it
  auto barrier = []() __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  if (nk > 0) {
    const int last = nk - 1;
    // Two stages: a stage is refilled right after the barrier that retires its reads, which
    // gives its load a whole step to land. More stages: it is refilled at the top of the next
    // step (issuing right after the barrier delays the next half's fragment reads and measured
    // slower), a load then has S - 1.5 steps to land.
    constexpr bool EARLY = S == 2;
    // past the last step the loads repeat the last step into its own stage (same bytes to the
    // same place), which keeps the per-step load count (and so the wait counts) uniform
#pragma unroll
    for (int p = 0; p < (EARLY ? S : S - 1); ++p) issue(min(p, last));
    __builtin_amdgcn_s_waitcnt(CF_WAITCNT((EARLY ? S - 1 : S - 2) * NL, 15));
    barrier();
    // The next half's fragment reads are spread evenly between this half's MFMAs (one LDS read,
    // then its share of the NM MFMAs, repeated) rather than issued as one block ahead of them.
    constexpr int NM = NSUB * FM * FN;
    auto interleave = [](auto sync_id) __attribute__((always_inline)) {
      sched_interleave<NM, NF, decltype(sync_id)::value>(std::make_integer_sequence<int, NF>{});
    };
    // the 256-row tile (full-row layers) keeps the single path: at its 256 registers a second
    // path makes the compiler spill
    constexpr bool SKIP = BM <= 128;
    if (!SKIP || m0 + wm * C::TM < a.M) {  // wave-uniform: some of this wave's rows are real
      FVec f0 = fread(0, 0), f1;
      for (int s = 0; s < nk; ++s) {
        if constexpr (!EARLY) issue(min(s + S - 1, last));  // the stage step s - 1 used
        f1 = fread(s % S, 1);
        fmma(f0);
        interleave(std::integral_constant<int, 0>{});
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(CF_WAITCNT((S - 2) * NL, 0));
        barrier();
        if constexpr (EARLY) issue(min(s + S, last));  // the stage step s used
        f0 = fread((s + 1) % S, 0);
        fmma(f1);
        interleave(std::integral_constant<int, 1>{});
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if constexpr (SKIP) {
      // every row of this wave lies past M (the padding of the last row tile): it still issues
      // its share of the tile loads and meets every barrier, but reads no fragments and runs no
      // MFMAs, so the matrix cores of its SIMD are left to the other waves and blocks (its
      // accumulators stay zero, and the epilogue skips rows past M)
      for (int s = 0; s < nk; ++s) {
        if constexpr (!EARLY) issue(min(s + S - 1, last));
        __builtin_amdgcn_s_waitcnt(CF_WAITCNT((S - 2) * NL, 0));
        barrier();
        if constexpr (EARLY) issue(min(s + S, last));
      }
    }
    __builtin_amdgcn_s_waitcnt(CF_WAITCNT(0, 0));  // drain the trailing repeat loads
  }
  epilogue<C>(a, acc, m0, n_tile, split, wm, wn, lane);
}

template <class C>
hipError_t launch_gemm_dtl(const GemmArgs& a, hipStream_t st) {
  const int tiles = ((a.M + C::BM - 1) / C::BM) *
                    (a.epi == EPI_SWIGLU ? (a.N + C::BN / 2 - 1) / (C::BN / 2) : (a.N + C::BN - 1) / C::BN) * a.splits;
  hipLaunchKernelGGL(gemm_bf16_dtl<C>, dim3(tiles), dim3(C::THREADS), 0, st, a);
  return hipGetLastError();
}

template <class C>
hipError_t launch_gemm_cfg(const GemmArgs& a, hipStream_t st) {
  const int tiles = ((a.M + C::BM - 1) / C::BM) *
                    (a.epi == EPI_SWIGLU ? (a.N + C::BN / 2 - 1) / (C::BN / 2) : (a.N + C::BN - 1) / C::BN) * a.splits;
  hipLaunchKernelGGL(gemm_bf16_kernel<C>, dim3(tiles), dim3(C::THREADS), 0, st, a);
  return hipGetLastError();
}

using GemmSmall = TileCfg<128, 128, 2, 2, 2, 2>;  // register-staged, 2 blocks per CU (K % 64 != 0)
// direct-to-LDS block heights for BN = 256, one block per CU, 8 waves each
// (16x16 MFMA tiles: the 32x32 shape measured slower in this loop on every projection shape)
using GemmDtl128 = DtlCfg<128, 256, 2, 4, 3, 1, 16>;  // waves 64x64, 3 x 48 KB stages
using GemmDtl96 = DtlCfg<96, 256, 2, 4, 3, 1, 16>;    // waves 48x64, 3 x 44 KB stages
using GemmDtl64 = DtlCfg<64, 256, 1, 8, 4, 1, 16>;    // waves 64x32, 4 x 40 KB stages
using GemmDtl256 = DtlCfg<256, 256, 2, 4, 2, 1, 16>;  // waves 128x64, 2 x 64 KB stages (many rows)
using GemmDtl224 = DtlCfg<224, 256, 2, 4, 2, 1, 16>;  // waves 112x64, 2 x 60 KB stages (3136 rows = 14 tiles)
using GemmDtl128n = DtlCfg<128, 192, 4, 2, 3, 1, 16>; // waves 32x96, 3 x 40 KB stages (finer weight tiles)
using GemmDtl64n = DtlCfg<64, 128, 1, 4, 3, 2, 16>;   // 4 waves 64x32, 3 x 24 KB stages, 2 blocks per CU (few rows)

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
  if (dt != BF16 || M <= 0 || N <= 0) return best;
  // The direct-to-LDS kernels need K % 64 == 0 (whole 64-wide K steps per split); otherwise the
  // register-staged kernel. Among the block shapes and split-K factors (K per split >= 512, at
  // most 4), pick the least
  //   rounds of resident blocks x (block area / 256 x K per split) / per-CU rate
  //   + the extra fp32 partial sums written and read back, (splits - 1) x M x N x 8 bytes,
  // with per-CU rates relative to the 128x256 block as measured on whole rounds of gate/up
  // products with the weights streaming from HBM (smaller blocks re-read the weight and
  // activation tiles more often). One cost unit is one row of a 256-wide block advancing one K
  // column (about 0.1 ns on a full round); the 8 bytes of one partial element (written once, then
  // read once by the short reduce or post-processing kernel, which moves about 4 TB/s) cost 0.02
  // units. (At 0.0131 the 3136-row QKV product took two splits: 187 against 176 us for one in the
  // standalone harness, before its post-processing read twice the partial sums.)
  struct Opt { int cfg, bm, bn, per_cu; double rate; };
  const Opt dtl_opts[7] = {{GEMM_DTL128, 128, 256, 1, 1.0},  {GEMM_DTL96, 96, 256, 1, 0.86},
                           {GEMM_DTL64, 64, 256, 1, 0.65},   {GEMM_DTL256, 256, 256, 1, 1.15},
                           {GEMM_DTL128N, 128, 192, 1, 1.0}, {GEMM_DTL224, 224, 256, 1, 1.05},
                           {GEMM_DTL64N, 64, 128, 2, 0.7}};
  const Opt small_opt[1] = {{GEMM_SMALL, 128, 128, 2, 0.85}};
  const bool dtl = K % 64 == 0;
  const Opt* opts = dtl ? dtl_opts : small_opt;
  // 64x128 blocks, two per CU, for few rows: the weights stream about once from HBM and the finer
  // column tiles put every CU on that stream. Measured faster on every projection at 64 rows and
  // on the split-K ones at 128 (down 37.6 against 53.0 us); slower on gate/up from 128 rows and
  // on the others from about 200, where the row tiles share each weight tile.
  const int n_opts = dtl ? (M <= 64 || (M <= 128 && !swiglu) ? 7 : 6) : 1;
  const int cols = swiglu ? 2 * N : N;
  double best_cost = 1e300;
  for (int o = 0; o < n_opts; ++o) {
    const long tiles = (long)((M + opts[o].bm - 1) / opts[o].bm) * ((cols + opts[o].bn - 1) / opts[o].bn);
    const long slots = (long)n_cu * opts[o].per_cu;
    const double work = (double)opts[o].bm * opts[o].bn / 256.0;  // of one block per K column
    for (int sp = 1; sp <= (allow_split ? 4 : 1); ++sp) {
      if (sp > 1 && K / sp < 512) break;
      const long rounds = (tiles * sp + slots - 1) / slots;
      const double cost = rounds * opts[o].per_cu * work * ((double)K / sp) / opts[o].rate +
                          (sp - 1) * (double)M * N * 0.02;
      if (cost < best_cost * 0.999) {
        best_cost = cost;
        best = GemmPlan{opts[o].cfg, sp};
      }
    }
  }
  return best;
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  if (a.dt == BF16) {
    if (a.cfg != GEMM_SMALL && (a.K % 64 != 0 || a.K < 64)) return hipErrorInvalidValue;
    switch (a.cfg) {
      case GEMM_DTL128: return launch_gemm_dtl<GemmDtl128>(a, st);
      case GEMM_DTL96: return launch_gemm_dtl<GemmDtl96>(a, st);
      case GEMM_DTL64: return launch_gemm_dtl<GemmDtl64>(a, st);
      case GEMM_DTL256: return launch_gemm_dtl<GemmDtl256>(a, st);
      case GEMM_DTL224: return launch_gemm_dtl<GemmDtl224>(a, st);
      case GEMM_DTL128N: return launch_gemm_dtl<GemmDtl128n>(a, st);
      case GEMM_DTL64N: return launch_gemm_dtl<GemmDtl64n>(a, st);
      default: return launch_gemm_cfg<GemmSmall>(a, st);
    }
  }
  dim3 grid((a.N + 63) / 64, (a.M + 63) / 64, 1);
  hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace cf
