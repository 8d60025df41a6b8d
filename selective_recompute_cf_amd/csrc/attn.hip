// Sparse-query causal attention: n selected query rows (absolute positions pos[j], ascending)
// attend over the full blended K/V cache, key t visible to row j iff t <= pos[j].
// CacheBlend ("Selective Recompute Without Skipping"): selected queries attend over the full
// blended K/V, n_sel x L instead of L x L; QCFuse Eq. 7: a selected position reads its prefix
// through the partially fused cache.
//
// bf16 path (head_dim 64/128): one block = 128 query rows of one kv head, 8 waves; keys stream
// in blocks of 64 through a ring of LDS stages filled by direct global->LDS loads; K and V tiles
// are stored row-major with a 16-byte-chunk XOR swizzle by key, and the V^T operand is read with
// gfx950's transposing LDS read (ds_read_b64_tr_b16).
// S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_16x16x32_bf16: in this orientation every lane
// holds one query row (lane % 16) for both S and O, so the online-softmax state needs no
// cross-lane exchange beyond 2 xor-shuffles. Softmax in fp32 with exp2; P rounded to bf16 for
// the PV product. Split-KV over key ranges, merged with log-sum-exp weights.
//
// fp32 path: one block per query row, one wave per query head, online softmax per 64 keys.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace cf {

constexpr int KB = 64;  // keys per step

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// One block = 128 query rows of one kv head (128/G selected rows x the G query heads), NW waves
// of RG groups of 16 rows: every K/V fragment read from LDS serves the wave's RG row groups, and
// every K/V tile read from memory serves the block's 128 rows. K and V tiles of 64 keys stream
// straight from global memory into a ring of S LDS stages (global_load_lds_dwordx4 from inline
// assembly, as in the GEMM; M0 is set right before each load and used by nothing else in the
// kernel): lane l of a load lands in 16-byte slot l of a 1 KB row group, so the swizzle is
// applied on the global side (the lane that fills chunk slot c' of key t fetches chunk
// c' ^ (t & SWM), or c' ^ vswz(t) in a V tile). Per key block: wait for this wave's loads of the
// block | barrier | load the block S - 1 ahead into the stage the previous block used | S^T,
// softmax, O^T on the block.
//
// Swizzle of the V tiles. The K fragment reads (16 keys x one 16-byte chunk per 16 lanes) are
// conflict-free with chunk c of key t at c ^ (t & 15); the transposing V reads are not (each 32-lane
// half reads 8 consecutive keys x two neighbouring chunks, which that XOR maps onto the same 8
// physical chunks: a 2-way bank conflict on every read, measured on gfx950). At head_dim 128 the V
// tiles therefore rotate the key's low 4 bits left by one, which spreads each half's 16 chunk reads
// over all 16 chunks (measured conflict-free) while staying a permutation of the chunks per key.
template <int HD>
__device__ __forceinline__ int vswz(int t) {
  if constexpr (HD == 128) return ((t & 7) << 1) | ((t >> 3) & 1);
  else return t & (HD / 8 - 1);
}

#define CF_ATTN_WAITCNT(vm) ((((vm) & 15) | (((vm) >> 4) << 14)) | 0x70 | (15 << 8))

template <int HD, int NW, int RG, int S, int MINB>
__global__ __launch_bounds__(NW * WAVE, MINB) void attn_dtl_kernel(AttnArgs a) {
  constexpr int NCH = HD / 8;       // 16-byte chunks per key row
  constexpr int SWM = NCH - 1;      // chunk c of K tile key t is stored at c ^ (t & SWM)
  constexpr int TILE = KB * HD;     // elements of one K (or V) tile
  constexpr int RPI = WAVE / NCH;   // key rows per load instruction
  constexpr int NI = 2 * KB / RPI;  // load instructions per key block (K then V)
  constexpr int NL = NI / NW;       // per wave
  static_assert(NW * RG * 16 == 128, "128 query rows per block");
  static_assert(NI % NW == 0, "load instructions must split over the waves");
  static_assert(S >= 2 && (S - 2) * NL <= 63, "stages");
  __shared__ __attribute__((aligned(1024))) bf16 smem[S * 2 * TILE];
  const int G = a.hq / a.hkv;
  const int rpt = 128 / G;  // selected rows per block
  const int q_tiles = (a.n + rpt - 1) / rpt;
  // the block's query tile j0.., kv head g, key range [kbeg, kend) and where its result goes:
  // piece >= 0 writes partial sums to piece slot `piece`, else the normalised output
  int j0, g, kbeg, kend, piece = -1;
  if (a.sched) {  // balanced pieces: blocks t * hkv + g, t < P <= ATTN_MAXP
    g = blockIdx.x % a.hkv;
    const int t = blockIdx.x / a.hkv;
    const int4 pc = a.sched->piece[t];  // read beside T: one round trip before the first loads
    if (t >= a.sched->T) return;        // block-uniform
    j0 = pc.x;
    kbeg = pc.y;
    kend = pc.z;
    piece = pc.w;
  } else {  // whole query tiles, latest first (they see the most keys); each kv head on one XCD
    const int lt = xcd_tile(blockIdx.x, q_tiles * a.hkv);
    j0 = (q_tiles - 1 - lt % q_tiles) * rpt;
    g = lt / q_tiles;
    kbeg = 0;
    kend = min(a.pos[min(j0 + rpt - 1, a.n - 1)] + 1, a.L);
  }
  const int tid = threadIdx.x, lane = tid % WAVE, w = tid / WAVE;
  const int lg = lane / 16, lr = lane % 16;
  const int kvd = a.hkv * HD;
  const int nkb = kend > kbeg ? (kend - kbeg + KB - 1) / KB : 0;

  // load q of this wave: instruction gi = q * NW + w covers key rows [ii * RPI, ii * RPI + RPI)
  // of tensor gi / (NI / 2) (0 = K, 1 = V), ii = gi % (NI / 2). The tile row of a lane is
  // ii * RPI + lane / NCH; ii * RPI is wave-uniform and, for every q, congruent to w * RPI modulo
  // NCH, so the swizzled chunk of a lane is one value for all its K loads and one for all its V
  // loads. Each load is the scalar base of the head's K or V columns plus a 32-bit lane offset.
  static_assert((NI / 2) % NW == 0 && (NW * RPI) % NCH == 0, "one swizzled chunk per lane and tensor");
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) bf16*)smem;
  const bf16* kbase_p = (const bf16*)a.k + g * HD;
  const bf16* vbase_p = (const bf16*)a.v + g * HD;
  const int t0 = (w * RPI) % KB + lane / NCH;  // congruent modulo NCH to every load's tile row
  const uint32_t colk = 16u * (uint32_t)((lane % NCH) ^ (t0 & SWM));
  const uint32_t colv = 16u * (uint32_t)((lane % NCH) ^ vswz<HD>(t0));
  const int lrow = lane / NCH;
  const uint32_t row_bytes = 2u * (uint32_t)kvd;
  auto issue = [&](int step) __attribute__((always_inline)) {
    const int stage = step % S;
    const int kbase = kbeg + step * KB;
#pragma unroll
    for (int q = 0; q < NL; ++q) {
      // with (NI / 2) % NW == 0 the tensor depends on q alone: the first NL / 2 loads are K
      constexpr int HALF = NL / 2;
      const bool vt = q >= HALF;
      const int ii = (q % HALF) * NW + w;
      const uint32_t off = (uint32_t)min(kbase + ii * RPI + lrow, a.L - 1) * row_bytes + (vt ? colv : colk);
      const uint32_t dst = __builtin_amdgcn_readfirstlane(
          lds0 + 2u * (uint32_t)(stage * 2 * TILE + (vt ? TILE : 0) + ii * RPI * HD));
      if (vt)
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(vbase_p), "s"(dst)
                     : "memory", "m0");
      else
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(kbase_p), "s"(dst)
                     : "memory", "m0");
    }
  };
  // the first S - 1 key blocks go out before the queries are read: their latency overlaps
  if (nkb > 0) {
#pragma unroll
    for (int q = 0; q < S - 1; ++q) issue(min(q, nkb - 1));
  }

  // row group rg of this wave: block rows (w * RG + rg) * 16 + lr
  int jrow[RG], head[RG], p[RG];
  bf16x8 qf[RG][HD / 32];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    const int r = (w * RG + rg) * 16 + lr;
    const int j = j0 + r / G;
    jrow[rg] = j;
    head[rg] = g * G + r % G;
    const int jc = min(j, a.n - 1);
    p[rg] = a.pos[jc];
    const bf16* qrow = (const bf16*)a.q + (int64_t)jc * a.ldq + head[rg] * HD;
#pragma unroll
    for (int kk = 0; kk < HD / 32; ++kk) qf[rg][kk] = *reinterpret_cast<const bf16x8*>(qrow + kk * 32 + 8 * lg);
  }
  f32x4 o[RG][HD / 16];
  float m_i[RG], l_i[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
#pragma unroll
    for (int nt = 0; nt < HD / 16; ++nt) o[rg][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_i[rg] = -INFINITY;
    l_i[rg] = 0.f;
  }
  const float sl2 = 1.4426950408889634f / sqrtf((float)HD);
  // smallest position among the wave's rows (lanes l, l + 16, l + 32, l + 48 share a row)
  int p_min = p[0];
#pragma unroll
  for (int rg = 1; rg < RG; ++rg) p_min = min(p_min, p[rg]);
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) p_min = min(p_min, __shfl_xor(p_min, off, WAVE));
  p_min = __builtin_amdgcn_readfirstlane(p_min);

  // V^T operand through the transposing LDS read: within each 16-lane group, lane q reads the
  // 4 dims 16nt + 4(q%4).. of tile key kb + q/4 and lane lr receives V[kb + 0..3][16nt + lr]
  auto vread = [&](const bf16* Vt, int kb, int nt) __attribute__((always_inline)) {
    const int t = kb + lr / 4;
    const int col = nt * 16 + 4 * (lr % 4);
    const int c = col / 8;
    const bf16* ptr = &Vt[t * HD + ((c ^ vswz<HD>(t)) * 8) + (col % 8)];
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)ptr);
  };
  auto step = [&](int it) __attribute__((always_inline)) {
    const bf16* Kt = smem + (it % S) * 2 * TILE;
    const bf16* Vt = Kt + TILE;
    const int kbase = kbeg + it * KB;
    f32x4 s[RG][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) s[rg][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int t = kt * 16 + lr;
#pragma unroll
      for (int kk = 0; kk < HD / 32; ++kk) {
        const int c = kk * 4 + lg;
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&Kt[t * HD + ((c ^ (t & SWM)) * 8)]);
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
          s[rg][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[rg][kk], s[rg][kt], 0, 0, 0);
      }
    }
    // s[rg][kt][i] = S[row of group rg][key kbase + 16kt + 4lg + i]. Softmax: unscaled scores,
    // masks only on blocks that reach past a row of the wave, exp2 of one fused multiply-add, and
    // a reference max that moves only on growth above 8 (log2).
    bf16x8 pf[RG][2];
    const bool unmasked = kbase + KB - 1 <= min(p_min, kend - 1);  // wave-uniform
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      if (!unmasked) {
        const int lim = min(p[rg], kend - 1) - kbase - 4 * lg;  // last visible key, block-relative
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (kt * 16 + i > lim) s[rg][kt][i] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[rg][kt][i]);
      // A row's reference moves only if some lane of the row sees a score above it by more than 8,
      // so the cross-lane maximum is needed only when some lane of the wave does (after the first
      // block, rarely); otherwise every row keeps its reference, whatever the row maximum is.
      bool upd = false;
      float m_use = m_i[rg];
      if (__builtin_amdgcn_ballot_w64(mx * sl2 > m_i[rg] + 8.f)) {
        mx = fmaxf(mx, __shfl_xor(mx, 16, WAVE));
        mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));
        const float m_cand = fmaxf(m_i[rg], mx * sl2);
        upd = m_cand > m_i[rg] + 8.f;
        m_use = upd ? m_cand : m_i[rg];
      }
      const float m_ref = m_use == -INFINITY ? 0.f : m_use;
      const float alpha = upd ? __builtin_amdgcn_exp2f(m_i[rg] - m_ref) : 1.f;
      // the row sum stays split over the row's four lanes (each its own keys) until the end
      float ps = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __builtin_amdgcn_exp2f(fmaf(s[rg][kt][i], sl2, -m_ref));
          s[rg][kt][i] = e;
          ps += e;
        }
      l_i[rg] = l_i[rg] * alpha + ps;
      m_i[rg] = m_use;
      if (__builtin_amdgcn_ballot_w64(upd)) {
#pragma unroll
        for (int nt = 0; nt < HD / 16; ++nt) o[rg][nt] *= alpha;
      }
#pragma unroll
      for (int mm = 0; mm < 2; ++mm)
#pragma unroll
        for (int tp = 0; tp < 2; ++tp)
#pragma unroll
          for (int i = 0; i < 4; ++i) pf[rg][mm][tp * 4 + i] = (bf16)s[rg][2 * mm + tp][i];
    }
    // O^T += V^T P^T over fragments f = 2 nt + mm. At 4 waves per SIMD the kernel has 128 VGPRs,
    // and left alone the compiler reads each fragment's V^T operand (two transposing reads) into
    // the same registers right before its product, exposing the LDS latency on all 16 products;
    // here each operand is read two fragments ahead (the groups are pinned for the scheduler)
    auto vfrag = [&](int f) __attribute__((always_inline)) {
      const int nt = f / 2, mm = f % 2;
      const i16x4 lo = vread(Vt, 32 * mm + 4 * lg, nt);
      const i16x4 hi = vread(Vt, 32 * mm + 16 + 4 * lg, nt);
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    constexpr int NF = 2 * (HD / 16);
    bf16x8 vcur = vfrag(0), vn1 = vfrag(1);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      bf16x8 vn2 = vn1;
      if (f + 2 < NF) {
        vn2 = vfrag(f + 2);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
        o[rg][f / 2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vcur, pf[rg][f % 2], o[rg][f / 2], 0, 0, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, RG, 0);
      vcur = vn1;
      vn1 = vn2;
    }
  };

  if (nkb > 0) {
    const int last = nkb - 1;
    // past the last block the loads repeat the last block into a stage nobody reads again, so
    // every wave issues NL loads per block and the wait counts hold (the query loads, issued
    // after the first blocks, only make the first wait stricter)
    for (int it = 0; it < nkb; ++it) {
      __builtin_amdgcn_s_waitcnt(CF_ATTN_WAITCNT((S - 2) * NL));
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      issue(min(it + S - 1, last));
      step(it);
    }
    __builtin_amdgcn_s_waitcnt(CF_ATTN_WAITCNT(0));
  }
  // the row sums over the four lanes of each row
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    l_i[rg] += __shfl_xor(l_i[rg], 16, WAVE);
    l_i[rg] += __shfl_xor(l_i[rg], 32, WAVE);
  }
  // o[rg][nt][i] = O[row of group rg][hd 16nt + 4lg + i] (unnormalised)
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    const int j = jrow[rg];
    if (j >= a.n) continue;
    if (piece >= 0) {
      const int64_t slot = ((int64_t)g * a.P + piece) * 128 + (w * RG + rg) * 16 + lr;
      float* op = a.o_part + slot * HD;
#pragma unroll
      for (int nt = 0; nt < HD / 16; ++nt)
        *reinterpret_cast<float4*>(op + nt * 16 + 4 * lg) =
            make_float4(o[rg][nt][0], o[rg][nt][1], o[rg][nt][2], o[rg][nt][3]);
      if (lg == 0) {
        float* ml = a.ml_part + slot * 2;
        ml[0] = m_i[rg];
        ml[1] = l_i[rg];
      }
    } else {
      if (a.ml_out && lg == 0) {
        float* ml = a.ml_out + ((int64_t)j * a.hq + head[rg]) * 2;
        ml[0] = m_i[rg] == -INFINITY ? 0.f : m_i[rg];
        ml[1] = l_i[rg];
      }
      const float inv = l_i[rg] > 0.f ? 1.0f / l_i[rg] : 0.f;
      bf16* out = (bf16*)a.out + (int64_t)j * a.ldo + head[rg] * HD;
#pragma unroll
      for (int nt = 0; nt < HD / 16; ++nt) {
        bf16x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (bf16)(o[rg][nt][i] * inv);
        *reinterpret_cast<bf16x4*>(out + nt * 16 + 4 * lg) = v;
      }
    }
  }
}

// Launch configuration: waves per block, 16-row groups per wave, LDS stages, blocks per CU.
template <int NW, int RG, int S, int MINB>
struct AttnCfg {
  static constexpr int nw = NW, rg = RG, stages = S, minb = MINB;
};

template <class C>
hipError_t launch_attention_cfg(const AttnArgs& a, hipStream_t st) {
  // the tile loads address a head's K/V columns with 32-bit byte offsets from the cache start
  if ((int64_t)a.L * a.hkv * a.hd * 2 >= (int64_t(1) << 32)) return hipErrorInvalidValue;
  const int G = a.hq / a.hkv, rpt = 128 / G;
  dim3 grid(a.sched ? a.P * a.hkv : ((a.n + rpt - 1) / rpt) * a.hkv);
  if (a.hd == 128)
    hipLaunchKernelGGL((attn_dtl_kernel<128, C::nw, C::rg, C::stages, C::minb>), grid, dim3(C::nw * WAVE), 0, st, a);
  else
    hipLaunchKernelGGL((attn_dtl_kernel<64, C::nw, C::rg, C::stages, C::minb>), grid, dim3(C::nw * WAVE), 0, st, a);
  return hipGetLastError();
}

// Whole query tiles (full causal layers) and balanced pieces (the selected rows of a blended
// layer): two blocks per CU over 2-stage rings, whose phases interleave (measured faster on both
// than one block per CU over deeper rings).
using AttnWide = AttnCfg<8, 1, 2, 2>;

// Combine the pieces of a query tile: weights 2^(m_s - max m) (scores are in log2 units). One
// thread per 4 consecutive output elements of one (row, head): 16-byte partial loads, one store.
template <typename T>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
  const unsigned q4 = (unsigned)a.hd / 4, per_row = (unsigned)a.hq * q4;
  const unsigned gid = blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (unsigned)a.n * per_row) return;
  const int j = (int)(gid / per_row), idx = (int)(gid % per_row);
  const int head = idx / (int)q4, d = (idx % (int)q4) * 4;
  // the row's parts: pieces off[qt] .. off[qt + 1] - 1 of its query tile
  const int G = a.hq / a.hkv, rpt = 128 / G, qt = j / rpt;
  const int first = a.sched->off[qt], parts = a.sched->off[qt + 1] - first;
  if (parts <= 1) return;  // a single piece wrote the normalised output itself
  const int64_t base = ((int64_t)(head / G) * a.P + first) * 128 + (j % rpt) * G + head % G, stride = 128;
  float mx = -INFINITY;
  for (int s = 0; s < parts; ++s) mx = fmaxf(mx, a.ml_part[(base + s * stride) * 2]);
  float n0 = 0.f, n1 = 0.f, n2 = 0.f, n3 = 0.f, den = 0.f;
  for (int s = 0; s < parts; ++s) {
    const int64_t r = base + s * stride;
    const float m = a.ml_part[r * 2], l = a.ml_part[r * 2 + 1];
    const float wgt = m == -INFINITY ? 0.f : exp2f(m - mx);
    const float4 o = *reinterpret_cast<const float4*>(a.o_part + r * a.hd + d);
    n0 += wgt * o.x, n1 += wgt * o.y, n2 += wgt * o.z, n3 += wgt * o.w;
    den += wgt * l;
  }
  T* out = (T*)a.out + (int64_t)j * a.ldo + head * a.hd + d;
  const bool ok = den > 0.f;
  if (a.ml_out && d == 0) {
    a.ml_out[((int64_t)j * a.hq + head) * 2] = mx == -INFINITY ? 0.f : mx;
    a.ml_out[((int64_t)j * a.hq + head) * 2 + 1] = den;
  }
  out[0] = from_f<T>(ok ? n0 / den : 0.f);
  out[1] = from_f<T>(ok ? n1 / den : 0.f);
  out[2] = from_f<T>(ok ? n2 / den : 0.f);
  out[3] = from_f<T>(ok ? n3 / den : 0.f);
}

// ----------------------------------------------------------------------------- plain path
template <typename T>
__global__ __launch_bounds__(256) void attn_simple_kernel(AttnArgs a) {
  __shared__ float qs[4][128];
  const int j = blockIdx.x;
  const int w = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int hd = a.hd, G = a.hq / a.hkv, kvd = a.hkv * hd;
  const int p = clampi(a.pos[j], 0, a.L - 1);
  const float scale = 1.0f / sqrtf((float)hd);
  for (int head = w; head < a.hq; head += blockDim.x / WAVE) {
    const int g = head / G;
    const T* qrow = (const T*)a.q + (int64_t)j * a.ldq + head * hd;
    for (int d = lane; d < hd; d += WAVE) qs[w][d] = to_f(qrow[d]);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    float m = -INFINITY, l = 0.f, acc0 = 0.f, acc1 = 0.f;
    for (int t0 = 0; t0 <= p; t0 += WAVE) {
      const int t = t0 + lane;
      float s = -INFINITY;
      if (t <= p) {
        const T* kr = (const T*)a.k + (int64_t)t * kvd + g * hd;
        float dot = 0.f;
        for (int d = 0; d < hd; ++d) dot += qs[w][d] * to_f(kr[d]);
        s = dot * scale;
      }
      const float m_new = fmaxf(m, wave_max(s));
      const float alpha = expf(m - m_new);
      const float pv = t <= p ? expf(s - m_new) : 0.f;
      l = l * alpha + wave_sum(pv);
      acc0 *= alpha;
      acc1 *= alpha;
      for (int tt = 0; tt < WAVE; ++tt) {
        const float pt = __shfl(pv, tt, WAVE);
        if (t0 + tt > p) break;
        const T* vr = (const T*)a.v + (int64_t)(t0 + tt) * kvd + g * hd;
        if (lane < hd) acc0 += pt * to_f(vr[lane]);
        if (lane + WAVE < hd) acc1 += pt * to_f(vr[lane + WAVE]);
      }
      m = m_new;
    }
    T* out = (T*)a.out + (int64_t)j * a.ldo + head * hd;
    if (a.ml_out && lane == 0) {  // natural-log max to log2 units
      a.ml_out[((int64_t)j * a.hq + head) * 2] = m * 1.4426950408889634f;
      a.ml_out[((int64_t)j * a.hq + head) * 2 + 1] = l;
    }
    if (lane < hd) out[lane] = from_f<T>(acc0 / l);
    if (lane + WAVE < hd) out[lane + WAVE] = from_f<T>(acc1 / l);
    __builtin_amdgcn_wave_barrier();
  }
}

hipError_t launch_attention_merge(const AttnArgs& a, hipStream_t st) {
  if (a.n == 0 || !a.sched) return hipSuccess;
  {
    const int64_t total = (int64_t)a.n * a.hq * (a.hd / 4);
    const dim3 grid((unsigned)((total + 255) / 256));
    if (a.dt == BF16)
      hipLaunchKernelGGL(attn_merge_kernel<bf16>, grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(attn_merge_kernel<float>, grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

// One workgroup: key blocks per query tile, then the smallest piece length (in key blocks) whose
// pieces fit in P blocks per kv head, then the piece table. The query tiles of the selected rows
// see very different numbers of keys (the latest rows see them all); cutting every tile into
// pieces of the same length gives each block about the same work.
constexpr int MIN_PIECE = 2;  // key blocks (128 keys); 1 to 12 measured within 0.3% of each other

__global__ __launch_bounds__(256) void attn_sched_kernel(const int* __restrict__ pos, int n, int rpt, int P, int L,
                                                         AttnSched* __restrict__ s) {
  __shared__ int c[ATTN_MAXQ];
  __shared__ int best, sum_c, max_c;
  const int Q = (n + rpt - 1) / rpt, tid = threadIdx.x;
  for (int qt = tid; qt < Q; qt += blockDim.x) c[qt] = (pos[min((qt + 1) * rpt, n) - 1] + KB) / KB;
  __syncthreads();
  if (tid == 0) {
    int sc = 0, mc = 0;
    for (int qt = 0; qt < Q; ++qt) sc += c[qt], mc = max(mc, c[qt]);
    sum_c = sc;
    max_c = mc;
    best = mc;  // one piece per tile always fits: Q <= P
  }
  __syncthreads();
  // pieces of at least MIN_PIECE key blocks: shorter ones cost more in merging than they save
  for (int chunk = max((sum_c + P - 1) / P, min(MIN_PIECE, max_c)) + tid; chunk < max_c; chunk += blockDim.x) {
    int pieces = 0;
    for (int qt = 0; qt < Q; ++qt) pieces += (c[qt] + chunk - 1) / chunk;
    if (pieces <= P) atomicMin(&best, chunk);
  }
  __syncthreads();
  if (tid == 0) {
    const int chunk = best;
    int t = 0;
    for (int qt = 0; qt < Q; ++qt) {
      s->off[qt] = t;
      const int np = (c[qt] + chunk - 1) / chunk, j0 = qt * rpt;
      const int last_pos = pos[min(j0 + rpt - 1, n - 1)];
      for (int e = 0; e < np; ++e, ++t) {
        const int kb0 = e * chunk, kb1 = min(kb0 + chunk, c[qt]);
        s->piece[t] = make_int4(j0, kb0 * KB, min(min(last_pos + 1, kb1 * KB), L), np > 1 ? t : -1);
      }
    }
    s->off[Q] = t;
    s->T = t;
  }
}

hipError_t launch_attention_sched(const AttnArgs& a, AttnSched* s, hipStream_t st) {
  const int rpt = 128 / (a.hq / a.hkv), Q = (a.n + rpt - 1) / rpt;
  if (a.n <= 0 || Q > ATTN_MAXQ || a.P < Q || a.P > ATTN_MAXP) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_sched_kernel, dim3(1), dim3(256), 0, st, a.pos, a.n, rpt, a.P, a.L, s);
  return hipGetLastError();
}

void attn_plan(Dt dt, int n, int hq, int hkv, int n_cu, int* P) {
  // When the query tiles fit in two blocks per CU (the selected rows of a blended layer), balanced
  // pieces (2 n_cu / hkv blocks per kv head): the tiles see very different numbers of keys, so
  // whole tiles leave most CUs waiting for the latest ones. Otherwise whole tiles (many of them:
  // full causal layers).
  *P = 0;
  if (dt != BF16 || n == 0) return;
  const int G = hq / hkv, q_tiles = (n + 128 / G - 1) / (128 / G), per_head = 2 * n_cu / hkv;
  if (n_cu % hkv == 0 && q_tiles <= ATTN_MAXQ && q_tiles <= per_head && per_head <= ATTN_MAXP) *P = per_head;
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t st) {
  if (a.n == 0) return hipSuccess;
  if (a.dt == BF16) return launch_attention_cfg<AttnWide>(a, st);
  hipLaunchKernelGGL(attn_simple_kernel<float>, dim3(a.n), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace cf
