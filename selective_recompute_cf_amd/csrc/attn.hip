// Sparse-query causal attention: n selected query rows (absolute positions pos[j], ascending)
// attend over the full blended K/V cache, key t visible to row j iff t <= pos[j].
// CacheBlend ("Selective Recompute Without Skipping"): selected queries attend over the full
// blended K/V, n_sel x L instead of L x L; QCFuse Eq. 7: a selected position reads its prefix
// through the partially fused cache.
//
// bf16 path (head_dim 64/128): one block = 64 query rows of one kv head (64/G selected rows x
// the G query heads sharing that kv head), 4 waves of 16 rows. Keys stream in blocks of 64
// through double-buffered LDS: K row-major with a 16-byte XOR swizzle, V transposed (hd-major)
// with keys permuted so that one 16-byte read gives the 8 keys an MFMA lane group needs.
// S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_16x16x32_bf16: in this orientation every lane
// holds one query row (lane % 16) for both S and O, so the online-softmax state needs no
// cross-lane exchange beyond 2 xor-shuffles. Softmax in fp32 with exp2; P rounded to bf16 for
// the PV product. Split-KV over key ranges, merged with log-sum-exp weights.
//
// fp32 path: one block per query row, one wave per query head, online softmax per 64 keys.
#include "common.h"
#include "kernels.h"

namespace cf {

constexpr int KB = 64;  // keys per step

template <int HD>
__global__ __launch_bounds__(256, 2) void attn_mfma_kernel(AttnArgs a) {
  constexpr int NCH = HD / 8;  // 16-byte chunks per key row
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][KB * HD];
  __shared__ __attribute__((aligned(16))) bf16 Vt[2][HD * KB];
  const int G = a.hq / a.hkv;
  const int rpt = 64 / G;  // selected rows per block
  // logical tile: query tile fastest, then split, then kv head: tiles reading the same K/V head
  // are neighbours and run on the same XCD
  const int q_tiles = (a.n + rpt - 1) / rpt;
  const int lt = xcd_tile(blockIdx.x, q_tiles * a.splits * a.hkv);
  const int j0 = (lt % q_tiles) * rpt, split = (lt / q_tiles) % a.splits, g = lt / (q_tiles * a.splits);
  const int tid = threadIdx.x, lane = tid % WAVE, w = tid / WAVE;
  const int lg = lane / 16, lr = lane % 16;
  const int r = w * 16 + lr;
  const int jl = r / G, hl = r % G;
  const int j = j0 + jl;
  const bool row_ok = j < a.n;
  const int jc = min(j, a.n - 1);
  const int head = g * G + hl;
  const int p = a.pos[jc];
  const int pmax = a.pos[min(j0 + rpt - 1, a.n - 1)];
  const int kvd = a.hkv * HD;
  const int kbeg = split * a.split_len;
  const int kend = min(min(pmax + 1, kbeg + a.split_len), a.L);
  const int nkb = kend > kbeg ? (kend - kbeg + KB - 1) / KB : 0;
  const bf16* K = (const bf16*)a.k + g * HD;
  const bf16* V = (const bf16*)a.v + g * HD;

  bf16x8 qf[HD / 32];
  {
    const bf16* qrow = (const bf16*)a.q + (int64_t)jc * a.ldq + head * HD;
#pragma unroll
    for (int kk = 0; kk < HD / 32; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(qrow + kk * 32 + 8 * lg);
  }
  f32x4 o[HD / 16];
#pragma unroll
  for (int nt = 0; nt < HD / 16; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_i = -INFINITY, l_i = 0.f;
  const float sl2 = 1.4426950408889634f / sqrtf((float)HD);

  constexpr int KCH = KB * NCH / 256;        // K chunks per thread per step
  constexpr int VUN = (KB / 4) * NCH;        // V units (4 keys x 8 dims) per step
  uint4 rk[KCH];
  uint4 rv[4];
  auto gload = [&](int kbase) {
#pragma unroll
    for (int it = 0; it < KCH; ++it) {
      const int ci = tid + 256 * it;
      const int t = ci / NCH, c = ci % NCH;
      const int key = min(kbase + t, a.L - 1);
      rk[it] = *reinterpret_cast<const uint4*>(K + (int64_t)key * kvd + c * 8);
    }
    if (tid < VUN) {
      const int kq = tid / NCH, hc = tid % NCH;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int key = min(kbase + kq * 4 + q, a.L - 1);
        rv[q] = *reinterpret_cast<const uint4*>(V + (int64_t)key * kvd + hc * 8);
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int it = 0; it < KCH; ++it) {
      const int ci = tid + 256 * it;
      const int t = ci / NCH, c = ci % NCH;
      *reinterpret_cast<uint4*>(&Ks[buf][t * HD + ((c ^ (t & 7)) * 8)]) = rk[it];
    }
    if (tid < VUN) {
      const int kq = tid / NCH, hc = tid % NCH;
      const int t0 = kq * 4;  // keys t0..t0+3: t0 = 32m + 16t' + 4g'
      const int mm = t0 / 32, tp = (t0 / 16) & 1, gp = (t0 / 4) & 3;
      const int chunk = 4 * mm + gp, off = 4 * tp;
      const bf16* v0 = reinterpret_cast<const bf16*>(&rv[0]);
      const bf16* v1 = reinterpret_cast<const bf16*>(&rv[1]);
      const bf16* v2 = reinterpret_cast<const bf16*>(&rv[2]);
      const bf16* v3 = reinterpret_cast<const bf16*>(&rv[3]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int n = hc * 8 + e;
        bf16x4 pk;
        pk[0] = v0[e]; pk[1] = v1[e]; pk[2] = v2[e]; pk[3] = v3[e];
        *reinterpret_cast<bf16x4*>(&Vt[buf][n * KB + ((chunk ^ (n & 7)) * 8) + off]) = pk;
      }
    }
  };

  if (nkb > 0) {
    gload(kbeg);
    sstore(0);
  }
  __syncthreads();
  for (int it = 0; it < nkb; ++it) {
    const int cur = it & 1;
    const int kbase = kbeg + it * KB;
    if (it + 1 < nkb) gload(kbase + KB);
    f32x4 s[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      s[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int t = kt * 16 + lr;
#pragma unroll
      for (int kk = 0; kk < HD / 32; ++kk) {
        const int c = kk * 4 + lg;
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&Ks[cur][t * HD + ((c ^ (t & 7)) * 8)]);
        s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[kk], s[kt], 0, 0, 0);
      }
    }
    // s[kt][i] = S[row r][key kbase + 16kt + 4lg + i]
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kbase + kt * 16 + 4 * lg + i;
        const float v = (key <= p && key < kend) ? s[kt][i] * sl2 : -INFINITY;
        s[kt][i] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, WAVE));
    mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));
    const float m_new = fmaxf(m_i, mx);
    const bool live = m_new != -INFINITY;
    const float alpha = live ? exp2f(m_i - m_new) : 1.f;
    float ps = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = live ? exp2f(s[kt][i] - m_new) : 0.f;
        s[kt][i] = e;
        ps += e;
      }
    ps += __shfl_xor(ps, 16, WAVE);
    ps += __shfl_xor(ps, 32, WAVE);
    l_i = l_i * alpha + ps;
    m_i = m_new;
#pragma unroll
    for (int nt = 0; nt < HD / 16; ++nt) o[nt] *= alpha;
    bf16x8 pf[2];
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
#pragma unroll
      for (int tp = 0; tp < 2; ++tp)
#pragma unroll
        for (int i = 0; i < 4; ++i) pf[mm][tp * 4 + i] = (bf16)s[2 * mm + tp][i];
#pragma unroll
    for (int nt = 0; nt < HD / 16; ++nt) {
      const int n = nt * 16 + lr;
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const int c = 4 * mm + lg;
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(&Vt[cur][n * KB + ((c ^ (n & 7)) * 8)]);
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[mm], o[nt], 0, 0, 0);
      }
    }
    if (it + 1 < nkb) sstore(cur ^ 1);
    __syncthreads();
  }
  if (!row_ok) return;
  // o[nt][i] = O[row r][hd 16nt + 4lg + i] (unnormalised)
  if (a.splits > 1) {
    float* op = a.o_part + (((int64_t)split * a.n + j) * a.hq + head) * HD;
#pragma unroll
    for (int nt = 0; nt < HD / 16; ++nt)
      *reinterpret_cast<float4*>(op + nt * 16 + 4 * lg) = make_float4(o[nt][0], o[nt][1], o[nt][2], o[nt][3]);
    if (lg == 0) {
      float* ml = a.ml_part + (((int64_t)split * a.n + j) * a.hq + head) * 2;
      ml[0] = m_i;
      ml[1] = l_i;
    }
  } else {
    const float inv = l_i > 0.f ? 1.0f / l_i : 0.f;
    bf16* out = (bf16*)a.out + (int64_t)j * a.ldo + head * HD;
#pragma unroll
    for (int nt = 0; nt < HD / 16; ++nt) {
      bf16x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = (bf16)(o[nt][i] * inv);
      *reinterpret_cast<bf16x4*>(out + nt * 16 + 4 * lg) = v;
    }
  }
}

// Combine split-KV partials: weights 2^(m_s - max m) (scores are in log2 units).
template <typename T>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)a.n * a.hq * a.hd) return;
  const int j = (int)(gid / (a.hq * a.hd));
  {
    const int idx = (int)(gid % (a.hq * a.hd));
    const int head = idx / a.hd, d = idx % a.hd;
    float mx = -INFINITY;
    for (int s = 0; s < a.splits; ++s) mx = fmaxf(mx, a.ml_part[(((int64_t)s * a.n + j) * a.hq + head) * 2]);
    float num = 0.f, den = 0.f;
    for (int s = 0; s < a.splits; ++s) {
      const float* ml = a.ml_part + (((int64_t)s * a.n + j) * a.hq + head) * 2;
      const float wgt = ml[0] == -INFINITY ? 0.f : exp2f(ml[0] - mx);
      num += wgt * a.o_part[(((int64_t)s * a.n + j) * a.hq + head) * a.hd + d];
      den += wgt * ml[1];
    }
    ((T*)a.out)[(int64_t)j * a.ldo + idx] = from_f<T>(den > 0.f ? num / den : 0.f);
  }
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
    if (lane < hd) out[lane] = from_f<T>(acc0 / l);
    if (lane + WAVE < hd) out[lane + WAVE] = from_f<T>(acc1 / l);
    __builtin_amdgcn_wave_barrier();
  }
}

hipError_t launch_attention_merge(const AttnArgs& a, hipStream_t st) {
  if (a.n == 0 || a.splits <= 1) return hipSuccess;
  {
    const int64_t total = (int64_t)a.n * a.hq * a.hd;
    const dim3 grid((unsigned)((total + 255) / 256));
    if (a.dt == BF16)
      hipLaunchKernelGGL(attn_merge_kernel<bf16>, grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(attn_merge_kernel<float>, grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

void attn_plan(Dt dt, int n, int L, int hq, int hkv, int hd, int n_cu, int* splits, int* split_len) {
  *splits = 1;
  *split_len = ((L + KB - 1) / KB) * KB;
  if (dt != BF16 || n == 0) return;
  const int G = hq / hkv;
  const int items = ((n + 64 / G - 1) / (64 / G)) * hkv;
  int s = 1;
  while (s < 8 && items * s < 2 * n_cu && L / (2 * s) >= 512) s *= 2;
  *splits = s;
  *split_len = (((L + s - 1) / s + KB - 1) / KB) * KB;
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t st) {
  if (a.n == 0) return hipSuccess;
  if (a.dt == BF16) {
    const int G = a.hq / a.hkv, rpt = 64 / G;
    dim3 grid(((a.n + rpt - 1) / rpt) * a.hkv * a.splits);
    if (a.hd == 128)
      hipLaunchKernelGGL(attn_mfma_kernel<128>, grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(attn_mfma_kernel<64>, grid, dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL(attn_simple_kernel<float>, dim3(a.n), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace cf
