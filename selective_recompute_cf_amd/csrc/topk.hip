// Selection of the recompute set P (exact, deterministic; one workgroup of 1024 threads).
//
// Token mode (CacheBlend "Quantifying the Damage": HKVD tokens; Request Order Matters §2.2):
// the k positions of largest deviation, ties to the lower index, written ascending. Deviations
// are mapped to order-preserving 32-bit keys (NaN -> +inf, -0 -> +0, handled on the bit
// pattern so denormals are never flushed); a most-significant-digit-first radix select (4
// passes of 8 bits, integer LDS histograms) finds the exact k-th key T and how many keys equal
// to T must be taken; a stable compaction in index order then writes the positions.
//
// Span mode (Request Order Matters §2.3, Eq. 3): fp64 sequential span sums, spans ranked by
// (mean desc, span index asc), whole spans taken while they fit (stopping at the first that
// does not), the remainder filled by the window of largest fp64 running-sum difference in that
// span (smallest start among equals).
#include "common.h"
#include "kernels.h"

namespace cf {

constexpr int TK_THREADS = 1024;

__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) u = 0x7f800000u;  // NaN -> +inf
  if ((u & 0x7fffffffu) == 0u) u = 0u;                    // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive scan of one int per thread over the block (1024 threads = 16 waves).
__device__ int block_excl_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x % WAVE, w = threadIdx.x / WAVE;
  int x = v;
#pragma unroll
  for (int o = 1; o < WAVE; o <<= 1) {
    const int y = __shfl_up(x, o, WAVE);
    if (lane >= o) x += y;
  }
  __syncthreads();
  if (lane == WAVE - 1) wsum[w] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int i = 0; i < TK_THREADS / WAVE; ++i) {
      const int t = wsum[i];
      wsum[i] = acc;
      acc += t;
    }
    *total = acc;
  }
  __syncthreads();
  return x - v + wsum[w];
}

// Write, in ascending index order, every i with take(i) true. Each thread owns a contiguous
// segment of the index range so that a single exclusive scan orders the output.
template <typename Take>
__device__ void compact(int n, int k, Take take, int* out, int* wsum, int* total) {
  const int seg = (n + TK_THREADS - 1) / TK_THREADS;
  const int b = min(n, (int)threadIdx.x * seg), e = min(n, b + seg);
  int cnt = 0;
  for (int i = b; i < e; ++i) cnt += take(i) ? 1 : 0;
  int o = block_excl_scan(cnt, wsum, total);
  for (int i = b; i < e; ++i)
    if (take(i) && o < k) out[o++] = i;
}

__global__ __launch_bounds__(TK_THREADS) void topk_token_kernel(const float* __restrict__ dev, int n, int k,
                                                                int* __restrict__ out) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_prefix;
  __shared__ int s_kk;
  __shared__ int wsum[TK_THREADS / WAVE];
  __shared__ int total;
  uint32_t prefix = 0, mask = 0;
  int kk = k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = threadIdx.x; i < 256; i += TK_THREADS) hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += TK_THREADS) {
      const uint32_t key = order_key(dev[i]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int cum = 0;
      for (int b = 255; b >= 0; --b) {
        const int h = (int)hist[b];
        if (cum + h >= kk) {
          s_prefix = prefix | ((uint32_t)b << shift);
          s_kk = kk - cum;
          break;
        }
        cum += h;
      }
    }
    __syncthreads();
    prefix = s_prefix;
    kk = s_kk;
    mask |= 255u << shift;
  }
  const uint32_t T = prefix;
  // rank of each key equal to T among the equal keys, in index order
  const int seg = (n + TK_THREADS - 1) / TK_THREADS;
  const int b = min(n, (int)threadIdx.x * seg), e = min(n, b + seg);
  int eq = 0;
  for (int i = b; i < e; ++i) eq += order_key(dev[i]) == T ? 1 : 0;
  const int eq_before = block_excl_scan(eq, wsum, &total);
  int cnt = 0;
  {
    int r = eq_before;
    for (int i = b; i < e; ++i) {
      const uint32_t key = order_key(dev[i]);
      const bool t = key > T || (key == T && r < kk);
      r += key == T ? 1 : 0;
      cnt += t ? 1 : 0;
    }
  }
  int o = block_excl_scan(cnt, wsum, &total);
  int r = eq_before;
  for (int i = b; i < e; ++i) {
    const uint32_t key = order_key(dev[i]);
    const bool t = key > T || (key == T && r < kk);
    r += key == T ? 1 : 0;
    if (t && o < k) out[o++] = i;
  }
}

hipError_t launch_topk_token(const float* dev, int n, int k, int* out, hipStream_t st) {
  if (k <= 0 || n <= 0) return hipSuccess;
  hipLaunchKernelGGL(topk_token_kernel, dim3(1), dim3(TK_THREADS), 0, st, dev, n, k, out);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- spans
__device__ __forceinline__ double canon_d(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) u = 0x7f800000u;
  if ((u & 0x7fffffffu) == 0u) u = 0u;
  return (double)__uint_as_float(u);
}

__global__ __launch_bounds__(TK_THREADS) void topk_spans_kernel(const float* __restrict__ dev, int n, int k,
                                                                SpanArgs sp, int* __restrict__ out,
                                                                double* __restrict__ run) {
  __shared__ double score[MAX_SPANS];
  __shared__ int order[MAX_SPANS];
  __shared__ int take[MAX_SPANS];
  __shared__ int s_part, s_rem, s_wa;
  __shared__ double bestv[TK_THREADS / WAVE];
  __shared__ int besta[TK_THREADS / WAVE];
  __shared__ int wsum[TK_THREADS / WAVE];
  __shared__ int total;
  const int ns = sp.n_spans;
  // 1. span means (fp64, sequential within the span)
  for (int j = threadIdx.x; j < ns; j += TK_THREADS) {
    double s = 0.0;
    for (int i = sp.b[j]; i < sp.b[j + 1]; ++i) s += canon_d(dev[i]);
    score[j] = s / (double)(sp.b[j + 1] - sp.b[j]);
    take[j] = 0;
  }
  __syncthreads();
  // 2. ranking by (score desc, index asc)
  for (int j = threadIdx.x; j < ns; j += TK_THREADS) {
    int r = 0;
    for (int i = 0; i < ns; ++i) r += (score[i] > score[j] || (score[i] == score[j] && i < j)) ? 1 : 0;
    order[r] = j;
  }
  __syncthreads();
  // 3. whole spans while they fit; remember the first that does not
  if (threadIdx.x == 0) {
    int rem = k, part = -1;
    for (int r = 0; r < ns && rem > 0; ++r) {
      const int j = order[r];
      const int len = sp.b[j + 1] - sp.b[j];
      if (len <= rem) {
        take[j] = 1;
        rem -= len;
      } else {
        part = j;
        break;
      }
    }
    s_part = part;
    s_rem = part >= 0 ? rem : 0;
    s_wa = -1;
    if (part >= 0) {  // running fp64 sum of the partial span, from its start
      double acc = 0.0;
      run[0] = 0.0;
      const int a = sp.b[part], len = sp.b[part + 1] - a;
      for (int i = 0; i < len; ++i) {
        acc += canon_d(dev[a + i]);
        run[i + 1] = acc;
      }
    }
  }
  __syncthreads();
  // 4. best window [a, a + rem) in the partial span: largest total, smallest a among equals
  if (s_part >= 0) {
    const int a0 = sp.b[s_part], len = sp.b[s_part + 1] - a0, rem = s_rem;
    double bv = -1.0;
    int ba = 0x7fffffff;
    __threadfence_block();
    for (int a = threadIdx.x; a + rem <= len; a += TK_THREADS) {
      const double t = run[a + rem] - run[a];
      if (ba == 0x7fffffff || t > bv) {
        bv = t;
        ba = a;
      }
    }
    // reduce (value desc, start asc) across the wave, then across waves
    for (int o = 32; o > 0; o >>= 1) {
      const double ov = __shfl_xor(bv, o, WAVE);
      const int oa = __shfl_xor(ba, o, WAVE);
      const bool better = oa != 0x7fffffff && (ba == 0x7fffffff || ov > bv || (ov == bv && oa < ba));
      if (better) {
        bv = ov;
        ba = oa;
      }
    }
    if (threadIdx.x % WAVE == 0) {
      bestv[threadIdx.x / WAVE] = bv;
      besta[threadIdx.x / WAVE] = ba;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      double v = 0.0;
      int a = 0x7fffffff;
      for (int w = 0; w < TK_THREADS / WAVE; ++w) {
        const int oa = besta[w];
        if (oa == 0x7fffffff) continue;
        if (a == 0x7fffffff || bestv[w] > v || (bestv[w] == v && oa < a)) {
          v = bestv[w];
          a = oa;
        }
      }
      s_wa = a0 + a;
    }
  }
  __syncthreads();
  // 5. ascending output
  const int wa = s_wa, wl = s_rem;
  auto in_span_taken = [&](int i) {
    int lo = 0, hi = ns - 1;  // span containing i (binary search over bounds)
    while (lo < hi) {
      const int mid = (lo + hi + 1) / 2;
      if (sp.b[mid] <= i) lo = mid; else hi = mid - 1;
    }
    return take[lo] != 0 || (wa >= 0 && i >= wa && i < wa + wl);
  };
  compact(n, k, in_span_taken, out, wsum, &total);
}

hipError_t launch_topk_spans(const float* dev, int n, int k, const SpanArgs& sp, int* out, double* ws,
                             hipStream_t st) {
  if (k <= 0 || n <= 0) return hipSuccess;
  hipLaunchKernelGGL(topk_spans_kernel, dim3(1), dim3(TK_THREADS), 0, st, dev, n, k, sp, out, ws);
  return hipGetLastError();
}

}  // namespace cf
