// Selection of the recompute set P (exact, deterministic; one workgroup of 1024 threads, or the
// whole GPU for large n in token mode).
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
#include <algorithm>

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
    // the digit: the bin b where the keys in bins above b number fewer than kk and those in bins
    // b and above at least kk. Thread t < 256 takes bin 255 - t, so an inclusive scan over the
    // threads counts the keys from the top bin down.
    int h = 0, incl = 0;
    if (threadIdx.x < 256) {
      h = (int)hist[255 - threadIdx.x];
      incl = h;
#pragma unroll
      for (int off = 1; off < WAVE; off <<= 1) {
        const int y = __shfl_up(incl, off, WAVE);
        if ((int)(threadIdx.x % WAVE) >= off) incl += y;
      }
      if (threadIdx.x % WAVE == WAVE - 1) wsum[threadIdx.x / WAVE] = incl;
    }
    __syncthreads();
    if (threadIdx.x < 256) {
      for (int wv = 0; wv < (int)threadIdx.x / WAVE; ++wv) incl += wsum[wv];
      const int above = incl - h;
      if (above < kk && incl >= kk) {
        s_prefix = prefix | ((uint32_t)(255 - threadIdx.x) << shift);
        s_kk = kk - above;
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

// ----------------------------------------------------------------------------- token, large n
// The same exact selection spread over the whole GPU for n >= TK_MB_MIN, reading the n keys once
// in the usual case.
//
// The index range is cut into sub-ranges of sw indices, one wave each. A gather over many blocks
// draws a stratified sample of TK_SAMPLE keys (one at a hashed offset inside each of TK_SAMPLE
// near-equal strata), and one block takes two of its order statistics as bounds lo <= hi that
// bracket the threshold key T (the k-th largest) with a margin of four standard deviations of the
// sample rank. One pass
// over the n keys then writes a map of 2 bits per index (taken: key > hi; undecided: lo <= key <=
// hi) and appends the undecided keys, in index order, to their sub-range's slice of a candidate
// list, counting both per sub-range. If fewer than k keys lie above hi and at least k at or above
// lo, T lies in the band: when lo == hi it is lo itself; otherwise, if the undecided keys fit the
// list, T is the (k - above)-th largest candidate, which 8-bit digit passes over the (small) list
// find (a digit that lo and hi share needs no pass). The candidates of each sub-range are then
// counted above / equal to T, a one-block scan turns the counts into output offsets and ranks
// among equal keys (lower index first), and the ordered write reads only the map and the
// candidates.
//
// Otherwise (a sample that missed, or too many undecided keys for the workspace) two 8-bit
// histogram passes over the n keys fix T's top 16 bits and the same collect pass runs with the
// keys sharing them as the undecided band; if those do not fit either, the last two digits come
// from histograms over all n keys and a counting pass over the n keys rewrites the map against T
// itself (taken: key > T; undecided: key == T). Every route gives the same positions; no block
// waits for another.
constexpr int TK_MB_MIN = 1 << 16;
constexpr int TK_SUB_MIN = 1024;      // indices per sub-range at least (a multiple of 1024)
constexpr int TK_MAX_SUB = 4096;      // sub-ranges at most: every wave of a per-range kernel resident at once
constexpr int TK_SUB_PER = (TK_MAX_SUB + TK_THREADS - 1) / TK_THREADS;  // sub-ranges per scan thread
constexpr int TK_HIST_BLOCKS = 1024;  // histogram blocks over all n (grid-stride)
constexpr int TK_SAMPLE = 32768;      // sampled keys
constexpr int TK_SPT = TK_SAMPLE / TK_THREADS;  // per thread: strata 32 t .. 32 t + 31
constexpr int TK_COARSE = 8;          // every 8th sampled key (4096, evenly spread) for the coarse band
constexpr int TK_WPB = 4;             // waves (sub-ranges) per block in the per-range kernels

enum : int { TK_UNSET = 0, TK_SAMPLED = 1, TK_FALLBACK = 2, TK_BIN = 3, TK_OVERFLOW = 4, TK_EXACT = 5 };

struct TopkState {
  uint32_t prefix[5];  // prefix[p]: the top 8p bits of T fixed by digit passes < p
  int kk[5];           // kk[p]: keys still owed among those matching prefix[p]
  uint32_t lo, hi;     // the undecided band of the current collect pass
  int mode;            // TK_*: which route the selection takes
  int n_cand;          // keys in the candidate list
};
static_assert(sizeof(TopkState) <= 256, "state slot");

// sw: indices per sub-range, n_sub: sub-ranges (n_sub * sw >= n; 64-bit: n may be near INT_MAX)
static void tk_geom(int n, int& sw, int& n_sub) {
  const int64_t per = ((int64_t)n + TK_MAX_SUB - 1) / TK_MAX_SUB;
  sw = (int)std::max<int64_t>(TK_SUB_MIN, (per + TK_SUB_MIN - 1) / TK_SUB_MIN * TK_SUB_MIN);
  n_sub = (int)(((int64_t)n + sw - 1) / sw);
}

// per sub-range: taken, undecided and equal counts, candidate offset, output offset, equal keys before
constexpr int TK_SUB_ARRAYS = 6;
static size_t tk_sub_bytes(int n_sub) { return ((size_t)n_sub * TK_SUB_ARRAYS * sizeof(int) + 255) / 256 * 256; }

constexpr size_t TK_HEAD_BYTES = 4 * 256 * sizeof(uint32_t) + 256 + TK_SAMPLE * sizeof(uint32_t);

// histograms, state, sampled keys, per-sub-range arrays and the 2-bit map; the candidate slices
// and list follow
static size_t tk_mb_fixed_bytes(int n) {
  int sw, n_sub;
  tk_geom(n, sw, n_sub);
  return TK_HEAD_BYTES + tk_sub_bytes(n_sub) + (size_t)n_sub * sw / 4;
}

size_t topk_token_ws_min_bytes(int n) { return n < TK_MB_MIN ? 0 : tk_mb_fixed_bytes(n); }

size_t topk_token_ws_bytes(int n) {
  if (n < TK_MB_MIN) return 0;
  int sw, n_sub;
  tk_geom(n, sw, n_sub);
  // a list of n/16 candidates, then slices of sw/16 per sub-range
  return tk_mb_fixed_bytes(n) + (size_t)(n / 16) * sizeof(uint32_t) + (size_t)n_sub * (sw / 16) * sizeof(uint32_t);
}

__device__ __forceinline__ uint32_t tk_hash(uint32_t x) {  // Wellons' "lowbias32" integer hash
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// Exclusive scan over the wave's 64 lanes with DPP moves (row shifts within each row of 16 lanes,
// then the row totals broadcast down): six adds and no LDS traffic. total: the wave's sum.
__device__ __forceinline__ int wave_excl_scan(int v, int& total) {
  int x = v;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1 and 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2 and 3
  total = __builtin_amdgcn_readlane(x, WAVE - 1);
  return x - v;
}

// The walk's keys: the order-preserving key without the -0 and positive-NaN rewrites (those are
// absorbed by the walk's bounds, see tk_bounds); negative NaNs, which would order below -inf, are
// mapped to +inf's key here. tk_canon finishes the canonical key for a stored candidate.
__device__ __forceinline__ uint32_t tk_raw_key(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t r = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
  return r < 0x007fffffu ? 0xff800000u : r;
}
__device__ __forceinline__ uint32_t tk_canon(uint32_t r) {
  return r == 0x7fffffffu ? 0x80000000u : (r > 0xff800000u ? 0xff800000u : r);  // -0 -> +0, NaN -> +inf
}

__device__ __forceinline__ int wave_isum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

// orders one wave's LDS writes before its other lanes' reads (no block barrier)
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// 16 copies of the 256 bins (lane % 16 picks the copy): most float keys fall into a few top-byte
// bins, and same-address LDS atomics serialise. Rows of 257 words put the copies of a bin in
// different banks.
constexpr int TK_HCOPIES = 16;

constexpr int TK_SCOPIES = 4;  // the sample's selects see few keys a thread: fewer copies to clear and add

struct TkSel {
  uint32_t h[2][TK_SCOPIES][257];
  int wtot[2][256 / WAVE];
  uint32_t pre[2];
  int rem[2];
  int cnt[2];
};

// Two radix selects in one block (4 passes of 8 bits, shared): the keys at descending ranks
// r0 and r1 (1-based; a search with act false is skipped) among key[j] for j = 0, STEP, 2 STEP, ...
// that lie in [blo, bhi]. Every thread of the block calls it.
template <int STEP>
__device__ void tk_select2(const uint32_t (&key)[TK_SPT], uint32_t blo, uint32_t bhi, int r0, int r1, bool a0,
                           bool a1, TkSel& s, uint32_t& out0, uint32_t& out1) {
  __syncthreads();  // earlier readers of s are done
  if (threadIdx.x == 0) {
    s.pre[0] = s.pre[1] = 0;
    s.rem[0] = r0;
    s.rem[1] = r1;
  }
  const int lane = threadIdx.x % WAVE, q = (threadIdx.x / 256) & 1, t = threadIdx.x % 256;
  const bool act_mine = q == 0 ? a0 : a1;
  for (int pass = 0; pass < 4; ++pass) {
    for (int i = threadIdx.x; i < 2 * TK_SCOPIES * 257; i += TK_THREADS) (&s.h[0][0][0])[i] = 0u;
    __syncthreads();
    const uint32_t mask = pass == 0 ? 0u : (0xffffffffu << (32 - 8 * pass));
    const int shift = 24 - 8 * pass;
    const uint32_t p0 = s.pre[0], p1 = s.pre[1], pre_mine = s.pre[q];
    const int r_mine = s.rem[q];
    const int c = threadIdx.x % TK_SCOPIES;
#pragma unroll
    for (int j = 0; j < TK_SPT; j += STEP) {
      const uint32_t x = key[j];
      if (x < blo || x > bhi) continue;
      const uint32_t d = (x >> shift) & 255u;
      if (a0 && (x & mask) == p0) atomicAdd(&s.h[0][c][d], 1u);
      if (a1 && (x & mask) == p1) atomicAdd(&s.h[1][c][d], 1u);
    }
    __syncthreads();
    // threads 0..511: search q takes bin 255 - t; counts accumulate from the top bin down
    int cnt = 0;
    if (threadIdx.x < 512)
#pragma unroll
      for (int cc = 0; cc < TK_SCOPIES; ++cc) cnt += (int)s.h[q][cc][255 - t];
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < WAVE; off <<= 1) {
      const int y = __shfl_up(incl, off, WAVE);
      if (lane >= off) incl += y;
    }
    if (threadIdx.x < 512 && lane == WAVE - 1) s.wtot[q][t / WAVE] = incl;
    __syncthreads();
    if (threadIdx.x < 512 && act_mine) {
      for (int wv = 0; wv < t / WAVE; ++wv) incl += s.wtot[q][wv];
      const int above = incl - cnt;
      if (above < r_mine && incl >= r_mine) {
        s.pre[q] = pre_mine | ((uint32_t)(255 - t) << shift);
        s.rem[q] = r_mine - above;
      }
    }
    __syncthreads();
  }
  out0 = s.pre[0];
  out1 = s.pre[1];
}

// The stratified sample, one key a thread over many blocks (random reads need many CUs): stratum s
// (indices from s n / S to (s + 1) n / S, rounded down) gives the key at a hashed offset inside it, stored at
// (s % 32) * 1024 + s / 32 so that the selecting block reads its keys coalesced.
__global__ __launch_bounds__(256) void tk_mb_gather_kernel(const float* __restrict__ dev, int n, uint32_t* skey) {
  const int sidx = blockIdx.x * 256 + (int)threadIdx.x;
  const int64_t jit = (int64_t)(((uint64_t)tk_hash((uint32_t)sidx) * (uint32_t)n) >> 32);  // in [0, n)
  const int64_t pos = ((int64_t)sidx * n + jit) / TK_SAMPLE;                               // in stratum sidx
  skey[(sidx % TK_SPT) * TK_THREADS + sidx / TK_SPT] = order_key(dev[pos]);
}

// Bounds of the undecided band from the sample: the keys at descending sample ranks
// mu -/+ (4 sd + 2), mu = k S / n, sd = sqrt(S p (1 - p)), p = k / n. A coarse band from every 8th
// sampled key (ranks mu' -/+ (6 sd' + 3) of those 4096) first, then the exact order statistics
// among the sampled keys inside it, so that the histograms see few keys. A rank below 1 leaves hi
// at the largest key, one past S leaves lo at the smallest; a target outside the coarse band
// (which only widens the band) takes the coarse bound or the extreme key.
// Also clears the digit histograms and the state.
__global__ __launch_bounds__(TK_THREADS) void tk_mb_sample_kernel(const uint32_t* __restrict__ skey, int n, int k,
                                                                  uint32_t* hist, TopkState* st) {
  __shared__ TkSel s;
  hist[threadIdx.x] = 0;  // 4 x 256 bins
  if (threadIdx.x == 0) {
    st->prefix[0] = 0;
    st->kk[0] = 0;
    st->mode = TK_UNSET;
    st->n_cand = 0;
  }
  uint32_t key[TK_SPT];  // key[j]: stratum TK_SPT * thread + j
#pragma unroll
  for (int j = 0; j < TK_SPT; ++j) key[j] = skey[j * TK_THREADS + threadIdx.x];
  const double p = (double)k / n;
  constexpr int S1 = TK_SAMPLE / TK_COARSE;
  const double mu1 = p * S1, sd1 = sqrt(S1 * p * (1.0 - p));
  const double ch_r = floor(mu1 - 6.0 * sd1 - 3.0), cl_r = ceil(mu1 + 6.0 * sd1 + 3.0);
  const bool ca0 = ch_r >= 1.0, ca1 = cl_r <= (double)S1;
  uint32_t ch = 0xffffffffu, cl = 0u;
  tk_select2<TK_COARSE>(key, 0u, 0xffffffffu, ca0 ? (int)ch_r : 0, ca1 ? (int)cl_r : 0, ca0, ca1, s, ch, cl);
  if (!ca0) ch = 0xffffffffu;
  if (!ca1) cl = 0u;
  // sampled keys above the coarse band and inside it
  int above = 0, inside = 0;
#pragma unroll
  for (int j = 0; j < TK_SPT; ++j) {
    above += key[j] > ch;
    inside += key[j] >= cl && key[j] <= ch;
  }
  above = wave_isum(above);
  inside = wave_isum(inside);
  if (threadIdx.x == 0) s.cnt[0] = s.cnt[1] = 0;
  __syncthreads();
  if (threadIdx.x % WAVE == 0) atomicAdd(&s.cnt[0], above), atomicAdd(&s.cnt[1], inside);
  __syncthreads();
  const int c_above = s.cnt[0], c_in = s.cnt[1];
  const double mu = p * TK_SAMPLE, sd = sqrt(TK_SAMPLE * p * (1.0 - p));
  const double rh = floor(mu - 4.0 * sd - 2.0), rl = ceil(mu + 4.0 * sd + 2.0);
  const bool act_h = rh >= 1.0, act_l = rl <= (double)TK_SAMPLE;
  const int rh2 = act_h ? (int)rh - c_above : 0, rl2 = act_l ? (int)rl - c_above : 0;
  const bool sh = act_h && rh2 >= 1 && rh2 <= c_in, sl = act_l && rl2 >= 1 && rl2 <= c_in;
  uint32_t hi = 0xffffffffu, lo = 0u;
  tk_select2<1>(key, cl, ch, sh ? rh2 : 0, sl ? rl2 : 0, sh, sl, s, hi, lo);
  if (threadIdx.x == 0) {
    st->hi = !act_h ? 0xffffffffu : sh ? hi : rh2 < 1 ? 0xffffffffu : cl;
    st->lo = !act_l ? 0u : sl ? lo : rl2 < 1 ? ch : 0u;
  }
}

// 16 keys of one step per lane: v[4 j + e] is index base + 256 j + 4 lane + e (0 past n), so that
// each load instruction covers 1 KB
__device__ __forceinline__ void tk_load_step(const float* __restrict__ dev, int64_t n, int64_t base, bool vec,
                                             float (&v)[16]) {
  const int lane = threadIdx.x % WAVE;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t i0 = base + 256 * j + 4 * lane;
    if (vec && i0 + 4 <= n) {
      const float4 x = *reinterpret_cast<const float4*>(dev + i0);
      v[4 * j] = x.x, v[4 * j + 1] = x.y, v[4 * j + 2] = x.z, v[4 * j + 3] = x.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * j + e] = i0 + e < n ? dev[i0 + e] : 0.f;
    }
  }
}

// One step of tk_walk: the map bytes of the step's 1024 indices (sub-step j in bits 8j..8j+7 of
// bytes) and, when STAGE, its undecided keys in index order at stage[0..), the others written to
// the lane's spare word stage[1024 + lane]. Returns the step's undecided count (wave-uniform).
template <bool FULL>
__device__ __forceinline__ int tk_classify(const float (&cur)[16], int64_t base, int64_t n, uint32_t lo2,
                                           uint32_t span, uint32_t hi2, bool stage_keys, uint32_t* stage,
                                           uint32_t& bytes) {
  const int lane = threadIdx.x % WAVE;
  int staged = 0;
  bytes = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t key[4], und[4];
    uint32_t byte = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      key[e] = tk_raw_key(cur[4 * j + e]);
      bool up = key[e] > hi2, u = key[e] - lo2 <= span;
      if (!FULL) {
        const bool in = base + 256 * j + 4 * lane + e < n;
        up = up && in;
        u = u && in;
      }
      und[e] = u ? 1u : 0u;
      byte |= (up ? 1u << (2 * e) : 0u) | (u ? 2u << (2 * e) : 0u);
    }
    bytes |= byte << (8 * j);
    uint64_t bal[4];
    int tot = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bal[e] = __ballot(und[e] != 0);
      tot += __popcll(bal[e]);
    }
    if (stage_keys && tot) {  // wave-uniform
      uint32_t slot = staged;  // + undecided keys of lower lanes in this sub-step
#pragma unroll
      for (int e = 0; e < 4; ++e)
        slot = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal[e] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal[e], slot));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        stage[und[e] ? slot : 1024u + lane] = key[e];
        slot += und[e];
      }
    }
    staged += tot;
  }
  return staged;
}

// Walks the indices [i_begin, i_begin + sw) that lie below n, 1024 per step. Per index, the map
// gets bit 2e "taken" (key > hi) and bit 2e + 1 "undecided" (lo <= key <= hi) for index 4b + e in
// byte b; undecided keys (raw: tk_canon gives the canonical key) are staged in the wave's LDS
// buffer in index order and written to cand[0..cap) (counted beyond cap, not written). The bounds
// are moved so that raw keys compare as canonical ones: -0's raw key sits just below +0's, and
// positive NaNs' above +inf's, where no canonical key lies. A step's stores are issued at the start
// of the next step, before that step's loads of the following keys (a wait for a load also waits
// for every memory operation issued before it). Returns the lane's taken count and the wave's
// undecided count (the same in every lane). stage: 1024 + 64 words (the last 64 take the writes
// of keys that are not staged).
template <bool MAP>
__device__ __forceinline__ void tk_walk(const float* __restrict__ dev, int64_t n, int64_t i_begin, int sw,
                                        uint32_t lo, uint32_t hi, bool vec, uint8_t* map, uint32_t* cand,
                                        int cap, uint32_t* stage, int& n_taken, int& n_und) {
  const int lane = threadIdx.x % WAVE;
  const int64_t i_end = i_begin + sw;
  const uint32_t lo2 = lo - (lo == 0x80000000u);
  const uint32_t hi2 = hi >= 0xff800000u ? 0xffffffffu : hi - (hi == 0x7fffffffu);
  const uint32_t span = hi2 - lo2;
  int a = 0, m = 0;
  float cur[16], nxt[16];
  uint32_t bytes = 0;     // the previous step's map bytes (sub-step j in bits 8j..8j+7)
  int staged = 0;         // the previous step's staged candidates (wave-uniform)
  int64_t prev = -1;      // the previous step's first index
  auto flush = [&]() {
    if (MAP && prev >= 0)
#pragma unroll
      for (int j = 0; j < 4; ++j) map[(prev + 256 * j) / 4 + lane] = (uint8_t)(bytes >> (8 * j));
    if (cand && staged) {
      wave_sync();
      for (int i = lane; i < staged; i += WAVE)
        if (m + i < cap) cand[m + i] = stage[i];
      wave_sync();  // the stage is read before this step writes it
    }
    m += staged;
  };
  tk_load_step(dev, n, i_begin, vec, nxt);
  for (int64_t base = i_begin; base < i_end; base += 1024) {
#pragma unroll
    for (int x = 0; x < 16; ++x) cur[x] = nxt[x];
    flush();
    if (base + 1024 < i_end) tk_load_step(dev, n, base + 1024, vec, nxt);
    // wave-uniform: a step with no index past n classifies without bounds checks
    if (base + 1024 <= n)
      staged = tk_classify<true>(cur, base, n, lo2, span, hi2, cand != nullptr, stage, bytes);
    else
      staged = tk_classify<false>(cur, base, n, lo2, span, hi2, cand != nullptr, stage, bytes);
    a += __popc(bytes & 0x55555555u);
    prev = base;
  }
  flush();
  n_taken = a;
  n_und = m;
}

// Round 0 (the sample's band) always; round 1 (T's 16-bit bin) only when the sample route failed.
__global__ __launch_bounds__(TK_WPB * WAVE) void tk_mb_collect_kernel(const float* __restrict__ dev, int n, int sw,
                                                                      int n_sub, int round,
                                                                      const TopkState* __restrict__ st, int* sub_a,
                                                                      int* sub_m, uint8_t* map, uint32_t* slices,
                                                                      int cap_w) {
  if (round == 1 && st->mode != TK_FALLBACK) return;
  __shared__ uint32_t stage[TK_WPB][1024 + WAVE];
  const int r = blockIdx.x * TK_WPB + (int)threadIdx.x / WAVE;
  if (r >= n_sub) return;  // whole waves
  const bool vec = ((uintptr_t)dev & 15) == 0;
  int a, m;
  tk_walk<true>(dev, n, (int64_t)r * sw, sw, st->lo, st->hi, vec, map, slices + (size_t)r * cap_w, cap_w,
                stage[threadIdx.x / WAVE], a, m);
  a = wave_isum(a);
  if (threadIdx.x % WAVE == 0) sub_a[r] = a, sub_m[r] = m;
}

// Candidate offsets and the route: round 0 checks that T lies in the sample's band, then whether
// the band is one key or fits the list; round 1 (after the bin picks) only whether the bin's keys
// fit. Each thread loads its TK_SUB_PER entries at once.
__global__ __launch_bounds__(TK_THREADS) void tk_mb_scan_cand_kernel(int n_sub, int k, int round, int cap_c,
                                                                     TopkState* st, const int* __restrict__ sub_a,
                                                                     const int* __restrict__ sub_m, int* coff) {
  if (round == 1 && st->mode != TK_FALLBACK) return;
  __shared__ int wsum[TK_THREADS / WAVE];
  __shared__ int total;
  const int r0 = (int)threadIdx.x * TK_SUB_PER;
  int vm[TK_SUB_PER], va[TK_SUB_PER];
#pragma unroll
  for (int j = 0; j < TK_SUB_PER; ++j) {
    const bool in = r0 + j < n_sub;
    vm[j] = in ? sub_m[r0 + j] : 0;
    va[j] = in ? sub_a[r0 + j] : 0;
  }
  int m = 0, a = 0;
#pragma unroll
  for (int j = 0; j < TK_SUB_PER; ++j) m += vm[j], a += va[j];
  int mb = block_excl_scan(m, wsum, &total);
  const int tm = total;
#pragma unroll
  for (int j = 0; j < TK_SUB_PER; ++j) {
    if (r0 + j < n_sub) coff[r0 + j] = mb;
    mb += vm[j];
  }
  (void)block_excl_scan(a, wsum, &total);
  const int ta = total;
  if (threadIdx.x == 0) {
    if (round == 0) {
      const bool in_band = ta < k && (int64_t)ta + tm >= k;
      const bool one_key = in_band && st->lo == st->hi;
      const bool ok = in_band && !one_key && tm <= cap_c;
      st->mode = one_key ? TK_EXACT : ok ? TK_SAMPLED : TK_FALLBACK;
      st->kk[0] = ok ? k - ta : k;
      st->n_cand = ok ? tm : 0;
      if (one_key) st->prefix[4] = st->lo, st->kk[4] = k - ta;
    } else {
      const bool fit = tm <= cap_c;
      st->mode = fit ? TK_BIN : TK_OVERFLOW;
      st->n_cand = fit ? tm : 0;
    }
  }
}

// Moves each sub-range's candidates to its place in the list; a sub-range whose slice overflowed
// reads its keys again.
__global__ __launch_bounds__(TK_WPB * WAVE) void tk_mb_compact_kernel(const float* __restrict__ dev, int n, int sw,
                                                                      int n_sub, int round,
                                                                      const TopkState* __restrict__ st,
                                                                      const int* __restrict__ sub_m,
                                                                      const int* __restrict__ coff,
                                                                      const uint32_t* __restrict__ slices, int cap_w,
                                                                      uint32_t* cand, int cap_c) {
  const int mode = st->mode;
  if (!((round == 0 && mode == TK_SAMPLED) || (round == 1 && mode == TK_BIN))) return;
  __shared__ uint32_t stage[TK_WPB][1024 + WAVE];
  const int r = blockIdx.x * TK_WPB + (int)threadIdx.x / WAVE;
  if (r >= n_sub) return;
  const int m = sub_m[r], o = coff[r];
  if (m <= cap_w) {
    const uint32_t* src = slices + (size_t)r * cap_w;
    for (int j = threadIdx.x % WAVE; j < m; j += WAVE) cand[o + j] = src[j];
  } else {
    const bool vec = ((uintptr_t)dev & 15) == 0;
    int a, mm;
    tk_walk<false>(dev, n, (int64_t)r * sw, sw, st->lo, st->hi, vec, nullptr, cand + o, cap_c - o,
                   stage[threadIdx.x / WAVE], a, mm);
  }
}

// Digit histograms: from the candidate list on the sampled route (a digit that lo and hi share is
// every candidate's and needs no histogram) and on the bin route (the last two digits), else from
// all n keys. Over the list only enough blocks for 16 keys a thread take part, so that few blocks
// merge into the global bins.
__global__ __launch_bounds__(256) void tk_mb_hist_kernel(const float* __restrict__ dev, int n, int pass,
                                                         const TopkState* __restrict__ st,
                                                         const uint32_t* __restrict__ cand, uint32_t* hist) {
  const int mode = st->mode;
  const int shift = 24 - 8 * pass;
  if (mode == TK_EXACT || (mode == TK_SAMPLED && ((st->lo ^ st->hi) >> shift) == 0)) return;
  const bool from_cand = mode == TK_SAMPLED || (pass >= 2 && mode == TK_BIN);
  const int m = from_cand ? st->n_cand : n;
  const int64_t used = from_cand ? std::min<int64_t>(gridDim.x, ((int64_t)m + 4095) / 4096) : gridDim.x;
  if ((int64_t)blockIdx.x >= used) return;  // block-uniform
  __shared__ uint32_t h[TK_HCOPIES][257];
#pragma unroll
  for (int c = 0; c < TK_HCOPIES; ++c) h[c][threadIdx.x] = 0;
  __syncthreads();
  const uint32_t prefix = st->prefix[pass];
  const uint32_t mask = pass == 0 ? 0u : (0xffffffffu << (32 - 8 * pass));
  uint32_t* mine = h[threadIdx.x % TK_HCOPIES];
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x, stride = used * blockDim.x;
  auto add = [&](uint32_t key) {
    if ((key & mask) == prefix) atomicAdd(&mine[(key >> shift) & 255u], 1u);
  };
  if (from_cand) {
    for (int64_t i = gid; i < m; i += stride) add(tk_canon(cand[i]));
  } else {
    const int64_t n4 = ((uintptr_t)dev & 15) == 0 ? n / 4 : 0;
    for (int64_t i = gid; i < n4; i += stride) {
      const float4 v = reinterpret_cast<const float4*>(dev)[i];
      add(order_key(v.x)), add(order_key(v.y)), add(order_key(v.z)), add(order_key(v.w));
    }
    for (int64_t i = 4 * n4 + gid; i < n; i += stride) add(order_key(dev[i]));
  }
  __syncthreads();
  uint32_t c = 0;
#pragma unroll
  for (int k = 0; k < TK_HCOPIES; ++k) c += h[k][threadIdx.x];
  if (c) atomicAdd(&hist[pass * 256 + threadIdx.x], c);
}

__global__ __launch_bounds__(256) void tk_mb_pick_kernel(int pass, TopkState* st, const uint32_t* hist) {
  const int mode = st->mode;
  if (mode == TK_EXACT) return;
  const int shift = 24 - 8 * pass;
  if (mode == TK_SAMPLED && ((st->lo ^ st->hi) >> shift) == 0) {  // a digit lo and hi share
    if (threadIdx.x == 0) {
      st->prefix[pass + 1] = st->lo & (0xffffffffu << shift);
      st->kk[pass + 1] = st->kk[pass];
    }
    return;
  }
  // thread t takes bin 255 - t and an inclusive scan over the threads counts the keys from the top
  // bin down; the bin where the count first reaches kk wins
  __shared__ int wtot[256 / WAVE];
  const int t = threadIdx.x, lane = t % WAVE;
  const int h = (int)hist[pass * 256 + 255 - t];
  int incl = h;
#pragma unroll
  for (int off = 1; off < WAVE; off <<= 1) {
    const int y = __shfl_up(incl, off, WAVE);
    if (lane >= off) incl += y;
  }
  if (lane == WAVE - 1) wtot[t / WAVE] = incl;
  __syncthreads();
  for (int wv = 0; wv < t / WAVE; ++wv) incl += wtot[wv];
  const int kk = st->kk[pass], above = incl - h;
  if (above < kk && incl >= kk) {
    const uint32_t p = st->prefix[pass] | ((uint32_t)(255 - t) << shift);
    st->prefix[pass + 1] = p;
    st->kk[pass + 1] = kk - above;
    if (pass == 1 && mode == TK_FALLBACK) st->lo = p, st->hi = p | 0xffffu;  // T's 16-bit bin
  }
}

// Per sub-range: keys above / equal to T. From the candidates on the sampled and bin routes (keys
// above the band were counted by the collect pass); when the band is the one key T, its undecided
// keys are the equal ones; on the overflow route from all of the sub-range's keys, rewriting its
// map against T (taken: key > T, undecided: key == T).
__global__ __launch_bounds__(TK_WPB * WAVE) void tk_mb_count_kernel(const float* __restrict__ dev, int n, int sw,
                                                                    int n_sub, const TopkState* __restrict__ st,
                                                                    int* sub_a, const int* __restrict__ sub_m,
                                                                    int* sub_e, const int* __restrict__ coff,
                                                                    const uint32_t* __restrict__ cand, uint8_t* map) {
  const int r = blockIdx.x * TK_WPB + (int)threadIdx.x / WAVE;
  if (r >= n_sub) return;
  const uint32_t T = st->prefix[4];
  const int mode = st->mode;
  const bool lane0 = threadIdx.x % WAVE == 0;
  if (mode == TK_EXACT) {
    if (lane0) sub_e[r] = sub_m[r];
  } else if (mode == TK_OVERFLOW) {
    const bool vec = ((uintptr_t)dev & 15) == 0;
    int a, e;
    tk_walk<true>(dev, n, (int64_t)r * sw, sw, T, T, vec, map, nullptr, 0, nullptr, a, e);
    a = wave_isum(a);
    if (lane0) sub_a[r] = a, sub_e[r] = e;
  } else {
    const int m = sub_m[r], o = coff[r];
    int gt = 0, eq = 0;
    for (int j = threadIdx.x % WAVE; j < m; j += WAVE) {
      const uint32_t key = tk_canon(cand[o + j]);
      gt += key > T;
      eq += key == T;
    }
    gt = wave_isum(gt);
    eq = wave_isum(eq);
    if (lane0) sub_a[r] += gt, sub_e[r] = eq;
  }
}

// ooff[r]: output offset of sub-range r; eqb[r]: keys equal to T in sub-ranges before r
__global__ __launch_bounds__(TK_THREADS) void tk_mb_scan_out_kernel(int n_sub, const TopkState* __restrict__ st,
                                                                    const int* __restrict__ sub_a,
                                                                    const int* __restrict__ sub_e, int* ooff,
                                                                    int* eqb) {
  __shared__ int wsum[TK_THREADS / WAVE];
  __shared__ int total;
  const int kk = st->kk[4];
  const int r0 = (int)threadIdx.x * TK_SUB_PER;
  int va[TK_SUB_PER], ve[TK_SUB_PER];
#pragma unroll
  for (int j = 0; j < TK_SUB_PER; ++j) {
    const bool in = r0 + j < n_sub;
    va[j] = in ? sub_a[r0 + j] : 0;
    ve[j] = in ? sub_e[r0 + j] : 0;
  }
  int eq = 0;
#pragma unroll
  for (int j = 0; j < TK_SUB_PER; ++j) eq += ve[j];
  int eq_before = block_excl_scan(eq, wsum, &total);
  int sel = 0;
  {
    int e = eq_before;
#pragma unroll
    for (int j = 0; j < TK_SUB_PER; ++j) {
      sel += va[j] + min(max(kk - e, 0), ve[j]);
      e += ve[j];
    }
  }
  int sel_before = block_excl_scan(sel, wsum, &total);
#pragma unroll
  for (int j = 0; j < TK_SUB_PER; ++j) {
    if (r0 + j < n_sub) ooff[r0 + j] = sel_before, eqb[r0 + j] = eq_before;
    sel_before += va[j] + min(max(kk - eq_before, 0), ve[j]);
    eq_before += ve[j];
  }
}

// Ordered write of sub-range r from its map: each lane takes one 32-bit word (16 consecutive
// indices) per step; the words of 4 steps are loaded together and the 4 steps unrolled (a store
// between a load and its use makes the wait cover every earlier memory operation, so loads are
// batched rather than prefetched one step ahead). Undecided indices take their keys from the
// sub-range's candidates in order, which the wave reads 1024 at a time into its LDS buffer (when
// the band is the one key T, or on the overflow route, they are the keys equal to T); keys equal to
// T are taken in index order while fewer than kk precede them. Two wave scans order the lanes; the
// step's positions are staged in the wave's LDS buffer and written out contiguously.
__global__ __launch_bounds__(TK_WPB * WAVE) void tk_mb_write_kernel(int n, int sw, int n_sub, int k,
                                                                    const TopkState* __restrict__ st,
                                                                    const uint32_t* __restrict__ map,
                                                                    const int* __restrict__ sub_m,
                                                                    const int* __restrict__ coff,
                                                                    const int* __restrict__ ooff,
                                                                    const int* __restrict__ eqb,
                                                                    const uint32_t* __restrict__ cand, int cap_c,
                                                                    int* out) {
  __shared__ int stage_all[TK_WPB][1024];
  __shared__ uint32_t cbuf_all[TK_WPB][1024];
  const int r = blockIdx.x * TK_WPB + (int)threadIdx.x / WAVE;
  if (r >= n_sub) return;
  int* stage = stage_all[threadIdx.x / WAVE];
  uint32_t* cbuf = cbuf_all[threadIdx.x / WAVE];
  const int lane = threadIdx.x % WAVE;
  const uint32_t T = st->prefix[4];
  const int kk = st->kk[4];
  const bool all_eq = st->mode == TK_OVERFLOW || st->mode == TK_EXACT;
  int o_run = ooff[r], e_run = eqb[r], c_run = all_eq ? 0 : coff[r];
  const int c_stop = all_eq ? 0 : min(cap_c, c_run + sub_m[r]);
  int buf_base = c_run, buf_end = c_run;  // candidate ordinals held in cbuf
  const int i_begin = r * sw;  // r * sw < n <= INT_MAX
  const int steps = (int)((std::min<int64_t>(n, (int64_t)i_begin + sw) - i_begin + 1023) / 1024);
  const uint32_t* mr = map + (size_t)i_begin / 16;  // the sub-range's sw / 16 map words
  const int last = sw / 16 - 1;
  auto step = [&](uint32_t w, int idx_step) {  // idx_step: the step's first index
    uint32_t take = w & 0x55555555u, eqm = 0;
    const uint32_t und = (w >> 1) & 0x55555555u;
    if (all_eq) {
      eqm = und;
    } else {
      int mtot;
      const int mpre = wave_excl_scan(__popc(und), mtot);
      if (c_run + mtot > buf_end) {  // wave-uniform: refill from c_run (mtot <= 1024)
        wave_sync();
        buf_base = c_run;
        buf_end = min(c_stop, c_run + 1024);
        const int cnt = buf_end - buf_base;  // >= mtot >= 1
        uint32_t v[1024 / WAVE];
#pragma unroll
        for (int i = 0; i < 1024 / WAVE; ++i) v[i] = cand[buf_base + min(lane + WAVE * i, cnt - 1)];
#pragma unroll
        for (int i = 0; i < 1024 / WAVE; ++i)
          if (lane + WAVE * i < cnt) cbuf[lane + WAVE * i] = v[i];
        wave_sync();
      }
      int c = c_run + mpre - buf_base;
      for (uint32_t rest = und; rest; rest &= rest - 1) {
        const uint32_t bit = rest & (0u - rest);
        const uint32_t key = c < 1024 ? tk_canon(cbuf[c]) : 0u;
        ++c;
        if (key > T) take |= bit;
        else if (key == T) eqm |= bit;
      }
      c_run += mtot;
    }
    int ptot;
    const int pk = wave_excl_scan((__popc(eqm) << 16) | __popc(take), ptot);
    const int owed = max(kk - e_run, 0);  // keys equal to T still to take at this step's start
    int o = (pk & 0xffff) + min(pk >> 16, owed);
    // equal keys of this lane still owed (fewer than kk precede them): its first ones in index order
    int eq_owed = min(max(owed - (pk >> 16), 0), __popc(eqm));
    for (uint32_t rest = eqm; eq_owed > 0; --eq_owed) {
      take |= rest & (0u - rest);
      rest &= rest - 1;
    }
    const int idx0 = idx_step + 16 * lane;
    for (uint32_t rest = take; rest; rest &= rest - 1, ++o)
      if (o < 1024) stage[o] = idx0 + (__ffs(rest) - 1) / 2;
    const int taken = (ptot & 0xffff) + min(ptot >> 16, owed);
    wave_sync();
    for (int i = lane; i < taken; i += WAVE)
      if (o_run + i < k) out[o_run + i] = stage[i];
    wave_sync();  // the stage is read before the next step writes it
    e_run += ptot >> 16;
    o_run += taken;
  };
  for (int s0 = 0; s0 < steps; s0 += 4) {
    uint32_t mw[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) mw[q] = mr[min((s0 + q) * WAVE + lane, last)];
    // every word is used (a step past the last runs on an empty word), so the loads stay together
#pragma unroll
    for (int q = 0; q < 4; ++q)  // (an empty step's index is clamped: it must not pass INT_MAX)
      step(s0 + q < steps ? mw[q] : 0u, i_begin + min(s0 + q, steps - 1) * 1024);
  }
}

hipError_t launch_topk_token(const float* dev, int n, int k, int* out, void* ws, size_t ws_bytes, hipStream_t st) {
  if (k <= 0 || n <= 0) return hipSuccess;
  if (n < TK_MB_MIN) {
    hipLaunchKernelGGL(topk_token_kernel, dim3(1), dim3(TK_THREADS), 0, st, dev, n, k, out);
    return hipGetLastError();
  }
  const size_t fixed = tk_mb_fixed_bytes(n);
  if (!ws || ws_bytes < fixed) return hipErrorInvalidValue;
  int sw, n_sub;
  tk_geom(n, sw, n_sub);
  char* w = reinterpret_cast<char*>(ws);
  uint32_t* hist = reinterpret_cast<uint32_t*>(w);
  TopkState* state = reinterpret_cast<TopkState*>(w + 4 * 256 * sizeof(uint32_t));
  uint32_t* skey = reinterpret_cast<uint32_t*>(w + 4 * 256 * sizeof(uint32_t) + 256);
  int* sub = reinterpret_cast<int*>(w + TK_HEAD_BYTES);
  int *sub_a = sub, *sub_m = sub + n_sub, *sub_e = sub + 2 * n_sub, *coff = sub + 3 * n_sub, *ooff = sub + 4 * n_sub,
      *eqb = sub + 5 * n_sub;
  uint8_t* map = reinterpret_cast<uint8_t*>(w + TK_HEAD_BYTES + tk_sub_bytes(n_sub));
  // beyond the fixed part: up to n/16 list entries first, then up to sw/16 slice entries per
  // sub-range, then whatever is left extends the list
  size_t room = (ws_bytes - fixed) / sizeof(uint32_t);
  size_t cap_c = std::min<size_t>((size_t)n / 16, room);
  room -= cap_c;
  const size_t cap_w = std::min<size_t>((size_t)sw / 16, room / n_sub);
  room -= cap_w * n_sub;
  cap_c += std::min<size_t>((size_t)n - cap_c, room);
  uint32_t* slices = reinterpret_cast<uint32_t*>(w + fixed);
  uint32_t* cand = slices + cap_w * n_sub;
  const int gw = (n_sub + TK_WPB - 1) / TK_WPB, cw = (int)cap_w, cc = (int)cap_c;
  const int hist_blocks = (int)std::min<int64_t>(TK_HIST_BLOCKS, ((int64_t)n + 1023) / 1024);
  hipLaunchKernelGGL(tk_mb_gather_kernel, dim3(TK_SAMPLE / 256), dim3(256), 0, st, dev, n, skey);
  hipLaunchKernelGGL(tk_mb_sample_kernel, dim3(1), dim3(TK_THREADS), 0, st, skey, n, k, hist, state);
  for (int round = 0; round < 2; ++round) {
    if (round == 1)
      for (int pass = 0; pass < 2; ++pass) {
        hipLaunchKernelGGL(tk_mb_hist_kernel, dim3(hist_blocks), dim3(256), 0, st, dev, n, pass, state, cand, hist);
        hipLaunchKernelGGL(tk_mb_pick_kernel, dim3(1), dim3(256), 0, st, pass, state, hist);
      }
    hipLaunchKernelGGL(tk_mb_collect_kernel, dim3(gw), dim3(TK_WPB * WAVE), 0, st, dev, n, sw, n_sub, round, state,
                       sub_a, sub_m, map, slices, cw);
    hipLaunchKernelGGL(tk_mb_scan_cand_kernel, dim3(1), dim3(TK_THREADS), 0, st, n_sub, k, round, cc, state, sub_a,
                       sub_m, coff);
    hipLaunchKernelGGL(tk_mb_compact_kernel, dim3(gw), dim3(TK_WPB * WAVE), 0, st, dev, n, sw, n_sub, round, state,
                       sub_m, coff, slices, cw, cand, cc);
  }
  for (int pass = 2; pass < 4; ++pass) {
    hipLaunchKernelGGL(tk_mb_hist_kernel, dim3(hist_blocks), dim3(256), 0, st, dev, n, pass, state, cand, hist);
    hipLaunchKernelGGL(tk_mb_pick_kernel, dim3(1), dim3(256), 0, st, pass, state, hist);
  }
  hipLaunchKernelGGL(tk_mb_count_kernel, dim3(gw), dim3(TK_WPB * WAVE), 0, st, dev, n, sw, n_sub, state, sub_a, sub_m,
                     sub_e, coff, cand, map);
  hipLaunchKernelGGL(tk_mb_scan_out_kernel, dim3(1), dim3(TK_THREADS), 0, st, n_sub, state, sub_a, sub_e, ooff, eqb);
  hipLaunchKernelGGL(tk_mb_write_kernel, dim3(gw), dim3(TK_WPB * WAVE), 0, st, n, sw, n_sub, k, state,
                     reinterpret_cast<const uint32_t*>(map), sub_m, coff, ooff, eqb, cand, cc, out);
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
  const bool doc = sp.mode == SPAN_DOC;
  // take[j]: how many leading tokens of span j are selected (the whole span, a head, or none)
  // 1. span means (fp64, sequential within the span); document-aligned only
  for (int j = threadIdx.x; j < ns; j += TK_THREADS) {
    double s = 0.0;
    if (doc)
      for (int i = sp.b[j]; i < sp.b[j + 1]; ++i) s += canon_d(dev[i]);
    score[j] = s / (double)(sp.b[j + 1] - sp.b[j]);
    take[j] = 0;
  }
  __syncthreads();
  // 2. ranking: by (score desc, index asc), or the given order
  for (int j = threadIdx.x; j < ns; j += TK_THREADS) {
    if (doc) {
      int r = 0;
      for (int i = 0; i < ns; ++i) r += (score[i] > score[j] || (score[i] == score[j] && i < j)) ? 1 : 0;
      order[r] = j;
    } else {
      order[j] = sp.order[j];
    }
  }
  __syncthreads();
  // 3. heads of every span: the smallest head length T with sum min(len, T) >= k (bisection),
  //    then one token less for the last spans holding T until exactly k remain
  if (sp.mode == SPAN_HEADS) {
    if (threadIdx.x == 0) {
      int lo = 0, hi = 0;
      for (int j = 0; j < ns; ++j) hi = max(hi, sp.b[j + 1] - sp.b[j]);
      while (lo < hi) {
        const int mid = (lo + hi) / 2;
        int tot = 0;
        for (int j = 0; j < ns; ++j) tot += min(sp.b[j + 1] - sp.b[j], mid);
        if (tot >= k) hi = mid; else lo = mid + 1;
      }
      int excess = -k;
      for (int j = 0; j < ns; ++j) {
        take[j] = min(sp.b[j + 1] - sp.b[j], lo);
        excess += take[j];
      }
      for (int j = ns - 1; j >= 0 && excess > 0; --j)
        if (lo > 0 && take[j] == lo) --take[j], --excess;
      s_part = -1;
      s_rem = 0;
      s_wa = -1;
    }
    __syncthreads();
  }
  // 3. whole spans while they fit; the first that does not gives its best window (document-
  //    aligned) or its head (ranked)
  else if (threadIdx.x == 0) {
    int rem = k, part = -1;
    for (int r = 0; r < ns && rem > 0; ++r) {
      const int j = order[r];
      const int len = sp.b[j + 1] - sp.b[j];
      if (len <= rem) {
        take[j] = len;
        rem -= len;
      } else {
        part = j;
        break;
      }
    }
    if (!doc && part >= 0) {
      take[part] = rem;
      part = -1;
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
    return i - sp.b[lo] < take[lo] || (wa >= 0 && i >= wa && i < wa + wl);
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
