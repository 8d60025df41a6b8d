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
// The same exact selection spread over the whole GPU for n >= TK_MB_MIN. Two 8-bit histogram
// passes over the n keys (LDS histograms merged with global atomics), each followed by a
// one-thread pick of the digit, fix the top 16 bits of the threshold key T. One collect pass then
// counts, per block range, the keys whose top 16 bits lie above T's and appends the keys that
// share them (the only ones still undecided) to a candidate list with their indices. The last two
// digits of T and the per-range counts of keys above / equal to T come from that list alone. A
// one-block scan turns the counts into output offsets and ranks among equal keys (lower index
// first), and an ordered write of each block's range, the fourth and last read of the n keys,
// writes the positions. When the threshold's 16-bit bin holds more keys than the candidate list
// has room for (known from the second histogram before anything is collected), the last two
// digits and the counts come from passes over all n keys instead. No block waits for another.
constexpr int TK_MB_MIN = 1 << 16;
constexpr int TK_MB_SEG = 16384;       // indices per count / write block (at least)
constexpr int TK_MB_MAX_BLOCKS = 2048;
constexpr int TK_HIST_BLOCKS = 1024;   // histogram blocks (grid-stride), fewer merges into the global bins

struct TopkState {
  uint32_t prefix[5];  // prefix[p]: the top 8p bits of T fixed by passes < p
  int kk[5];           // kk[p]: keys still owed among those matching prefix[p]
  int overflow;        // 1: the threshold's 16-bit bin does not fit the candidate list
  int n_cand;          // candidates appended by the collect pass
};
static_assert(sizeof(TopkState) <= 256, "state slot");

static int tk_mb_blocks(int n) {
  return (int)std::min<int64_t>(TK_MB_MAX_BLOCKS, ((int64_t)n + TK_MB_SEG - 1) / TK_MB_SEG);
}

// histograms, state, per-block counts and offsets; the candidate list follows
static size_t tk_mb_fixed_bytes(int n) {
  return 4 * 256 * sizeof(uint32_t) + 256 + (size_t)tk_mb_blocks(n) * 4 * sizeof(int);
}

size_t topk_token_ws_min_bytes(int n) { return n < TK_MB_MIN ? 0 : tk_mb_fixed_bytes(n); }

size_t topk_token_ws_bytes(int n) {
  if (n < TK_MB_MIN) return 0;
  return tk_mb_fixed_bytes(n) + (size_t)(n / 16) * 2 * sizeof(uint32_t);  // room for n/16 candidates
}

__global__ __launch_bounds__(TK_THREADS) void tk_mb_init_kernel(uint32_t* hist, TopkState* st, int k) {
  hist[threadIdx.x] = 0;  // 4 x 256 bins
  if (threadIdx.x == 0) {
    st->prefix[0] = 0;
    st->kk[0] = k;
    st->overflow = 0;
    st->n_cand = 0;
  }
}

// 16 copies of the 256 bins per block (lane % 16 picks the copy): deviations, like most float
// data, put most keys into a few top-byte bins, and same-address LDS atomics serialise. Passes 0
// and 1 read the n keys; passes 2 and 3 read the candidate list unless it overflowed.
constexpr int TK_HCOPIES = 16;

__global__ __launch_bounds__(256) void tk_mb_hist_kernel(const float* __restrict__ dev, int n, int pass,
                                                         const TopkState* __restrict__ st,
                                                         const uint32_t* __restrict__ cand, uint32_t* hist) {
  const bool from_cand = pass >= 2 && !st->overflow;
  const int m = from_cand ? st->n_cand : n;
  if (from_cand && (int64_t)blockIdx.x * blockDim.x >= m) return;  // block-uniform: no candidate here
  __shared__ uint32_t h[TK_HCOPIES][257];  // rows of 257 words: the copies of a bin in different banks
#pragma unroll
  for (int c = 0; c < TK_HCOPIES; ++c) h[c][threadIdx.x] = 0;
  __syncthreads();
  const uint32_t prefix = st->prefix[pass];
  const uint32_t mask = pass == 0 ? 0u : (0xffffffffu << (32 - 8 * pass));
  const int shift = 24 - 8 * pass;
  uint32_t* mine = h[threadIdx.x % TK_HCOPIES];
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x, stride = (int64_t)gridDim.x * blockDim.x;
  auto add = [&](uint32_t key) {
    if ((key & mask) == prefix) atomicAdd(&mine[(key >> shift) & 255u], 1u);
  };
  if (from_cand) {
    for (int64_t i = gid; i < m; i += stride) add(cand[i]);
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

__global__ __launch_bounds__(256) void tk_mb_pick_kernel(int pass, TopkState* st, const uint32_t* hist,
                                                         int cap) {
  // as in the one-workgroup kernel: thread t takes bin 255 - t and an inclusive scan over the
  // threads counts the keys from the top bin down; the bin where the count first reaches kk wins
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
    st->prefix[pass + 1] = st->prefix[pass] | ((uint32_t)(255 - t) << (24 - 8 * pass));
    st->kk[pass + 1] = kk - above;
    if (pass == 1) st->overflow = h > cap;  // h keys share T's top 16 bits
  }
}

// Collect pass over block b's index range (the count / write partition): blk[2b] = keys whose top
// 16 bits exceed T's, blk[2b+1] = 0; keys sharing T's top 16 bits go to the candidate list. They
// are staged in LDS (wave-aggregated LDS atomics) and reserve their global slots with one atomic
// per flush of the stage, so a block's candidates land contiguously and the one global counter
// sees about one atomic per block. The list holds at most cap entries: the pick of pass 1 set the
// overflow flag otherwise, and then this pass does nothing.
constexpr int TK_CSTAGE = 8192;  // staged candidates per block: 64 KB of LDS
constexpr int TK_CTILE = 4 * TK_THREADS;

__global__ __launch_bounds__(TK_THREADS) void tk_mb_collect_kernel(const float* __restrict__ dev, int n, int seg,
                                                                   TopkState* st, int* blk, uint32_t* ckey,
                                                                   int* cidx) {
  if (st->overflow) return;
  __shared__ uint32_t sk[TK_CSTAGE];
  __shared__ int si[TK_CSTAGE];
  __shared__ int red[TK_THREADS / WAVE];
  __shared__ int cnt, gbase;
  const uint32_t p16 = st->prefix[2] >> 16;
  const int b0 = blockIdx.x * seg, b1 = (int)min((int64_t)n, (int64_t)b0 + seg);
  const int lane = threadIdx.x % WAVE;
  if (threadIdx.x == 0) cnt = 0;
  int gt = 0;
  auto visit = [&](uint32_t key, int i, bool in) {
    const uint32_t d = key >> 16;
    gt += in && d > p16;
    const bool c = in && d == p16;
    const uint64_t bal = __ballot(c);
    if (bal == 0) return;
    int base = 0;
    if (lane == 0) base = atomicAdd(&cnt, __popcll(bal));
    base = __shfl(base, 0, WAVE);
    if (c) {
      const int slot = base + __popcll(bal & ((1ull << lane) - 1));
      sk[slot] = key;
      si[slot] = i;
    }
  };
  // moves the staged candidates to the global list; every thread of the block calls it
  auto flush = [&]() {
    if (threadIdx.x == 0) gbase = cnt ? atomicAdd(&st->n_cand, cnt) : 0;
    __syncthreads();
    const int m = cnt, g = gbase;
    for (int j = threadIdx.x; j < m; j += TK_THREADS) {
      ckey[g + j] = sk[j];
      cidx[g + j] = si[j];
    }
    __syncthreads();
    if (threadIdx.x == 0) cnt = 0;
    __syncthreads();  // the reset is seen before any wave stages again
  };
  // b0 is a multiple of 64, so with a 16-byte aligned dev the 4-wide loads are aligned. Tiles of
  // TK_CTILE indices: each tile adds at most TK_CTILE candidates, so the stage is flushed before a
  // tile whenever less room than that is left; every lane of a wave runs the same iterations, so
  // the ballots see the whole wave
  const bool vec = ((uintptr_t)dev & 15) == 0;
  const int v1 = vec ? b0 + (b1 - b0) / 4 * 4 : b0;
  for (int64_t base = b0; base < b1; base += TK_CTILE) {
    __syncthreads();
    if (cnt > TK_CSTAGE - TK_CTILE) flush();
    if (base + TK_CTILE <= v1) {
      const int i = (int)base + 4 * (int)threadIdx.x;
      const float4 v = *reinterpret_cast<const float4*>(dev + i);
      visit(order_key(v.x), i, true), visit(order_key(v.y), i + 1, true), visit(order_key(v.z), i + 2, true),
          visit(order_key(v.w), i + 3, true);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t i = base + e * TK_THREADS + (int)threadIdx.x;
        const bool in = i < b1;
        visit(in ? order_key(dev[i]) : 0u, in ? (int)i : 0, in);
      }
    }
  }
  __syncthreads();
  flush();
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) gt += __shfl_xor(gt, o, WAVE);
  const int w = threadIdx.x / WAVE;
  if (lane == 0) red[w] = gt;
  __syncthreads();
  if (threadIdx.x == 0) {
    int a = 0;
    for (int i = 0; i < TK_THREADS / WAVE; ++i) a += red[i];
    blk[2 * blockIdx.x] = a;
    blk[2 * blockIdx.x + 1] = 0;
  }
}

// Adds each candidate above / equal to T to its block range's counts. A wave's candidates come in
// runs from one range (a collect block flushes its staged candidates at once), so the lanes
// sharing a range are counted together: one atomic per range and wave.
__global__ __launch_bounds__(256) void tk_mb_count_cand_kernel(int seg, const TopkState* __restrict__ st,
                                                               const uint32_t* __restrict__ ckey,
                                                               const int* __restrict__ cidx, int* blk) {
  if (st->overflow) return;
  const int m = st->n_cand;
  const uint32_t T = st->prefix[4];
  const int lane = threadIdx.x % WAVE;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  // whole waves step together so the ballots see every lane
  for (int64_t base = (int64_t)blockIdx.x * blockDim.x; base < m; base += stride) {
    const int64_t i = base + threadIdx.x;
    const bool in = i < m;
    const uint32_t key = in ? ckey[i] : 0u;
    const int b = in ? cidx[i] / seg : -1;
    uint64_t todo = __ballot(in && key >= T);
    while (todo) {
      const int leader = __ffsll((unsigned long long)todo) - 1;
      const int bl = __shfl(b, leader, WAVE);
      const uint64_t same = todo & __ballot(b == bl);
      const int gt = __popcll(same & __ballot(key > T)), eq = __popcll(same) - gt;
      if (lane == leader) {
        if (gt) atomicAdd(&blk[2 * bl], gt);
        if (eq) atomicAdd(&blk[2 * bl + 1], eq);
      }
      todo &= ~same;
    }
  }
}

// blk[2b], blk[2b+1]: keys above / equal to T in block b's index range, from all n keys (overflow)
__global__ __launch_bounds__(TK_THREADS) void tk_mb_count_kernel(const float* __restrict__ dev, int n, int seg,
                                                                 const TopkState* __restrict__ st, int* blk) {
  if (!st->overflow) return;  // the collect pass and the candidate list gave the counts
  __shared__ int red[2][TK_THREADS / WAVE];
  const uint32_t T = st->prefix[4];
  const int b0 = blockIdx.x * seg, b1 = (int)min((int64_t)n, (int64_t)b0 + seg);
  int gt = 0, eq = 0;
  auto cnt = [&](float x) {
    const uint32_t key = order_key(x);
    gt += key > T;
    eq += key == T;
  };
  // b0 is a multiple of 64, so with a 16-byte aligned dev the 4-wide loads are aligned
  const bool vec = ((uintptr_t)dev & 15) == 0;
  const int v1 = vec ? b0 + (b1 - b0) / 4 * 4 : b0;
  for (int64_t i = b0 + 4 * (int)threadIdx.x; i < v1; i += 4 * TK_THREADS) {
    const float4 v = *reinterpret_cast<const float4*>(dev + i);
    cnt(v.x), cnt(v.y), cnt(v.z), cnt(v.w);
  }
  for (int64_t i = v1 + (int)threadIdx.x; i < b1; i += TK_THREADS) cnt(dev[i]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    gt += __shfl_xor(gt, o, WAVE);
    eq += __shfl_xor(eq, o, WAVE);
  }
  const int w = threadIdx.x / WAVE;
  if (threadIdx.x % WAVE == 0) red[0][w] = gt, red[1][w] = eq;
  __syncthreads();
  if (threadIdx.x == 0) {
    int a = 0, e = 0;
    for (int i = 0; i < TK_THREADS / WAVE; ++i) a += red[0][i], e += red[1][i];
    blk[2 * blockIdx.x] = a;
    blk[2 * blockIdx.x + 1] = e;
  }
}

// off[2b]: output offset of block b; off[2b+1]: keys equal to T in blocks before b
__global__ __launch_bounds__(TK_THREADS) void tk_mb_scan_kernel(int nb, const TopkState* __restrict__ st,
                                                                const int* __restrict__ blk, int* off) {
  __shared__ int wsum[TK_THREADS / WAVE];
  __shared__ int total;
  const int kk = st->kk[4];
  const int per = (nb + TK_THREADS - 1) / TK_THREADS;
  const int b0 = min(nb, (int)threadIdx.x * per), b1 = min(nb, b0 + per);
  int eq = 0;
  for (int b = b0; b < b1; ++b) eq += blk[2 * b + 1];
  int eq_before = block_excl_scan(eq, wsum, &total);
  int sel = 0;
  {
    int e = eq_before;
    for (int b = b0; b < b1; ++b) {
      const int eb = blk[2 * b + 1];
      sel += blk[2 * b] + min(max(kk - e, 0), eb);
      e += eb;
    }
  }
  int sel_before = block_excl_scan(sel, wsum, &total);
  for (int b = b0; b < b1; ++b) {
    const int eb = blk[2 * b + 1];
    off[2 * b] = sel_before;
    off[2 * b + 1] = eq_before;
    sel_before += blk[2 * b] + min(max(kk - eq_before, 0), eb);
    eq_before += eb;
  }
}

// Each thread owns TK_EPT consecutive indices of a tile (one 16-byte load, coalesced across the
// wave), so one block scan orders TK_THREADS * TK_EPT positions. The scan runs over (keys equal to
// T) << 16 | (keys above T) per thread (a tile's counts fit 16 bits): keys equal to T are taken in
// index order while fewer than kk of them precede, so the positions taken before a thread are its
// keys-above prefix plus min(equal prefix, kk - equal keys of earlier tiles). The next tile's keys
// are loaded before the current tile's scan; a tile's positions are staged in LDS and written out
// contiguously.
constexpr int TK_EPT = 4;
static_assert(TK_THREADS * TK_EPT < (1 << 16), "packed tile counts");

__device__ __forceinline__ void tk_load_tile(const float* __restrict__ dev, int64_t i0, int b1, bool vec,
                                             uint32_t (&key)[TK_EPT]) {
  if (vec && i0 + TK_EPT <= b1) {
#pragma unroll
    for (int e = 0; e < TK_EPT; e += 4) {
      const float4 v = *reinterpret_cast<const float4*>(dev + i0 + e);
      key[e] = order_key(v.x), key[e + 1] = order_key(v.y), key[e + 2] = order_key(v.z), key[e + 3] = order_key(v.w);
    }
  } else {
#pragma unroll
    for (int e = 0; e < TK_EPT; ++e) key[e] = i0 + e < b1 ? order_key(dev[i0 + e]) : 0u;
  }
}

__global__ __launch_bounds__(TK_THREADS) void tk_mb_write_kernel(const float* __restrict__ dev, int n, int seg,
                                                                 const TopkState* __restrict__ st,
                                                                 const int* __restrict__ off, int k, int* out) {
  constexpr int TILE = TK_THREADS * TK_EPT;
  __shared__ int wsum[TK_THREADS / WAVE];
  __shared__ int total;
  __shared__ int stage[TILE];
  const uint32_t T = st->prefix[4];
  const int kk = st->kk[4];
  const int b0 = blockIdx.x * seg, b1 = (int)min((int64_t)n, (int64_t)b0 + seg);
  int o_run = off[2 * blockIdx.x], e_run = off[2 * blockIdx.x + 1];
  const bool vec = ((uintptr_t)dev & 15) == 0;  // b0 and i0 are multiples of 4 elements
  uint32_t key[TK_EPT], nxt[TK_EPT];
  if (b0 < b1) tk_load_tile(dev, b0 + (int)threadIdx.x * TK_EPT, b1, vec, nxt);
  for (int64_t base = b0; base < b1; base += TILE) {
    const int64_t i0 = base + (int)threadIdx.x * TK_EPT;
#pragma unroll
    for (int e = 0; e < TK_EPT; ++e) key[e] = nxt[e];
    if (base + TILE < b1) tk_load_tile(dev, i0 + TILE, b1, vec, nxt);
    int n_eq = 0, n_gt = 0;
#pragma unroll
    for (int e = 0; e < TK_EPT; ++e) {
      const bool in = i0 + e < b1;
      n_eq += in && key[e] == T;
      n_gt += in && key[e] > T;
    }
    const int pre = block_excl_scan((n_eq << 16) | n_gt, wsum, &total);
    const int tot = total;
    const int owed = max(kk - e_run, 0);  // keys equal to T still to take at this tile's start
    int r = e_run + (pre >> 16);
    int o = (pre & 0xffff) + min(pre >> 16, owed);  // within the tile
#pragma unroll
    for (int e = 0; e < TK_EPT; ++e) {
      const bool in = i0 + e < b1, eq = in && key[e] == T;
      if (in && (key[e] > T || (eq && r < kk))) stage[o++] = (int)(i0 + e);
      r += eq;
    }
    const int take = (tot & 0xffff) + min(tot >> 16, owed);
    __syncthreads();
    for (int j = threadIdx.x; j < take; j += TK_THREADS)
      if (o_run + j < k) out[o_run + j] = stage[j];
    // the next tile's scan starts with a barrier, so stage is not overwritten while it is read
    e_run += tot >> 16;
    o_run += take;
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
  char* w = reinterpret_cast<char*>(ws);
  uint32_t* hist = reinterpret_cast<uint32_t*>(w);
  TopkState* state = reinterpret_cast<TopkState*>(w + 4 * 256 * sizeof(uint32_t));
  int* blk = reinterpret_cast<int*>(w + 4 * 256 * sizeof(uint32_t) + 256);
  const int nb = tk_mb_blocks(n);
  int* off = blk + 2 * nb;
  // candidate list: keys, then indices, in what the workspace holds beyond the fixed part
  const int cap = (int)std::min<size_t>((ws_bytes - fixed) / (2 * sizeof(uint32_t)), (size_t)n);
  uint32_t* ckey = reinterpret_cast<uint32_t*>(w + fixed);
  int* cidx = reinterpret_cast<int*>(ckey + cap);
  const int seg = (int)((((int64_t)n + nb - 1) / nb + 63) / 64 * 64);  // block ranges start at multiples of 64
  hipLaunchKernelGGL(tk_mb_init_kernel, dim3(1), dim3(TK_THREADS), 0, st, hist, state, k);
  const int hist_blocks = (int)std::min<int64_t>(TK_HIST_BLOCKS, ((int64_t)n + 1023) / 1024);
  for (int pass = 0; pass < 4; ++pass) {
    if (pass == 2)
      hipLaunchKernelGGL(tk_mb_collect_kernel, dim3(nb), dim3(TK_THREADS), 0, st, dev, n, seg, state, blk, ckey, cidx);
    hipLaunchKernelGGL(tk_mb_hist_kernel, dim3(hist_blocks), dim3(256), 0, st, dev, n, pass, state, ckey, hist);
    hipLaunchKernelGGL(tk_mb_pick_kernel, dim3(1), dim3(256), 0, st, pass, state, hist, cap);
  }
  hipLaunchKernelGGL(tk_mb_count_cand_kernel, dim3(hist_blocks), dim3(256), 0, st, seg, state, ckey, cidx, blk);
  hipLaunchKernelGGL(tk_mb_count_kernel, dim3(nb), dim3(TK_THREADS), 0, st, dev, n, seg, state, blk);
  hipLaunchKernelGGL(tk_mb_scan_kernel, dim3(1), dim3(TK_THREADS), 0, st, nb, state, blk, off);
  hipLaunchKernelGGL(tk_mb_write_kernel, dim3(nb), dim3(TK_THREADS), 0, st, dev, n, seg, state, off, k, out);
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
