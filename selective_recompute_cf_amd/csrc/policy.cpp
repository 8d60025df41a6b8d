// libcf host-side policy arithmetic: the recompute budget, the gradual-filtering schedule, the
// loading controller, the span bounds of the span-policy ablations, the chunk-anchor positions and
// the selection diagnostics.
// These are plain host computations on host arrays (no device memory, no stream); they live in the
// library so that every step of the method, including its integer bookkeeping, is one C call.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <vector>

#include "cf.h"
#include "status.h"

namespace {

cf_status bad(cf_status s, const char* msg) { return cf::set_error(s, msg); }

// k = max(1, floor(N num / den)) for num > 0, 0 for num = 0 or N = 0 (64-bit integer arithmetic).
int64_t budget_of(int64_t n, int64_t num, int64_t den) {
  if (num == 0 || n == 0) return 0;
  return std::max<int64_t>(1, n * num / den);
}

bool ratio_ok(int32_t num, int32_t den) { return num >= 0 && den > 0 && num <= den; }

}  // namespace

extern "C" {

cf_status cf_budget(int32_t n_ctx, int32_t rho_num, int32_t rho_den, int32_t* k) {
  cf::clear_error();
  if (!k) return bad(CF_EINVAL, "null output");
  if (n_ctx < 0) return bad(CF_EINVAL, "negative context size");
  if (!ratio_ok(rho_num, rho_den)) return bad(CF_EINVAL, "ratio must be num/den with 0 <= num <= den, den > 0");
  *k = (int32_t)budget_of(n_ctx, rho_num, rho_den);
  return CF_OK;
}

cf_status cf_gradual_schedule(int32_t n_ctx, int32_t n_sched, int32_t first_num, int32_t first_den,
                              int32_t keep_num, int32_t keep_den, int32_t final_num, int32_t final_den,
                              int32_t* k_sched) {
  cf::clear_error();
  if (n_ctx < 0 || n_sched < 0) return bad(CF_EINVAL, "negative size");
  if (n_sched > 0 && !k_sched) return bad(CF_EINVAL, "null output");
  if (!ratio_ok(first_num, first_den) || !ratio_ok(final_num, final_den))
    return bad(CF_EINVAL, "ratios must be num/den with 0 <= num <= den, den > 0");
  if (!ratio_ok(keep_num, keep_den)) return bad(CF_EINVAL, "keep fraction must be in [0, 1]");
  const int64_t top = budget_of(n_ctx, first_num, first_den), low = budget_of(n_ctx, final_num, final_den);
  if (low > top) return bad(CF_EINVAL, "the final ratio must not exceed the first");
  int64_t cur = top;
  for (int32_t i = 0; i < n_sched; ++i) {
    k_sched[i] = (int32_t)cur;
    if (cur > 0) cur = std::max(low, std::max<int64_t>(1, cur * keep_num / keep_den));
  }
  return CF_OK;
}

cf_status cf_loading_ratio(double load_ms, const int32_t* ratios, const double* recompute_ms, int32_t n,
                           int32_t floor_num, int32_t floor_den, int32_t* out_num, int32_t* out_den) {
  cf::clear_error();
  if (!out_num || !out_den || n < 0 || (n > 0 && (!ratios || !recompute_ms)))
    return bad(CF_EINVAL, "null pointer or negative count");
  if (!ratio_ok(floor_num, floor_den)) return bad(CF_EINVAL, "floor must be num/den with 0 <= num <= den, den > 0");
  int best = -1;
  for (int32_t i = 0; i < n; ++i) {
    const int64_t a = ratios[2 * i], b = ratios[2 * i + 1];
    if (!ratio_ok((int32_t)a, (int32_t)b)) return bad(CF_EINVAL, "ratio entries must be num/den in [0, 1]");
    if (!(recompute_ms[i] <= load_ms)) continue;  // recompute of this ratio does not hide under the load
    if (best < 0 || a * ratios[2 * best + 1] > (int64_t)ratios[2 * best] * b) best = i;
  }
  if (best < 0 || (int64_t)ratios[2 * best] * floor_den < (int64_t)floor_num * ratios[2 * best + 1]) {
    *out_num = floor_num;
    *out_den = floor_den;
  } else {
    *out_num = ratios[2 * best];
    *out_den = ratios[2 * best + 1];
  }
  return CF_OK;
}

cf_status cf_single_window_bounds(int32_t n_ctx, int32_t* bounds, int32_t cap, int32_t* n_bounds) {
  cf::clear_error();
  if (n_ctx < 0 || !n_bounds || (cap > 0 && !bounds)) return bad(CF_EINVAL, "bad arguments");
  *n_bounds = 2;
  if (cap < 2) return bad(CF_EINVAL, "bounds array needs 2 entries");
  bounds[0] = 0;
  bounds[1] = n_ctx;
  return CF_OK;
}

cf_status cf_fixed_chunk_bounds(int32_t n_ctx, int32_t size, int32_t offset, int32_t* bounds, int32_t cap,
                                int32_t* n_bounds) {
  cf::clear_error();
  if (n_ctx < 0 || !n_bounds || (cap > 0 && !bounds)) return bad(CF_EINVAL, "bad arguments");
  if (size <= 0 || offset < 0 || offset >= size) return bad(CF_EINVAL, "need size > 0 and 0 <= offset < size");
  std::vector<int32_t> b{0};
  if (n_ctx > 0) {
    for (int64_t at = offset > 0 ? offset : size; at < n_ctx; at += size) b.push_back((int32_t)at);
  }
  b.push_back(n_ctx);
  *n_bounds = (int32_t)b.size();
  if ((int64_t)b.size() > cap) return bad(CF_EINVAL, "bounds array too small (n_bounds holds the size needed)");
  std::copy(b.begin(), b.end(), bounds);
  return CF_OK;
}

cf_status cf_anchor_positions(int32_t rule, const int32_t* chunk_tab, int32_t m, int32_t ra_num, int32_t ra_den,
                              const float* scores, int32_t store_rows, int32_t* anchors, int32_t cap,
                              int32_t* n_anchors) {
  cf::clear_error();
  if (!n_anchors || m < 0 || (m > 0 && !chunk_tab) || (cap > 0 && !anchors)) return bad(CF_EINVAL, "bad arguments");
  if (rule != CF_ANCHOR_SINK && rule != CF_ANCHOR_KNORM && rule != CF_ANCHOR_KNORM_LOW)
    return bad(CF_EINVAL, "unknown anchor rule");
  if (!ratio_ok(ra_num, ra_den)) return bad(CF_EINVAL, "anchor ratio must be num/den with 0 <= num <= den, den > 0");
  if (rule != CF_ANCHOR_SINK && !scores) return bad(CF_EINVAL, "key-norm anchors need the per-row scores");
  std::vector<int32_t> out;
  std::vector<int32_t> idx;
  for (int32_t i = 0; i < m; ++i) {
    const int32_t row = chunk_tab[4 * i], dst = chunk_tab[4 * i + 2], len = chunk_tab[4 * i + 3];
    if (len <= 0 || row < 0 || dst < 0 || (rule != CF_ANCHOR_SINK && (int64_t)row + len > store_rows))
      return bad(CF_EINVAL, "chunk rows outside the store or empty chunk");
    const int64_t n_a = ((int64_t)len * ra_num + ra_den - 1) / ra_den;  // ceil(r_a |c_i|)
    idx.resize(len);
    for (int32_t r = 0; r < len; ++r) idx[r] = r;
    if (rule != CF_ANCHOR_SINK) {
      // TopK of the score (largest norm, or smallest for the low rule); equal scores keep the lower
      // position; NaN ranks as +inf
      const float* g = scores + row;
      const bool low = rule == CF_ANCHOR_KNORM_LOW;
      auto key = [&](int32_t r) { const double v = g[r]; return std::isnan(v) ? INFINITY : (low ? -v : v); };
      std::stable_sort(idx.begin(), idx.end(), [&](int32_t a, int32_t b) { return key(a) > key(b); });
    }
    std::sort(idx.begin(), idx.begin() + n_a);
    for (int64_t r = 0; r < n_a; ++r) out.push_back(dst + idx[r]);
  }
  std::sort(out.begin(), out.end());
  for (size_t i = 1; i < out.size(); ++i)
    if (out[i] == out[i - 1]) return bad(CF_EINVAL, "chunk destinations overlap");
  *n_anchors = (int32_t)out.size();
  if ((int64_t)out.size() > cap) return bad(CF_EINVAL, "anchor array too small (n_anchors holds the size needed)");
  std::copy(out.begin(), out.end(), anchors);
  return CF_OK;
}

cf_status cf_selection_stats(const int32_t* sel, int32_t k, const float* dev, int32_t n, int32_t* segments,
                             double* captured) {
  cf::clear_error();
  if (!segments || !captured || k < 0 || n < 0 || (k > 0 && !sel) || (n > 0 && !dev))
    return bad(CF_EINVAL, "bad arguments");
  std::vector<int32_t> s(sel, sel + k);
  std::sort(s.begin(), s.end());
  for (int32_t i = 0; i < k; ++i) {
    if (s[i] < 0 || s[i] >= n) return bad(CF_EINVAL, "selected position outside [0, n)");
    if (i && s[i] == s[i - 1]) return bad(CF_EINVAL, "selected positions must be distinct");
  }
  int32_t seg = 0;
  for (int32_t i = 0; i < k; ++i)
    if (i == 0 || s[i] != s[i - 1] + 1) ++seg;
  // deviation with NaN counted as +inf (the order the selection uses), summed in fp64
  auto val = [&](int32_t i) { const double v = dev[i]; return std::isnan(v) ? INFINITY : v; };
  double total = 0.0, taken = 0.0;
  for (int32_t i = 0; i < n; ++i) total += val(i);
  for (int32_t i = 0; i < k; ++i) taken += val(s[i]);
  *segments = seg;
  *captured = total > 0.0 ? taken / total : 0.0;
  return CF_OK;
}

}  // extern "C"
