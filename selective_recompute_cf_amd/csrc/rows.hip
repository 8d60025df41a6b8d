// Row-wise and element-wise kernels of libcf (HBM-bound): RoPE re-positioning and stitching,
// embedding gather, RMSNorm gather, projection post-processing (qk-norm, RoPE, K/V scatter,
// fused KV deviation), split-K reduction with residual, SwiGLU, standalone deviation.
#include "common.h"
#include "kernels.h"

namespace cf {

// ----------------------------------------------------------------------------- re-position
// QCFuse Eq. 4 (remap + stitch) with the rotation composition of CacheBlend ("Why You Can't
// Just Concatenate"): a key encoded at p is moved to p + delta by rotating every pair
// (x_j, x_{j+hd/2}) by delta * omega_j; values are copied. One block moves up to
// REPOS_ROWS_PER_BLOCK rows of one chunk of one layer; each thread moves 8 pairs of K
// (two 16-byte loads for bf16) or 8 elements of V per step.
template <typename T>
__global__ __launch_bounds__(256) void reposition_kernel(const T* __restrict__ ks, const T* __restrict__ vs,
                                                         int64_t sls, T* __restrict__ kb, T* __restrict__ vb,
                                                         int64_t bls, ChunkBatch cb, int kvd, int hd,
                                                         const float* __restrict__ cos_t,
                                                         const float* __restrict__ sin_t, int layer_begin) {
  const int blk = blockIdx.x;
  int c = 0;
  while (c + 1 < cb.n && cb.blk0[c + 1] <= blk) ++c;
  const int r0 = (blk - cb.blk0[c]) * REPOS_ROWS_PER_BLOCK;
  const int nrows = min(REPOS_ROWS_PER_BLOCK, cb.len[c] - r0);
  const int64_t l = layer_begin + blockIdx.y;
  const int64_t src_row = cb.row[c] + r0, dst_row = cb.dst[c] + r0;
  const T* ksrc = ks + l * sls + src_row * kvd;
  const T* vsrc = vs + l * sls + src_row * kvd;
  T* kdst = kb + l * bls + dst_row * kvd;
  T* vdst = vb + l * bls + dst_row * kvd;
  const int delta = cb.delta[c];
  const int half = hd / 2;
  const float sgn = delta < 0 ? -1.f : 1.f;
  const float* cs = cos_t + (int64_t)abs(delta) * half;
  const float* sn = sin_t + (int64_t)abs(delta) * half;

  const int upr = kvd / 16;  // units of 8 pairs per row
  for (int u = threadIdx.x; u < nrows * upr; u += blockDim.x) {
    const int row = u / upr, w = u % upr;
    const int head = w / (half / 8), j0 = (w % (half / 8)) * 8;
    const int64_t off = (int64_t)row * kvd + head * hd + j0;
    float x1[8], x2[8], c8[8], s8[8];
    load8(ksrc + off, x1);
    load8(ksrc + off + half, x2);
    load8(cs + j0, c8);
    load8(sn + j0, s8);
    float y1[8], y2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float s = sgn * s8[e];
      y1[e] = x1[e] * c8[e] - x2[e] * s;
      y2[e] = x1[e] * s + x2[e] * c8[e];
    }
    store8(kdst + off, y1);
    store8(kdst + off + half, y2);
  }
  const int vpr = kvd / 8;
  for (int u = threadIdx.x; u < nrows * vpr; u += blockDim.x) {
    const int64_t off = (int64_t)(u / vpr) * kvd + (u % vpr) * 8;
    copy8(vdst + off, vsrc + off);
  }
}

hipError_t launch_reposition(Dt dt, const void* ks, const void* vs, int64_t sls, void* kb, void* vb,
                             int64_t bls, const ChunkBatch& cb, int kvd, int hd, const float* cos_t,
                             const float* sin_t, int layer_begin, int n_layers, hipStream_t st) {
  const int nblk = cb.blk0[cb.n];
  if (nblk == 0 || n_layers == 0) return hipSuccess;
  dim3 grid(nblk, n_layers);
  if (dt == BF16)
    hipLaunchKernelGGL(reposition_kernel<bf16>, grid, dim3(256), 0, st, (const bf16*)ks, (const bf16*)vs,
                       sls, (bf16*)kb, (bf16*)vb, bls, cb, kvd, hd, cos_t, sin_t, layer_begin);
  else
    hipLaunchKernelGGL(reposition_kernel<float>, grid, dim3(256), 0, st, (const float*)ks, (const float*)vs,
                       sls, (float*)kb, (float*)vb, bls, cb, kvd, hd, cos_t, sin_t, layer_begin);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- embedding
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const int* __restrict__ tok, const T* __restrict__ emb,
                                                    int vocab, int d, float* __restrict__ h) {
  const int r = blockIdx.x;
  const int t = tok[r];
  const bool ok = t >= 0 && t < vocab;
  const T* src = emb + (int64_t)(ok ? t : 0) * d;
  float* dst = h + (int64_t)r * d;
  for (int c = threadIdx.x * 8; c < d; c += blockDim.x * 8) {
    float v[8];
    load8(src + c, v);
    if (!ok) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = __builtin_nanf("");
    }
    store8(dst + c, v);
  }
}

hipError_t launch_embed(Dt dt, const int* tok, int L, const void* emb, int vocab, int d, float* h,
                        hipStream_t st) {
  if (L == 0) return hipSuccess;
  if (dt == BF16)
    hipLaunchKernelGGL(embed_kernel<bf16>, dim3(L), dim3(256), 0, st, tok, (const bf16*)emb, vocab, d, h);
  else
    hipLaunchKernelGGL(embed_kernel<float>, dim3(L), dim3(256), 0, st, tok, (const float*)emb, vocab, d, h);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- RMSNorm rows
template <typename To>
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(const float* __restrict__ x, const int* __restrict__ rows,
                                                           int L, int d, const float* __restrict__ g, float eps,
                                                           To* __restrict__ out, int64_t ldo) {
  __shared__ float red[4];
  const int j = blockIdx.x;
  const int r = rows ? clampi(rows[j], 0, L - 1) : j;
  const float* xr = x + (int64_t)r * d;
  float ss = 0.f;
  for (int c = threadIdx.x * 8; c < d; c += blockDim.x * 8) {
    float v[8];
    load8(xr + c, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
  }
  ss = block_sum(ss, red);
  const float inv = 1.0f / sqrtf(ss / (float)d + eps);
  To* o = out + (int64_t)j * ldo;
  for (int c = threadIdx.x * 8; c < d; c += blockDim.x * 8) {
    float v[8], gg[8];
    load8(xr + c, v);
    load8(g + c, gg);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = v[e] * inv * gg[e];
    store8(o + c, v);
  }
}

hipError_t launch_rmsnorm_rows(Dt out_dt, const float* x, const int* rows, int n, int L, int d,
                               const float* g, float eps, void* out, int64_t ldo, hipStream_t st) {
  if (n == 0) return hipSuccess;
  if (out_dt == BF16)
    hipLaunchKernelGGL(rmsnorm_rows_kernel<bf16>, dim3(n), dim3(256), 0, st, x, rows, L, d, g, eps, (bf16*)out, ldo);
  else
    hipLaunchKernelGGL(rmsnorm_rows_kernel<float>, dim3(n), dim3(256), 0, st, x, rows, L, d, g, eps, (float*)out, ldo);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- QKV post
// Store mode: block (row j, head group y), wave w handles head 4y + w, so every head's loads are
// in flight at once. Deviation mode: one block per row, wave w handles heads w, w+4, ... (the
// block sums the row's deviation). Lane j < hd/2 owns the RoPE pair (j, j + hd/2) of its head. qk-norm (per-head RMS over hd) happens before RoPE, as in the
// decoder definition. In deviation mode (p.dev set) the rows hold K only and the rotated keys
// are compared with the stitched keys instead of being stored (Request Order Matters Eq. 1).
template <typename T>
__global__ __launch_bounds__(256) void qkv_post_kernel(QkvPost p) {
  __shared__ float red[4];
  const int j = blockIdx.x;
  const int w = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int hd = p.hd, half = hd / 2;
  const bool devmode = p.dev != nullptr;
  const int pos = devmode ? j : clampi(p.rows[j], 0, p.L - 1);
  const float* src = p.qkv + (int64_t)j * p.ld;
  const int splits = p.splits > 1 ? p.splits : 1;
  const int64_t sst = p.split_stride;
  auto at = [&](int c) {  // projection value: the sum of the split-K partials
    float v = src[c];
    for (int s2 = 1; s2 < splits; ++s2) v += src[s2 * sst + c];
    return v;
  };
  const int64_t rp = (int64_t)pos + p.rope_off;  // RoPE position (the stored row plus an offset)
  const float c = lane < half ? p.cos_t[rp * half + lane] : 0.f;
  const float s = lane < half ? p.sin_t[rp * half + lane] : 0.f;
  const int nq = devmode ? 0 : p.hq;
  const int nkv = p.hkv;
  const int nh = nq + nkv + (devmode ? 0 : nkv);
  const int koff = nq * hd, voff = koff + nkv * hd;
  const int qd = p.hq * hd, kvd = nkv * hd;
  float dacc = 0.f;
  const int h0 = devmode ? w : blockIdx.y * (blockDim.x / WAVE) + w;
  const int hstep = devmode ? blockDim.x / WAVE : nh;  // store mode: one head per wave
  for (int h = h0; h < nh; h += hstep) {
    if (h < nq + nkv) {
      const bool isq = h < nq;
      const int hh = isq ? h : h - nq;
      const int xo = isq ? hh * hd : koff + hh * hd;
      float x1 = lane < half ? at(xo + lane) : 0.f;
      float x2 = lane < half ? at(xo + lane + half) : 0.f;
      if (p.qk_norm) {
        const float ss = wave_sum(x1 * x1 + x2 * x2);
        const float inv = 1.0f / sqrtf(ss / (float)hd + p.eps);
        const float* gn = isq ? p.qn : p.kn;
        if (lane < half) {
          x1 = x1 * inv * gn[lane];
          x2 = x2 * inv * gn[lane + half];
        }
      }
      const float y1 = x1 * c - x2 * s;
      const float y2 = x1 * s + x2 * c;
      if (lane < half) {
        if (isq) {
          T* q = (T*)p.q_out + (int64_t)j * qd + hh * hd;
          q[lane] = from_f<T>(y1);
          q[lane + half] = from_f<T>(y2);
        } else if (devmode) {
          const T* r = (const T*)p.k_ref + (int64_t)j * kvd + hh * hd;
          const float d1 = y1 - to_f(r[lane]), d2 = y2 - to_f(r[lane + half]);
          dacc += d1 * d1 + d2 * d2;
        } else {
          T* kc = (T*)p.k_cache + (int64_t)pos * kvd + hh * hd;
          kc[lane] = from_f<T>(y1);
          kc[lane + half] = from_f<T>(y2);
        }
      }
    } else {
      const int hh = h - nq - nkv;
      T* vc = (T*)p.v_cache + (int64_t)pos * kvd + hh * hd;
      for (int e = lane; e < hd; e += WAVE) vc[e] = from_f<T>(at(voff + hh * hd + e));
    }
  }
  if (devmode) {
    dacc = block_sum(dacc, red);
    if (threadIdx.x == 0) p.dev[j] = dacc;
  }
}

// Store mode with 16-byte accesses: thread e of a head handles dims [4e, 4e + 4) of both halves
// (the rotation pairs dim i with i + hd/2), so a head is hd/8 threads and a 256-thread block covers
// 2048/hd heads of one row; qk-norm sums over the head's threads with xor shuffles.
template <typename T, int HD>
__global__ __launch_bounds__(256) void qkv_post_vec_kernel(QkvPost p) {
  constexpr int HALF = HD / 2, TPH = HALF / 4, HPB = 256 / TPH;
  const int j = blockIdx.x;
  const int h = blockIdx.y * HPB + threadIdx.x / TPH, e = (threadIdx.x % TPH) * 4;
  const int nq = p.hq, nkv = p.hkv, nh = nq + 2 * nkv;
  if (h >= nh) return;  // whole heads: the shuffle groups below stay complete
  const int pos = clampi(p.rows[j], 0, p.L - 1);
  const float* src = p.qkv + (int64_t)j * p.ld;
  const int splits = p.splits > 1 ? p.splits : 1;
  auto at4 = [&](int c) {  // 4 projection values: the sum of the split-K partials
    float4 v = *reinterpret_cast<const float4*>(src + c);
    for (int s2 = 1; s2 < splits; ++s2) {
      const float4 w = *reinterpret_cast<const float4*>(src + s2 * p.split_stride + c);
      v.x += w.x, v.y += w.y, v.z += w.z, v.w += w.w;
    }
    return v;
  };
  const int kvd = nkv * HD;
  auto store4 = [](T* dst, float a, float b, float c, float d) {
    dst[0] = from_f<T>(a), dst[1] = from_f<T>(b), dst[2] = from_f<T>(c), dst[3] = from_f<T>(d);
  };
  if (h >= nq + nkv) {  // V: copied
    const int hh = h - nq - nkv, xo = (nq + nkv) * HD + hh * HD;
    const float4 a = at4(xo + e), b = at4(xo + e + HALF);
    T* vc = (T*)p.v_cache + (int64_t)pos * kvd + hh * HD;
    store4(vc + e, a.x, a.y, a.z, a.w);
    store4(vc + e + HALF, b.x, b.y, b.z, b.w);
    return;
  }
  const bool isq = h < nq;
  const int hh = isq ? h : h - nq, xo = isq ? hh * HD : nq * HD + hh * HD;
  float4 x1 = at4(xo + e), x2 = at4(xo + e + HALF);
  if (p.qk_norm) {
    float ss = x1.x * x1.x + x1.y * x1.y + x1.z * x1.z + x1.w * x1.w + x2.x * x2.x + x2.y * x2.y + x2.z * x2.z +
               x2.w * x2.w;
#pragma unroll
    for (int off = 1; off < TPH; off <<= 1) ss += __shfl_xor(ss, off, WAVE);
    const float inv = 1.0f / sqrtf(ss / (float)HD + p.eps);
    const float* gn = isq ? p.qn : p.kn;
    x1.x = x1.x * inv * gn[e], x1.y = x1.y * inv * gn[e + 1], x1.z = x1.z * inv * gn[e + 2];
    x1.w = x1.w * inv * gn[e + 3];
    x2.x = x2.x * inv * gn[e + HALF], x2.y = x2.y * inv * gn[e + HALF + 1], x2.z = x2.z * inv * gn[e + HALF + 2];
    x2.w = x2.w * inv * gn[e + HALF + 3];
  }
  const int64_t rp = (int64_t)pos + p.rope_off;  // RoPE position (the stored row plus an offset)
  const float4 c = *reinterpret_cast<const float4*>(p.cos_t + rp * HALF + e);
  const float4 sn = *reinterpret_cast<const float4*>(p.sin_t + rp * HALF + e);
  T* dst = isq ? (T*)p.q_out + (int64_t)j * (nq * HD) + hh * HD : (T*)p.k_cache + (int64_t)pos * kvd + hh * HD;
  const float y1[4] = {x1.x * c.x - x2.x * sn.x, x1.y * c.y - x2.y * sn.y, x1.z * c.z - x2.z * sn.z,
                       x1.w * c.w - x2.w * sn.w};
  const float y2[4] = {x1.x * sn.x + x2.x * c.x, x1.y * sn.y + x2.y * c.y, x1.z * sn.z + x2.z * c.z,
                       x1.w * sn.w + x2.w * c.w};
  if (!isq && p.dev_heads && j < p.n_dev) {  // uniform over the head's TPH threads
    // deviation of the fresh key from the stitched key it replaces (Request Order Matters Eq. 1),
    // per head; the row sum over heads is taken by launch_dev_rows
    float dd = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = y1[i] - to_f(dst[e + i]), b = y2[i] - to_f(dst[e + HALF + i]);
      dd += a * a + b * b;
    }
#pragma unroll
    for (int off = 1; off < TPH; off <<= 1) dd += __shfl_xor(dd, off, WAVE);
    if (e == 0) p.dev_heads[(int64_t)j * nkv + hh] = dd;
  }
  store4(dst + e, y1[0], y1[1], y1[2], y1[3]);
  store4(dst + e + HALF, y2[0], y2[1], y2[2], y2[3]);
}

hipError_t launch_qkv_post(Dt dt, const QkvPost& p, hipStream_t st) {
  if (p.n == 0) return hipSuccess;
  if (!p.dev && (p.hd == 64 || p.hd == 128) && p.ld % 4 == 0 && p.split_stride % 4 == 0) {
    const int nh = p.hq + 2 * p.hkv, hpb = 256 / (p.hd / 8);
    const dim3 grid(p.n, (nh + hpb - 1) / hpb);
    if (dt == BF16) {
      if (p.hd == 128) hipLaunchKernelGGL((qkv_post_vec_kernel<bf16, 128>), grid, dim3(256), 0, st, p);
      else hipLaunchKernelGGL((qkv_post_vec_kernel<bf16, 64>), grid, dim3(256), 0, st, p);
    } else {
      if (p.hd == 128) hipLaunchKernelGGL((qkv_post_vec_kernel<float, 128>), grid, dim3(256), 0, st, p);
      else hipLaunchKernelGGL((qkv_post_vec_kernel<float, 64>), grid, dim3(256), 0, st, p);
    }
    return hipGetLastError();
  }
  if (p.dev_heads) return hipErrorInvalidValue;  // the per-head deviation lives in the vector kernel only
  const int nh = p.dev ? 1 : p.hq + 2 * p.hkv;
  const dim3 grid(p.n, p.dev ? 1 : (nh + 3) / 4);
  if (dt == BF16)
    hipLaunchKernelGGL(qkv_post_kernel<bf16>, grid, dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL(qkv_post_kernel<float>, grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

// dst[j] = src[idx ? clamp(idx[j]) : j] for j < n, rows of row16 16-byte words: a 256-thread block
// copies 4 rows, one wave per row, with 16-byte accesses.
__global__ __launch_bounds__(256) void gather_rows_kernel(const char* __restrict__ src, int64_t src_ld,
                                                          int src_rows, const int* __restrict__ idx, int n,
                                                          int row16, char* __restrict__ dst, int64_t dst_ld) {
  const int j = blockIdx.x * 4 + threadIdx.x / 64;
  if (j >= n) return;
  const int r = idx ? clampi(idx[j], 0, src_rows - 1) : j;
  const uint4* s = reinterpret_cast<const uint4*>(src + (int64_t)r * src_ld);
  uint4* d = reinterpret_cast<uint4*>(dst + (int64_t)j * dst_ld);
  for (int e = threadIdx.x % 64; e < row16; e += 64) d[e] = s[e];
}

hipError_t launch_gather_rows(Dt dt, const void* src, int64_t src_ld, int src_rows, const int* idx, int n,
                              int row_elems, void* dst, int64_t dst_ld, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int es = dt == BF16 ? 2 : 4;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((n + 3) / 4), dim3(256), 0, st, (const char*)src, src_ld * es,
                     src_rows, idx, n, row_elems * es / 16, (char*)dst, dst_ld * es);
  return hipGetLastError();
}

// norms[r] = sum over layers [lb, le) and the kvd entries of K[l][r]^2 (fp32, layer by layer, each
// row's entries summed across one wave): one wave per store row.
template <typename T>
__global__ __launch_bounds__(256) void key_norms_kernel(const T* __restrict__ k, int64_t sls, int rows, int kvd,
                                                        int lb, int le, float* __restrict__ norms) {
  const int r = blockIdx.x * 4 + threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  if (r >= rows) return;
  float acc = 0.f;
  for (int l = lb; l < le; ++l) {
    const T* row = k + (int64_t)l * sls + (int64_t)r * kvd;
    float part = 0.f;
    for (int c = lane; c < kvd; c += WAVE) {
      const float x = to_f(row[c]);
      part += x * x;
    }
    acc += wave_sum(part);
  }
  if (lane == 0) norms[r] = acc;
}

hipError_t launch_key_norms(Dt dt, const void* k, int64_t sls, int rows, int kvd, int lb, int le, float* norms,
                            hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (dt == BF16)
    hipLaunchKernelGGL(key_norms_kernel<bf16>, dim3((rows + 3) / 4), dim3(256), 0, st, (const bf16*)k, sls, rows,
                       kvd, lb, le, norms);
  else
    hipLaunchKernelGGL(key_norms_kernel<float>, dim3((rows + 3) / 4), dim3(256), 0, st, (const float*)k, sls, rows,
                       kvd, lb, le, norms);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void dev_rows_kernel(const float* __restrict__ dh, int n, int hkv,
                                                        float* __restrict__ dev) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= n) return;
  float s = 0.f;
  for (int h = 0; h < hkv; ++h) s += dh[(int64_t)j * hkv + h];
  dev[j] = s;
}

hipError_t launch_dev_rows(const float* dev_heads, int n, int hkv, float* dev, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(dev_rows_kernel, dim3((n + 255) / 256), dim3(256), 0, st, dev_heads, n, hkv, dev);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void sel_map_kernel(int* __restrict__ sel, const int* __restrict__ prev, int k,
                                                       int U, int n_ctx) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j < k) sel[j] = prev[sel[j]];
  else if (j < k + U) sel[j] = n_ctx + (j - k);
}

hipError_t launch_sel_map(int* sel, const int* prev, int k, int U, int n_ctx, hipStream_t st) {
  if (k + U <= 0) return hipSuccess;
  hipLaunchKernelGGL(sel_map_kernel, dim3((k + U + 255) / 256), dim3(256), 0, st, sel, prev, k, U, n_ctx);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- small helpers
__global__ void iota_kernel(int* out, int n, int start) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = start + i;
}
hipError_t launch_iota(int* out, int n, int start, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(iota_kernel, dim3((n + 255) / 256), dim3(256), 0, st, out, n, start);
  return hipGetLastError();
}
template <typename T>
__global__ void copy_kernel(T* dst, const T* src, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}
hipError_t launch_copy_i32(int* dst, const int* src, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(copy_kernel<int>, dim3((n + 255) / 256), dim3(256), 0, st, dst, src, n);
  return hipGetLastError();
}
hipError_t launch_copy_f32(float* dst, const float* src, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(copy_kernel<float>, dim3((n + 255) / 256), dim3(256), 0, st, dst, src, n);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- split-K reduce
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int splits, int M, int N,
                                                            const float* __restrict__ resid, const int* __restrict__ rrows,
                                                            float* __restrict__ out, const int* __restrict__ orows, int L) {
  const int m = blockIdx.x;
  const int64_t rr = rrows ? clampi(rrows[m], 0, L - 1) : m;
  const int64_t orr = orows ? clampi(orows[m], 0, L - 1) : m;
  for (int c = threadIdx.x * 4; c < N; c += blockDim.x * 4) {
    float4 a = resid ? *reinterpret_cast<const float4*>(resid + rr * N + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < splits; ++s) {
      const float4 b = *reinterpret_cast<const float4*>(part + ((int64_t)s * M + m) * N + c);
      a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
    }
    *reinterpret_cast<float4*>(out + orr * N + c) = a;
  }
}
hipError_t launch_splitk_reduce(const float* part, int splits, int M, int N, const float* resid,
                                const int* resid_rows, float* out, const int* out_rows, int L,
                                hipStream_t st) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(M), dim3(256), 0, st, part, splits, M, N, resid, resid_rows,
                     out, out_rows, L);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- reduce + residual + norm
// out[orow(m)] = resid[rrow(m)] + sum_s part[s][m]; x[m] = RMSNorm(out row) * g. Closes a split-K
// projection and prepares the next bf16 GEMM input in one pass: after the O projection (residual
// gathered from the selected rows, output h' dense, the MLP norm) and after the down projection
// (residual h' dense, output scattered back to the selected rows, the next layer's attention norm).
template <typename T>
__global__ __launch_bounds__(256) void reduce_resid_norm_kernel(const float* __restrict__ part, int splits, int M, int d,
                                                                const float* __restrict__ resid,
                                                                const int* __restrict__ rrows,
                                                                float* __restrict__ out,
                                                                const int* __restrict__ orows, int L,
                                                                const float* __restrict__ g, float eps,
                                                                T* __restrict__ x) {
  constexpr int KEEP = 4;  // chunks of 8 per thread kept in registers: rows up to 256 * 8 * 4 = 8192
  __shared__ float red[4];
  const int m = blockIdx.x;
  const int64_t rr = rrows ? clampi(rrows[m], 0, L - 1) : m;
  const int64_t orr = orows ? clampi(orows[m], 0, L - 1) : m;
  float keep[KEEP][8];
  float ss = 0.f;
  int it = 0;
  for (int c = threadIdx.x * 8; c < d; c += blockDim.x * 8, ++it) {
    float v[8], t[8];
    load8(resid + rr * d + c, v);
    for (int s = 0; s < splits; ++s) {
      load8(part + ((int64_t)s * M + m) * d + c, t);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] += t[e];
    }
    store8(out + orr * d + c, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
    if (it < KEEP)
#pragma unroll
      for (int e = 0; e < 8; ++e) keep[it < KEEP ? it : 0][e] = v[e];
  }
  ss = block_sum(ss, red);
  const float inv = 1.0f / sqrtf(ss / (float)d + eps);
  it = 0;
  for (int c = threadIdx.x * 8; c < d; c += blockDim.x * 8, ++it) {
    float v[8], gg[8];
    if (it < KEEP) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = keep[it < KEEP ? it : 0][e];
    } else {
      load8(out + orr * d + c, v);
    }
    load8(g + c, gg);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = v[e] * inv * gg[e];
    store8(x + (int64_t)m * d + c, v);
  }
}
hipError_t launch_reduce_resid_norm(Dt dt, const float* part, int splits, int M, int d, const float* resid,
                                    const int* resid_rows, float* out, const int* out_rows, int L, const float* g,
                                    float eps, void* x, hipStream_t st) {
  if (M == 0) return hipSuccess;
  if (dt == BF16)
    hipLaunchKernelGGL(reduce_resid_norm_kernel<bf16>, dim3(M), dim3(256), 0, st, part, splits, M, d, resid,
                       resid_rows, out, out_rows, L, g, eps, (bf16*)x);
  else
    hipLaunchKernelGGL(reduce_resid_norm_kernel<float>, dim3(M), dim3(256), 0, st, part, splits, M, d, resid,
                       resid_rows, out, out_rows, L, g, eps, (float*)x);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- SwiGLU (fp32 path)
template <typename T>
__global__ void swiglu_kernel(const float* __restrict__ gu, int M, int F, T* __restrict__ act) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)M * F) return;
  const int64_t m = i / F, c = i % F;
  const float g = gu[m * 2 * F + c], u = gu[m * 2 * F + F + c];
  act[i] = from_f<T>(g / (1.0f + expf(-g)) * u);
}
hipError_t launch_swiglu(Dt dt, const float* gu, int M, int F, void* act, hipStream_t st) {
  const int64_t n = (int64_t)M * F;
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (dt == BF16)
    hipLaunchKernelGGL(swiglu_kernel<bf16>, grid, dim3(256), 0, st, gu, M, F, (bf16*)act);
  else
    hipLaunchKernelGGL(swiglu_kernel<float>, grid, dim3(256), 0, st, gu, M, F, (float*)act);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- deviation
// Request Order Matters §2.2 Eq. 1 on two key arrays: one block per token, fp32 accumulation.
template <typename TA, typename TB>
__global__ __launch_bounds__(256) void deviation_kernel(const TA* __restrict__ a, int64_t lda, const TB* __restrict__ b,
                                                        int64_t ldb, float* __restrict__ dev, int kvd) {
  __shared__ float red[4];
  const int i = blockIdx.x;
  const TA* ar = a + (int64_t)i * lda;
  const TB* br = b + (int64_t)i * ldb;
  float acc = 0.f;
  for (int c = threadIdx.x * 8; c < kvd; c += blockDim.x * 8) {
    float x[8], y[8];
    load8(ar + c, x);
    load8(br + c, y);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float t = x[e] - y[e];
      acc += t * t;
    }
  }
  acc = block_sum(acc, red);
  if (threadIdx.x == 0) dev[i] = acc;
}
hipError_t launch_deviation(Dt dn, const void* a, int64_t lda, Dt dr, const void* b, int64_t ldb,
                            float* dev, int n, int kvd, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const dim3 g(n), blk(256);
  if (dn == BF16 && dr == BF16)
    hipLaunchKernelGGL((deviation_kernel<bf16, bf16>), g, blk, 0, st, (const bf16*)a, lda, (const bf16*)b, ldb, dev, kvd);
  else if (dn == F32 && dr == BF16)
    hipLaunchKernelGGL((deviation_kernel<float, bf16>), g, blk, 0, st, (const float*)a, lda, (const bf16*)b, ldb, dev, kvd);
  else if (dn == BF16 && dr == F32)
    hipLaunchKernelGGL((deviation_kernel<bf16, float>), g, blk, 0, st, (const bf16*)a, lda, (const float*)b, ldb, dev, kvd);
  else
    hipLaunchKernelGGL((deviation_kernel<float, float>), g, blk, 0, st, (const float*)a, lda, (const float*)b, ldb, dev, kvd);
  return hipGetLastError();
}

}  // namespace cf
