// Query-aware token scores (QCFuse §3.2.1, Eq. 10 and Eq. 20): at a scored layer, the attention
// weight that the query rows put on each context position, summed over query rows and heads.
// The weights are the rows' softmax over every cache row they see; the rows sit after the
// context, so every context key is visible to every row and the context columns need no mask.
// Each row's softmax maximum and sum (log2 units) come from the layer's own attention pass.
//   qmass_cols_kernel: one block per (64 context keys, kv head): lane = key, its key row held in
//     registers; the rows x heads of that kv head pass through LDS in chunks of 64, the four waves
//     sharing each chunk; partial masses per kv head.
//   qmass_cols_mfma_kernel: the same for bf16 models on the matrix cores.
//   qmass_sum_kernel: score[t] (+)= sum over kv heads in head order (fixed order: deterministic).
#include "common.h"
#include "kernels.h"

namespace cf {

constexpr int QM_CHUNK = 64;  // rows x heads staged in LDS at a time

template <typename T, int HD>
__global__ __launch_bounds__(256) void qmass_cols_kernel(QMassArgs a) {
  __shared__ float qs[QM_CHUNK][HD];
  __shared__ float red[4][WAVE];
  const int g = blockIdx.y, G = a.hq / a.hkv, R = a.n * G, kvd = a.hkv * HD;
  const int w = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int t = blockIdx.x * WAVE + lane;
  const float sl2 = 1.4426950408889634f / sqrtf((float)HD);
  float kr[HD];
  const T* kp = (const T*)a.k + (int64_t)min(t, a.n_ctx - 1) * kvd + g * HD;
#pragma unroll
  for (int d = 0; d < HD; ++d) kr[d] = to_f(kp[d]);
  float acc = 0.f;
  for (int r0 = 0; r0 < R; r0 += QM_CHUNK) {
    const int rc = min(QM_CHUNK, R - r0);
    __syncthreads();  // the previous chunk is no longer read
    for (int i = threadIdx.x; i < rc * HD; i += 256) {
      const int r = r0 + i / HD, d = i % HD, j = r / G, h = g * G + r % G;
      qs[i / HD][d] = to_f(((const T*)a.q)[(int64_t)j * a.ldq + h * HD + d]);
    }
    __syncthreads();
    for (int rr = w; rr < rc; rr += 4) {
      const int r = r0 + rr, j = r / G, h = g * G + r % G;
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < HD; ++d) s = fmaf(qs[rr][d], kr[d], s);
      const float m = a.ml[((int64_t)j * a.hq + h) * 2], l = a.ml[((int64_t)j * a.hq + h) * 2 + 1];
      acc += l > 0.f ? __builtin_amdgcn_exp2f(s * sl2 - m) / l : 0.f;
    }
  }
  red[w][lane] = acc;
  __syncthreads();
  if (w == 0 && t < a.n_ctx) a.part[(int64_t)g * a.n_ctx + t] = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
}

// bf16 models: the same sums on the matrix cores. Each wave keeps the 64 keys' fragments in
// registers (16 keys x 32 dims per v_mfma_f32_16x16x32_bf16 operand) and takes 16 rows x heads at
// a time: S^T = K Q^T gives lane l the scores of keys 16 kt + 4 (l / 16) + i for row-head l % 16;
// the weights are summed over the 16 row-heads with xor shuffles inside each 16-lane group.
template <int HD>
__global__ __launch_bounds__(256) void qmass_cols_mfma_kernel(QMassArgs a) {
  __shared__ float red[4][WAVE];
  const int g = blockIdx.y, G = a.hq / a.hkv, R = a.n * G, kvd = a.hkv * HD;
  const int w = threadIdx.x / WAVE, lane = threadIdx.x % WAVE, lr = lane % 16, lg = lane / 16;
  const int t0 = blockIdx.x * WAVE;
  const float sl2 = 1.4426950408889634f / sqrtf((float)HD);
  bf16x8 kf[4][HD / 32];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const int t = min(t0 + kt * 16 + lr, a.n_ctx - 1);
    const bf16* kp = (const bf16*)a.k + (int64_t)t * kvd + g * HD + 8 * lg;
#pragma unroll
    for (int kk = 0; kk < HD / 32; ++kk) kf[kt][kk] = *reinterpret_cast<const bf16x8*>(kp + kk * 32);
  }
  float col[4][4] = {};  // column sums: keys 16 kt + 4 lg + i
  for (int r0 = w * 16; r0 < R; r0 += 64) {
    const int r = r0 + lr;
    const bool live = r < R;
    const int rc = live ? r : R - 1, j = rc / G, h = g * G + rc % G;
    const bf16* qp = (const bf16*)a.q + (int64_t)j * a.ldq + h * HD + 8 * lg;
    bf16x8 qf[HD / 32];
#pragma unroll
    for (int kk = 0; kk < HD / 32; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(qp + kk * 32);
    const float m = a.ml[((int64_t)j * a.hq + h) * 2], l = a.ml[((int64_t)j * a.hq + h) * 2 + 1];
    const float inv = live && l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < HD / 32; ++kk) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kt][kk], qf[kk], sc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float p = __builtin_amdgcn_exp2f(sc[i] * sl2 - m) * inv;
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) p += __shfl_xor(p, off, WAVE);
        col[kt][i] += p;
      }
    }
  }
  // lanes of a 16-lane group hold the same sums; lane 16 lg + 4 kt + i publishes key 16 kt + 4 lg + i
  float mine = 0.f;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (lr == kt * 4 + i) mine = col[kt][i];
  red[w][(lr / 4) * 16 + 4 * lg + (lr % 4)] = mine;
  __syncthreads();
  const int t = t0 + lane;
  if (w == 0 && t < a.n_ctx)
    a.part[(int64_t)g * a.n_ctx + t] = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
}

__global__ __launch_bounds__(256) void qmass_sum_kernel(const float* __restrict__ part, int hkv, int n_ctx, int first,
                                                         float* __restrict__ score) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= n_ctx) return;
  float s = first ? 0.f : score[t];
  for (int g = 0; g < hkv; ++g) s += part[(int64_t)g * n_ctx + t];
  score[t] = s;
}

hipError_t launch_query_mass(Dt dt, const QMassArgs& a, int first, hipStream_t st) {
  if (a.n <= 0 || a.n_ctx <= 0) return hipSuccess;
  if (a.hd != 64 && a.hd != 128) return hipErrorInvalidValue;
  const dim3 gc((a.n_ctx + WAVE - 1) / WAVE, a.hkv);
  if (dt == BF16) {
    if (a.hd == 128) hipLaunchKernelGGL(qmass_cols_mfma_kernel<128>, gc, dim3(256), 0, st, a);
    else hipLaunchKernelGGL(qmass_cols_mfma_kernel<64>, gc, dim3(256), 0, st, a);
  } else {
    if (a.hd == 128) hipLaunchKernelGGL((qmass_cols_kernel<float, 128>), gc, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((qmass_cols_kernel<float, 64>), gc, dim3(256), 0, st, a);
  }
  hipLaunchKernelGGL(qmass_sum_kernel, dim3((a.n_ctx + 255) / 256), dim3(256), 0, st, a.part, a.hkv, a.n_ctx, first,
                     a.score);
  return hipGetLastError();
}

}  // namespace cf
