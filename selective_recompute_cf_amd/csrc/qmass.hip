// Query-aware token scores (QCFuse §3.2.1, Eq. 10 and Eq. 20): at a scored layer, the attention
// weight that the query rows put on each context position, summed over query rows and heads.
// The weights are the rows' softmax over every cache row they see; the rows sit after the
// context, so every context key is visible to every row and the context columns need no mask.
// Each row's softmax maximum and sum (log2 units) come from the layer's own attention pass.
//   qmass_cols_kernel: one block per (64 context keys, kv head): lane = key, its key row held in
//     registers; the rows x heads of that kv head pass through LDS in chunks of 64, the four waves
//     sharing each chunk; partial masses per kv head.
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
    if (a.hd == 128) hipLaunchKernelGGL((qmass_cols_kernel<bf16, 128>), gc, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((qmass_cols_kernel<bf16, 64>), gc, dim3(256), 0, st, a);
  } else {
    if (a.hd == 128) hipLaunchKernelGGL((qmass_cols_kernel<float, 128>), gc, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((qmass_cols_kernel<float, 64>), gc, dim3(256), 0, st, a);
  }
  hipLaunchKernelGGL(qmass_sum_kernel, dim3((a.n_ctx + 255) / 256), dim3(256), 0, st, a.part, a.hkv, a.n_ctx, first,
                     a.score);
  return hipGetLastError();
}

}  // namespace cf
