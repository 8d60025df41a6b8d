// Measurement aids: the achievable rates of the device, the denominators the kernels' fractions
// can be read against besides the published peaks.
// * A matrix-core loop with no memory traffic: each 256-thread block issues iters x 4
//   independent v_mfma_f32_32x32x16_bf16 per wave; the sums are written so the work is kept.
// * A streaming copy (16-byte loads and stores, one contiguous range per block).
#include "common.h"
#include "kernels.h"

namespace cf {

__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* out) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (bf16)(threadIdx.x * 0.001f + i);
    b[i] = (bf16)(i * 0.5f);
  }
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x16{};
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) s += acc[j][0] + acc[j][15];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Streaming copy of n16 16-byte words: each block copies one contiguous 256 KB range, four
// 16-byte loads in flight per thread (the fastest of the layouts measured on the device).
constexpr int64_t COPY_PER_BLOCK = 16384;  // 16-byte words

__global__ __launch_bounds__(256) void copy_loop_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                        int64_t n16) {
  const int64_t b0 = (int64_t)blockIdx.x * COPY_PER_BLOCK;
  const int64_t b1 = b0 + COPY_PER_BLOCK < n16 ? b0 + COPY_PER_BLOCK : n16;
  for (int64_t i = b0 + threadIdx.x; i < b1; i += 4 * 256) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i + u * 256 < b1) v[u] = src[i + u * 256];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i + u * 256 < b1) dst[i + u * 256] = v[u];
  }
}

void launch_copy_loop(const void* src, void* dst, int64_t n16, hipStream_t st) {
  const int64_t blocks = (n16 + COPY_PER_BLOCK - 1) / COPY_PER_BLOCK;
  if (blocks > 0)
    hipLaunchKernelGGL(copy_loop_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (const u32x4*)src, (u32x4*)dst, n16);
}

double launch_mfma_loop(int blocks, int iters, float* out, hipStream_t st) {
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(256), 0, st, iters, out);
  return (double)blocks * 4 * iters * 4 * (2.0 * 32 * 32 * 16);
}

}  // namespace cf
