// Route-weighted combine back to token order (the fused MoE combine of
// "perf(ds4): accelerate ROCm decode and long-context selection", lucebox8
// gfx1151 A/B).  One workgroup per token row slice; each thread owns 4
// consecutive fp32 columns and sums its token's active routes in ascending
// route order from +0.0.  Masked routes are skipped by a branch, never
// multiplied by zero, so nothing they hold can reach the output.
#include "kernels.h"

namespace moe {

constexpr int kCombThreads = 256;

__global__ __launch_bounds__(kCombThreads) void combine_kernel(const float *__restrict__ y,
                                                               const int32_t *__restrict__ route_rows,
                                                               const float *__restrict__ topk_w,
                                                               const uint8_t *__restrict__ mask,
                                                               int T, int k, int d, int slices,
                                                               float *__restrict__ out) {
  const int t = blockIdx.x / slices;
  const int c = ((blockIdx.x - t * slices) * kCombThreads + threadIdx.x) * 4;
  if (c >= d) return;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int j = 0; j < k; ++j) {
    const int r = t * k + j;
    if (mask != nullptr && mask[r] == 0) continue;
    const float w = topk_w[r];
    const f32x4 v = *reinterpret_cast<const f32x4 *>(y + (size_t)route_rows[r] * d + c);
    acc[0] = __builtin_fmaf(w, v[0], acc[0]);
    acc[1] = __builtin_fmaf(w, v[1], acc[1]);
    acc[2] = __builtin_fmaf(w, v[2], acc[2]);
    acc[3] = __builtin_fmaf(w, v[3], acc[3]);
  }
  *reinterpret_cast<f32x4 *>(out + (size_t)t * d + c) = acc;
}

hipError_t launch_combine(const float *y, const int32_t *route_rows, const float *topk_w,
                          const uint8_t *mask, int T, int k, int d, float *out,
                          hipStream_t stream) {
  const int per_block = kCombThreads * 4;
  const int slices = (d + per_block - 1) / per_block;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)T * slices), dim3(kCombThreads), 0, stream, y,
                     route_rows, topk_w, mask, T, k, d, slices, out);
  return hipGetLastError();
}

}  // namespace moe
