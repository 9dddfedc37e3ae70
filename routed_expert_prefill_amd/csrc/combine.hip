// Route-weighted combine back to token order (the fused MoE combine of
// "perf(ds4): accelerate ROCm decode and long-context selection", lucebox8
// gfx1151 A/B).  One workgroup per token row slice; each thread owns 4
// consecutive fp32 columns and sums its token's active routes in ascending
// route order from +0.0.  Masked routes are skipped by a branch, never
// multiplied by zero, so nothing they hold can reach the output.  With a row
// limit (the number of rows of y the grouped FFN wrote, offsets[E] of the
// route build) a route whose row lies at or past it is skipped the same way:
// the route build sends masked routes and active routes with ids outside
// [0, E) to those trailing rows, which the FFN never writes.
//
// Shared-output form ("perf(ds4): extend sparse prefill scheduling to 10K",
// Historical fused-combine discriminator): the row of the shared expert's
// output is added once to the routed sum, and a bf16 copy (round to nearest
// even) can be written beside or instead of the fp32 row.
#include <climits>

#include "kernels.h"

namespace moe {

constexpr int kCombThreads = 256;

__global__ __launch_bounds__(kCombThreads) void combine_kernel(const float *__restrict__ y,
                                                               const int32_t *__restrict__ route_rows,
                                                               const float *__restrict__ topk_w,
                                                               const uint8_t *__restrict__ mask,
                                                               const int32_t *__restrict__ row_limit,
                                                               const float *__restrict__ shared,
                                                               int T, int k, int d, int slices,
                                                               float *__restrict__ out,
                                                               uint16_t *__restrict__ out_bf16) {
  const int t = blockIdx.x / slices;
  const int c = ((blockIdx.x - t * slices) * kCombThreads + threadIdx.x) * 4;
  if (c >= d) return;
  const int lim = row_limit != nullptr ? *row_limit : INT_MAX;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int j = 0; j < k; ++j) {
    const int r = t * k + j;
    if (mask != nullptr && mask[r] == 0) continue;
    const int row = route_rows[r];
    if (row >= lim) continue;
    const float w = topk_w[r];
    const f32x4 v = *reinterpret_cast<const f32x4 *>(y + (size_t)row * d + c);
    acc[0] = __builtin_fmaf(w, v[0], acc[0]);
    acc[1] = __builtin_fmaf(w, v[1], acc[1]);
    acc[2] = __builtin_fmaf(w, v[2], acc[2]);
    acc[3] = __builtin_fmaf(w, v[3], acc[3]);
  }
  const size_t o = (size_t)t * d + c;
  if (shared != nullptr) {
    const f32x4 sh = *reinterpret_cast<const f32x4 *>(shared + o);
    acc[0] += sh[0];
    acc[1] += sh[1];
    acc[2] += sh[2];
    acc[3] += sh[3];
  }
  if (out != nullptr) *reinterpret_cast<f32x4 *>(out + o) = acc;
  if (out_bf16 != nullptr) {
    uint2 v;
    v.x = (uint32_t)f32_to_bf16_bits(acc[0]) | ((uint32_t)f32_to_bf16_bits(acc[1]) << 16);
    v.y = (uint32_t)f32_to_bf16_bits(acc[2]) | ((uint32_t)f32_to_bf16_bits(acc[3]) << 16);
    *reinterpret_cast<uint2 *>(out_bf16 + o) = v;
  }
}

hipError_t launch_combine(const float *y, const int32_t *route_rows, const float *topk_w,
                          const uint8_t *mask, const int32_t *row_limit, const float *shared,
                          int T, int k, int d,
                          float *out, uint16_t *out_bf16, hipStream_t stream) {
  const int per_block = kCombThreads * 4;
  const int slices = (d + per_block - 1) / per_block;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)T * slices), dim3(kCombThreads), 0, stream, y,
                     route_rows, topk_w, mask, row_limit, shared, T, k, d, slices, out,
                     out_bf16);
  return hipGetLastError();
}

}  // namespace moe
