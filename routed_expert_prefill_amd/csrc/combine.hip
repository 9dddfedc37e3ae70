// Route-weighted combine back to token order (the fused MoE combine of
// "perf(ds4): accelerate ROCm decode and long-context selection", lucebox8
// gfx1151 A/B).  One workgroup per token row slice; each thread owns 4
// consecutive fp32 columns and sums its token's active routes in ascending
// route order from +0.0 (the loads of all routes in flight together).  Masked routes are skipped by a branch, never
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

// K routes per token, known at compile time: the token's masks, rows and
// gates are read once (uniform, scalar loads), then the rows of every route
// that is read are loaded together, and only then summed in ascending j.  A
// loop over j that loaded, waited and added route by route kept one row load
// in flight per thread and made the combine latency-bound.  The rows of y
// (and of the shared output) are read once, with non-temporal loads that
// leave the caches to other data: MI355X, 8192 tokens, 0.165-0.177 ->
// 0.141-0.143 ms (Zipf and fp8 workloads), unchanged at 401 and 2048.
// (Non-temporal stores of y in the down GEMM instead slowed that kernel
// by 8-17%.)
template <int K>
__global__ __launch_bounds__(kCombThreads) void combine_kernel(const float *__restrict__ y,
                                                               const int32_t *__restrict__ route_rows,
                                                               const float *__restrict__ topk_w,
                                                               const uint8_t *__restrict__ mask,
                                                               const int32_t *__restrict__ row_limit,
                                                               const float *__restrict__ shared,
                                                               int T, int d, int slices,
                                                               float *__restrict__ out,
                                                               uint16_t *__restrict__ out_bf16) {
  const int t = blockIdx.x / slices;
  const int c = ((blockIdx.x - t * slices) * kCombThreads + threadIdx.x) * 4;
  const int lim = row_limit != nullptr ? *row_limit : INT_MAX;
  const size_t r0 = (size_t)t * K;
  // lane j of every wave loads route j's mask, row and gate (one load of
  // each for the whole token); readlane hands them to the wave as uniform
  // values, so the row loads below depend on nothing in flight
  const int lane = lane_id();
  int m_l = 1, row_l = 0;
  float w_l = 0.0f;
  if (lane < K) {
    if (mask != nullptr) m_l = mask[r0 + lane];
    row_l = route_rows[r0 + lane];
    w_l = topk_w[r0 + lane];
  }
  bool on[K];
  int row[K];
  float w[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    row[j] = __builtin_amdgcn_readlane(row_l, j);
    w[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_l), j));
    on[j] = __builtin_amdgcn_readlane(m_l, j) != 0;
  }
  if (c >= d) return;
  f32x4 v[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    on[j] = on[j] && row[j] < lim;  // never read: masked, or past the rows the FFN wrote
    if (on[j]) v[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(y + (size_t)row[j] * d + c));
  }
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < K; ++j) {
    if (on[j]) {
      acc[0] = __builtin_fmaf(w[j], v[j][0], acc[0]);
      acc[1] = __builtin_fmaf(w[j], v[j][1], acc[1]);
      acc[2] = __builtin_fmaf(w[j], v[j][2], acc[2]);
      acc[3] = __builtin_fmaf(w[j], v[j][3], acc[3]);
    }
  }
  const size_t o = (size_t)t * d + c;
  if (shared != nullptr) {
    const f32x4 sh = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(shared + o));
    acc[0] += sh[0];
    acc[1] += sh[1];
    acc[2] += sh[2];
    acc[3] += sh[3];
  }
  if (out != nullptr) *reinterpret_cast<f32x4 *>(out + o) = acc;
  if (out_bf16 != nullptr) {
    uint2 b;
    b.x = (uint32_t)f32_to_bf16_bits(acc[0]) | ((uint32_t)f32_to_bf16_bits(acc[1]) << 16);
    b.y = (uint32_t)f32_to_bf16_bits(acc[2]) | ((uint32_t)f32_to_bf16_bits(acc[3]) << 16);
    *reinterpret_cast<uint2 *>(out_bf16 + o) = b;
  }
}

hipError_t launch_combine(const float *y, const int32_t *route_rows, const float *topk_w,
                          const uint8_t *mask, const int32_t *row_limit, const float *shared,
                          int T, int k, int d, float *out, uint16_t *out_bf16,
                          hipStream_t stream) {
  const int per_block = kCombThreads * 4;
  const int slices = (d + per_block - 1) / per_block;
  const dim3 grid((unsigned)T * slices), block(kCombThreads);
  switch (k) {
#define MOE_COMBINE_CASE(K)                                                                     \
  case K:                                                                                      \
    hipLaunchKernelGGL(combine_kernel<K>, grid, block, 0, stream, y, route_rows, topk_w, mask, \
                       row_limit, shared, T, d, slices, out, out_bf16);                        \
    break;
    MOE_COMBINE_CASE(1) MOE_COMBINE_CASE(2) MOE_COMBINE_CASE(3) MOE_COMBINE_CASE(4)
    MOE_COMBINE_CASE(5) MOE_COMBINE_CASE(6) MOE_COMBINE_CASE(7) MOE_COMBINE_CASE(8)
    MOE_COMBINE_CASE(9) MOE_COMBINE_CASE(10) MOE_COMBINE_CASE(11) MOE_COMBINE_CASE(12)
    MOE_COMBINE_CASE(13) MOE_COMBINE_CASE(14) MOE_COMBINE_CASE(15) MOE_COMBINE_CASE(16)
#undef MOE_COMBINE_CASE
    default:
      return hipErrorInvalidValue;  // the C ABI accepts 1 <= k <= 16 only
  }
  return hipGetLastError();
}

}  // namespace moe
