// Top-k expert selection and renormalised gates from router logits.
//
// The routing step ahead of the route build: the pages keep the model's
// native top-6 routing and its selected-row order ("perf(ds4): extend sparse
// prefill scheduling to 10K", Summary); the arithmetic is the workloads'
// router: z = logits (+ bias, one fp32 addition), the k largest z in
// descending order with equal z going to the lower expert index, and gates
// equal to the softmax over the selected experts, exp(z_j - z_max) / sum,
// evaluated in fp64 (summed in ascending j) and rounded once to fp32.
//
// One wave per token: lane l holds experts l, l + 64, l + 128, l + 192; each
// of the k rounds picks the best remaining candidate of every lane and
// reduces across the wave with xor shuffles.
#include <math.h>

#include "kernels.h"

namespace moe {

constexpr int kTkThreads = 256;
constexpr int kTkWaves = kTkThreads / kWave;
constexpr int kTkPerLane = 4;  // 64 lanes x 4 >= 256 experts
constexpr int kTkNone = 0x7fffffff;

// (va, ia) ranks before (vb, ib): larger value, or the same value and a lower index
__device__ __forceinline__ bool tk_before(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

__global__ __launch_bounds__(kTkThreads) void route_topk_kernel(const float *__restrict__ logits,
                                                                const float *__restrict__ bias,
                                                                int T, int E, int k,
                                                                int32_t *__restrict__ ids,
                                                                float *__restrict__ gates) {
  const int lane = lane_id();
  const int nwaves = gridDim.x * kTkWaves;
  for (int t = blockIdx.x * kTkWaves + threadIdx.x / kWave; t < T; t += nwaves) {
    float z[kTkPerLane];
    bool live[kTkPerLane];
#pragma unroll
    for (int i = 0; i < kTkPerLane; ++i) {
      const int e = lane + kWave * i;
      live[i] = e < E;
      z[i] = 0.f;
      if (live[i]) {
        z[i] = logits[(size_t)t * E + e];
        if (bias) z[i] = __fadd_rn(z[i], bias[e]);
      }
    }
    float zsel = 0.f;  // lane j keeps the j-th selected value
    for (int j = 0; j < k; ++j) {
      float bv = -INFINITY;
      int bi = kTkNone;
#pragma unroll
      for (int i = 0; i < kTkPerLane; ++i) {
        const int e = lane + kWave * i;
        if (live[i] && tk_before(z[i], e, bv, bi)) {
          bv = z[i];
          bi = e;
        }
      }
#pragma unroll
      for (int m = 1; m < kWave; m <<= 1) {
        const float ov = __shfl_xor(bv, m);
        const int oi = __shfl_xor(bi, m);
        if (tk_before(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
        }
      }
      // every lane now holds the winner
#pragma unroll
      for (int i = 0; i < kTkPerLane; ++i)
        if (lane + kWave * i == bi) live[i] = false;
      if (lane == j) zsel = bv;
      if (lane == 0) ids[(size_t)t * k + j] = bi;
    }
    const double zmax = (double)__shfl(zsel, 0);
    const double p = lane < k ? exp((double)zsel - zmax) : 0.0;
    double s = 0.0;
    for (int j = 0; j < k; ++j) s += __shfl(p, j);
    if (lane < k) gates[(size_t)t * k + lane] = (float)(p / s);
  }
}

hipError_t launch_route_topk(const float *logits, const float *bias, int T, int E, int k,
                             int32_t *ids, float *gates, int grid_cap, hipStream_t stream) {
  const long long want = ((long long)T + kTkWaves - 1) / kTkWaves;
  const int grid = (int)(want < grid_cap ? want : grid_cap);
  hipLaunchKernelGGL(route_topk_kernel, dim3(grid), dim3(kTkThreads), 0, stream, logits, bias, T, E,
                     k, ids, gates);
  return hipGetLastError();
}

}  // namespace moe
