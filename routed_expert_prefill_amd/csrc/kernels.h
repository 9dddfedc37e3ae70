// Launch entry points of the gfx950 kernels, called by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"

namespace moe {

hipError_t launch_route_build(const int32_t *ids, const uint8_t *mask, int R, int E,
                              int32_t *counts, int32_t *offsets, int32_t *sorted_routes,
                              int32_t *route_rows, int32_t *ws, hipStream_t stream);
size_t route_build_ws_bytes(int R, int E);

// The route build on the library's own device scratch (no workspace, no
// allocation), for up to kRouteNoAllocMaxR routes.
constexpr int kRouteNoAllocMaxR = 1 << 20;
hipError_t launch_route_build_noalloc(const int32_t *ids, const uint8_t *mask, int R, int E,
                                      int32_t *counts, int32_t *offsets, int32_t *sorted_routes,
                                      int32_t *route_rows, hipStream_t stream);

// row_limit (one int32: rows of y at or past it are never read), shared
// (fp32 [T,d]) and out_bf16 may be null; out may be null if out_bf16 is not.
hipError_t launch_combine(const float *y, const int32_t *route_rows, const float *topk_w,
                          const uint8_t *mask, const int32_t *row_limit, const float *shared,
                          int T, int k, int d, float *out, uint16_t *out_bf16,
                          hipStream_t stream);

hipError_t launch_route_topk(const float *logits, const float *bias, int T, int E, int k,
                             int32_t *ids, float *gates, int grid_cap, hipStream_t stream);

int quant_max_cols();
hipError_t launch_quant_rows(const uint16_t *x, int rows, const int32_t *rows_dev, int cols,
                             uint8_t *q, float *s, int grid_cap, hipStream_t stream);

// Tile list of the grouped FFN from the expert offsets (one thread per
// expert); also zeroes the work-queue heads.
hipError_t launch_grouped_schedule(const int32_t *offsets, int E, Schedule *sch, Tile *tiles,
                                   hipStream_t stream);

// Stages of the grouped FFN (bit mask).
enum : int { kStagePlan = 1, kStageGateUp = 2, kStageDown = 4, kStageAll = 7 };

// bf16 grouped FFN: schedule, gate/up + SwiGLU, down.
struct FfnLaunch {
  const uint16_t *x;
  const int32_t *offsets;
  const int32_t *sorted_routes;
  const uint16_t *wg, *wu, *wd;
  float *y;
  uint16_t *h;
  Schedule *sch;
  Tile *tiles;
  int T, k, E, d, f, R;
  int num_cus;  // workgroups of each persistent GEMM launch
};
hipError_t launch_grouped_ffn_bf16(const FfnLaunch &L, int stages, hipStream_t stream);

// fp8 grouped FFN: plan (schedule, per-row quantisation of x into qx, sx,
// row maxima of h cleared), gate/up + SwiGLU (h in bf16, its row maxima
// kept), down (per-row quantisation of h with those maxima, then GEMM).
struct FfnLaunchFp8 {
  const uint16_t *x;
  uint8_t *qx;
  float *sx;
  const int32_t *offsets;
  const int32_t *sorted_routes;
  const uint8_t *wg, *wu, *wd;
  const float *sg, *su, *sd;
  float *y;
  uint16_t *h;
  uint8_t *qh;
  float *sh;
  uint32_t *hmax;  // [R] bits of max |h| per row (the gate/up epilogue keeps them)
  Schedule *sch;
  Tile *tiles;
  int T, k, E, d, f, R;
  int grid_cap;  // workgroups of a row-quantisation launch
  int num_cus;
};
hipError_t launch_ffn_fp8(const FfnLaunchFp8 &L, int stages, hipStream_t stream);

// Per-row E4M3 quantisation of bf16 rows whose maxima are known: amax_bits[r]
// holds the fp32 bits of max |x[r, :]|; same codes and scales as
// launch_quant_rows.  rows_dev as there.
hipError_t launch_quant_rows_known_max(const uint16_t *x, int rows, const int32_t *rows_dev,
                                       int cols, const uint32_t *amax_bits, uint8_t *q, float *s,
                                       int grid_cap, hipStream_t stream);
// zero n 32-bit words (a kernel, not a memset: the path stays graph-capturable)
hipError_t launch_zero_u32(uint32_t *p, int n, hipStream_t stream);

}  // namespace moe
