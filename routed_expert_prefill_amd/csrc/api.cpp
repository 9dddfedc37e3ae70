// Host side of the C ABI declared in include/moe_prefill.h: argument checks
// (all before any HIP call), workspace layout and launch sequencing.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "moe_prefill.h"
#include "kernels.h"


namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool misaligned(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// Scalars read once by a kernel (the combine's row limit) need only their
// own alignment.
bool misaligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) != 0; }

int status_from(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

int num_cus_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return 256;
  return cus;
}

// Workgroups of a row-quantisation launch: four per compute unit, each
// looping over rows.
int grid_cap_for_current_device() { return num_cus_current_device() * 4; }

struct FfnLayout {
  size_t sched, tiles, h, qx, sx, qh, sh, hmax, total;
};

bool ffn_desc_status(const moe_ffn_desc *d, int *st) {
  if (d == nullptr) {
    *st = MOE_EINVAL;
    return false;
  }
  if (d->T < 1 || d->k < 1 || d->E < 1 || d->d < 1 || d->f < 1) {
    *st = MOE_EINVAL;
    return false;
  }
  if ((long long)d->T * d->k >= (1LL << 31)) {
    *st = MOE_EINVAL;
    return false;
  }
  if (d->E > MOE_MAX_EXPERTS || d->k > MOE_MAX_TOPK || d->k > d->E || d->d % 128 != 0 ||
      d->f % 128 != 0) {
    *st = MOE_EUNSUPPORTED;
    return false;
  }
  const bool w8 = d->weight_dtype == MOE_W_FP8_E4M3_B128;
  const bool a8 = d->act_dtype == MOE_ACT_FP8_E4M3_ROW;
  const bool wok = d->weight_dtype == MOE_W_BF16 || w8;
  const bool aok = d->act_dtype == MOE_ACT_BF16 || a8;
  if (!wok || !aok || w8 != a8) {
    *st = MOE_EUNSUPPORTED;
    return false;
  }
  if (a8 && (d->d > moe::quant_max_cols() || d->f > moe::quant_max_cols())) {
    *st = MOE_EUNSUPPORTED;
    return false;
  }
  *st = MOE_OK;
  return true;
}

FfnLayout ffn_layout(const moe_ffn_desc *d) {
  const size_t R = (size_t)d->T * d->k;
  const bool fp8 = d->weight_dtype == MOE_W_FP8_E4M3_B128;
  FfnLayout L{};
  size_t off = 0;
  L.sched = off;
  off += align_up(sizeof(moe::Schedule));
  L.tiles = off;  // at most R / 256 full tiles plus one remainder per expert
  off += align_up(sizeof(moe::Tile) * (R / moe::kTileRows + (size_t)d->E));
  L.h = off;
  off += align_up(R * (size_t)d->f * 2);
  if (fp8) {
    L.qx = off;
    off += align_up((size_t)d->T * d->d);
    L.sx = off;
    off += align_up((size_t)d->T * 4);
    L.qh = off;
    off += align_up(R * (size_t)d->f);
    L.sh = off;
    off += align_up(R * 4);
    L.hmax = off;  // row maxima of |h|, kept by the gate/up epilogue
    off += align_up(R * 4);
  }
  L.total = off;
  return L;
}

}  // namespace

extern "C" {

const char *moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_EINVAL: return "MOE_EINVAL: invalid argument (null pointer, size or overflow)";
    case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED: shape or dtype outside the supported set";
    case MOE_EALIGN: return "MOE_EALIGN: device pointer not 16-byte aligned";
    case MOE_EWORKSPACE: return "MOE_EWORKSPACE: workspace missing or too small";
    case MOE_EHIP: return "MOE_EHIP: HIP runtime error";
    case MOE_ETOOLARGE:
      return "MOE_ETOOLARGE: larger than the fixed device scratch of a no-allocation call";
    default: return "unknown moe_status";
  }
}

int moe_abi_version(void) { return 2; }

size_t moe_route_build_workspace(int T, int k, int E) {
  if (T < 1 || k < 1 || E < 1 || E > MOE_MAX_EXPERTS || (long long)T * k >= (1LL << 31)) return 0;
  return align_up(moe::route_build_ws_bytes(T * k, E));
}

int moe_route_build(const int32_t *topk_ids, const uint8_t *route_mask, int T, int k, int E,
                    int32_t *counts, int32_t *offsets, int32_t *sorted_routes,
                    int32_t *route_rows, void *workspace, size_t workspace_bytes,
                    moe_stream_t stream) {
  if (!topk_ids || !counts || !offsets || !sorted_routes || !route_rows) return MOE_EINVAL;
  if (T < 1 || k < 1 || (long long)T * k >= (1LL << 31)) return MOE_EINVAL;
  if (E < 1 || E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK || k > E) return MOE_EUNSUPPORTED;
  if (misaligned(topk_ids) || misaligned(counts) || misaligned(offsets) ||
      misaligned(sorted_routes) || misaligned(route_rows) || misaligned(workspace) ||
      (route_mask && misaligned(route_mask)))
    return MOE_EALIGN;
  const size_t need = moe_route_build_workspace(T, k, E);
  if (!workspace || workspace_bytes < need) return MOE_EWORKSPACE;
  return status_from(moe::launch_route_build(topk_ids, route_mask, T * k, E, counts, offsets,
                                             sorted_routes, route_rows,
                                             static_cast<int32_t *>(workspace),
                                             static_cast<hipStream_t>(stream)));
}

int moe_route_build_noalloc(const int32_t *topk_ids, const uint8_t *route_mask, int T, int k,
                            int E, int32_t *counts, int32_t *offsets, int32_t *sorted_routes,
                            int32_t *route_rows, moe_stream_t stream) {
  static_assert(MOE_ROUTE_NOALLOC_MAX_ROUTES == moe::kRouteNoAllocMaxR, "one limit");
  if (!topk_ids || !counts || !offsets || !sorted_routes || !route_rows) return MOE_EINVAL;
  if (T < 1 || k < 1 || (long long)T * k >= (1LL << 31)) return MOE_EINVAL;
  if (E < 1 || E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK || k > E) return MOE_EUNSUPPORTED;
  if ((long long)T * k > MOE_ROUTE_NOALLOC_MAX_ROUTES) return MOE_ETOOLARGE;
  if (misaligned(topk_ids) || misaligned(counts) || misaligned(offsets) ||
      misaligned(sorted_routes) || misaligned(route_rows) || (route_mask && misaligned(route_mask)))
    return MOE_EALIGN;
  return status_from(moe::launch_route_build_noalloc(topk_ids, route_mask, T * k, E, counts,
                                                     offsets, sorted_routes, route_rows,
                                                     static_cast<hipStream_t>(stream)));
}

size_t moe_grouped_ffn_workspace(const moe_ffn_desc *desc) {
  int st;
  if (!ffn_desc_status(desc, &st)) return 0;
  return ffn_layout(desc).total;
}

}  // extern "C"

namespace {

// Shared body of moe_grouped_ffn and its stage calls.
int ffn_call(const moe_ffn_desc *desc, int stages, const void *x, const int32_t *offsets,
             const int32_t *sorted_routes, const void *w_gate, const void *w_up,
             const void *w_down, const float *s_gate, const float *s_up, const float *s_down,
             float *y, void *workspace, size_t workspace_bytes, moe_stream_t stream) {
  int st;
  if (!ffn_desc_status(desc, &st)) return st;
  const bool fp8 = desc->weight_dtype == MOE_W_FP8_E4M3_B128;
  const bool plan = stages & moe::kStagePlan, gu = stages & moe::kStageGateUp,
             dn = stages & moe::kStageDown;
  // pointers each requested stage reads or writes
  if (plan && (!offsets || (fp8 && !x))) return MOE_EINVAL;
  if (gu && (!x || !sorted_routes || !w_gate || !w_up || (fp8 && (!s_gate || !s_up))))
    return MOE_EINVAL;
  if (dn && (!offsets || !w_down || !y || (fp8 && !s_down))) return MOE_EINVAL;
  const void *ptrs[] = {x, offsets, sorted_routes, w_gate, w_up, w_down, s_gate, s_up, s_down, y,
                        workspace};
  for (const void *p : ptrs)
    if (p && misaligned(p)) return MOE_EALIGN;
  const FfnLayout lay = ffn_layout(desc);
  if (!workspace || workspace_bytes < lay.total) return MOE_EWORKSPACE;

  char *ws = static_cast<char *>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int R = desc->T * desc->k;
  if (!fp8) {
    moe::FfnLaunch L{};
    L.x = static_cast<const uint16_t *>(x);
    L.offsets = offsets;
    L.sorted_routes = sorted_routes;
    L.wg = static_cast<const uint16_t *>(w_gate);
    L.wu = static_cast<const uint16_t *>(w_up);
    L.wd = static_cast<const uint16_t *>(w_down);
    L.y = y;
    L.h = reinterpret_cast<uint16_t *>(ws + lay.h);
    L.sch = reinterpret_cast<moe::Schedule *>(ws + lay.sched);
    L.tiles = reinterpret_cast<moe::Tile *>(ws + lay.tiles);
    L.num_cus = num_cus_current_device();
    L.T = desc->T;
    L.k = desc->k;
    L.E = desc->E;
    L.d = desc->d;
    L.f = desc->f;
    L.R = R;
    return status_from(moe::launch_grouped_ffn_bf16(L, stages, s));
  }
  moe::FfnLaunchFp8 L{};
  L.x = static_cast<const uint16_t *>(x);
  L.qx = reinterpret_cast<uint8_t *>(ws + lay.qx);
  L.sx = reinterpret_cast<float *>(ws + lay.sx);
  L.offsets = offsets;
  L.sorted_routes = sorted_routes;
  L.wg = static_cast<const uint8_t *>(w_gate);
  L.wu = static_cast<const uint8_t *>(w_up);
  L.wd = static_cast<const uint8_t *>(w_down);
  L.sg = s_gate;
  L.su = s_up;
  L.sd = s_down;
  L.y = y;
  L.h = reinterpret_cast<uint16_t *>(ws + lay.h);
  L.qh = reinterpret_cast<uint8_t *>(ws + lay.qh);
  L.sh = reinterpret_cast<float *>(ws + lay.sh);
  L.hmax = reinterpret_cast<uint32_t *>(ws + lay.hmax);
  L.sch = reinterpret_cast<moe::Schedule *>(ws + lay.sched);
  L.tiles = reinterpret_cast<moe::Tile *>(ws + lay.tiles);
  L.num_cus = num_cus_current_device();
  L.T = desc->T;
  L.k = desc->k;
  L.E = desc->E;
  L.d = desc->d;
  L.f = desc->f;
  L.R = R;
  L.grid_cap = grid_cap_for_current_device();
  return status_from(moe::launch_ffn_fp8(L, stages, s));
}

}  // namespace

extern "C" {

int moe_grouped_ffn(const moe_ffn_desc *desc, const void *x, const int32_t *offsets,
                    const int32_t *sorted_routes, const void *w_gate, const void *w_up,
                    const void *w_down, const float *s_gate, const float *s_up,
                    const float *s_down, float *y, void *workspace, size_t workspace_bytes,
                    moe_stream_t stream) {
  return ffn_call(desc, moe::kStageAll, x, offsets, sorted_routes, w_gate, w_up, w_down, s_gate,
                  s_up, s_down, y, workspace, workspace_bytes, stream);
}

int moe_ffn_plan(const moe_ffn_desc *desc, const void *x, const int32_t *offsets,
                 void *workspace, size_t workspace_bytes, moe_stream_t stream) {
  return ffn_call(desc, moe::kStagePlan, x, offsets, nullptr, nullptr, nullptr, nullptr, nullptr,
                  nullptr, nullptr, nullptr, workspace, workspace_bytes, stream);
}

int moe_ffn_gate_up(const moe_ffn_desc *desc, const void *x, const int32_t *sorted_routes,
                    const void *w_gate, const void *w_up, const float *s_gate, const float *s_up,
                    void *workspace, size_t workspace_bytes, moe_stream_t stream) {
  return ffn_call(desc, moe::kStageGateUp, x, nullptr, sorted_routes, w_gate, w_up, nullptr,
                  s_gate, s_up, nullptr, nullptr, workspace, workspace_bytes, stream);
}

int moe_ffn_down(const moe_ffn_desc *desc, const int32_t *offsets, const void *w_down,
                 const float *s_down, float *y, void *workspace, size_t workspace_bytes,
                 moe_stream_t stream) {
  return ffn_call(desc, moe::kStageDown, nullptr, offsets, nullptr, nullptr, nullptr, w_down,
                  nullptr, nullptr, s_down, y, workspace, workspace_bytes, stream);
}

int moe_combine(const float *y, const int32_t *route_rows, const float *topk_w,
                const uint8_t *route_mask, const int32_t *row_limit, int T, int k, int d,
                float *out, moe_stream_t stream) {
  if (!y || !route_rows || !topk_w || !out) return MOE_EINVAL;
  if (T < 1 || k < 1 || d < 4 || d % 4 != 0 || (long long)T * k >= (1LL << 31)) return MOE_EINVAL;
  if (k > MOE_MAX_TOPK) return MOE_EUNSUPPORTED;
  if (misaligned(y) || misaligned(route_rows) || misaligned(topk_w) || misaligned(out) ||
      (route_mask && misaligned(route_mask)) || (row_limit && misaligned4(row_limit)))
    return MOE_EALIGN;
  return status_from(moe::launch_combine(y, route_rows, topk_w, route_mask, row_limit, nullptr, T,
                                         k, d, out, nullptr, static_cast<hipStream_t>(stream)));
}

int moe_combine_shared(const float *y, const int32_t *route_rows, const float *topk_w,
                       const uint8_t *route_mask, const int32_t *row_limit, const float *shared,
                       int T, int k, int d, float *out, void *out_bf16, moe_stream_t stream) {
  if (!y || !route_rows || !topk_w || (!out && !out_bf16)) return MOE_EINVAL;
  if (T < 1 || k < 1 || d < 4 || d % 4 != 0 || (long long)T * k >= (1LL << 31)) return MOE_EINVAL;
  if (k > MOE_MAX_TOPK) return MOE_EUNSUPPORTED;
  const void *ptrs[] = {y, route_rows, topk_w, route_mask, shared, out, out_bf16};
  for (const void *p : ptrs)
    if (p && misaligned(p)) return MOE_EALIGN;
  if (row_limit && misaligned4(row_limit)) return MOE_EALIGN;
  return status_from(moe::launch_combine(y, route_rows, topk_w, route_mask, row_limit, shared, T,
                                         k, d, out, static_cast<uint16_t *>(out_bf16),
                                         static_cast<hipStream_t>(stream)));
}

int moe_route_topk(const float *logits, const float *bias, int T, int E, int k,
                   int32_t *topk_ids, float *topk_w, moe_stream_t stream) {
  if (!logits || !topk_ids || !topk_w) return MOE_EINVAL;
  if (T < 1 || E < 1 || k < 1 || (long long)T * E >= (1LL << 31)) return MOE_EINVAL;
  if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK || k > E) return MOE_EUNSUPPORTED;
  if (misaligned(logits) || misaligned(topk_ids) || misaligned(topk_w) || (bias && misaligned(bias)))
    return MOE_EALIGN;
  return status_from(moe::launch_route_topk(logits, bias, T, E, k, topk_ids, topk_w,
                                            num_cus_current_device() * 8,
                                            static_cast<hipStream_t>(stream)));
}

int moe_quant_rows_fp8(const void *x, int rows, int cols, uint8_t *q, float *s,
                       moe_stream_t stream) {
  if (!x || !q || !s || rows < 1 || cols < 1) return MOE_EINVAL;
  if (cols % 128 != 0 || cols > moe::quant_max_cols()) return MOE_EUNSUPPORTED;
  if (misaligned(x) || misaligned(q) || misaligned(s)) return MOE_EALIGN;
  return status_from(moe::launch_quant_rows(static_cast<const uint16_t *>(x), rows, nullptr, cols,
                                            q, s, grid_cap_for_current_device(),
                                            static_cast<hipStream_t>(stream)));
}

}  // extern "C"
