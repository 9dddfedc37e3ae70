/*
 * moe_prefill.h -- C ABI of the grouped routed-MoE prefill library (gfx950).
 *
 * The library computes one routed-expert MoE layer for a prefill chunk of T
 * tokens, each routed to k of E experts, in expert-major order:
 *
 *   moe_route_topk    (optional, ahead of the path) top-k experts and
 *                     renormalised gates from router logits;
 *   moe_route_build   route histogram, prefix and scatter into
 *                     expert-contiguous order ("perf(ds4): batch heterogeneous
 *                     MoE prefill by expert", Summary: GPU-native route
 *                     histogram, prefix and scatter for up to 256 experts);
 *   moe_grouped_ffn   grouped gate/up GEMM with SwiGLU fused into its epilogue,
 *                     then the grouped down GEMM (same page, Summary: grouped
 *                     gate/up/down matmuls per owner; SwiGLU between them,
 *                     "perf(ggml): reuse ROCmFP4 weights across q=4 columns",
 *                     DS4 SwiGLU split op);
 *   moe_combine       route-weighted sum back to token order in which masked
 *                     routes contribute exact zeros (the fused MoE combine of
 *                     "perf(ds4): accelerate ROCm decode and long-context
 *                     selection", lucebox8 gfx1151 A/B; exact-zero masked
 *                     routes: "... by expert", Summary).
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless marked "host".  The caller owns every
 *    buffer; the library never allocates, frees or synchronises.  Work is
 *    enqueued on `stream` (a hipStream_t; NULL = the null stream) and is
 *    asynchronous.
 *  - All argument checks run on the host before any HIP call, so a rejected
 *    call touches no device memory.  Return value: MOE_OK (0) or a negative
 *    moe_status.  MOE_EHIP reports a launch error from the HIP runtime.
 *  - Device base pointers must be 16-byte aligned (MOE_EALIGN otherwise):
 *    the kernels use 16-byte vector loads and stores.  This is the
 *    library's alignment admission rule.
 *  - The library keeps no mutable global state: calls on different streams
 *    with distinct outputs and workspaces are independent.
 *  - Route r = t*k + j is route j of token t.  Arrays [T,k] are row-major.
 */
#ifndef MOE_PREFILL_H
#define MOE_PREFILL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_EINVAL = -1,       /* null pointer, non-positive size, T*k overflow */
  MOE_EUNSUPPORTED = -2, /* E > 256, k > 16 or k > E, d or f not a multiple of 128, dtype mix */
  MOE_EALIGN = -3,       /* a device base pointer is not 16-byte aligned */
  MOE_EWORKSPACE = -4,   /* workspace pointer null or smaller than the size query */
  MOE_EHIP = -5,         /* the HIP runtime reported an error */
  MOE_ETOOLARGE = -6     /* larger than the fixed device scratch of a no-allocation call */
} moe_status;

/* Weight storage formats. */
typedef enum moe_weight_dtype {
  MOE_W_BF16 = 0,          /* bf16 weights */
  MOE_W_FP8_E4M3_B128 = 1  /* OCP E4M3FN codes, one fp32 scale per 128x128 block */
} moe_weight_dtype;

/* Activation formats fed to the GEMMs. */
typedef enum moe_act_dtype {
  MOE_ACT_BF16 = 0,        /* x and h stay bf16 */
  MOE_ACT_FP8_E4M3_ROW = 1 /* x and h quantised per row to E4M3 with an fp32 scale */
} moe_act_dtype;

#define MOE_MAX_EXPERTS 256
#define MOE_MAX_TOPK 16

typedef void *moe_stream_t; /* a hipStream_t */

/* Shapes and formats of one MoE layer (host struct). */
typedef struct moe_ffn_desc {
  int32_t T;            /* tokens, >= 1 */
  int32_t k;            /* routes per token, 1 <= k <= min(E, 16) */
  int32_t E;            /* experts, 1 <= E <= 256 */
  int32_t d;            /* model width, multiple of 128 */
  int32_t f;            /* expert FFN width, multiple of 128 */
  int32_t weight_dtype; /* moe_weight_dtype */
  int32_t act_dtype;    /* moe_act_dtype; FP8_E4M3_ROW iff weights are FP8_E4M3_B128 */
} moe_ffn_desc;

/* Human-readable name of a status code (static string, never NULL). */
const char *moe_status_string(int status);

/* Library ABI version: 2. */
int moe_abi_version(void);

/* ------------------------------------------------------------ route build
 * Route histogram, prefix and scatter ("perf(ds4): batch heterogeneous MoE
 * prefill by expert", Summary).  Integer results, identical on every call.
 *
 *   key[r]   = topk_ids[r] if route r is active and 0 <= topk_ids[r] < E,
 *              else E (masked routes, and ids outside [0,E), fill the
 *              trailing bin E and are never computed)
 *   counts[b]    = #{r : key[r] = b}, b in [0, E]        int32 [E+1]
 *   offsets[0]   = 0, offsets[b+1] = offsets[b] + counts[b]   int32 [E+2]
 *   sorted_routes[offsets[key[r]] + #{r' < r : key[r'] = key[r]}] = r
 *                                                        int32 [T*k]
 *   route_rows   = the inverse permutation of sorted_routes   int32 [T*k]
 *
 * Each expert's segment keeps the route order, so the selected-row order is
 * preserved ("perf(ds4): extend sparse prefill scheduling to 10K", Summary of
 * the earlier description).
 *
 * topk_ids    int32 [T,k]
 * route_mask  uint8 [T,k], nonzero = active; NULL = every route active
 * workspace   device scratch of at least moe_route_build_workspace(T,k,E)
 *             bytes; contents on entry are ignored.
 * Errors: MOE_EINVAL (null output, T < 1, k < 1, T*k >= 2^31),
 *         MOE_EUNSUPPORTED (E < 1 or E > 256, k > 16 or k > E), MOE_EALIGN,
 *         MOE_EWORKSPACE.
 */
size_t moe_route_build_workspace(int T, int k, int E);
int moe_route_build(const int32_t *topk_ids, const uint8_t *route_mask, int T, int k, int E,
                    int32_t *counts, int32_t *offsets, int32_t *sorted_routes,
                    int32_t *route_rows, void *workspace, size_t workspace_bytes,
                    moe_stream_t stream);

/* ------------------------------------------------------------ route build, no allocation
 * For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: the same
 * route build as moe_route_build, with the same outputs bit for bit, but
 * without a workspace.  Its kernels use a fixed device array of the library
 * (MOE_ROUTE_NOALLOC_MAX_ROUTES routes' worth of chunk histograms, about
 * 1 MiB per GPU, held until the process ends); the call allocates and frees
 * nothing.  The caller still owns topk_ids, route_mask and the four outputs.
 *
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (on different streams) race and must not be issued.  Nothing in the
 * array has to be cleared between calls (each call writes what it reads).
 * Arguments as for moe_route_build.
 * Errors: as moe_route_build, and MOE_ETOOLARGE if T*k exceeds
 *         MOE_ROUTE_NOALLOC_MAX_ROUTES.
 */
#define MOE_ROUTE_NOALLOC_MAX_ROUTES (1 << 20)
int moe_route_build_noalloc(const int32_t *topk_ids, const uint8_t *route_mask, int T, int k,
                            int E, int32_t *counts, int32_t *offsets, int32_t *sorted_routes,
                            int32_t *route_rows, moe_stream_t stream);

/* ------------------------------------------------------------ grouped FFN
 * Grouped gate/up GEMM + SwiGLU + grouped down GEMM over expert-contiguous
 * rows ("perf(ds4): batch heterogeneous MoE prefill by expert", Summary).
 * For every expert e and every sorted row i in [offsets[e], offsets[e+1]),
 * with token t = sorted_routes[i] / k:
 *
 *   g = Wg[e] . x[t],  u = Wu[e] . x[t]             (fp32 accumulation)
 *   h = bf16_rne(silu(g) * u),  silu(z) = z / (1 + e^-z)
 *   y[i] = Wd[e] . h                                 (fp32)
 *
 * Rows i >= offsets[E] (masked routes) of y are never written.
 *
 * x             bf16 [T,d]
 * offsets       int32 [E+2], sorted_routes int32 [T*k]: from moe_route_build
 * w_gate, w_up  [E,f,d]  (row n of expert e holds output feature n; d contiguous)
 * w_down        [E,d,f]
 *               bf16, or E4M3 codes (uint8) for MOE_W_FP8_E4M3_B128
 * s_gate, s_up  fp32 [E, f/128, d/128]; s_down fp32 [E, d/128, f/128]:
 *               block scales, element [n,c] of expert e is multiplied by
 *               s[e, n/128, c/128].  NULL for bf16 weights.
 * y             fp32 [T*k, d]
 * workspace     at least moe_grouped_ffn_workspace(desc) bytes; holds the
 *               tile schedule, h and (fp8) the quantised activations.
 *
 * fp8 mode (weights FP8_E4M3_B128, activations FP8_E4M3_ROW): x rows and h
 * rows are quantised as s = fp32(max|v|)/448, q = e4m3_rne_saturate(v / s)
 * (IEEE fp32 division; an all-zero row gets s = 1, q = 0), and the GEMMs
 * consume decode(q) * s.
 * Errors: MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EALIGN, MOE_EWORKSPACE, MOE_EHIP.
 */
size_t moe_grouped_ffn_workspace(const moe_ffn_desc *desc /* host */);
int moe_grouped_ffn(const moe_ffn_desc *desc /* host */, const void *x, const int32_t *offsets,
                    const int32_t *sorted_routes, const void *w_gate, const void *w_up,
                    const void *w_down, const float *s_gate, const float *s_up,
                    const float *s_down, float *y, void *workspace, size_t workspace_bytes,
                    moe_stream_t stream);

/* ------------------------------------------------------------ FFN stages
 * moe_grouped_ffn is exactly these three calls, in this order, on one stream
 * with one workspace.  They are exposed for callers that time or overlap the
 * stages; the workspace carries the tile schedule and h between them.
 *
 * moe_ffn_plan     builds the tile schedule from offsets (device work list of
 *                  expert row tiles; fp8: also quantises x into the workspace).
 * moe_ffn_gate_up  gate/up GEMM with SwiGLU fused into the epilogue -> h
 *                  (fp8: the epilogue also keeps each row's max |h|).
 * moe_ffn_down     (fp8: quantises h per row with those maxima) down GEMM -> y.
 * Arguments mean what they mean for moe_grouped_ffn; unused ones may be NULL
 * (x is used by plan only in fp8 mode).  Errors as for moe_grouped_ffn.
 * After one plan, moe_ffn_gate_up and moe_ffn_down may each run again (for
 * instance for timing): the GEMM kernels leave their work-queue state in
 * the workspace as the plan left it.  A new offsets array needs a new plan.
 * The stage calls issue no memset and allocate nothing, so a sequence of
 * them (or of moe_grouped_ffn) can be captured in a HIP graph and replayed.
 */
int moe_ffn_plan(const moe_ffn_desc *desc /* host */, const void *x, const int32_t *offsets,
                 void *workspace, size_t workspace_bytes, moe_stream_t stream);
int moe_ffn_gate_up(const moe_ffn_desc *desc /* host */, const void *x,
                    const int32_t *sorted_routes, const void *w_gate, const void *w_up,
                    const float *s_gate, const float *s_up, void *workspace,
                    size_t workspace_bytes, moe_stream_t stream);
int moe_ffn_down(const moe_ffn_desc *desc /* host */, const int32_t *offsets, const void *w_down,
                 const float *s_down, float *y, void *workspace, size_t workspace_bytes,
                 moe_stream_t stream);

/* ------------------------------------------------------------ combine
 * Route-weighted combine back to token order (the fused MoE combine,
 * "perf(ds4): accelerate ROCm decode and long-context selection", lucebox8
 * gfx1151 A/B; "perf(ds4): extend sparse prefill scheduling to 10K",
 * Historical fused-combine discriminator):
 *
 *   out[t] = sum over j = 0..k-1 ascending, route read, of
 *            topk_w[t,j] * y[route_rows[t*k+j]]          (fp32, from +0.0)
 *
 * Route r is read when route_mask[r] != 0 (or route_mask is NULL) and, if
 * row_limit is given, route_rows[r] < *row_limit.  A route that is not read
 * -- its gate, its route_rows entry and its row of y may hold anything, NaN
 * included -- contributes an exact zero ("perf(ds4): batch heterogeneous MoE
 * prefill by expert", Summary and Correctness and validation).  A token with
 * no route read gets +0.0.
 *
 * row_limit is the bound that makes the combine agree with moe_route_build:
 * pass offsets + E (device pointer to offsets[E], the number of rows of y
 * moe_grouped_ffn writes).  moe_route_build sends masked routes AND active
 * routes whose id lies outside [0,E) to rows at or past offsets[E], which the
 * FFN never writes, so with the bound such routes are skipped like masked
 * ones.  With row_limit NULL, route_mask alone decides.
 *
 * y           fp32 [rows, d] with route_rows[r] < rows for every route read
 * route_rows  int32 [T*k]; topk_w fp32 [T,k]; route_mask uint8 [T,k] or NULL
 * row_limit   int32 [1] or NULL (4-byte aligned; read once by the kernel)
 * out         fp32 [T,d]
 * Errors: MOE_EINVAL (null, T < 1, k < 1, d < 4 or d not a multiple of 4),
 *         MOE_EUNSUPPORTED (k > 16), MOE_EALIGN, MOE_EHIP.
 */
int moe_combine(const float *y, const int32_t *route_rows, const float *topk_w,
                const uint8_t *route_mask, const int32_t *row_limit, int T, int k, int d,
                float *out, moe_stream_t stream);

/* ------------------------------------------------------------ combine, shared-output form
 * The combine writing into the layer's shared-expert output (the fused
 * combine's "shared-output" cases, "perf(ds4): extend sparse prefill
 * scheduling to 10K", Historical fused-combine discriminator):
 *
 *   routed[t]   = the moe_combine sum (fp32, ascending j from +0.0, routes
 *                 not read contribute nothing)
 *   out[t]      = routed[t] + shared[t]   (one fp32 addition; out = routed if shared is NULL)
 *   out_bf16[t] = bf16 round-to-nearest-even of out[t]
 *
 * shared fp32 [T,d] or NULL; out fp32 [T,d] or NULL; out_bf16 bf16 [T,d] or
 * NULL (at least one of out, out_bf16).  Other arguments, row_limit
 * included, as for moe_combine.
 * Errors: MOE_EINVAL (null y/route_rows/topk_w, both outputs null, T < 1,
 *         k < 1, d < 4 or d not a multiple of 4), MOE_EUNSUPPORTED (k > 16),
 *         MOE_EALIGN, MOE_EHIP.
 */
int moe_combine_shared(const float *y, const int32_t *route_rows, const float *topk_w,
                       const uint8_t *route_mask, const int32_t *row_limit, const float *shared,
                       int T, int k, int d, float *out, void *out_bf16, moe_stream_t stream);

/* ------------------------------------------------------------ router
 * Top-k expert selection and gates from router logits, the step ahead of
 * moe_route_build.  The pages keep the model's native top-6 routing and its
 * selected-row order ("perf(ds4): extend sparse prefill scheduling to 10K",
 * Summary); the arithmetic is the usual renormalised-softmax router:
 *
 *   z[t,e]      = logits[t,e] + bias[e]        (one fp32 addition; z = logits if bias is NULL)
 *   topk_ids[t] = the k largest z[t,.], descending; equal z go to the lower expert index
 *   topk_w[t,j] = exp(z_j - z_max) / sum_i exp(z_i - z_max), i over the selected experts,
 *                 evaluated in fp64 (sum in ascending j) and rounded once to fp32
 *
 * logits fp32 [T,E] row-major, finite; bias fp32 [E] or NULL;
 * topk_ids int32 [T,k] and topk_w fp32 [T,k] are written in full.
 * Errors: MOE_EINVAL (null logits or outputs, T < 1, E < 1, k < 1, T*E
 *         overflows int), MOE_EUNSUPPORTED (E > 256, k > 16 or k > E),
 *         MOE_EALIGN, MOE_EHIP.
 */
int moe_route_topk(const float *logits, const float *bias, int T, int E, int k,
                   int32_t *topk_ids, float *topk_w, moe_stream_t stream);

/* ------------------------------------------------------------ fp8 row quantisation
 * The activation quantisation the fp8 mode applies to x (exposed so callers
 * and tests can inspect codes and scales):
 *   s[i] = fp32(max_c |x[i,c]|) / 448  (IEEE fp32 division; 1 for an all-zero row)
 *   q[i,c] = e4m3_rne_saturate(x[i,c] / s[i])  (IEEE fp32 division, |.| >= 448 -> 448)
 * x bf16 [rows, cols]; q uint8 [rows, cols]; s fp32 [rows].
 * Errors: MOE_EINVAL (null, rows < 1), MOE_EUNSUPPORTED (cols not a multiple
 *         of 128), MOE_EALIGN, MOE_EHIP.
 */
int moe_quant_rows_fp8(const void *x, int rows, int cols, uint8_t *q, float *s,
                       moe_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PREFILL_H */
