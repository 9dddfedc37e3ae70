// Grouped gate/up (+ fused SwiGLU) and down GEMMs over expert-sorted rows, bf16.
//
// The expert-major grouping of "perf(ds4): batch heterogeneous MoE prefill by
// expert" (Summary): each expert's routed rows form one contiguous segment
// of the sorted route order, and its weights are multiplied against that
// whole segment at once.  A device-built schedule splits segments into row
// tiles (a persistent compact work list, as in the MoE work queue of
// "perf(ds4): unify gfx1151 sparse-prefill stack", Composition) whose shape
// depends on the rows an expert received (adaptive MoE tiles, same passage):
//
//  * skinny tiles (<= 32 rows): the expert's weights are the bandwidth-bound
//    stream.  Each wave loads its weight rows straight from HBM into MFMA
//    operand registers (each weight byte is read once and used once), and
//    reads the few activation rows from L2.  No LDS, no barriers.
//  * fat tiles (<= 128 rows): both operands are staged through LDS so one
//    weight tile serves 128 rows.
//
// MFMA orientation: the first operand is a 16-feature slab of weights, the
// second a 16-row slab of activations, so each lane ends up holding four
// consecutive output features of one row (8- or 16-byte stores).
#include "kernels.h"

namespace moe {

struct GemmArgs {
  const uint16_t *act;           // gate/up: x [T, K]; down: h [R, K]
  const int32_t *sorted_routes;  // gate/up: token of sorted row i is sorted_routes[i] / k
  int k;
  const uint16_t *w0;  // gate (or down) weights [E, N, K]
  const uint16_t *w1;  // up weights [E, N, K] (gate/up only)
  void *out;           // gate/up: h bf16 [R, N]; down: y fp32 [R, N]
  int N, K;
  const Tile *tiles;
  const int *ntiles;
};

// ------------------------------------------------------------------ schedule

constexpr int kSchedThreads = 256;

__device__ int block_excl_scan(int v, int *total, int *buf) {
  const int t = threadIdx.x;
  buf[t] = v;
  __syncthreads();
  for (int off = 1; off < kSchedThreads; off <<= 1) {
    const int a = (t >= off) ? buf[t - off] : 0;
    __syncthreads();
    buf[t] += a;
    __syncthreads();
  }
  const int incl = buf[t];
  *total = buf[kSchedThreads - 1];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(const int32_t *__restrict__ offsets,
                                                                 int E, Schedule *sch,
                                                                 Tile *__restrict__ skinny,
                                                                 Tile *__restrict__ fat) {
  __shared__ int buf[kSchedThreads];
  const int e = threadIdx.x;
  int n = 0, row0 = 0;
  if (e < E) {
    row0 = offsets[e];
    n = offsets[e + 1] - row0;
  }
  const int nfull = n / kFatRows;
  const int rem = n - nfull * kFatRows;
  const int cs = (rem > 0 && rem <= kSkinnyMaxRows) ? 1 : 0;
  const int cf = nfull + (rem > kSkinnyMaxRows ? 1 : 0);
  int tot_s, tot_f;
  const int ps = block_excl_scan(cs, &tot_s, buf);
  const int pf = block_excl_scan(cf, &tot_f, buf);
  for (int i = 0; i < cf; ++i) {
    Tile t;
    t.e = e;
    t.row0 = row0 + i * kFatRows;
    t.nrows = min(kFatRows, n - i * kFatRows);
    t.pad = 0;
    fat[pf + i] = t;
  }
  if (cs) {
    Tile t;
    t.e = e;
    t.row0 = row0 + nfull * kFatRows;
    t.nrows = rem;
    t.pad = 0;
    skinny[ps] = t;
  }
  if (e == 0) {
    sch->n_skinny = tot_s;
    sch->n_fat = tot_f;
  }
}

// ------------------------------------------------------------------ epilogues

template <bool GATEUP>
__device__ __forceinline__ void store_out(const GemmArgs &a, int row, int n, const f32x4 &g,
                                          const f32x4 &u) {
  if constexpr (GATEUP) {
    uint32_t lo = (uint32_t)f32_to_bf16_bits(swiglu(g[0], u[0])) |
                  ((uint32_t)f32_to_bf16_bits(swiglu(g[1], u[1])) << 16);
    uint32_t hi = (uint32_t)f32_to_bf16_bits(swiglu(g[2], u[2])) |
                  ((uint32_t)f32_to_bf16_bits(swiglu(g[3], u[3])) << 16);
    uint2 v;
    v.x = lo;
    v.y = hi;
    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + (size_t)row * a.N + n) = v;
  } else {
    *reinterpret_cast<f32x4 *>(static_cast<float *>(a.out) + (size_t)row * a.N + n) = g;
  }
}

// ------------------------------------------------------------------ skinny tiles

constexpr int kSkThreads = 256;
constexpr int kSkWaves = kSkThreads / kWave;
template <bool GATEUP>
constexpr int sk_tn() { return GATEUP ? 2 : 4; }
template <bool GATEUP>
constexpr int sk_feat() { return kSkWaves * sk_tn<GATEUP>() * 16; }
constexpr int kSkU = 2;  // 32-wide reduction steps per pipeline stage

template <bool GATEUP, int TM>
__device__ __forceinline__ void skinny_item(const GemmArgs &a, const Tile &t, int n_item0) {
  constexpr int TN = sk_tn<GATEUP>();
  constexpr int NB = GATEUP ? 2 : 1;
  constexpr int S = 32 * kSkU;
  const int lane = lane_id();
  const int wv = threadIdx.x / kWave;
  const int m = lane & 15, q = lane >> 4;
  const int n_w = n_item0 + wv * TN * 16;
  const int K = a.K;
  if (n_w >= a.N) return;  // tail item of an N that is not a multiple of the item width

  const uint16_t *arow[TM];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int r = min(tm * 16 + m, t.nrows - 1);
    const int i = t.row0 + r;
    const size_t src = GATEUP ? (size_t)(a.sorted_routes[i] / a.k) : (size_t)i;
    arow[tm] = a.act + src * K + q * 8;
  }
  const uint16_t *wrow[NB][TN];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
      wrow[b][tn] = (b == 0 ? a.w0 : a.w1) + ((size_t)t.e * a.N + n_w + tn * 16 + m) * K + q * 8;

  f32x4 acc[NB][TN][TM];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) acc[b][tn][tm] = f32x4{0.f, 0.f, 0.f, 0.f};

  bf16x8 wA[kSkU][NB][TN], xA[kSkU][TM], wB[kSkU][NB][TN], xB[kSkU][TM];

  auto load = [&](bf16x8(&w)[kSkU][NB][TN], bf16x8(&x)[kSkU][TM], int k0) {
#pragma unroll
    for (int u = 0; u < kSkU; ++u) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) w[u][b][tn] = load_bf16x8(wrow[b][tn] + k0 + u * 32);
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) x[u][tm] = load_bf16x8(arow[tm] + k0 + u * 32);
    }
  };
  auto compute = [&](bf16x8(&w)[kSkU][NB][TN], bf16x8(&x)[kSkU][TM]) {
#pragma unroll
    for (int u = 0; u < kSkU; ++u)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
          for (int tm = 0; tm < TM; ++tm) acc[b][tn][tm] = mfma_bf16(w[u][b][tn], x[u][tm], acc[b][tn][tm]);
  };

  load(wA, xA, 0);
  for (int k0 = 0; k0 < K; k0 += 2 * S) {
    if (k0 + S < K) load(wB, xB, k0 + S);
    compute(wA, xA);
    if (k0 + 2 * S < K) load(wA, xA, k0 + 2 * S);
    if (k0 + S < K) compute(wB, xB);
  }

#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int row = tm * 16 + m;
    if (row < t.nrows) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const int n = n_w + tn * 16 + q * 4;
        store_out<GATEUP>(a, t.row0 + row, n, acc[0][tn][tm], acc[NB - 1][tn][tm]);
      }
    }
  }
}

template <bool GATEUP>
__global__ __launch_bounds__(kSkThreads) void skinny_kernel(GemmArgs a) {
  const int per_tile = (a.N + sk_feat<GATEUP>() - 1) / sk_feat<GATEUP>();
  const int total = *a.ntiles * per_tile;
  for (int it = blockIdx.x; it < total; it += gridDim.x) {
    const int ti = it / per_tile;
    const int j = it - ti * per_tile;
    const Tile t = a.tiles[ti];
    if (t.nrows <= 16)
      skinny_item<GATEUP, 1>(a, t, j * sk_feat<GATEUP>());
    else
      skinny_item<GATEUP, 2>(a, t, j * sk_feat<GATEUP>());
  }
}

// ------------------------------------------------------------------ fat tiles

constexpr int kFtThreads = 256;
constexpr int kFtBN = 128;  // output features per item
constexpr int kFtKT = 64;   // reduction slice per LDS stage
constexpr int kFtLd = kFtKT + 8;  // padded LDS row (elements)

template <bool GATEUP>
__global__ __launch_bounds__(kFtThreads) void fat_kernel(GemmArgs a) {
  constexpr int NB = GATEUP ? 2 : 1;
  constexpr int BM = kFatRows;
  constexpr int TN = 4, TM = 4;  // per wave: 64 features x 64 rows
  constexpr int CH = kFtKT / 8;  // 16-byte chunks per row per stage
  constexpr int LOADS = BM * CH / kFtThreads;  // chunks per thread per operand (4)
  __shared__ __attribute__((aligned(16))) uint16_t sW[NB][kFtBN][kFtLd];
  __shared__ __attribute__((aligned(16))) uint16_t sX[BM][kFtLd];

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wv = tid / kWave;
  const int wf = wv & 1, wt = wv >> 1;
  const int m = lane & 15, q = lane >> 4;
  const int K = a.K;
  const int per_tile = a.N / kFtBN;
  const int total = *a.ntiles * per_tile;

  for (int it = blockIdx.x; it < total; it += gridDim.x) {
    const int ti = it / per_tile;
    const int n0 = (it - ti * per_tile) * kFtBN;
    const Tile t = a.tiles[ti];

    const uint16_t *xsrc[LOADS];
    const uint16_t *wsrc[NB][LOADS];
    int lrow[LOADS], lcol[LOADS];
#pragma unroll
    for (int c = 0; c < LOADS; ++c) {
      const int chunk = tid + c * kFtThreads;
      lrow[c] = chunk / CH;
      lcol[c] = (chunk % CH) * 8;
      const int r = min(lrow[c], t.nrows - 1);
      const int i = t.row0 + r;
      const size_t src = GATEUP ? (size_t)(a.sorted_routes[i] / a.k) : (size_t)i;
      xsrc[c] = a.act + src * K + lcol[c];
#pragma unroll
      for (int b = 0; b < NB; ++b)
        wsrc[b][c] = (b == 0 ? a.w0 : a.w1) + ((size_t)t.e * a.N + n0 + lrow[c]) * K + lcol[c];
    }

    f32x4 acc[NB][TN][TM];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) acc[b][tn][tm] = f32x4{0.f, 0.f, 0.f, 0.f};

    bf16x8 rx[LOADS], rw[NB][LOADS];
    auto gload = [&](int k0) {
#pragma unroll
      for (int c = 0; c < LOADS; ++c) {
        rx[c] = load_bf16x8(xsrc[c] + k0);
#pragma unroll
        for (int b = 0; b < NB; ++b) rw[b][c] = load_bf16x8(wsrc[b][c] + k0);
      }
    };
    gload(0);
    for (int k0 = 0; k0 < K; k0 += kFtKT) {
      __syncthreads();
#pragma unroll
      for (int c = 0; c < LOADS; ++c) {
        *reinterpret_cast<bf16x8 *>(&sX[lrow[c]][lcol[c]]) = rx[c];
#pragma unroll
        for (int b = 0; b < NB; ++b) *reinterpret_cast<bf16x8 *>(&sW[b][lrow[c]][lcol[c]]) = rw[b][c];
      }
      __syncthreads();
      if (k0 + kFtKT < K) gload(k0 + kFtKT);
#pragma unroll
      for (int kk = 0; kk < kFtKT; kk += 32) {
        bf16x8 fw[NB][TN], fx[TM];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int tn = 0; tn < TN; ++tn)
            fw[b][tn] = *reinterpret_cast<const bf16x8 *>(&sW[b][wf * 64 + tn * 16 + m][kk + q * 8]);
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
          fx[tm] = *reinterpret_cast<const bf16x8 *>(&sX[wt * 64 + tm * 16 + m][kk + q * 8]);
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int tn = 0; tn < TN; ++tn)
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) acc[b][tn][tm] = mfma_bf16(fw[b][tn], fx[tm], acc[b][tn][tm]);
      }
    }

#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      const int row = wt * 64 + tm * 16 + m;
      if (row < t.nrows) {
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const int n = n0 + wf * 64 + tn * 16 + q * 4;
          store_out<GATEUP>(a, t.row0 + row, n, acc[0][tn][tm], acc[NB - 1][tn][tm]);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ host side

hipError_t launch_schedule(const int32_t *offsets, int E, Schedule *sch, Tile *skinny, Tile *fat,
                           hipStream_t stream) {
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, offsets, E, sch,
                     skinny, fat);
  return hipGetLastError();
}

static int cap_grid(long long items, int cap) {
  if (items < 1) items = 1;
  return (int)(items < cap ? items : cap);
}

hipError_t launch_ffn_bf16(const FfnLaunch &L, int stages, hipStream_t stream) {
  if (stages & kStagePlan) {
    hipError_t err = launch_schedule(L.offsets, L.E, L.sch, L.skinny, L.fat, stream);
    if (err != hipSuccess) return err;
  }
  const long long max_skinny = L.E < L.R ? L.E : L.R;
  const long long max_fat = L.R / kFatRows + L.E;

  GemmArgs gu{};
  gu.act = L.x;
  gu.sorted_routes = L.sorted_routes;
  gu.k = L.k;
  gu.w0 = L.wg;
  gu.w1 = L.wu;
  gu.out = L.h;
  gu.N = L.f;
  gu.K = L.d;

  GemmArgs dn{};
  dn.act = L.h;
  dn.sorted_routes = nullptr;
  dn.k = L.k;
  dn.w0 = L.wd;
  dn.w1 = nullptr;
  dn.out = L.y;
  dn.N = L.d;
  dn.K = L.f;

  if (stages & kStageGateUp) {
  gu.tiles = L.skinny;
  gu.ntiles = &L.sch->n_skinny;
  hipLaunchKernelGGL(skinny_kernel<true>,
                     dim3(cap_grid(max_skinny * (L.f / sk_feat<true>()), L.grid_cap)),
                     dim3(kSkThreads), 0, stream, gu);
  gu.tiles = L.fat;
  gu.ntiles = &L.sch->n_fat;
  hipLaunchKernelGGL(fat_kernel<true>, dim3(cap_grid(max_fat * (L.f / kFtBN), L.grid_cap)),
                     dim3(kFtThreads), 0, stream, gu);
  }
  if (stages & kStageDown) {
  dn.tiles = L.skinny;
  dn.ntiles = &L.sch->n_skinny;
  hipLaunchKernelGGL(skinny_kernel<false>,
                     dim3(cap_grid(max_skinny * ((L.d + sk_feat<false>() - 1) / sk_feat<false>()), L.grid_cap)),
                     dim3(kSkThreads), 0, stream, dn);
  dn.tiles = L.fat;
  dn.ntiles = &L.sch->n_fat;
  hipLaunchKernelGGL(fat_kernel<false>, dim3(cap_grid(max_fat * (L.d / kFtBN), L.grid_cap)),
                     dim3(kFtThreads), 0, stream, dn);
  }
  return hipGetLastError();
}

}  // namespace moe
