// Grouped gate/up (+ fused SwiGLU) and down GEMMs, E4M3 weights with one fp32
// scale per 128x128 block and E4M3 activations with one fp32 scale per row.
//
// Same schedule and tile classes as the bf16 path.  One 16x16x128 MFMA covers
// exactly one 128-wide scale block of the reduction, so each block's partial
// product P is formed with a zero accumulator and folded in as
//   acc += s_w[n/128, kb] * P
// (the 16 output features of one MFMA lie in one 128-row scale block).  The
// per-row activation scale is constant along the reduction and multiplies the
// accumulator once in the epilogue.  Between the GEMMs, h is written in bf16
// and quantised per row by the row-quantisation kernel.
#include "kernels.h"

namespace moe {

struct GemmArgs8 {
  const uint8_t *act;            // gate/up: qx [T, K]; down: qh [R, K]
  const float *act_scale;        // gate/up: sx [T]; down: sh [R]
  const int32_t *sorted_routes;  // gate/up only
  int k;
  const uint8_t *w0, *w1;  // [E, N, K] codes (w1: up, gate/up only)
  const float *s0, *s1;    // [E, N/128, K/128]
  void *out;               // gate/up: h bf16 [R, N]; down: y fp32 [R, N]
  int N, K;
  const Tile *tiles;
  const int *ntiles;
};

__device__ __forceinline__ i32x8 load_i32x8(const uint8_t *p) {
  const i32x4 lo = *reinterpret_cast<const i32x4 *>(p);
  const i32x4 hi = *reinterpret_cast<const i32x4 *>(p + 16);
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ void fold(f32x4 &acc, float s, const f32x4 &p) {
  acc[0] = __builtin_fmaf(s, p[0], acc[0]);
  acc[1] = __builtin_fmaf(s, p[1], acc[1]);
  acc[2] = __builtin_fmaf(s, p[2], acc[2]);
  acc[3] = __builtin_fmaf(s, p[3], acc[3]);
}

template <bool GATEUP>
__device__ __forceinline__ void store_out8(const GemmArgs8 &a, int row, int n, float rs,
                                           const f32x4 &g, const f32x4 &u) {
  if constexpr (GATEUP) {
    uint32_t lo = (uint32_t)f32_to_bf16_bits(swiglu(g[0] * rs, u[0] * rs)) |
                  ((uint32_t)f32_to_bf16_bits(swiglu(g[1] * rs, u[1] * rs)) << 16);
    uint32_t hi = (uint32_t)f32_to_bf16_bits(swiglu(g[2] * rs, u[2] * rs)) |
                  ((uint32_t)f32_to_bf16_bits(swiglu(g[3] * rs, u[3] * rs)) << 16);
    uint2 v;
    v.x = lo;
    v.y = hi;
    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + (size_t)row * a.N + n) = v;
  } else {
    const f32x4 v = {g[0] * rs, g[1] * rs, g[2] * rs, g[3] * rs};
    *reinterpret_cast<f32x4 *>(static_cast<float *>(a.out) + (size_t)row * a.N + n) = v;
  }
}

// ------------------------------------------------------------------ schedule
//
// Tiles of the fp8 path: each expert's segment is cut into 128-row fat tiles
// and a remainder (a fat tile if it holds more than 32 rows, else a skinny
// tile), written to two lists.

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
                                                                 Tile *__restrict__ fat,
                                                                 Tile *__restrict__ big) {
  __shared__ int buf[kSchedThreads];
  const int e = threadIdx.x;
  int n = 0, row0 = 0;
  if (e < E) {
    row0 = offsets[e];
    n = offsets[e + 1] - row0;
  }
  // full big tiles, then one tile for the remainder chosen by its size
  int nb = 0, rem = n;
  if (big != nullptr) {
    nb = n / kBigRows;
    rem = n - nb * kBigRows;
    if (rem > kFatRows) {
      ++nb;
      rem = 0;
    }
  }
  int nf = 0;
  if (big == nullptr) {  // no big class: cut into fat tiles
    nf = rem / kFatRows;
    rem -= nf * kFatRows;
  }
  if (rem > kSkinnyMaxRows) {
    ++nf;
    rem = -rem;  // marks "remainder is one fat tile"
  }
  const int cs = rem > 0 ? 1 : 0;
  int tot_s, tot_f, tot_b;
  const int ps = block_excl_scan(cs, &tot_s, buf);
  const int pf = block_excl_scan(nf, &tot_f, buf);
  const int pb = block_excl_scan(nb, &tot_b, buf);
  int r = row0;
  for (int i = 0; i < nb; ++i) {
    Tile t;
    t.e = e;
    t.row0 = r;
    t.nrows = min(kBigRows, row0 + n - r);
    t.pad = 0;
    big[pb + i] = t;
    r += t.nrows;
  }
  for (int i = 0; i < nf; ++i) {
    Tile t;
    t.e = e;
    t.row0 = r;
    t.nrows = min(kFatRows, row0 + n - r);
    t.pad = 0;
    fat[pf + i] = t;
    r += t.nrows;
  }
  if (cs) {
    Tile t;
    t.e = e;
    t.row0 = r;
    t.nrows = rem;
    t.pad = 0;
    skinny[ps] = t;
  }
  if (e == 0) {
    sch->n_skinny = tot_s;
    sch->n_fat = tot_f;
    sch->n_big = tot_b;
  }
}

// ------------------------------------------------------------------ skinny tiles

constexpr int kSk8Threads = 256;
constexpr int kSk8Waves = kSk8Threads / kWave;
template <bool GATEUP>
constexpr int sk8_tn() { return GATEUP ? 2 : 4; }
template <bool GATEUP>
constexpr int sk8_feat() { return kSk8Waves * sk8_tn<GATEUP>() * 16; }

template <bool GATEUP, int TM>
__device__ __forceinline__ void skinny8_item(const GemmArgs8 &a, const Tile &t, int n_item0) {
  constexpr int TN = sk8_tn<GATEUP>();
  constexpr int NB = GATEUP ? 2 : 1;
  const int lane = lane_id();
  const int wv = threadIdx.x / kWave;
  const int m = lane & 15, q = lane >> 4;
  const int n_w = n_item0 + wv * TN * 16;
  const int K = a.K;
  const int KB = K / 128;
  if (n_w >= a.N) return;

  const uint8_t *arow[TM];
  float rs[TM];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int r = min(tm * 16 + m, t.nrows - 1);
    const int i = t.row0 + r;
    const size_t src = GATEUP ? (size_t)(a.sorted_routes[i] / a.k) : (size_t)i;
    arow[tm] = a.act + src * K + q * 32;
    rs[tm] = a.act_scale[src];
  }
  const uint8_t *wrow[NB][TN];
  const float *srow[NB][TN];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const int n = n_w + tn * 16;
      wrow[b][tn] = (b == 0 ? a.w0 : a.w1) + ((size_t)t.e * a.N + n + m) * K + q * 32;
      srow[b][tn] = (b == 0 ? a.s0 : a.s1) + ((size_t)t.e * (a.N / 128) + n / 128) * KB;
    }

  f32x4 acc[NB][TN][TM];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) acc[b][tn][tm] = f32x4{0.f, 0.f, 0.f, 0.f};

  i32x8 wA[NB][TN], xA[TM], wB[NB][TN], xB[TM];
  auto load = [&](i32x8(&w)[NB][TN], i32x8(&x)[TM], int kb) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) w[b][tn] = load_i32x8(wrow[b][tn] + kb * 128);
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) x[tm] = load_i32x8(arow[tm] + kb * 128);
  };
  auto compute = [&](i32x8(&w)[NB][TN], i32x8(&x)[TM], int kb) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const float s = srow[b][tn][kb];
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          const f32x4 p = mfma_fp8(w[b][tn], x[tm], f32x4{0.f, 0.f, 0.f, 0.f});
          fold(acc[b][tn][tm], s, p);
        }
      }
  };

  load(wA, xA, 0);
  for (int kb = 0; kb < KB; kb += 2) {
    if (kb + 1 < KB) load(wB, xB, kb + 1);
    compute(wA, xA, kb);
    if (kb + 2 < KB) load(wA, xA, kb + 2);
    if (kb + 1 < KB) compute(wB, xB, kb + 1);
  }

#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int row = tm * 16 + m;
    if (row < t.nrows) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const int n = n_w + tn * 16 + q * 4;
        store_out8<GATEUP>(a, t.row0 + row, n, rs[tm], acc[0][tn][tm], acc[NB - 1][tn][tm]);
      }
    }
  }
}

template <bool GATEUP>
__global__ __launch_bounds__(kSk8Threads) void skinny8_kernel(GemmArgs8 a) {
  const int per_tile = (a.N + sk8_feat<GATEUP>() - 1) / sk8_feat<GATEUP>();
  const int total = *a.ntiles * per_tile;
  for (int it = blockIdx.x; it < total; it += gridDim.x) {
    const int ti = it / per_tile;
    const int j = it - ti * per_tile;
    const Tile t = a.tiles[ti];
    if (t.nrows <= 16)
      skinny8_item<GATEUP, 1>(a, t, j * sk8_feat<GATEUP>());
    else
      skinny8_item<GATEUP, 2>(a, t, j * sk8_feat<GATEUP>());
  }
}

// ------------------------------------------------------------------ fat tiles

constexpr int kFt8Threads = 256;
constexpr int kFt8BN = 128;
constexpr int kFt8KT = 128;          // one scale block per LDS stage
constexpr int kFt8Ld = kFt8KT + 16;  // padded LDS row (bytes)

template <bool GATEUP>
__global__ __launch_bounds__(kFt8Threads) void fat8_kernel(GemmArgs8 a) {
  constexpr int NB = GATEUP ? 2 : 1;
  constexpr int BM = kFatRows;
  constexpr int TN = 4, TM = 4;
  constexpr int CH = kFt8KT / 16;                  // 16-byte chunks per row per stage
  constexpr int LOADS = BM * CH / kFt8Threads;     // 4
  __shared__ __attribute__((aligned(16))) uint8_t sW[NB][kFt8BN][kFt8Ld];
  __shared__ __attribute__((aligned(16))) uint8_t sX[BM][kFt8Ld];

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wv = tid / kWave;
  const int wf = wv & 1, wt = wv >> 1;
  const int m = lane & 15, q = lane >> 4;
  const int K = a.K;
  const int KB = K / 128;
  const int per_tile = a.N / kFt8BN;
  const int total = *a.ntiles * per_tile;

  for (int it = blockIdx.x; it < total; it += gridDim.x) {
    const int ti = it / per_tile;
    const int n0 = (it - ti * per_tile) * kFt8BN;
    const Tile t = a.tiles[ti];

    const uint8_t *xsrc[LOADS];
    const uint8_t *wsrc[NB][LOADS];
    int lrow[LOADS], lcol[LOADS];
#pragma unroll
    for (int c = 0; c < LOADS; ++c) {
      const int chunk = tid + c * kFt8Threads;
      lrow[c] = chunk / CH;
      lcol[c] = (chunk % CH) * 16;
      const int r = min(lrow[c], t.nrows - 1);
      const int i = t.row0 + r;
      const size_t src = GATEUP ? (size_t)(a.sorted_routes[i] / a.k) : (size_t)i;
      xsrc[c] = a.act + src * K + lcol[c];
#pragma unroll
      for (int b = 0; b < NB; ++b)
        wsrc[b][c] = (b == 0 ? a.w0 : a.w1) + ((size_t)t.e * a.N + n0 + lrow[c]) * K + lcol[c];
    }
    // the 128 output features of this item share one scale row per matrix
    const float *srow[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
      srow[b] = (b == 0 ? a.s0 : a.s1) + ((size_t)t.e * (a.N / 128) + n0 / 128) * KB;
    float rs[TM];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      const int r = min(wt * 64 + tm * 16 + m, t.nrows - 1);
      const int i = t.row0 + r;
      const size_t src = GATEUP ? (size_t)(a.sorted_routes[i] / a.k) : (size_t)i;
      rs[tm] = a.act_scale[src];
    }

    f32x4 acc[NB][TN][TM];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) acc[b][tn][tm] = f32x4{0.f, 0.f, 0.f, 0.f};

    i32x4 rx[LOADS], rw[NB][LOADS];
    auto gload = [&](int kb) {
#pragma unroll
      for (int c = 0; c < LOADS; ++c) {
        rx[c] = *reinterpret_cast<const i32x4 *>(xsrc[c] + kb * 128);
#pragma unroll
        for (int b = 0; b < NB; ++b) rw[b][c] = *reinterpret_cast<const i32x4 *>(wsrc[b][c] + kb * 128);
      }
    };
    gload(0);
    for (int kb = 0; kb < KB; ++kb) {
      __syncthreads();
#pragma unroll
      for (int c = 0; c < LOADS; ++c) {
        *reinterpret_cast<i32x4 *>(&sX[lrow[c]][lcol[c]]) = rx[c];
#pragma unroll
        for (int b = 0; b < NB; ++b) *reinterpret_cast<i32x4 *>(&sW[b][lrow[c]][lcol[c]]) = rw[b][c];
      }
      __syncthreads();
      if (kb + 1 < KB) gload(kb + 1);
      float s[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) s[b] = srow[b][kb];
      i32x8 fw[NB][TN], fx[TM];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) fw[b][tn] = load_i32x8(&sW[b][wf * 64 + tn * 16 + m][q * 32]);
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) fx[tm] = load_i32x8(&sX[wt * 64 + tm * 16 + m][q * 32]);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
          for (int tm = 0; tm < TM; ++tm) {
            const f32x4 p = mfma_fp8(fw[b][tn], fx[tm], f32x4{0.f, 0.f, 0.f, 0.f});
            fold(acc[b][tn][tm], s[b], p);
          }
    }

#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      const int row = wt * 64 + tm * 16 + m;
      if (row < t.nrows) {
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const int n = n0 + wf * 64 + tn * 16 + q * 4;
          store_out8<GATEUP>(a, t.row0 + row, n, rs[tm], acc[0][tn][tm], acc[NB - 1][tn][tm]);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ host side

hipError_t launch_schedule(const int32_t *offsets, int E, Schedule *sch, Tile *skinny, Tile *fat,
                           Tile *big, hipStream_t stream) {
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, offsets, E, sch,
                     skinny, fat, big);
  return hipGetLastError();
}


static int cap_grid8(long long items, int cap) {
  if (items < 1) items = 1;
  return (int)(items < cap ? items : cap);
}

hipError_t launch_ffn_fp8(const FfnLaunchFp8 &L, int stages, hipStream_t stream) {
  hipError_t err = hipSuccess;
  if (stages & kStagePlan) {
    err = launch_schedule(L.offsets, L.E, L.sch, L.skinny, L.fat, nullptr, stream);
    if (err != hipSuccess) return err;
    err = launch_quant_rows(L.x, L.T, nullptr, L.d, L.qx, L.sx, L.grid_cap, stream);
    if (err != hipSuccess) return err;
  }
  const long long max_skinny = L.E < L.R ? L.E : L.R;
  const long long max_fat = L.R / kFatRows + L.E;  // no big class: fat tiles only

  GemmArgs8 gu{};
  gu.act = L.qx;
  gu.act_scale = L.sx;
  gu.sorted_routes = L.sorted_routes;
  gu.k = L.k;
  gu.w0 = L.wg;
  gu.w1 = L.wu;
  gu.s0 = L.sg;
  gu.s1 = L.su;
  gu.out = L.h;
  gu.N = L.f;
  gu.K = L.d;

  if (stages & kStageGateUp) {
  gu.tiles = L.skinny;
  gu.ntiles = &L.sch->n_skinny;
  hipLaunchKernelGGL(skinny8_kernel<true>,
                     dim3(cap_grid8(max_skinny * ((L.f + sk8_feat<true>() - 1) / sk8_feat<true>()),
                                    L.grid_cap)),
                     dim3(kSk8Threads), 0, stream, gu);
  gu.tiles = L.fat;
  gu.ntiles = &L.sch->n_fat;
  hipLaunchKernelGGL(fat8_kernel<true>, dim3(cap_grid8(max_fat * (L.f / kFt8BN), L.grid_cap)),
                     dim3(kFt8Threads), 0, stream, gu);
  }
  if (!(stages & kStageDown)) return hipGetLastError();

  // h -> per-row E4M3; the active row count is offsets[E]
  err = launch_quant_rows(L.h, L.R, L.offsets + L.E, L.f, L.qh, L.sh, L.grid_cap, stream);
  if (err != hipSuccess) return err;

  GemmArgs8 dn{};
  dn.act = L.qh;
  dn.act_scale = L.sh;
  dn.sorted_routes = nullptr;
  dn.k = L.k;
  dn.w0 = L.wd;
  dn.w1 = nullptr;
  dn.s0 = L.sd;
  dn.s1 = nullptr;
  dn.out = L.y;
  dn.N = L.d;
  dn.K = L.f;
  dn.tiles = L.skinny;
  dn.ntiles = &L.sch->n_skinny;
  hipLaunchKernelGGL(skinny8_kernel<false>,
                     dim3(cap_grid8(max_skinny * ((L.d + sk8_feat<false>() - 1) / sk8_feat<false>()),
                                    L.grid_cap)),
                     dim3(kSk8Threads), 0, stream, dn);
  dn.tiles = L.fat;
  dn.ntiles = &L.sch->n_fat;
  hipLaunchKernelGGL(fat8_kernel<false>, dim3(cap_grid8(max_fat * (L.d / kFt8BN), L.grid_cap)),
                     dim3(kFt8Threads), 0, stream, dn);
  return hipGetLastError();
}

}  // namespace moe
