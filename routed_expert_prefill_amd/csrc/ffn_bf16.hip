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

#ifndef MOE_SK_U
#define MOE_SK_U 2
#endif
#ifndef MOE_SK_TN_GU
#define MOE_SK_TN_GU 2
#endif
#ifndef MOE_SK_TN_DN
#define MOE_SK_TN_DN 4
#endif
#ifndef MOE_SK_MINW
#define MOE_SK_MINW 1
#endif
constexpr int kSkThreads = 256;
constexpr int kSkWaves = kSkThreads / kWave;
template <bool GATEUP>
constexpr int sk_tn() { return GATEUP ? MOE_SK_TN_GU : MOE_SK_TN_DN; }  // 16-feature slabs per wave
template <bool GATEUP>
constexpr int sk_feat() { return kSkWaves * sk_tn<GATEUP>() * 16; }
constexpr int kSkU = MOE_SK_U;  // 32-wide reduction steps per pipeline stage

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
__global__ __launch_bounds__(kSkThreads, MOE_SK_MINW) void skinny_kernel(GemmArgs a) {
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


// ------------------------------------------------------------------ big tiles
//
// One item = up to 256 rows x 256 weight rows (gate/up: 128 output features of
// both matrices; down: 256 output features).  The reduction is streamed in
// stages of 32 elements (64 bytes per row): each stage is 512 rows x 64 bytes =
// 32 KB of LDS filled by direct global->LDS loads (each wave moves 8 KB per
// stage, no VGPR staging), in a ring of four stages, so three stages (96 KB per
// CU) are in flight while one is consumed.  Inside a stage, the four 16-byte
// chunks of row R are stored at chunk slot q ^ ((R >> 1) & 3): eight
// consecutive rows read at the same chunk then hit eight different bank
// groups.  Each wave owns a 128-row x 128-weight-row quadrant: 8 x 8 MFMA
// tiles, 256 fp32 accumulators per lane.

constexpr int kBgThreads = 256;
constexpr int kBgWRows = 256;
constexpr int kBgLdsRows = kBigRows + kBgWRows;  // 512 rows of 64 bytes
constexpr int kBgStage = kBgLdsRows * 64;        // 32 KB
constexpr int kBgLoads = kBgLdsRows / 16 / (kBgThreads / kWave);  // 8 wave loads per stage

typedef __attribute__((address_space(3))) void lds_ptr_t;

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(lds_ptr_t *)p;
}

// Direct global->LDS load of 16 bytes per lane: lane i's bytes land at LDS
// byte address m0 + 16 i.  Issued as inline assembly so that the compiler's
// wait-count insertion does not track it: a tracked load into one ring
// buffer makes the compiler drain every outstanding load before reads of
// another buffer.  Completion is awaited explicitly with wait_vm(); nothing
// else in these kernels uses m0.
__device__ __forceinline__ void dma16(const void *src, uint32_t lds_byte_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds_byte_addr)
               : "memory");
}

template <bool GATEUP>
struct BigItem {
  const uint16_t *src[kBgLoads];  // this lane's global chunk for each of its 8 loads (stage 0)
};

template <bool GATEUP>
__device__ __forceinline__ void big_issue(const BigItem<GATEUP> &it, uint32_t stage_lds, int s) {
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
#pragma unroll
  for (int j = 0; j < kBgLoads; ++j)
    dma16(it.src[j] + s * 32, stage_lds + (uint32_t)(wv * kBgLoads + j) * 1024u);
}

// Workgroup barrier without a memory fence.  __syncthreads() would make the
// compiler drain every outstanding vector-memory operation first (the direct
// global->LDS loads count as LDS writes), which would empty the stage ring at
// every stage.  Each wave instead waits for its own loads of the stage about
// to be read (wait_vm) and then meets the others here; the "memory" clobber
// keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void ring_barrier() { asm volatile("s_barrier" ::: "memory"); }

// wait until at most n (a multiple of 8, <= 32) of this wave's vector-memory
// operations are outstanding (s_waitcnt vmcnt: bits 3:0 and 15:14)
__device__ __forceinline__ void wait_vm(int n) {
  if (n >= 32)
    __builtin_amdgcn_s_waitcnt(0x8F70);  // vmcnt(32)
  else if (n >= 24)
    __builtin_amdgcn_s_waitcnt(0x4F78);  // vmcnt(24)
  else if (n >= 16)
    __builtin_amdgcn_s_waitcnt(0x4F70);  // vmcnt(16)
  else if (n >= 8)
    __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8)
  else
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
}

#ifndef MOE_BIG_SWZ
#define MOE_BIG_SWZ 1
#endif
// 16-byte chunk slot of chunk q in row r (0..15) of a 16-row block: the 16
// rows read at one chunk by a 16-lane group land on 16 distinct 16-byte slots
// of a 256-byte window, and each 8-lane half on 8 distinct slots of a
// 128-byte window.
__device__ __forceinline__ int big_slot(int r, int q) {
#if MOE_BIG_SWZ
  return q ^ (((r >> 1) ^ (r >> 3)) & 3);
#else
  return q ^ ((r >> 1) & 3);
#endif
}

// One stage's operand fragments of a wave: two 16-wide reduction steps, four
// 32-row token tiles and four 32-row weight tiles (gate/up: gate features
// [0,32), [32,64) then up features [0,32), [32,64) of the wave's 64; down:
// four 32-feature tiles of the wave's 128).
struct BigFrags {
  bf16x8 a[2][4];
  bf16x8 w[2][4];
};

template <bool GATEUP>
__device__ __forceinline__ void big_read(const uint8_t *buf, const int (&lane_off)[2], int wt,
                                         int wf, BigFrags &F) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
      F.a[ks][tt] = *reinterpret_cast<const bf16x8 *>(buf + (wt * 4 + tt) * 2048 + lane_off[ks]);
#pragma unroll
    for (int tw = 0; tw < 4; ++tw) {
      const int wrow = GATEUP ? ((tw >> 1) * 128 + wf * 64 + (tw & 1) * 32) : (wf * 128 + tw * 32);
      F.w[ks][tw] =
          *reinterpret_cast<const bf16x8 *>(buf + (kBigRows + wrow) * 64 + lane_off[ks]);
    }
  }
}

__device__ __forceinline__ void big_mfma(const BigFrags &F, f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int tw = 0; tw < 4; ++tw)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) acc[tw][tt] = mfma32_bf16(F.w[ks][tw], F.a[ks][tt], acc[tw][tt]);
}

#ifndef MOE_BIG_STAGES
#define MOE_BIG_STAGES 4
#endif
#ifndef MOE_BIG_PIPE
#define MOE_BIG_PIPE 0
#endif
constexpr int kBgStages = MOE_BIG_STAGES;  // ring depth: kBgStages - 1 stages in flight
static_assert(kBgStages >= 2 && kBgStages <= 5, "LDS holds at most five 32 KB stages");

template <bool GATEUP>
__global__ __launch_bounds__(kBgThreads, 1) void big_kernel(GemmArgs a) {
  constexpr int FEAT = GATEUP ? 128 : 256;  // output features per item
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kBgStages * kBgStage];

  const uint32_t ring_lds = lds_addr(ring);
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wv = tid / kWave;
  const int wt = wv >> 1, wf = wv & 1;
  const int K = a.K;
  const int nst = K / 32;
  const int per_tile = (a.N + FEAT - 1) / FEAT;
  const int total = *a.ntiles * per_tile;
  // reader: row (lane & 31) of a 32-row tile; reduction step ks reads chunk
  // 2 ks + (lane >> 5) of the row's four, at its swizzled slot
  const int rr = lane & 31, rh = lane >> 5;
  const int lane_off[2] = {rr * 64 + big_slot(rr & 15, rh) * 16,
                           rr * 64 + big_slot(rr & 15, 2 + rh) * 16};
  // loader: lane i fills slot (i & 3) of row (i >> 2) of a 16-row block, so it
  // fetches the chunk that belongs in that slot (the swizzle is an involution)
  const int lr = lane >> 2;
  const int lq = big_slot(lr, lane & 3);

  for (int it = blockIdx.x; it < total; it += gridDim.x) {
    const int ti = it / per_tile;
    const int n0 = (it - ti * per_tile) * FEAT;
    const Tile t = a.tiles[ti];

    BigItem<GATEUP> item;
#pragma unroll
    for (int j = 0; j < kBgLoads; ++j) {
      const int R = (wv * kBgLoads + j) * 16 + lr;  // LDS row 0..511
      if (R < kBigRows) {
        const int i = t.row0 + min(R, t.nrows - 1);
        const size_t src = GATEUP ? (size_t)(a.sorted_routes[i] / a.k) : (size_t)i;
        item.src[j] = a.act + src * K + lq * 8;
      } else {
        const int wr = R - kBigRows;
        const uint16_t *w;
        int n;
        if (GATEUP) {
          w = wr < 128 ? a.w0 : a.w1;
          n = n0 + (wr & 127);
        } else {
          w = a.w0;
          n = min(n0 + wr, a.N - 1);
        }
        item.src[j] = w + ((size_t)t.e * a.N + n) * K + lq * 8;
      }
    }

    f32x16 acc[4][4];
#pragma unroll
    for (int tw = 0; tw < 4; ++tw)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[tw][tt][j] = 0.f;

    wait_vm(0);
    ring_barrier();  // the previous item's last stages have been read by every wave
#pragma unroll
    for (int s = 0; s < kBgStages - 1; ++s)
      if (s < nst) big_issue<GATEUP>(item, ring_lds + s * kBgStage, s);
#if MOE_BIG_PIPE
    // Fragments of stage s + 1 are read from LDS while the MFMAs of stage s
    // run from registers (two fragment sets, alternating by stage parity).
    BigFrags F0, F1;
    wait_vm(8 * min(kBgStages - 2, nst - 1));
    ring_barrier();
    big_read<GATEUP>(ring, lane_off, wt, wf, F0);
    int slot = 0;  // ring slot of stage s
    // one stage: make stage st + 1 visible, refill the ring, read st + 1's
    // fragments into `next`, multiply stage st from `cur`
    auto step = [&](int st, BigFrags &cur, BigFrags &next) {
      const int nslot = slot == kBgStages - 1 ? 0 : slot + 1;  // slot of stage st + 1
      if (st + 1 < nst) {
        wait_vm(8 * max(0, min(kBgStages - 3, nst - 2 - st)));
        ring_barrier();  // everyone's stage st + 1 is in LDS; stage st - 1 is consumed
        const int ahead = st + kBgStages - 1;
        if (ahead < nst) {
          const int aslot = slot == 0 ? kBgStages - 1 : slot - 1;  // slot of stage st - 1
          big_issue<GATEUP>(item, ring_lds + aslot * kBgStage, ahead);
        }
        big_read<GATEUP>(ring + nslot * kBgStage, lane_off, wt, wf, next);
      }
      big_mfma(cur, acc);
      slot = nslot;
    };
    for (int s = 0; s < nst; s += 2) {  // nst is even: K is a multiple of 128
      step(s, F0, F1);
      step(s + 1, F1, F0);
    }
#else
    int slot = 0;  // ring slot of stage s
    for (int s = 0; s < nst; ++s) {
      // stage s must have landed; up to kBgStages - 2 later stages may still be in flight
      wait_vm(8 * min(kBgStages - 2, nst - 1 - s));
      ring_barrier();  // everyone's stage s is in LDS; everyone is done with stage s - 1
      const int ahead = s + kBgStages - 1;
      if (ahead < nst) {
        const int aslot = slot == 0 ? kBgStages - 1 : slot - 1;  // the slot of stage s - 1
        big_issue<GATEUP>(item, ring_lds + aslot * kBgStage, ahead);
      }
      BigFrags F;
      big_read<GATEUP>(ring + slot * kBgStage, lane_off, wt, wf, F);
      big_mfma(F, acc);
      slot = slot == kBgStages - 1 ? 0 : slot + 1;
    }
#endif

    // register j of a 32x32 tile holds feature 8*(j/4) + 4*rh + j%4, token rr
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int row = wt * 128 + tt * 32 + rr;
      if (row < t.nrows) {
#pragma unroll
        for (int tw = 0; tw < (GATEUP ? 2 : 4); ++tw)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int n = n0 + wf * (FEAT / 2) + tw * 32 + g * 8 + rh * 4;
            const f32x4 v0 = {acc[tw][tt][4 * g], acc[tw][tt][4 * g + 1], acc[tw][tt][4 * g + 2],
                              acc[tw][tt][4 * g + 3]};
            if (GATEUP) {
              const f32x4 v1 = {acc[tw + 2][tt][4 * g], acc[tw + 2][tt][4 * g + 1],
                                acc[tw + 2][tt][4 * g + 2], acc[tw + 2][tt][4 * g + 3]};
              store_out<GATEUP>(a, t.row0 + row, n, v0, v1);
            } else if (n < a.N) {
              store_out<GATEUP>(a, t.row0 + row, n, v0, v0);
            }
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

static int cap_grid(long long items, int cap) {
  if (items < 1) items = 1;
  return (int)(items < cap ? items : cap);
}

hipError_t launch_ffn_bf16(const FfnLaunch &L, int stages, hipStream_t stream) {
  if (stages & kStagePlan) {
    hipError_t err = launch_schedule(L.offsets, L.E, L.sch, L.skinny, L.fat, L.big, stream);
    if (err != hipSuccess) return err;
  }
  const long long max_skinny = L.E < L.R ? L.E : L.R;
  const long long max_fat = L.E;
  const long long max_big = L.R / kBigRows + L.E;

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
  gu.tiles = L.big;
  gu.ntiles = &L.sch->n_big;
  hipLaunchKernelGGL(big_kernel<true>, dim3(cap_grid(max_big * (L.f / 128), L.num_cus)),
                     dim3(kBgThreads), 0, stream, gu);
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
  dn.tiles = L.big;
  dn.ntiles = &L.sch->n_big;
  hipLaunchKernelGGL(big_kernel<false>, dim3(cap_grid(max_big * ((L.d + 255) / 256), L.num_cus)),
                     dim3(kBgThreads), 0, stream, dn);
  }
  return hipGetLastError();
}

}  // namespace moe
