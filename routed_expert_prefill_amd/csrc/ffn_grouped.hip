// Persistent grouped GEMM for the bf16 routed-MoE FFN: one kernel per
// projection (gate/up with the SwiGLU epilogue, then down) that pulls work
// items from a device queue.
//
// The expert-major grouping of "perf(ds4): batch heterogeneous MoE prefill by
// expert" (Summary): every expert's routed rows form one contiguous segment
// of the sorted route order and are multiplied by its weights together.  The
// schedule cuts each segment into row tiles whose height adapts to the rows
// the expert received (adaptive MoE tiles and a persistent compact work
// queue, "perf(ds4): unify gfx1151 sparse-prefill stack", Composition):
// 256-row tiles, then one remainder tile of 32, 64, 128, 192 or 256 rows
// (192-row tiles use the 256-row layout here).  The tile list is ordered
// tallest class first, the 256-row tiles of experts with several tiles ahead
// of the rest, and each workgroup repeatedly takes the next item from one of
// two atomic counters: a tile and 128 gate/up output features, or a tile and
// one to four blocks of 256 down-projection features streamed through one
// ring fill.  One counter hands out the items of experts with several tiles
// (compute-bound), the other those of single-tile experts (each a weight
// stream); part of the workgroups start on each, so memory-bound items of
// small experts run on some compute units while compute-bound items of large
// experts run on others.  The weights of an expert with a single tile are
// read once and go through non-temporal loads.
//
// Every item streams both operands through the LDS stage ring (ring.h): 256
// weight rows and 32 x ablk activation rows per 64-element reduction stage
// (128-byte rows), with as many stages as the 160 KB of LDS holds (2 to 4).
// MFMAs are 32x32x16
// bf16; eight waves (two per SIMD, so one wave's matrix work covers the
// other's barrier and LDS waits) each own 32-row weight tiles:
//   ablk = 8 (256 rows): wave w takes weight tiles 2(w%4), 2(w%4)+1 and the
//                        four activation tiles of half w/4;
//   ablk < 8:            wave w takes weight tile w and every activation tile.
// Gate/up weight rows are interleaved in 16-row groups (16 gate features,
// the same 16 up features, ...), so one 32x32 tile holds both halves of the
// SwiGLU for 16 features: registers 0-7 gate, 8-15 up.
#include "kernels.h"
#include "ring.h"

#ifndef MOE_SSW4_GU
#define MOE_SSW4_GU 6
#endif
#ifndef MOE_SSW4_DN
#define MOE_SSW4_DN 9
#endif

namespace moe {

struct GgArgs {
  const uint16_t *act;           // gate/up: x [T, K]; down: h [R, K]
  const int32_t *sorted_routes;  // gate/up: token of sorted row i is sorted_routes[i] / k
  int k;
  const uint16_t *w0;  // gate (or down) weights [E, N, K]
  const uint16_t *w1;  // up weights [E, N, K] (gate/up only)
  void *out;           // gate/up: h bf16 [R, N]; down: y fp32 [R, N]
  int N, K;
  const Tile *tiles;
  const int *ntiles;
  int *counter;        // compute-queue head (TwoQueue), zeroed by the schedule
  int wr;              // weight rows per item: 256, 128 or 64 (at most 32 routed rows), or 0:
                       // 128 if every tile is a 32-row tile, else 256 (decided on the device)
  int nb;              // feature blocks per item (streamed through one ring fill)
  int nb_skinny;       // the same for 32-row tiles when nearly all tiles are 32-row ones
  const int *n_small;  // 32-row tiles at the end of the tile list
  const int *n_multi;  // tiles of experts with several tiles, at the start of the list
  int *counter_s;      // head of the second queue (items of the other tiles)
  int static_items;    // 1: workgroup b takes items b, b + grid, ... (no queue)
};

constexpr int kGgThreads = 512;
constexpr int kGgWaves = kGgThreads / kWave;
constexpr int kGgWRows = 256;
constexpr int kGgRing = 160 * 1024;  // the whole LDS of a workgroup

// Ring geometry of an item with 32 * AB activation rows: a stage is
// (32 AB + 256) rows of 128 bytes, and the ring has as many slots as fit.
template <int AB, int WR = kGgWRows>
struct GgRing {
  static constexpr int kSlot = (32 * AB + WR) * 128;
  static constexpr int kDepth = (kGgRing / kSlot) < 12 ? (kGgRing / kSlot) : 12;
};

// ------------------------------------------------------------------ schedule

constexpr int kGsThreads = 256;

constexpr int kGsWaves = kGsThreads / kWave;

// Inclusive sum of v over the lanes of a wave up to this one.
__device__ __forceinline__ int gs_wave_scan(int v) {
  const int lane = threadIdx.x & (kWave - 1);
  for (int off = 1; off < kWave; off <<= 1) {
    const int x = __shfl_up(v, off, kWave);
    if (lane >= off) v += x;
  }
  return v;
}

// One thread per expert: full 256-row tiles, then one remainder tile whose
// height is the smallest of 32, 64, 128, 192, 256 that holds it.  Tiles are
// written tallest class first.
__global__ __launch_bounds__(kGsThreads) void grouped_schedule_kernel(
    const int32_t *__restrict__ offsets, int E, Schedule *sch, Tile *__restrict__ tiles) {
  constexpr int NC = 6;
  __shared__ int wave_tot[kGsWaves][NC];
  const int e = threadIdx.x;
  int n = 0, row0 = 0;
  if (e < E) {
    row0 = offsets[e];
    n = offsets[e + 1] - row0;
  }
  const int nfull = n / kTileRows;
  const int rem = n - nfull * kTileRows;
  const int rab = rem == 0       ? 0
                  : rem <= 32    ? 1
                  : rem <= 64    ? 2
                  : rem <= 128   ? 4
                  : rem <= 192   ? 6
                                 : 8;
  // classes, tallest first: ablk 8 of experts with several tiles, ablk 8 of
  // single-tile experts, then 6, 4, 2, 1
  const int n8 = nfull + (rab == 8);
  const bool multi = n > kTileRows;
  int cnt[NC] = {multi ? n8 : 0, multi ? 0 : n8, rab == 6, rab == 4, rab == 2, rab == 1};
  // per class: exclusive prefix over the experts (wave scans, then the
  // totals of the waves before this one) and the total over all experts
  int pos[NC], tot[NC];
  const int wave = threadIdx.x / kWave;
  for (int c = 0; c < NC; ++c) {
    pos[c] = gs_wave_scan(cnt[c]);
    if ((threadIdx.x & (kWave - 1)) == kWave - 1) wave_tot[wave][c] = pos[c];
  }
  __syncthreads();
  for (int c = 0; c < NC; ++c) {
    int before = 0, all = 0;
    for (int w = 0; w < kGsWaves; ++w) {
      const int v = wave_tot[w][c];
      before += w < wave ? v : 0;
      all += v;
    }
    pos[c] += before - cnt[c];
    tot[c] = all;
  }
  int base = 0;
  for (int c = 0; c < NC; ++c) {
    pos[c] += base;
    base += tot[c];
  }
  const int stream = n <= kTileRows ? kTileStream : 0;  // the expert's only tile
  for (int i = 0; i < n8; ++i) {
    Tile t;
    t.e = e;
    t.row0 = row0 + i * kTileRows;
    t.nrows = min(kTileRows, n - i * kTileRows);
    t.ablk = 8 | stream;
    tiles[pos[multi ? 0 : 1] + i] = t;
  }
  if (rab > 0 && rab < 8) {
    const int c = rab == 6 ? 2 : rab == 4 ? 3 : rab == 2 ? 4 : 5;
    Tile t;
    t.e = e;
    t.row0 = row0 + nfull * kTileRows;
    t.nrows = rem;
    t.ablk = rab | stream;
    tiles[pos[c]] = t;
  }
  if (e == 0) {
    sch->n_tiles = base;
    sch->counter[0] = 0;
    sch->counter[1] = 0;
    sch->n_small = tot[NC - 1];
    sch->n_multi = tot[0];
    sch->counter_s[0] = 0;
    sch->counter_s[1] = 0;
  }
}

// ------------------------------------------------------------------ one item

template <bool GATEUP>
__device__ __forceinline__ void gg_store(const GgArgs &a, int row, int n, const f32x4 &g,
                                         const f32x4 &u) {
  if constexpr (GATEUP) {
    uint2 v;
    v.x = (uint32_t)f32_to_bf16_bits(swiglu(g[0], u[0])) |
          ((uint32_t)f32_to_bf16_bits(swiglu(g[1], u[1])) << 16);
    v.y = (uint32_t)f32_to_bf16_bits(swiglu(g[2], u[2])) |
          ((uint32_t)f32_to_bf16_bits(swiglu(g[3], u[3])) << 16);
    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + (size_t)row * a.N + n) = v;
  } else {
    *reinterpret_cast<f32x4 *>(static_cast<float *>(a.out) + (size_t)row * a.N + n) = g;
  }
}

__device__ __forceinline__ f32x4 quad(const f32x16 &v, int g) {
  return f32x4{v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]};
}

// Operand tiles a wave multiplies for one stage: TT activation tiles and TW
// weight tiles of 32 rows, for the four 16-wide reduction steps.
// With fewer weight rows per item (WR < 256, 32-row tiles only) waves
// WR/32 .. 7 only load.
template <int AB, int WR = kGgWRows>
struct GgLayout {
  static constexpr int TT = AB == 8 ? 4 : AB;
  static constexpr int TW = AB == 8 ? 2 : 1;
  __device__ static bool active(int wv) { return WR == kGgWRows || wv < WR / 32; }
  // LDS row (within the stage) of activation tile tt / weight tile tw of wave wv
  __device__ static int arow(int wv, int tt) { return AB == 8 ? ((wv >> 2) * 128 + tt * 32) : tt * 32; }
  __device__ static int wtile(int wv, int tw) { return AB == 8 ? ((wv & 3) * 2 + tw) : wv; }
  __device__ static int wrow(int wv, int tw) { return 32 * AB + 32 * wtile(wv, tw); }
};

// NT: weight rows go through non-temporal loads (the tile carries
// kTileStream); a template parameter because a per-load choice inside the
// stage loop cost the MFMA-bound tiles up to 4%.
// MB: the item may carry several feature blocks (nb); without it nb is 1 and
// the stage loop has no block bookkeeping.
template <bool GATEUP, bool NT, bool MB, int AB, int WR = kGgWRows>
__device__ __forceinline__ void gg_item(const GgArgs &a, const Tile &t, int n0, int nb_arg,
                                        uint8_t *ring, uint32_t ring_lds) {
  const int nb = MB ? nb_arg : 1;
  using L = GgLayout<AB, WR>;
  constexpr int FEAT = GATEUP ? WR / 2 : WR;  // output features per block
  constexpr int TT = L::TT, TW = L::TW;
  constexpr int NA = 4 * AB;       // activation loads (8 rows each) per stage
  constexpr int NL = NA + WR / 8;  // all loads per stage
  constexpr int MAXJ = (NL + kGgWaves - 1) / kGgWaves;
  const int lane = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int K = a.K;
  const int nst = K / 64;
  const int cnt = (NL - wv + kGgWaves - 1) / kGgWaves;  // loads this wave issues per stage

  // this lane's source chunk for each of its loads (stage 0): load i fills
  // stage rows 8 i .. 8 i + 7; lane fills slot (lane & 7) of row 8 i + (lane >> 3)
  const int lr = lane >> 3;
  const uint16_t *src[MAXJ];
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    const int i = wv + kGgWaves * j;
    const int lq = ring_slot(i * 8 + lr, lane & 7);  // the chunk that belongs in that slot
    src[j] = a.act;
    if (i < NA) {
      const int R = i * 8 + lr;
      const int row = t.row0 + min(R, t.nrows - 1);
      const size_t s = GATEUP ? (size_t)(a.sorted_routes[row] / a.k) : (size_t)row;
      src[j] = a.act + s * K + lq * 8;
    } else if (i < NL) {
      const int wr = (i - NA) * 8 + lr;
      const uint16_t *w;
      int n;
      if (GATEUP) {  // 16-row groups alternate gate and up
        w = ((wr >> 4) & 1) ? a.w1 : a.w0;
        n = n0 + (wr >> 5) * 16 + (wr & 15);
      } else {
        w = a.w0;
        n = min(n0 + wr, a.N - 1);
      }
      src[j] = w + ((size_t)t.e * a.N + n) * K + lq * 8;
    }
  }
  constexpr int NS = GgRing<AB, WR>::kDepth;
  constexpr int SLOT = GgRing<AB, WR>::kSlot;
  // stage s of feature block b: weight rows move on by FEAT rows per block,
  // activation rows stay
  const size_t bstep = (size_t)FEAT * K;
  auto issue = [&](int s, int b, int slot) {
    const uint32_t base = ring_lds + (uint32_t)(slot * SLOT);
    const size_t woff = MB ? (size_t)b * bstep : 0;
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
      const int i = wv + kGgWaves * j;
      const uint16_t *p = src[j] + s * 64;
      if (MB && i >= NA) p += woff;
      if (NT && i >= NA) {
        if (i < NL) dma16_nt(p, base + (uint32_t)i * 1024u);
      } else if (i < NL) {
        dma16(p, base + (uint32_t)i * 1024u);
      }
    }
  };

  // reader: row (lane & 31) of a 32-row tile; reduction step ks (16 elements)
  // reads chunk 2 ks + (lane >> 5) of the row's eight, at its swizzled slot
  const int rr = lane & 31, rh = lane >> 5;
  int lane_off[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) lane_off[ks] = rr * 128 + ring_slot(rr, 2 * ks + rh) * 16;

  f32x16 acc[TW][TT];
  auto zero_acc = [&]() {
#pragma unroll
    for (int tw = 0; tw < TW; ++tw)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[tw][tt][j] = 0.f;
  };
  // register j of a 32x32 tile holds weight row 8*(j/4) + 4*rh + j%4, activation row rr
  auto epilogue = [&](int nb0) {
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int row = L::arow(wv, tt) + rr;
      if (row < t.nrows) {
#pragma unroll
        for (int tw = 0; tw < TW; ++tw) {
          const int wt = L::wtile(wv, tw);
          if (GATEUP) {
            // rows 0-15 of the tile are gate features 16 wt + [0,16), rows 16-31 the same up features
#pragma unroll
            for (int g = 0; g < 2; ++g) {
              const int n = nb0 + wt * 16 + g * 8 + rh * 4;
              gg_store<true>(a, t.row0 + row, n, quad(acc[tw][tt], g), quad(acc[tw][tt], g + 2));
            }
          } else {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int n = nb0 + wt * 32 + g * 8 + rh * 4;
              if (n < a.N) gg_store<false>(a, t.row0 + row, n, quad(acc[tw][tt], g), f32x4{});
            }
          }
        }
      }
    }
  };
  zero_acc();

  // the MFMAs of one ring stage
  auto mma_stage = [&](const uint8_t *buf) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (!L::active(wv)) break;
      bf16x8 fa[TT], fw[TW];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
        fa[tt] = *reinterpret_cast<const bf16x8 *>(buf + L::arow(wv, tt) * 128 + lane_off[ks]);
#pragma unroll
      for (int tw = 0; tw < TW; ++tw)
        fw[tw] = *reinterpret_cast<const bf16x8 *>(buf + L::wrow(wv, tw) * 128 + lane_off[ks]);
#pragma unroll
      for (int tw = 0; tw < TW; ++tw)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) acc[tw][tt] = mfma32_bf16(fw[tw], fa[tt], acc[tw][tt]);
    }
  };

  wait_vm(0);
  ring_barrier();  // every wave is done with the ring contents of the previous item
  if constexpr (!MB) {
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
      if (s < nst) issue(s, 0, s);
    int slot = 0;
    for (int s = 0; s < nst; ++s) {
      // this wave's loads of stage s are done; later stages may stay in flight
      wait_vm(cnt * min(NS - 2, nst - 1 - s));
      ring_barrier();  // stage s is in LDS for everyone; stage s - 1 is consumed
      const int ahead = s + NS - 1;
      if (ahead < nst) issue(ahead, 0, slot == 0 ? NS - 1 : slot - 1);
      mma_stage(ring + slot * SLOT);
      slot = slot == NS - 1 ? 0 : slot + 1;
    }
    if (L::active(wv)) epilogue(n0);
  } else {
    // nb feature blocks of nst stages each run through the ring back to
    // back; a block's results are written while the next block's first
    // stages load
    const int total = nb * nst;
    int ib = 0, is = 0;  // block and stage of the next stage to load
    auto issue_next = [&](int slot) {
      issue(is, ib, slot);
      if (++is == nst) {
        is = 0;
        ++ib;
      }
    };
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
      if (s < total) issue_next(s);
    int slot = 0, cb = 0, cs = 0;  // block and stage being multiplied
    for (int sg = 0; sg < total; ++sg) {
      // as above; stores of an earlier block, counted too, only make the
      // wait longer
      wait_vm(cnt * min(NS - 2, total - 1 - sg));
      ring_barrier();
      if (sg + NS - 1 < total) issue_next(slot == 0 ? NS - 1 : slot - 1);
      mma_stage(ring + slot * SLOT);
      slot = slot == NS - 1 ? 0 : slot + 1;
      if (++cs == nst) {
        if (L::active(wv)) epilogue(n0 + cb * FEAT);
        cs = 0;
        ++cb;
        if (cb < nb) zero_acc();
      }
    }
  }
}

template <bool GATEUP, int AB, int WR = kGgWRows>
__device__ __forceinline__ void gg_item_any(const GgArgs &a, const Tile &t, int n0, int nb,
                                            uint8_t *ring, uint32_t ring_lds) {
  // several feature blocks per item only for the down projection: the
  // block bookkeeping slowed the MFMA-bound gate/up items
  constexpr bool MB = !GATEUP;
  if (t.ablk & kTileStream)
    gg_item<GATEUP, true, MB, AB, WR>(a, t, n0, nb, ring, ring_lds);
  else
    gg_item<GATEUP, false, MB, AB, WR>(a, t, n0, nb, ring, ring_lds);
}

// ------------------------------------------------------------------ kernel

// The item order and shape of the bf16 persistent kernels: which tile and
// which output features item `it` covers.  Its state lives in vector
// registers (there is room there; the inputs go through vreg()), so that the
// compiler neither holds it nor values hoisted from it in the scalar
// registers while the workgroup multiplies, and only thread 0 decodes items.
template <bool GATEUP>
struct GgDispatch {
  int nbig, nsm, ptb, pts, ptt, FEATB, FEATS, FIB, FIS, nbb, nbs, items_big, items_mid, total, N,
      grid, wrb, wrs;
  __device__ __forceinline__ explicit GgDispatch(const GgArgs &a) {
    N = vreg(a.N);
    grid = vreg((int)gridDim.x);
    const int nsmall = vreg(*a.n_small);
    nbig = vreg(*a.ntiles) - nsmall;
    // weight rows per item of the taller tiles (wrb) and of the 32-row tiles
    // (wrs).  Left to the device (0), 32-row tiles take 128-row items when
    // there are no taller tiles (or few, below): on MI355X at 401 tokens (every expert under
    // 32 rows) gate/up 1.349 -> 1.313 ms and down 0.703 -> 0.687 ms, one
    // expert owner's share 0.348 -> 0.320 ms per step: twice the items to
    // balance, and a 20 KB stage leaves eight ring slots where a 36 KB one
    // leaves four.
    const int wr = vreg(a.wr);
    // Mixed lists narrow their 32-row tiles too while the tiles of experts
    // with several tiles are under an eighth of the list (2048 tokens:
    // 2.295 -> 2.267 ms per step); with many of those (8192 Zipf-routed
    // tokens) narrowing cost 4%, with few it changes nothing there.
    const bool narrow = wr == 0 && (nbig == 0 || vreg(*a.n_multi) * 8 < vreg(*a.ntiles));
    wrb = wr == 0 ? kGgWRows : wr;
    wrs = narrow ? kGgWRows / 2 : wrb;
    // output features per block: half the weight rows for gate/up (gate and
    // up rows of the same features), all of them for down
    FEATB = GATEUP ? wrb / 2 : wrb;
    FEATS = GATEUP ? wrs / 2 : wrs;
    // items of taller tiles first (the list is tallest first), then of the
    // 32-row tiles; the 32-row tiles take nb_skinny blocks per item when the
    // taller ones are at most an eighth as many (on MI355X, 4 blocks were
    // best there and 2 elsewhere, for 200 to 8192 tokens; narrowed items take
    // one block)
    const bool skinny = nbig * 8 <= nsmall;
    nbb = vreg(a.nb);
    nbs = narrow ? 1 : skinny ? vreg(a.nb_skinny) : nbb;
    // narrowed down items take four blocks while the 32-row tiles are fewer
    // than the workgroups (MI355X: one expert owner's share, 32 tiles, down
    // 0.106 -> 0.102 ms; 16 tokens 0.636 -> 0.619 ms, 32 tokens 1.054 ->
    // 1.037 ms per step); with a tile per workgroup or more one block is
    // best (401 tokens, 256 tiles: down 0.689 ms, 0.715 with two, 0.699 with
    // four); in mixed lists one block (2048 tokens: down 0.801 -> 0.793 ms)
    if (narrow && nbig == 0 && !GATEUP && nsmall < grid && N % (4 * FEATS) == 0) nbs = 4;
    // with few tiles, halve the blocks per item until at least half the
    // workgroups have an item: a workgroup of a half-idle chip streams faster
    // than its even share, so long items on half of them still pay (measured:
    // 11 experts 0.175 -> 0.123 ms with the halving, 43 experts 4% slower if
    // every workgroup had to get one).  Block counts above one divide the
    // feature blocks of a tile.
    const int ptb1 = (N + FEATB - 1) / FEATB;
    ptt = (N + FEATS - 1) / FEATS;  // one-block items of a 32-row tile
    while ((nbb > 1 || nbs > 1) && 2 * (nbig * (ptb1 / nbb) + nsmall * (ptt / nbs)) < grid) {
      if (nbs >= nbb)
        nbs >>= 1;
      else
        nbb >>= 1;
    }
    FIB = FEATB * nbb;  // output features per item
    FIS = FEATS * nbs;
    ptb = (N + FIB - 1) / FIB;
    pts = (N + FIS - 1) / FIS;
    // when (nearly) all tiles are 32-row ones, the last of them (about two
    // rounds of items) go out one block per item, so that the end of the
    // queue balances at a fine grain (MI355X: down 0.725 -> 0.705 ms at 401
    // tokens, -3% at 200 and 1024; with many taller tiles it did not help)
    const int ntail = (skinny && nbs > 1) ? min(nsmall, (2 * grid + ptt - 1) / ptt) : 0;
    nsm = nsmall - ntail;
    items_big = nbig * ptb;
    items_mid = items_big + nsm * pts;
    total = items_mid + ntail * ptt;
  }
  // tile index, first output feature, feature blocks and weight rows per
  // block of item it
  __device__ __forceinline__ void decode(int it, int *ti, int *n0, int *nb, int *wr) const {
    int nbw, feat;
    if (it < items_big) {
      *ti = it / ptb;
      *n0 = (it - *ti * ptb) * FIB;
      nbw = nbb;
      feat = FEATB;
      *wr = wrb;
    } else if (it < items_mid) {
      const int is = it - items_big;
      const int q = is / pts;
      *ti = nbig + q;
      *n0 = (is - q * pts) * FIS;
      nbw = nbs;
      feat = FEATS;
      *wr = wrs;
    } else {
      const int is = it - items_mid;
      const int q = is / ptt;
      *ti = nbig + nsm + q;
      *n0 = (is - q * ptt) * FEATS;
      nbw = 1;
      feat = FEATS;
      *wr = wrs;
    }
    *nb = min(nbw, (N - *n0 + feat - 1) / feat);
  }
};

template <bool GATEUP>
__global__ __launch_bounds__(kGgThreads, 1) void grouped_gemm_kernel(GgArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kGgRing];
  // the next item (tile index, first feature, blocks; tile -1 = none left)
  // is passed from thread 0 through the idle ring between items
  int *next_item = reinterpret_cast<int *>(ring);
  const uint32_t ring_lds = lds_addr(ring);
  // two queues (TwoQueue): the items of the first n_multi tiles, whose
  // experts have several tiles, and the rest.  A compute item counts as 1.5
  // stream items for gate/up and 2.25 for down: on MI355X, 8192 Zipf-routed
  // tokens, against one tallest-first queue, gate/up 1.94-1.99 -> 1.86 ms
  // (1 to 2.5 all helped, 1.5 best) and down 1.12-1.14 -> 1.05-1.07 ms (1:
  // 1.09, 1.5: 1.08-1.09, 2: 1.12, 2.25: 1.05-1.07, 2.5: 1.09, 3: 1.11 -- not
  // monotonic, so tuned to this workload); 401 and 2048 tokens unchanged.
  const GgDispatch<GATEUP> D(a);
  TwoQueue queue(vreg(*a.n_multi) * D.ptb, D.total, GATEUP ? MOE_SSW4_GU : MOE_SSW4_DN, D.grid);
  int next_static = vreg((int)blockIdx.x);
  for (;;) {
    if (threadIdx.x == 0) {
      int it;
      if (a.static_items) {
        it = min(next_static, D.total);
        next_static += D.grid;
      } else {
        it = queue.next(a.counter, a.counter_s);
      }
      int ti = -1, n0 = 0, nb = 0, wr = 0;
      if (it < D.total) {
        D.decode(it, &ti, &n0, &nb, &wr);
      }
      next_item[0] = ti;
      next_item[1] = n0;
      next_item[2] = nb;
      next_item[3] = a.K;
      next_item[4] = wr;
    }
    __syncthreads();
    // read before gg_item's first barrier (its loads overwrite it); uniform,
    // so the tile fetch below is a scalar load.  The reduction length also
    // comes through LDS: read from the kernel arguments, everything derived
    // from it was hoisted out of the loop and held in scalar registers for
    // the kernel's lifetime, more than fit.
    const int ti = __builtin_amdgcn_readfirstlane(next_item[0]);
    if (ti < 0) break;
    const int n0 = __builtin_amdgcn_readfirstlane(next_item[1]);
    const int nb = __builtin_amdgcn_readfirstlane(next_item[2]);
    GgArgs ai = a;
    ai.K = __builtin_amdgcn_readfirstlane(next_item[3]);
    const int wr = __builtin_amdgcn_readfirstlane(next_item[4]);
    const Tile t = a.tiles[ti];
    if (wr == 128) {
      gg_item_any<GATEUP, 1, 128>(ai, t, n0, nb, ring, ring_lds);
    } else if (wr == 64) {
      gg_item_any<GATEUP, 1, 64>(ai, t, n0, nb, ring, ring_lds);
    } else {
      switch (tile_class(t)) {
        case 8:
        case 6: gg_item_any<GATEUP, 8>(ai, t, n0, nb, ring, ring_lds); break;
        case 4: gg_item_any<GATEUP, 4>(ai, t, n0, nb, ring, ring_lds); break;
        case 2: gg_item_any<GATEUP, 2>(ai, t, n0, nb, ring, ring_lds); break;
        default: gg_item_any<GATEUP, 1>(ai, t, n0, nb, ring, ring_lds); break;
      }
    }
    // the ring (and the item in it) is rewritten only after every wave has
    // passed this barrier
    __syncthreads();
  }
}

// ------------------------------------------------------------------ host side

hipError_t launch_grouped_schedule(const int32_t *offsets, int E, Schedule *sch, Tile *tiles,
                                   hipStream_t stream) {
  hipLaunchKernelGGL(grouped_schedule_kernel, dim3(1), dim3(kGsThreads), 0, stream, offsets, E,
                     sch, tiles);
  return hipGetLastError();
}

// Weight rows per item.  With at most 32 routed rows in all (decode-sized
// chunks) every tile is a 32-row tile and items may be narrowed to 128 or 64
// weight rows: the weight stream then spreads over more CUs.  The choice
// minimises (rounds of items over the CUs) x (weight rows per item + 32),
// counting at most min(R, E) tiles; the 32 rows stand for an item's fixed
// cost (ring fill and queue round trip, ~4 us, measured) and ties go to the
// wider item.  With more rows the kernel chooses (0 here): 128 when every
// tile is a 32-row tile, else 256.  n_out: output features of the
// projection; mats: weight matrices interleaved in an item (2 for gate/up).
static int item_weight_rows(const FfnLaunch &L, int n_out, int mats) {
  if (L.R > 32) return 0;  // the kernel decides from the tile list
  const long long tiles = L.R < L.E ? L.R : L.E;
  const int cus = L.num_cus > 0 ? L.num_cus : 1;
  int best = kGgWRows;
  long long best_cost = -1;
  for (int wr = kGgWRows; wr >= 64; wr /= 2) {
    const long long per_tile = (n_out + wr / mats - 1) / (wr / mats);
    const long long rounds = (tiles * per_tile + cus - 1) / cus;
    const long long cost = rounds * (wr + 32);
    if (best_cost < 0 || cost < best_cost) {
      best = wr;
      best_cost = cost;
    }
  }
  return best;
}

// With at most 32 routed rows every tile is a 32-row tile and every item
// streams the same weight bytes, so a fixed assignment (item b, b + grid,
// ... to workgroup b) balances as well as the work queues and saves their
// atomics at the start and end of every workgroup.
static int static_items(const FfnLaunch &L) { return L.R <= 32 ? 1 : 0; }

// Feature blocks per item: more than one only for full-width items (narrow
// items exist to make more of them) and when the blocks tile the output
// features exactly.
static int item_blocks(int wr, int n_out, int mats, int want) {
  if (wr == 0) wr = kGgWRows;  // the blocks of full-width items (narrowed ones take one)
  const int feat = wr / mats;
  return (want > 1 && wr == kGgWRows && n_out % (feat * want) == 0) ? want : 1;
}

hipError_t launch_grouped_ffn_bf16(const FfnLaunch &L, int stages, hipStream_t stream) {
  if (stages & kStagePlan) {
    const hipError_t err = launch_grouped_schedule(L.offsets, L.E, L.sch, L.tiles, stream);
    if (err != hipSuccess) return err;
  }
  GgArgs g{};
  g.k = L.k;
  g.tiles = L.tiles;
  g.ntiles = &L.sch->n_tiles;
  g.n_small = &L.sch->n_small;
  g.n_multi = &L.sch->n_multi;
  if (stages & kStageGateUp) {
    g.act = L.x;
    g.sorted_routes = L.sorted_routes;
    g.w0 = L.wg;
    g.w1 = L.wu;
    g.out = L.h;
    g.N = L.f;
    g.K = L.d;
    g.counter = &L.sch->counter[0];
    g.counter_s = &L.sch->counter_s[0];
    g.wr = item_weight_rows(L, L.f, 2);
    g.nb = 1;
    g.nb_skinny = 1;
    g.static_items = static_items(L);
    hipLaunchKernelGGL(grouped_gemm_kernel<true>, dim3(L.num_cus), dim3(kGgThreads), 0, stream, g);
  }
  if (stages & kStageDown) {
    g.act = L.h;
    g.sorted_routes = nullptr;
    g.w0 = L.wd;
    g.w1 = nullptr;
    g.out = L.y;
    g.N = L.d;
    g.K = L.f;
    g.counter = &L.sch->counter[1];
    g.counter_s = &L.sch->counter_s[1];
    g.wr = item_weight_rows(L, L.d, 1);
    g.nb = item_blocks(g.wr, L.d, 1, 2);
    g.nb_skinny = item_blocks(g.wr, L.d, 1, 4);
    g.static_items = static_items(L);
    hipLaunchKernelGGL(grouped_gemm_kernel<false>, dim3(L.num_cus), dim3(kGgThreads), 0, stream,
                       g);
  }
  return hipGetLastError();
}

}  // namespace moe
