// Persistent grouped GEMM for the fp8 routed-MoE FFN: E4M3 weights with one
// fp32 scale per 128 x 128 block, E4M3 activations with one fp32 scale per
// row (x per token, h per routed row).
//
// Same tile list, two work queues and LDS stage ring as the bf16 kernels
// (ffn_grouped.hip, ring.h).  A ring row is 128 bytes = 128 fp8 reduction
// elements = one weight scale block, so each stage's partial product P (two
// chained 32x32x64 fp8 MFMAs from zero) is folded into the fp32 accumulator
// once: acc += s_w[n / 128][stage] * P.  The activation row scale is constant
// along the reduction and multiplies the accumulator in the epilogue.  Items
// carry 128 weight rows (gate/up: 64 features of both matrices, interleaved
// in 16-row groups; down: one to four blocks of 128 features streamed
// through one ring fill), which keeps the fold of a wave in proportion to
// its MFMAs; 192-row tiles have a layout of their own.  Between the
// projections h is written in bf16, the gate/up epilogue keeps each row's
// max |h| (atomicMax), and the down stage quantises h per row with it.
#include "kernels.h"
#include "ring.h"

namespace moe {

struct Gg8Args {
  const uint8_t *act;            // gate/up: qx [T, K]; down: qh [R, K]
  const float *act_scale;        // gate/up: sx [T]; down: sh [R]
  const int32_t *sorted_routes;  // gate/up: token of sorted row i is sorted_routes[i] / k
  int k;
  const uint8_t *w0, *w1;  // [E, N, K] codes: gate (or down), up
  const float *s0, *s1;    // [E, N / 128, K / 128] block scales of w0, w1
  void *out;               // gate/up: h bf16 [R, N]; down: y fp32 [R, N]
  int N, K;                // K <= 16384: a lane pair holds the K / 128 scales of a row
  const Tile *tiles;
  const int *ntiles;
  const int *n_multi;  // tiles of experts with several tiles, at the start of the list
  int *counter;        // compute-queue head (TwoQueue)
  int *counter_s;      // stream-queue head
  int nb;  // feature blocks per item (streamed through one ring fill)
  uint32_t *hmax;  // gate/up: [R] fp32 bits of max |h| per row, kept with atomicMax
};

constexpr int kG8Threads = 512;
constexpr int kG8MaxBlocks = 4;
constexpr int kG8Waves = kG8Threads / kWave;
constexpr int kG8WRows = 128;
constexpr int kG8Ring = 160 * 1024;

template <int AB>
struct G8Ring {
  static constexpr int kSlot = (32 * AB + kG8WRows) * 128;
  static constexpr int kDepth = (kG8Ring / kSlot) < 8 ? (kG8Ring / kSlot) : 8;
};

// Wave wv multiplies TT activation tiles by TW weight tiles (32 rows each).
// An item has 4 weight tiles and AB activation tiles; with AB = 1 only waves
// 0-3 have a pair (waves 4-7 still load).  AB = 6 (192-row tiles): each wave
// takes three activation tiles against one weight tile.
template <int AB>
struct G8Layout {
  static constexpr int TT = AB == 6 ? 3 : AB >= 4 ? 2 : 1;
  static constexpr int TW = AB == 8 ? 2 : 1;
  __device__ static bool active(int wv) { return AB > 1 || wv < 4; }
  __device__ static int atile(int wv, int tt) {
    return AB == 8   ? (wv >> 1) * 2 + tt
           : AB == 6 ? (wv >> 2) * 3 + tt
           : AB == 4 ? (wv >> 2) * 2 + tt
           : AB == 2 ? (wv >> 2)
                     : 0;
  }
  __device__ static int wtile(int wv, int tw) { return AB == 8 ? (wv & 1) * 2 + tw : (wv & 3); }
};

// 32x32x64 E4M3 x E4M3 MFMA with unit block exponents (E8M0 127 = 2^0).  Lane
// l supplies row l % 32 of its operand and 32 reduction elements; both
// operands are read with the same lane -> element map, so the sum covers the
// 64 elements of the step whatever order the unit takes them in.  Result
// layout as for the bf16 32x32 shape.
__device__ __forceinline__ f32x16 mfma32_fp8(const i32x8 &a, const i32x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x8 lds_i32x8(const uint8_t *p0, const uint8_t *p1) {
  const i32x4 lo = *reinterpret_cast<const i32x4 *>(p0);
  const i32x4 hi = *reinterpret_cast<const i32x4 *>(p1);
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ f32x4 quad_scaled(const f32x16 &v, int g, float s) {
  return f32x4{v[4 * g] * s, v[4 * g + 1] * s, v[4 * g + 2] * s, v[4 * g + 3] * s};
}

// Scale of reduction block s (uniform) from the pair (lo: block lane, hi:
// block 64 + lane) that the lanes of a wave hold.
__device__ __forceinline__ float block_scale(float lo, float hi, int s) {
  const float v = s < 64 ? lo : hi;
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), s & 63));
}

// NT: weight rows through non-temporal loads (tile flagged kTileStream).
// MB: the item may carry up to kG8MaxBlocks feature blocks (nb) of 128
// outputs; without it nb is 1 and the stage loop has no block bookkeeping.
template <bool GATEUP, bool NT, bool MB, int AB>
__device__ __forceinline__ void g8_item(const Gg8Args &a, const Tile &t, int n0, int nb_arg,
                                        uint8_t *ring, uint32_t ring_lds) {
  using L = G8Layout<AB>;
  constexpr int FEAT = GATEUP ? 64 : 128;  // output features per block
  constexpr int NB = MB ? kG8MaxBlocks : 1;
  const int nb = MB ? nb_arg : 1;
  constexpr int TT = L::TT, TW = L::TW;
  constexpr int NA = 4 * AB;             // activation loads (8 rows each) per stage
  constexpr int NL = NA + kG8WRows / 8;  // all loads per stage
  constexpr int MAXJ = (NL + kG8Waves - 1) / kG8Waves;
  constexpr int NS = G8Ring<AB>::kDepth;
  constexpr int SLOT = G8Ring<AB>::kSlot;
  const int lane = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int K = a.K;
  const int nst = K / 128;
  const int cnt = (NL - wv + kG8Waves - 1) / kG8Waves;  // loads this wave issues per stage

  // load i fills stage rows 8 i .. 8 i + 7; this lane fills slot (lane & 7)
  // of row 8 i + (lane >> 3) with the chunk that belongs there
  const int lr = lane >> 3;
  const uint8_t *src[MAXJ];
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    const int i = wv + kG8Waves * j;
    const int lq = ring_slot(i * 8 + lr, lane & 7);
    src[j] = a.act;
    if (i < NA) {
      const int row = t.row0 + min(i * 8 + lr, t.nrows - 1);
      const size_t s = GATEUP ? (size_t)(a.sorted_routes[row] / a.k) : (size_t)row;
      src[j] = a.act + s * K + lq * 16;
    } else if (i < NL) {
      const int wr = (i - NA) * 8 + lr;
      const uint8_t *w;
      int n;
      if (GATEUP) {  // 16-row groups alternate gate and up
        w = ((wr >> 4) & 1) ? a.w1 : a.w0;
        n = n0 + (wr >> 5) * 16 + (wr & 15);
      } else {
        w = a.w0;
        n = min(n0 + wr, a.N - 1);
      }
      src[j] = w + ((size_t)t.e * a.N + n) * K + lq * 16;
    }
  }
  // stage s of feature block b: weight rows move on by FEAT rows per block,
  // activation rows stay
  const size_t bstep = (size_t)FEAT * K;
  auto issue = [&](int s, int b, int slot) {
    const uint32_t base = ring_lds + (uint32_t)(slot * SLOT);
    const size_t woff = MB ? (size_t)b * bstep : 0;
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
      const int i = wv + kG8Waves * j;
      const uint8_t *p = src[j] + s * 128;
      if (MB && i >= NA) p += woff;
      if (NT && i >= NA) {
        if (i < NL) dma16_nt(p, base + (uint32_t)i * 1024u);
      } else if (i < NL) {
        dma16(p, base + (uint32_t)i * 1024u);
      }
    }
  };

  // Everything the item reads besides the ring is loaded here, before the
  // ring fill: a compiler-tracked load between stages would make the
  // compiler wait for every load in flight, the ring's included.
  // Block scales: each 128-row scale block of the item's weight rows (one per
  // feature block; gate/up items lie in one), the K / 128 scales of a row
  // held two per lane.
  const int KB = nst;
  float sc0[NB][2], sc1[2];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const size_t srow = ((size_t)t.e * (a.N / 128) + (n0 + b * FEAT) / 128) * KB;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kb = lane + 64 * h;
      sc0[b][h] = (b < nb && kb < KB) ? a.s0[srow + kb] : 0.f;
    }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int kb = lane + 64 * h;
    const size_t srow = ((size_t)t.e * (a.N / 128) + n0 / 128) * KB;
    sc1[h] = (GATEUP && kb < KB) ? a.s1[srow + kb] : 0.f;
  }
  // activation row scales of this lane's rows
  float rsc[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const int row = L::atile(wv, tt) * 32 + (lane & 31);
    const int i = t.row0 + min(row, t.nrows - 1);
    rsc[tt] = a.act_scale[GATEUP ? (size_t)(a.sorted_routes[i] / a.k) : (size_t)i];
  }

  // reader: row (lane & 31) of a 32-row tile; 64-element step ks takes the
  // 32 bytes of chunks 4 ks + 2 (lane >> 5) and 4 ks + 2 (lane >> 5) + 1
  const int rr = lane & 31, rh = lane >> 5;
  int off0[2], off1[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    off0[ks] = rr * 128 + ring_slot(rr, 4 * ks + 2 * rh) * 16;
    off1[ks] = rr * 128 + ring_slot(rr, 4 * ks + 2 * rh + 1) * 16;
  }

  f32x16 acc[TW][TT];
  auto zero_acc = [&]() {
#pragma unroll
    for (int tw = 0; tw < TW; ++tw)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[tw][tt][j] = 0.f;
  };
  zero_acc();
  const bool on = L::active(wv);

  // the MFMAs of stage s of a block whose weight scales are (lo, hi)
  auto mma_stage = [&](const uint8_t *buf, int s, float lo, float hi) {
    const float sg = block_scale(lo, hi, s);
    const float su = GATEUP ? block_scale(sc1[0], sc1[1], s) : sg;
    i32x8 fa[TT][2], fw[TW][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        const uint8_t *r = buf + L::atile(wv, tt) * 32 * 128;
        fa[tt][ks] = lds_i32x8(r + off0[ks], r + off1[ks]);
      }
#pragma unroll
      for (int tw = 0; tw < TW; ++tw) {
        const uint8_t *r = buf + (32 * AB + L::wtile(wv, tw) * 32) * 128;
        fw[tw][ks] = lds_i32x8(r + off0[ks], r + off1[ks]);
      }
    }
#pragma unroll
    for (int tw = 0; tw < TW; ++tw)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        f32x16 p;
#pragma unroll
        for (int j = 0; j < 16; ++j) p[j] = 0.f;
        p = mfma32_fp8(fw[tw][0], fa[tt][0], p);
        p = mfma32_fp8(fw[tw][1], fa[tt][1], p);
        // gate/up: registers 0-7 hold gate rows of the tile, 8-15 up rows
#pragma unroll
        for (int j = 0; j < 16; ++j)
          acc[tw][tt][j] = __builtin_fmaf((GATEUP && j >= 8) ? su : sg, p[j], acc[tw][tt][j]);
      }
  };

  // register j of a 32x32 tile holds weight row 8*(j/4) + 4*rh + j%4, activation row rr
  auto epilogue = [&](int nb0) {
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int row = L::atile(wv, tt) * 32 + rr;
      if (row < t.nrows) {
        const int i = t.row0 + row;
        const float rs = rsc[tt];
        uint32_t hm = 0;  // gate/up: max |h| of this lane's values of row i, as bf16 bits
#pragma unroll
        for (int tw = 0; tw < TW; ++tw) {
          const int wt = L::wtile(wv, tw);
          if (GATEUP) {
            // rows 0-15 of the tile are gate features 16 wt + [0,16), rows 16-31 the same up features
#pragma unroll
            for (int g = 0; g < 2; ++g) {
              const f32x4 gv = quad_scaled(acc[tw][tt], g, rs);
              const f32x4 uv = quad_scaled(acc[tw][tt], g + 2, rs);
              uint32_t hb[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                hb[e] = f32_to_bf16_bits(swiglu(gv[e], uv[e]));
                const uint32_t ab = hb[e] & 0x7fffu;
                hm = ab <= 0x7f80u && ab > hm ? ab : hm;  // NaN left out
              }
              uint2 v;
              v.x = hb[0] | (hb[1] << 16);
              v.y = hb[2] | (hb[3] << 16);
              const int n = nb0 + wt * 16 + g * 8 + rh * 4;
              *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + (size_t)i * a.N + n) = v;
            }
          } else {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int n = nb0 + wt * 32 + g * 8 + rh * 4;
              if (n < a.N)
                *reinterpret_cast<f32x4 *>(static_cast<float *>(a.out) + (size_t)i * a.N + n) =
                    quad_scaled(acc[tw][tt], g, rs);
            }
          }
        }
        if (GATEUP) {
          // the row's maximum over this wave: lanes rr and rr + 32 hold the
          // same row; one atomic per row and wave (fp32 bits of a
          // non-negative value order like the values)
          const uint32_t other = (uint32_t)__shfl_xor((int)hm, 32);
          hm = other > hm ? other : hm;
          if (rh == 0) atomicMax(a.hmax + i, hm << 16);
        }
      }
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
      wait_vm(cnt * min(NS - 2, nst - 1 - s));
      ring_barrier();  // stage s is in LDS for everyone; stage s - 1 is consumed
      const int ahead = s + NS - 1;
      if (ahead < nst) issue(ahead, 0, slot == 0 ? NS - 1 : slot - 1);
      if (on) mma_stage(ring + slot * SLOT, s, sc0[0][0], sc0[0][1]);
      slot = slot == NS - 1 ? 0 : slot + 1;
    }
    if (on) epilogue(n0);
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
    float lo = sc0[0][0], hi = sc0[0][1];
    for (int sg = 0; sg < total; ++sg) {
      // as above; stores of an earlier block, counted too, only make the
      // wait longer
      wait_vm(cnt * min(NS - 2, total - 1 - sg));
      ring_barrier();
      if (sg + NS - 1 < total) issue_next(slot == 0 ? NS - 1 : slot - 1);
      if (on) mma_stage(ring + slot * SLOT, cs, lo, hi);
      slot = slot == NS - 1 ? 0 : slot + 1;
      if (++cs == nst) {
        if (on) epilogue(n0 + cb * FEAT);
        cs = 0;
        ++cb;
        if (cb < nb) {
          zero_acc();
#pragma unroll
          for (int b = 1; b < NB; ++b)
            if (b == cb) {
              lo = sc0[b][0];
              hi = sc0[b][1];
            }
        }
      }
    }
  }
}

template <bool GATEUP, int AB>
__device__ __forceinline__ void g8_item_any(const Gg8Args &a, const Tile &t, int n0, int nb,
                                            uint8_t *ring, uint32_t ring_lds) {
  // several feature blocks per item only for the down projection
  constexpr bool MB = !GATEUP;
  if (t.ablk & kTileStream)
    g8_item<GATEUP, true, MB, AB>(a, t, n0, nb, ring, ring_lds);
  else
    g8_item<GATEUP, false, MB, AB>(a, t, n0, nb, ring, ring_lds);
}

template <bool GATEUP>
__global__ __launch_bounds__(kG8Threads, 1) void grouped_gemm8_kernel(Gg8Args a) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kG8Ring];
  // the next item (tile index, first feature, blocks, reduction length; tile
  // -1 = none left) is passed from thread 0 through the idle ring between
  // items
  int *next_item = reinterpret_cast<int *>(ring);
  const uint32_t ring_lds = lds_addr(ring);
  constexpr int FEAT = GATEUP ? 64 : 128;  // output features per block
  // The dispatch state is built from vreg() values (common.h): it stays in
  // vector registers and nothing derived from it is hoisted into the scalar
  // registers the item loop needs.
  // blocks per item: halved while fewer than half the workgroups would get
  // an item (counts above one divide the feature blocks of a tile)
  const int N = vreg(a.N), grid = vreg((int)gridDim.x);
  const int ntiles = vreg(*a.ntiles);
  const int pt1 = (N + FEAT - 1) / FEAT;
  int nbi = vreg(a.nb);
  while (nbi > 1 && 2 * ntiles * (pt1 / nbi) < grid) nbi >>= 1;
  const int FI = FEAT * nbi;  // output features per item
  const int per_tile = (N + FI - 1) / FI;
  const int total = ntiles * per_tile;
  // two queues (TwoQueue): the items of the first n_multi tiles, whose
  // experts have several tiles, and the rest (a compute item weighed as in
  // the bf16 kernels)
  TwoQueue queue(vreg(*a.n_multi) * per_tile, total, GATEUP ? 6 : 9, grid);
  for (;;) {
    if (threadIdx.x == 0) {
      const int it = queue.next(a.counter, a.counter_s);
      int ti = -1, n0 = 0, nb = 0;
      if (it < total) {
        ti = it / per_tile;
        n0 = (it - ti * per_tile) * FI;
        nb = min(nbi, (N - n0 + FEAT - 1) / FEAT);
      }
      next_item[0] = ti;
      next_item[1] = n0;
      next_item[2] = nb;
      next_item[3] = a.K;
    }
    __syncthreads();
    // read before g8_item's first barrier (its loads overwrite it); the
    // reduction length comes through LDS so that nothing derived from it is
    // hoisted out of the loop into the scalar registers
    const int ti = __builtin_amdgcn_readfirstlane(next_item[0]);
    if (ti < 0) break;
    const int n0 = __builtin_amdgcn_readfirstlane(next_item[1]);
    const int nb = __builtin_amdgcn_readfirstlane(next_item[2]);
    Gg8Args ai = a;
    ai.K = __builtin_amdgcn_readfirstlane(next_item[3]);
    const Tile t = a.tiles[ti];
    switch (tile_class(t)) {
      case 8: g8_item_any<GATEUP, 8>(ai, t, n0, nb, ring, ring_lds); break;
      case 6: g8_item_any<GATEUP, 6>(ai, t, n0, nb, ring, ring_lds); break;
      case 4: g8_item_any<GATEUP, 4>(ai, t, n0, nb, ring, ring_lds); break;
      case 2: g8_item_any<GATEUP, 2>(ai, t, n0, nb, ring, ring_lds); break;
      default: g8_item_any<GATEUP, 1>(ai, t, n0, nb, ring, ring_lds); break;
    }
    // the ring (and the item in it) is rewritten only after every wave has
    // passed this barrier
    __syncthreads();
  }
}

hipError_t launch_ffn_fp8(const FfnLaunchFp8 &L, int stages, hipStream_t stream) {
  hipError_t err = hipSuccess;
  if (stages & kStagePlan) {
    err = launch_grouped_schedule(L.offsets, L.E, L.sch, L.tiles, stream);
    if (err != hipSuccess) return err;
    err = launch_quant_rows(L.x, L.T, nullptr, L.d, L.qx, L.sx, L.grid_cap, stream);
    if (err != hipSuccess) return err;
    err = launch_zero_u32(L.hmax, L.R, stream);  // the gate/up epilogue maxes into it
    if (err != hipSuccess) return err;
  }
  Gg8Args g{};
  g.k = L.k;
  g.tiles = L.tiles;
  g.ntiles = &L.sch->n_tiles;
  g.n_multi = &L.sch->n_multi;
  if (stages & kStageGateUp) {
    g.act = L.qx;
    g.act_scale = L.sx;
    g.sorted_routes = L.sorted_routes;
    g.w0 = L.wg;
    g.w1 = L.wu;
    g.s0 = L.sg;
    g.s1 = L.su;
    g.out = L.h;
    g.N = L.f;
    g.K = L.d;
    g.counter = &L.sch->counter[0];
    g.counter_s = &L.sch->counter_s[0];
    g.nb = 1;
    g.hmax = L.hmax;
    hipLaunchKernelGGL(grouped_gemm8_kernel<true>, dim3(L.num_cus), dim3(kG8Threads), 0, stream,
                       g);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (stages & kStageDown) {
    // h -> per-row E4M3 with the row maxima the gate/up epilogue kept; the
    // active row count is offsets[E]
    err = launch_quant_rows_known_max(L.h, L.R, L.offsets + L.E, L.f, L.hmax, L.qh, L.sh,
                                      L.grid_cap, stream);
    if (err != hipSuccess) return err;
    g.hmax = nullptr;
    g.act = L.qh;
    g.act_scale = L.sh;
    g.sorted_routes = nullptr;
    g.w0 = L.wd;
    g.w1 = nullptr;
    g.s0 = L.sd;
    g.s1 = nullptr;
    g.out = L.y;
    g.N = L.d;
    g.K = L.f;
    g.counter = &L.sch->counter[1];
    g.counter_s = &L.sch->counter_s[1];
    // the most blocks of 128 outputs, up to kG8MaxBlocks, that tile d
    // (MI355X, 8192 tokens: down 0.946 -> 0.877 ms with four, 0.884 with two)
    g.nb = kG8MaxBlocks;
    while (g.nb > 1 && L.d % (128 * g.nb) != 0) g.nb >>= 1;
    hipLaunchKernelGGL(grouped_gemm8_kernel<false>, dim3(L.num_cus), dim3(kG8Threads), 0, stream,
                       g);
  }
  return hipGetLastError();
}

}  // namespace moe
