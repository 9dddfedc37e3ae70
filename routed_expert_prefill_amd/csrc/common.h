// Internal definitions shared by the gfx950 kernels of the routed-MoE library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// v as an opaque vector-register value.  Loop-invariant bookkeeping of the
// persistent kernels (work dispatch) is built from such values: the
// compiler can then neither keep it nor anything it hoists from it in the
// scalar registers, which the inner loops need, and there is room for it in
// the vector registers.
__device__ __forceinline__ int vreg(int v) {
  asm("" : "+v"(v));
  return v;
}

// One row tile of one expert: rows [row0, row0 + nrows) of the expert-sorted
// route order all belong to expert e.  ablk = row capacity / 32 (1, 2, 4, 6
// or 8): an expert's segment is cut into full tiles of kTileRows rows and one
// remainder tile of the smallest capacity (32, 64, 128, 192 or 256) that
// holds it.  Kernels without a 192-row layout run class 6 as class 8.
struct Tile {
  int e;
  int row0;
  int nrows;
  int ablk;  // row capacity / 32 in the low byte, kTileStream flag above it
};

constexpr int kTileRows = 256;

// Set on the only tile of an expert with at most kTileRows rows: its weights
// are read by that tile's items alone, so they go through non-temporal loads
// and leave the caches to the activation rows, which every item re-reads.
// Experts with several tiles keep the default policy (their weights are
// re-read once per tile).
constexpr int kTileStream = 0x100;
__device__ __forceinline__ int tile_class(const Tile &t) { return t.ablk & 0xff; }

// Layout of the schedule at the start of the grouped-FFN workspace.
struct Schedule {
  int n_tiles;     // entries of the tile list, tallest capacity first
  int counter[2];  // work-queue heads of the gate/up and down kernels
  int n_small;     // 32-row tiles, the last n_small entries of the list
  int n_multi;     // tiles of experts with more than kTileRows rows, the first n_multi entries
  int counter_s[2];  // second queue heads (items of the other tiles) of the two kernels
  int pad[57];     // keeps the tile list 256-byte aligned
};
static_assert(sizeof(Schedule) == 256, "the tile list follows the schedule at 256 bytes");

// Work dispatch of the persistent grouped-GEMM kernels from two queues:
// items [0, nc) belong to experts with several 256-row tiles (compute-bound:
// their weights serve every tile) and items [nc, total) to all other tiles
// (each expert's weights read once: memory-bound streams, tallest first).
// The first ps workgroups start on the streams and the others on the compute
// items; each switches to the other queue when its own runs dry, so the
// weight streams run beside the matrix work instead of after it.  ps is the
// streams' share of the work, counting a compute item as weight4 / 4 stream
// items, between 1/16 and 1/2 of the grid.  Used by thread 0 of a workgroup
// only.  Both members are forced inline: as calls they kept the object in
// the private segment (scratch memory) and made the caller save registers.
//
// A workgroup never draws again from a queue that has once come back empty
// (its head only grows), and it stops when both have.  Every workgroup of
// the grid therefore draws exactly once past the end of each queue, each
// head ends at its item count + G, and the workgroup whose draw returns that
// value - 1 made the head's last access of the launch: it sets the head back
// to 0, so the same stage can run again on the same schedule with no
// arrival count or fence at the end of the kernel.  All G workgroups must
// draw until next() returns the end.
struct TwoQueue {
  int nc, ns, G;
  int src;  // 0 = compute queue, 1 = stream queue
  int dry;  // bit q set: queue q came back empty
  __device__ __forceinline__ TwoQueue(int nc_, int total, int weight4, int G_)
      : nc(nc_), ns(total - nc_), G(G_), dry(0) {
    const int ps =
        nc == 0 ? G
                : max(G / 16, min(G / 2, (int)((long long)G * 4 * ns /
                                                (4LL * ns + (long long)weight4 * nc))));
    src = vreg((int)blockIdx.x) < ps ? 1 : 0;
  }
  // the next item, or nc + ns when both queues are empty
  __device__ __forceinline__ int next(int *compute_head, int *stream_head) {
    for (int tries = 0; tries < 2; ++tries) {
      if (!((dry >> src) & 1)) {
        int *head = src ? stream_head : compute_head;
        const int n = src ? ns : nc;
        const int q = atomicAdd(head, 1);
        if (q < n) return src ? nc + q : q;
        if (q == n + G - 1) __hip_atomic_store(head, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        dry |= 1 << src;
      }
      src ^= 1;
    }
    return nc + ns;
  }
};

// 16x16x32 bf16 MFMA, fp32 accumulate.  Operand lane layout (gfx950): lane l
// supplies row (l % 16) of its operand and the 8 consecutive reduction
// indices 8*(l/16) .. 8*(l/16)+7; lane l receives D[4*(l/16) + r][l % 16],
// r = 0..3, where the first operand indexes D's rows.
__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 32x32x16 bf16 MFMA, fp32 accumulate.  Lane l supplies row (l % 32) of its
// operand and reduction indices 8*(l/32) .. 8*(l/32)+7; register j of lane l
// receives D[8*(j/4) + 4*(l/32) + j%4][l % 32].  On gfx950 this shape runs at
// the full bf16 rate; the 16x16x32 shape issues at half of it.
__device__ __forceinline__ f32x16 mfma32_bf16(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16x16x128 E4M3 x E4M3 MFMA with unit block exponents (E8M0 127 = 2^0).
// Each lane supplies 32 consecutive reduction indices 32*(l/16) .. +31 of
// row (l % 16); the result layout is the bf16 one.
__device__ __forceinline__ f32x4 mfma_fp8(const i32x8 &a, const i32x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
  uint32_t b = __float_as_uint(v);
  if ((b & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((b >> 16) | 0x40u);
  b += 0x7fffu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// silu(g) * u in fp32.
__device__ __forceinline__ float swiglu(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

__device__ __forceinline__ bf16x8 load_bf16x8(const void *p) {
  return *reinterpret_cast<const bf16x8 *>(p);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

}  // namespace moe
