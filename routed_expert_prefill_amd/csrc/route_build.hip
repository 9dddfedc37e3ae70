// Route histogram, prefix and stable scatter for up to 256 experts
// ("perf(ds4): batch heterogeneous MoE prefill by expert", Summary).
//
// Up to 5120 routes: one workgroup does all three steps (rb_fused_kernel).
// Beyond that, two launches over chunks of kChunk routes:
//   1. per-chunk histogram in LDS (integer atomics: order-independent);
//   2. per-chunk stable scatter.  Each workgroup first forms, from all the
//      chunk histograms, the bin totals, their exclusive prefix (the
//      offsets) and the counts of its bins in the chunks before its own, so
//      no launch between the two scans the histograms; then each wave walks
//      its routes 64 at a time in route order, finds equal keys among the 64
//      lanes with one ballot per key bit, and ranks each lane among its
//      earlier peers.
// Results are integers and do not depend on scheduling.
#include <mutex>

#include "kernels.h"

namespace moe {

constexpr int kRbThreads = 256;
constexpr int kRbWaves = kRbThreads / kWave;
// Measured on MI355X (route build alone, uniform routing over 256 experts,
// calls back to back): the one-workgroup path takes 11 us up to ~4k
// routes, 14 us at 6,144, 19 us at 8,196 and 25 us at 12,288; the chunked
// path in two launches 13-14 us from 6 to 49k routes (1,024-route chunks:
// 512 are ~1 us slower at 49k, 2,048 equal or slower).  The crossing lies
// between 4,098 routes (one workgroup 2.4 us faster) and 6,144 (0.5 us
// slower).
#ifndef MOE_RB_CHUNK
#define MOE_RB_CHUNK 1024
#endif
#ifndef MOE_RB_FUSED_MAX
#define MOE_RB_FUSED_MAX 5120
#endif
constexpr int kChunk = MOE_RB_CHUNK;  // routes per workgroup
constexpr int kMaxBins = 257; // E + 1 with E <= 256

__device__ __forceinline__ int route_key(const int32_t *ids, const uint8_t *mask, int r, int E) {
  const int e = ids[r];
  const bool act = (mask == nullptr || mask[r] != 0) && (unsigned)e < (unsigned)E;
  return act ? e : E;
}

__global__ __launch_bounds__(kRbThreads) void rb_hist_kernel(const int32_t *__restrict__ ids,
                                                             const uint8_t *__restrict__ mask,
                                                             int R, int E,
                                                             int32_t *__restrict__ chunk_hist) {
  __shared__ int h[kMaxBins];
  for (int b = threadIdx.x; b <= E; b += kRbThreads) h[b] = 0;
  __syncthreads();
  const int base = blockIdx.x * kChunk;
  for (int i = threadIdx.x; i < kChunk; i += kRbThreads) {
    const int r = base + i;
    if (r < R) atomicAdd(&h[route_key(ids, mask, r, E)], 1);
  }
  __syncthreads();
  for (int b = threadIdx.x; b <= E; b += kRbThreads) chunk_hist[(size_t)blockIdx.x * (E + 1) + b] = h[b];
}

// Exclusive prefix of v over the threads of the workgroup; *total = the sum.
__device__ __forceinline__ int rb_block_scan(int v, int *total, int *wave_sums) {
  const int lane = lane_id(), w = threadIdx.x / kWave;
  int x = v;
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  if (lane == kWave - 1) wave_sums[w] = x;
  __syncthreads();
  int before = 0, all = 0;
  for (int i = 0; i < kRbWaves; ++i) {
    const int s = wave_sums[i];
    before += i < w ? s : 0;
    all += s;
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

__global__ __launch_bounds__(kRbThreads) void rb_scatter_kernel(const int32_t *__restrict__ ids,
                                                                const uint8_t *__restrict__ mask,
                                                                int R, int E, int key_bits,
                                                                int nchunks,
                                                                const int32_t *__restrict__ chunk_hist,
                                                                int32_t *__restrict__ counts,
                                                                int32_t *__restrict__ offsets,
                                                                int32_t *__restrict__ sorted_routes,
                                                                int32_t *__restrict__ route_rows) {
  __shared__ int cnt[kRbWaves][kMaxBins];
  __shared__ int chunk_start[kMaxBins];  // bin b's first row for this chunk
  __shared__ int wave_sums[kRbWaves];
  const int w = threadIdx.x / kWave;
  const int lane = lane_id();
  for (int i = threadIdx.x; i < kRbWaves * kMaxBins; i += kRbThreads) (&cnt[0][0])[i] = 0;

  // bin totals over all chunks and the counts in the chunks before this
  // one; thread t holds bins t and (for E = 256) t + 256, and the exclusive
  // prefix of the totals is one scan over the threads of their pairs' sums
  int tot[2] = {0, 0}, before[2] = {0, 0};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int b = threadIdx.x + h * kRbThreads;
    if (b <= E) {
      // eight chunks at a time: their counts load together
      constexpr int U = 8;
      for (int c0 = 0; c0 < nchunks; c0 += U) {
        int v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
          v[u] = c0 + u < nchunks ? chunk_hist[(size_t)(c0 + u) * (E + 1) + b] : 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          tot[h] += v[u];
          before[h] += c0 + u < (int)blockIdx.x ? v[u] : 0;
        }
      }
    }
  }
  // bins 0..255 in thread order, bin 256 after all of them
  int all;
  const int excl = rb_block_scan(tot[0], &all, wave_sums);
  if (threadIdx.x <= E) chunk_start[threadIdx.x] = excl + before[0];
  if (threadIdx.x == 0 && E >= kRbThreads) chunk_start[kRbThreads] = all + before[1];
  if (blockIdx.x == 0) {
    if (threadIdx.x <= E) {
      counts[threadIdx.x] = tot[0];
      offsets[threadIdx.x] = excl;
    }
    if (threadIdx.x == 0) {
      if (E >= kRbThreads) {
        counts[kRbThreads] = tot[1];
        offsets[kRbThreads] = all;
      }
      offsets[E + 1] = R;
    }
  }
  __syncthreads();

  constexpr int kPerWave = kChunk / kRbWaves;
  const int wbase = blockIdx.x * kChunk + w * kPerWave;

  // pass 1: per-wave key counts
  for (int g = 0; g < kPerWave; g += kWave) {
    const int r = wbase + g + lane;
    if (r < R) atomicAdd(&cnt[w][route_key(ids, mask, r, E)], 1);
  }
  __syncthreads();
  // per bin: the chunk's base plus the counts of the earlier waves
  for (int b = threadIdx.x; b <= E; b += kRbThreads) {
    int s = chunk_start[b];
    for (int v = 0; v < kRbWaves; ++v) {
      const int c = cnt[v][b];
      cnt[v][b] = s;
      s += c;
    }
  }
  __syncthreads();

  // pass 2: ordered placement, 64 routes at a time
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int g = 0; g < kPerWave; g += kWave) {
    const int r = wbase + g + lane;
    const bool valid = r < R;
    const int key = valid ? route_key(ids, mask, r, E) : 0;
    uint64_t peers = __ballot(valid);
    for (int bit = 0; bit < key_bits; ++bit) {
      const bool set = (key >> bit) & 1;
      const uint64_t m = __ballot(set);
      peers &= set ? m : ~m;
    }
    const int rank = __popcll(peers & below);
    int pos = 0;
    if (valid) pos = cnt[w][key] + rank;
    __builtin_amdgcn_wave_barrier();
    if (valid && rank == 0) cnt[w][key] = pos + __popcll(peers);
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      sorted_routes[pos] = r;
      route_rows[r] = pos;
    }
  }
}

// ------------------------------------------------------------------ small R

// Up to kFusedMaxR routes: the same three steps in one workgroup, without the
// two extra launches.  The histogram is one pass of LDS atomics; the scatter
// walks the routes in order, 1024 at a time (64 per wave), and ranks each
// lane among equal keys of its wave (ballots) and of the earlier waves
// (per-wave counts in LDS) on top of the bin's running base.
constexpr int kFusedThreads = 1024;
constexpr int kFusedWaves = kFusedThreads / kWave;
constexpr int kFusedMaxR = MOE_RB_FUSED_MAX;

__global__ __launch_bounds__(kFusedThreads) void rb_fused_kernel(
    const int32_t *__restrict__ ids, const uint8_t *__restrict__ mask, int R, int E, int key_bits,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_routes,
    int32_t *__restrict__ route_rows) {
  __shared__ int base[kMaxBins];  // histogram, then the running start of each bin
  __shared__ int scan[kFusedThreads];
  __shared__ int cnt[kFusedWaves][kMaxBins];
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int lane = lane_id();
  if (tid <= E) base[tid] = 0;
  __syncthreads();
  for (int r = tid; r < R; r += kFusedThreads) atomicAdd(&base[route_key(ids, mask, r, E)], 1);
  __syncthreads();
  // exclusive prefix over the E + 1 bins (inclusive Hillis-Steele, shifted)
  const int c = tid <= E ? base[tid] : 0;
  scan[tid] = c;
  __syncthreads();
  for (int off = 1; off < kFusedThreads; off <<= 1) {
    const int v = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  const int excl = scan[tid] - c;
  if (tid <= E) {
    counts[tid] = c;
    base[tid] = excl;
  }
  if (tid <= E + 1) offsets[tid] = excl;  // offsets[E + 1] = R
  __syncthreads();

  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int r0 = 0; r0 < R; r0 += kFusedThreads) {
    for (int i = tid; i < kFusedWaves * kMaxBins; i += kFusedThreads) (&cnt[0][0])[i] = 0;
    __syncthreads();
    const int r = r0 + tid;
    const bool valid = r < R;
    const int key = valid ? route_key(ids, mask, r, E) : 0;
    uint64_t peers = __ballot(valid);
    for (int bit = 0; bit < key_bits; ++bit) {
      const bool set = (key >> bit) & 1;
      const uint64_t m = __ballot(set);
      peers &= set ? m : ~m;
    }
    const int rank = __popcll(peers & below);
    if (valid && rank == 0) cnt[w][key] = __popcll(peers);
    __syncthreads();
    // per bin: the running start plus the counts of the earlier waves
    if (tid <= E) {
      int s = base[tid];
      for (int v = 0; v < kFusedWaves; ++v) {
        const int n = cnt[v][tid];
        cnt[v][tid] = s;
        s += n;
      }
      base[tid] = s;
    }
    __syncthreads();
    if (valid) {
      const int pos = cnt[w][key] + rank;
      sorted_routes[pos] = r;
      route_rows[r] = pos;
    }
    __syncthreads();
  }
}

int route_chunks(int R) { return (R + kChunk - 1) / kChunk; }

hipError_t launch_route_build(const int32_t *ids, const uint8_t *mask, int R, int E,
                              int32_t *counts, int32_t *offsets, int32_t *sorted_routes,
                              int32_t *route_rows, int32_t *ws, hipStream_t stream) {
  const int nchunks = route_chunks(R);
  int32_t *chunk_hist = ws;
  int key_bits = 1;
  while ((1 << key_bits) < E + 1) ++key_bits;
  if (R <= kFusedMaxR) {
    hipLaunchKernelGGL(rb_fused_kernel, dim3(1), dim3(kFusedThreads), 0, stream, ids, mask, R, E,
                       key_bits, counts, offsets, sorted_routes, route_rows);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(rb_hist_kernel, dim3(nchunks), dim3(kRbThreads), 0, stream, ids, mask, R, E,
                     chunk_hist);
  hipLaunchKernelGGL(rb_scatter_kernel, dim3(nchunks), dim3(kRbThreads), 0, stream, ids, mask, R,
                     E, key_bits, nchunks, chunk_hist, counts, offsets, sorted_routes, route_rows);
  return hipGetLastError();
}

size_t route_build_ws_bytes(int R, int E) {
  return (size_t)route_chunks(R) * (E + 1) * sizeof(int32_t);
}

// ------------------------------------------------------------------ no allocation

// The route build for callers that cannot allocate: the chunk histograms
// live in this file-scope device array instead of a caller's workspace.
// Each GPU holds its own copy until the process ends; every call on a GPU
// uses that GPU's copy.  Every word the kernels read there is written
// earlier in the same call (the histogram launch, then the scatter reads),
// so nothing has to be cleared between calls; calls that overlap on one GPU
// race.
static __device__ __align__(256) int32_t scratch[(kRouteNoAllocMaxR / kChunk) * kMaxBins];
static_assert(kRouteNoAllocMaxR % kChunk == 0, "whole chunks");
static_assert(sizeof(scratch) >= (kRouteNoAllocMaxR / kChunk) * (size_t)kMaxBins * 4,
              "room for the chunk histograms of the largest call");

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
int32_t *scratch_dev[kMaxDevices];  // device address of `scratch` on each device, once looked up
}  // namespace

hipError_t route_build_scratch(int32_t **ptr) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_dev[dev] == nullptr) {
    // the host-side name `scratch` is not a device address: look the
    // device's copy up once, with that device current
    void *p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    scratch_dev[dev] = static_cast<int32_t *>(p);
  }
  *ptr = scratch_dev[dev];
  return hipSuccess;
}

hipError_t launch_route_build_noalloc(const int32_t *ids, const uint8_t *mask, int R, int E,
                                      int32_t *counts, int32_t *offsets, int32_t *sorted_routes,
                                      int32_t *route_rows, hipStream_t stream) {
  if (R > kRouteNoAllocMaxR) return hipErrorInvalidValue;  // the caller checks first
  int32_t *ws = nullptr;
  const hipError_t err = route_build_scratch(&ws);
  if (err != hipSuccess) return err;
  return launch_route_build(ids, mask, R, E, counts, offsets, sorted_routes, route_rows, ws,
                            stream);
}

}  // namespace moe
