// Per-row E4M3 quantisation of bf16 activations with one fp32 scale per row.
//
//   s = fp32(max|v|) / 448,  q = e4m3_rne_saturate(v / s)   (IEEE fp32 division)
//   an all-zero row gets s = 1 and q = 0.
//
// E4M3 is the OCP E4M3FN format (bias 7, 3 mantissa bits, no infinities,
// largest finite 448).  The pages define none of their own low-bit formats;
// this is the format gfx950's fp8 MFMA consumes.
//
// Rows of up to 4096 elements: one wave per row; longer rows (up to
// kQMaxCols): one workgroup per row.  Either way a row is read once into
// registers, reduced, then encoded and written.
#include "kernels.h"

namespace moe {

// fp32 -> E4M3FN code, round to nearest even, saturating |v| >= 448 to 448,
// sign of zero kept, NaN -> 0x7f.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t a = b & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;
  if (a >= 0x43e00000u) return sign | 0x7eu;  // 448.0f
  if (a >= 0x3c800000u) {                     // 2^-6: normal E4M3 range
    uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);  // RNE at the 4th significant bit
    r >>= 20;                                      // (exp32 << 3) | mantissa3
    return sign | (r - (120u << 3));               // rebias 127 -> 7
  }
  // subnormal range: multiples of 2^-9 (8 * 2^-9 = 2^-6 encodes as 0x08)
  const float s = __uint_as_float(a) * 512.0f;
  return sign | (uint32_t)__builtin_rintf(s);
}

constexpr int kQThreads = 256;
constexpr int kQPer = 16;  // bf16 elements per thread per pass
constexpr int kQMaxPass = 4;
constexpr int kQMaxCols = kQThreads * kQPer * kQMaxPass;  // 16384

// rows_dev: if non-null the row count is read from device memory (the active
// sorted rows of the grouped FFN); rows beyond it are skipped.
__global__ __launch_bounds__(kQThreads) void quant_rows_kernel(const uint16_t *__restrict__ x,
                                                               int rows, const int32_t *rows_dev,
                                                               int cols, uint8_t *__restrict__ q,
                                                               float *__restrict__ s) {
  __shared__ float red[kQThreads / kWave];
  const int nrows = rows_dev ? *rows_dev : rows;
  const int tid = threadIdx.x;
  const int npass = (cols + kQThreads * kQPer - 1) / (kQThreads * kQPer);
  for (int row = blockIdx.x; row < nrows; row += gridDim.x) {
    const uint16_t *src = x + (size_t)row * cols;
    i32x4 raw[kQMaxPass][2];
    float amax = 0.0f;
#pragma unroll
    for (int p = 0; p < kQMaxPass; ++p) {
      const int c = (p * kQThreads + tid) * kQPer;
      if (p < npass && c < cols) {
        raw[p][0] = *reinterpret_cast<const i32x4 *>(src + c);
        raw[p][1] = *reinterpret_cast<const i32x4 *>(src + c + 8);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t two = (uint32_t)raw[p][h][w];
            amax = fmaxf(amax, fabsf(bf16_bits_to_f32((uint16_t)(two & 0xffffu))));
            amax = fmaxf(amax, fabsf(bf16_bits_to_f32((uint16_t)(two >> 16))));
          }
      }
    }
    for (int off = kWave / 2; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    if ((tid & (kWave - 1)) == 0) red[tid / kWave] = amax;
    __syncthreads();
    amax = red[0];
#pragma unroll
    for (int w = 1; w < kQThreads / kWave; ++w) amax = fmaxf(amax, red[w]);
    __syncthreads();
    const bool zero = amax == 0.0f;
    const float sc = zero ? 1.0f : amax / 448.0f;
    if (tid == 0) s[row] = sc;
    uint8_t *dst = q + (size_t)row * cols;
#pragma unroll
    for (int p = 0; p < kQMaxPass; ++p) {
      const int c = (p * kQThreads + tid) * kQPer;
      if (p < npass && c < cols) {
        i32x4 out;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int w = 0; w < 4; w += 2) {
            uint32_t packed = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t two = (uint32_t)raw[p][h][w + (e >> 1)];
              const uint16_t bits = (e & 1) ? (uint16_t)(two >> 16) : (uint16_t)(two & 0xffffu);
              const uint32_t code = zero ? 0u : f32_to_e4m3(bf16_bits_to_f32(bits) / sc);
              packed |= code << (8 * e);
            }
            out[h * 2 + (w >> 1)] = (int)packed;
          }
        *reinterpret_cast<i32x4 *>(dst + c) = out;
      }
    }
  }
}

// Rows of at most kQWaveMaxCols elements: one wave per row (four rows per
// workgroup), lane l holding elements 8 l + 512 i .. +7, the row maximum
// reduced with shuffles only.  Same arithmetic as quant_rows_kernel.
constexpr int kQWaveMaxCols = 4096;
constexpr int kQWaveLoads = kQWaveMaxCols / (kWave * 8);  // 16-byte loads per lane

__global__ __launch_bounds__(kQThreads) void quant_rows_wave_kernel(
    const uint16_t *__restrict__ x, int rows, const int32_t *rows_dev, int cols,
    uint8_t *__restrict__ q, float *__restrict__ s) {
  const int nrows = rows_dev ? *rows_dev : rows;
  const int lane = lane_id();
  const int waves = gridDim.x * (kQThreads / kWave);
  for (int row = blockIdx.x * (kQThreads / kWave) + threadIdx.x / kWave; row < nrows; row += waves) {
    const uint16_t *src = x + (size_t)row * cols;
    i32x4 raw[kQWaveLoads];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < kQWaveLoads; ++i) {
      const int c = (i * kWave + lane) * 8;  // cols is a multiple of 8
      if (c < cols) {
        raw[i] = *reinterpret_cast<const i32x4 *>(src + c);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t two = (uint32_t)raw[i][w];
          amax = fmaxf(amax, fabsf(bf16_bits_to_f32((uint16_t)(two & 0xffffu))));
          amax = fmaxf(amax, fabsf(bf16_bits_to_f32((uint16_t)(two >> 16))));
        }
      }
    }
    for (int off = kWave / 2; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const bool zero = amax == 0.0f;
    const float sc = zero ? 1.0f : amax / 448.0f;
    if (lane == 0) s[row] = sc;
    uint8_t *dst = q + (size_t)row * cols;
#pragma unroll
    for (int i = 0; i < kQWaveLoads; ++i) {
      const int c = (i * kWave + lane) * 8;
      if (c < cols) {
        uint2 out;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uint32_t packed = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t two = (uint32_t)raw[i][h * 2 + (e >> 1)];
            const uint16_t bits = (e & 1) ? (uint16_t)(two >> 16) : (uint16_t)(two & 0xffffu);
            const uint32_t code = zero ? 0u : f32_to_e4m3(bf16_bits_to_f32(bits) / sc);
            packed |= code << (8 * e);
          }
          (h ? out.y : out.x) = packed;
        }
        *reinterpret_cast<uint2 *>(dst + c) = out;
      }
    }
  }
}

int quant_max_cols() { return kQMaxCols; }

hipError_t launch_quant_rows(const uint16_t *x, int rows, const int32_t *rows_dev, int cols,
                             uint8_t *q, float *s, int grid_cap, hipStream_t stream) {
  if (cols <= kQWaveMaxCols) {
    const int per_block = kQThreads / kWave;
    const long long want = ((long long)rows + per_block - 1) / per_block;
    const int grid = (int)(want < grid_cap ? want : grid_cap);
    hipLaunchKernelGGL(quant_rows_wave_kernel, dim3(grid > 0 ? grid : 1), dim3(kQThreads), 0,
                       stream, x, rows, rows_dev, cols, q, s);
    return hipGetLastError();
  }
  const int grid = rows < grid_cap ? rows : grid_cap;
  hipLaunchKernelGGL(quant_rows_kernel, dim3(grid > 0 ? grid : 1), dim3(kQThreads), 0, stream, x,
                     rows, rows_dev, cols, q, s);
  return hipGetLastError();
}

}  // namespace moe
