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
// registers, reduced, then encoded and written; the quotients are formed by
// a reciprocal multiply where that provably gives the same code and encoded
// by the conversion instruction (quant_e4m3_x4), by IEEE division and the
// bit-level encoder elsewhere.
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

// E4M3 codes of two fp32 values that are not NaN, in bytes 2 HI and 2 HI + 1
// of old: gfx950's conversion instruction (OCP E4M3FN, round to nearest
// even) on the values clamped to +-448.  On every fp32 pattern of magnitude
// below 464 it gives the same code as f32_to_e4m3 (subnormal codes and ties
// included; checked on MI355X), and from 464 on NaN, hence the clamp.
template <bool HI>
__device__ __forceinline__ uint32_t cvt_e4m3_x2(float a, float b, uint32_t old) {
  a = fminf(fmaxf(a, -448.0f), 448.0f);
  b = fminf(fmaxf(b, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

// q = e4m3_rne_saturate(fl32(v / sc)) without a division for nearly every
// element.  rcp = fl32(1 / sc); exact: the row needs the division throughout
// (sc not a normal float, or rcp not finite).
//
// y = v * rcp differs from fl32(v / sc) by a few units in the last place
// (two roundings of relative size 2^-24 each against one), i.e. by at most a
// handful of consecutive fp32 bit patterns.  E4M3 rounding is monotone and
// changes only at the midpoints between neighbouring codes, which in the
// normal range are the patterns whose low 20 bits are 0x80000.  So where y
// lies in the normal range and more than 16 patterns from a midpoint, the
// quotient has y's code.  Within that window (ties included), in the
// subnormal-code range, for NaN and for rows flagged exact the quotient is
// formed by IEEE division instead; the flag costs three compares, and the
// division runs behind one branch for the rare flagged elements.
__device__ __forceinline__ bool quant_needs_division(float y) {
  const uint32_t a = __float_as_uint(y) & 0x7fffffffu;
  return (a - 1u) < 0x3c7fffffu           // 0 < |y| < 2^-6: subnormal codes
         || a > 0x7f800000u               // NaN
         || ((a & 0xfffffu) - 0x7fff0u) < 32u;  // near a midpoint
}

// Four codes (one byte each) for the bf16 pairs lo and hi.  zero: the row is
// all zeros and every code is 0.
__device__ __forceinline__ uint32_t quant_e4m3_x4(uint32_t lo, uint32_t hi, float sc, float rcp,
                                                  bool exact, bool zero) {
  float v[4], y[4];
  v[0] = bf16_bits_to_f32((uint16_t)(lo & 0xffffu));
  v[1] = bf16_bits_to_f32((uint16_t)(lo >> 16));
  v[2] = bf16_bits_to_f32((uint16_t)(hi & 0xffffu));
  v[3] = bf16_bits_to_f32((uint16_t)(hi >> 16));
  bool any = exact;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    y[e] = v[e] * rcp;
    any = any || quant_needs_division(y[e]);
  }
  uint32_t packed = cvt_e4m3_x2<false>(y[0], y[1], 0u);
  packed = cvt_e4m3_x2<true>(y[2], y[3], packed);
  if (any) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (exact || quant_needs_division(y[e]))
        packed = (packed & ~(0xffu << (8 * e))) | (f32_to_e4m3(v[e] / sc) << (8 * e));
    }
  }
  return zero ? 0u : packed;
}

// The reciprocal of a row scale, and whether the row must divide throughout.
__device__ __forceinline__ float quant_rcp(float sc, bool *exact) {
  const float r = 1.0f / sc;
  *exact = !(sc >= 1.17549435e-38f) || !(r < 3.40282347e38f);  // sc subnormal, r overflowed
  return r;
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
    bool exact;
    const float rcp = quant_rcp(sc, &exact);
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
          for (int w = 0; w < 4; w += 2)
            out[h * 2 + (w >> 1)] = (int)quant_e4m3_x4((uint32_t)raw[p][h][w],
                                                       (uint32_t)raw[p][h][w + 1], sc, rcp, exact,
                                                       zero);
        *reinterpret_cast<i32x4 *>(dst + c) = out;
      }
    }
  }
}

// Rows of at most kQWaveMaxCols elements, one or two waves per row.  A wave
// holds NL 16-byte loads per lane of its part of the row, columns c0 + 8 l +
// 512 i .. +7 in lane l; the row maximum is reduced with shuffles (and, for
// two waves, one exchange through LDS).  Same arithmetic as
// quant_rows_kernel.
constexpr int kQWaveMaxCols = 4096;

// loads of one wave's part of a row (columns [c0, min(cols, c0 + NL * 512)))
// and the wave's maximum magnitude
template <int NL>
__device__ __forceinline__ float q_load_part(const uint16_t *row_src, int c0, int cols,
                                             i32x4 (&raw)[NL]) {
  const int lane = lane_id();
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int c = c0 + (i * kWave + lane) * 8;  // cols is a multiple of 8
    if (c < cols) raw[i] = __builtin_nontemporal_load(reinterpret_cast<const i32x4 *>(row_src + c));
  }
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int c = c0 + (i * kWave + lane) * 8;
    if (c < cols) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t two = (uint32_t)raw[i][w];
        amax = fmaxf(amax, fabsf(bf16_bits_to_f32((uint16_t)(two & 0xffffu))));
        amax = fmaxf(amax, fabsf(bf16_bits_to_f32((uint16_t)(two >> 16))));
      }
    }
  }
  for (int off = kWave / 2; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  return amax;
}

// codes of one wave's part of a row, given the row maximum
template <int NL>
__device__ __forceinline__ void q_store_part(uint8_t *row_dst, int c0, int cols,
                                             const i32x4 (&raw)[NL], float amax) {
  const int lane = lane_id();
  const bool zero = amax == 0.0f;
  const float sc = zero ? 1.0f : amax / 448.0f;
  bool exact;
  const float rcp = quant_rcp(sc, &exact);
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int c = c0 + (i * kWave + lane) * 8;
    if (c < cols) {
      uint2 out;
      out.x = quant_e4m3_x4((uint32_t)raw[i][0], (uint32_t)raw[i][1], sc, rcp, exact, zero);
      out.y = quant_e4m3_x4((uint32_t)raw[i][2], (uint32_t)raw[i][3], sc, rcp, exact, zero);
      *reinterpret_cast<uint2 *>(row_dst + c) = out;
    }
  }
}

__device__ __forceinline__ float q_scale(float amax) { return amax == 0.0f ? 1.0f : amax / 448.0f; }

// one wave per row, four rows per workgroup
template <int NL>
__global__ __launch_bounds__(kQThreads) void quant_rows_wave_kernel(
    const uint16_t *__restrict__ x, int rows, const int32_t *rows_dev, int cols,
    uint8_t *__restrict__ q, float *__restrict__ s) {
  const int nrows = rows_dev ? *rows_dev : rows;
  const int waves = gridDim.x * (kQThreads / kWave);
  for (int row = blockIdx.x * (kQThreads / kWave) + threadIdx.x / kWave; row < nrows; row += waves) {
    i32x4 raw[NL];
    const float amax = q_load_part<NL>(x + (size_t)row * cols, 0, cols, raw);
    if (lane_id() == 0) s[row] = q_scale(amax);
    q_store_part<NL>(q + (size_t)row * cols, 0, cols, raw, amax);
  }
}

// two waves per row (columns [0, NL * 512) and the rest), two rows per
// workgroup: for 4096-column rows the registers of one wave's half keep the
// kernel at twice the occupancy of a whole row per wave (MI355X, 8192 x 4096:
// 44 -> 36 us)
template <int NL>
__global__ __launch_bounds__(kQThreads) void quant_rows_pair_kernel(
    const uint16_t *__restrict__ x, int rows, const int32_t *rows_dev, int cols,
    uint8_t *__restrict__ q, float *__restrict__ s) {
  constexpr int kRowsPerBlock = kQThreads / kWave / 2;
  __shared__ float part[2][kQThreads / kWave];  // per wave, double-buffered by trip
  const int nrows = rows_dev ? *rows_dev : rows;
  const int wave = threadIdx.x / kWave;
  const int c0 = (wave & 1) * NL * kWave * 8;
  int trip = 0;
  // the trip count is the same for every wave of the workgroup, so all of
  // them meet each barrier
  for (int base = blockIdx.x * kRowsPerBlock; base < nrows;
       base += gridDim.x * kRowsPerBlock, trip ^= 1) {
    const int row = base + wave / 2;
    const bool on = row < nrows;
    i32x4 raw[NL];
    float amax = on ? q_load_part<NL>(x + (size_t)row * cols, c0, cols, raw) : 0.0f;
    if (lane_id() == 0) part[trip][wave] = amax;
    __syncthreads();
    amax = fmaxf(amax, part[trip][wave ^ 1]);
    if (!on) continue;
    if (lane_id() == 0 && c0 == 0) s[row] = q_scale(amax);
    q_store_part<NL>(q + (size_t)row * cols, c0, cols, raw, amax);
  }
}

// Rows whose maxima are known (amax_bits[r] = fp32 bits of max |x[r, :]|,
// NaN elements left out, as fmaxf does above): no reduction, so every
// thread encodes 8 consecutive elements of any row, 16-byte non-temporal
// loads and 8-byte stores, the row's scale written by the thread of its
// first 8 elements.  Same scale and codes as the kernels above.
__global__ __launch_bounds__(kQThreads) void quant_rows_known_max_kernel(
    const uint16_t *__restrict__ x, int rows, const int32_t *rows_dev, int cols,
    const uint32_t *__restrict__ amax_bits, uint8_t *__restrict__ q, float *__restrict__ s) {
  const int nrows = rows_dev ? *rows_dev : rows;
  const int per_row = cols / 8;  // cols is a multiple of 8
  const long long n = (long long)nrows * per_row;
  for (long long c = (long long)blockIdx.x * kQThreads + threadIdx.x; c < n;
       c += (long long)gridDim.x * kQThreads) {
    const int row = (int)(c / per_row);
    const int col = (int)(c - (long long)row * per_row) * 8;
    const float amax = __uint_as_float(amax_bits[row]);
    const bool zero = amax == 0.0f;
    const float sc = q_scale(amax);
    bool exact;
    const float rcp = quant_rcp(sc, &exact);
    const size_t o = (size_t)row * cols + col;
    const i32x4 raw = __builtin_nontemporal_load(reinterpret_cast<const i32x4 *>(x + o));
    uint2 out;
    out.x = quant_e4m3_x4((uint32_t)raw[0], (uint32_t)raw[1], sc, rcp, exact, zero);
    out.y = quant_e4m3_x4((uint32_t)raw[2], (uint32_t)raw[3], sc, rcp, exact, zero);
    *reinterpret_cast<uint2 *>(q + o) = out;
    if (col == 0) s[row] = sc;
  }
}

__global__ __launch_bounds__(kQThreads) void zero_u32_kernel(uint32_t *__restrict__ p, int n) {
  for (int i = blockIdx.x * kQThreads + threadIdx.x; i < n; i += gridDim.x * kQThreads) p[i] = 0u;
}

int quant_max_cols() { return kQMaxCols; }

hipError_t launch_quant_rows_known_max(const uint16_t *x, int rows, const int32_t *rows_dev,
                                       int cols, const uint32_t *amax_bits, uint8_t *q, float *s,
                                       int grid_cap, hipStream_t stream) {
  const long long chunks = (long long)rows * (cols / 8);
  const long long want = (chunks + kQThreads - 1) / kQThreads;
  const long long cap = (long long)grid_cap * 4;
  const int grid = (int)(want < cap ? want : cap);
  hipLaunchKernelGGL(quant_rows_known_max_kernel, dim3(grid > 0 ? grid : 1), dim3(kQThreads), 0,
                     stream, x, rows, rows_dev, cols, amax_bits, q, s);
  return hipGetLastError();
}

hipError_t launch_zero_u32(uint32_t *p, int n, hipStream_t stream) {
  const int grid = (n + kQThreads * 4 - 1) / (kQThreads * 4);
  hipLaunchKernelGGL(zero_u32_kernel, dim3(grid > 0 ? grid : 1), dim3(kQThreads), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_quant_rows(const uint16_t *x, int rows, const int32_t *rows_dev, int cols,
                             uint8_t *q, float *s, int grid_cap, hipStream_t stream) {
  if (cols <= kQWaveMaxCols) {
    const int nl = (cols + kWave * 8 - 1) / (kWave * 8);
    const int per_block = nl <= 4 ? kQThreads / kWave : kQThreads / kWave / 2;
    const long long want = ((long long)rows + per_block - 1) / per_block;
    // up to 16 workgroups per CU (four times grid_cap): more rows in flight
    // at once (MI355X, 46,700 x 2048: 4 per CU 106 us, 16 per CU 80 us)
    const long long cap = (long long)grid_cap * 4;
    const int grid = (int)(want < cap ? want : cap);
    if (nl <= 2)
      hipLaunchKernelGGL(quant_rows_wave_kernel<2>, dim3(grid > 0 ? grid : 1), dim3(kQThreads), 0,
                         stream, x, rows, rows_dev, cols, q, s);
    else if (nl <= 4)
      hipLaunchKernelGGL(quant_rows_wave_kernel<4>, dim3(grid > 0 ? grid : 1), dim3(kQThreads), 0,
                         stream, x, rows, rows_dev, cols, q, s);
    else  // up to 4096 columns: two waves of four loads per lane
      hipLaunchKernelGGL(quant_rows_pair_kernel<4>, dim3(grid > 0 ? grid : 1), dim3(kQThreads), 0,
                         stream, x, rows, rows_dev, cols, q, s);
    return hipGetLastError();
  }
  const int grid = rows < grid_cap ? rows : grid_cap;
  hipLaunchKernelGGL(quant_rows_kernel, dim3(grid > 0 ? grid : 1), dim3(kQThreads), 0, stream, x,
                     rows, rows_dev, cols, q, s);
  return hipGetLastError();
}

}  // namespace moe
