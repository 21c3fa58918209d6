// Blockwise fp32 -> e4m3 quantisation with one fp32 scale per block.
//
// Method: nxmr §3.1 (block amax; scale = amax / FP8 max; divide to quantise)
// and czchanglian §5.2 (max_val / 448 per block, computed independently).
// Rounding is to nearest, ties to even (nxmr §5.1). Per block:
//   amax = max |x| over the block, NaN skipped
//   s    = amax / 448            (IEEE fp32 division, correctly rounded)
//   q    = e4m3_rne(clamp(x / s, -448, 448))   (fp32 quotient, then e4m3)
// with s == 0 giving signed zeros and NaN elements the NaN code 0x7F|sign.
//
// Both kernels are HBM-streaming: each element is read once (4 B) and its
// code written once (1 B); a scale adds 4 B per block. Loads are 16-byte
// vectors, 32 lanes covering the 512 bytes of one 128-wide block row, and
// codes leave as one 32-bit store per lane (128 contiguous bytes per row).
//
// fp32 denormals are preserved (the default HIP denormal mode); the division
// is the compiler's correctly rounded sequence, never a reciprocal multiply.

#include "internal.h"

namespace fp8g {
namespace {

constexpr float kE4M3Max = 448.0f;

// e4m3 code of a finite fp32 value with |y| <= 448, round to nearest even.
// Normal range (|y| >= 2^-6): round the fp32 pattern at mantissa bit 20
// (3 bits kept), then rebias the exponent from 127 to 7; a mantissa carry
// correctly bumps the exponent. Subnormal range: the e4m3 grid is 2^-9, so
// the code is rint(|y| * 2^9) (exact scaling, hardware RNE); a result of 8 is
// the smallest normal, code 0x08, as it should be.
__device__ __forceinline__ uint32_t e4m3_code_sat(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  const uint32_t rounded = a + 0x7FFFFu + ((a >> 20) & 1u);
  const uint32_t code_n = (rounded >> 20) - (120u << 3);
  const uint32_t code_s = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  return (a >= 0x3C800000u ? code_n : code_s) | sign;
}

// Code of one element given its block scale.
__device__ __forceinline__ uint32_t quant_one(float x, float s) {
  const uint32_t xs = (__float_as_uint(x) >> 24) & 0x80u;
  if (__builtin_isnan(x)) return 0x7Fu | xs;
  if (s == 0.0f) return xs;
  const float y = x / s;
  if (__builtin_isnan(y)) return 0x7Fu | xs;            // inf / inf
  const float yc = __builtin_fminf(__builtin_fmaxf(y, -kE4M3Max), kE4M3Max);
  return e4m3_code_sat(yc);
}

__device__ __forceinline__ float amax4(float4 v, float m) {
  m = __builtin_fmaxf(m, __builtin_fabsf(v.x));
  m = __builtin_fmaxf(m, __builtin_fabsf(v.y));
  m = __builtin_fmaxf(m, __builtin_fabsf(v.z));
  m = __builtin_fmaxf(m, __builtin_fabsf(v.w));
  return m;
}

__device__ __forceinline__ uint32_t pack4(float4 v, float s) {
  return quant_one(v.x, s) | (quant_one(v.y, s) << 8) | (quant_one(v.z, s) << 16) |
         (quant_one(v.w, s) << 24);
}

// 1x128 blocks. Workgroup = 256 lanes = 8 half-waves; half-wave h handles row
// blockIdx.x*8 + h and the QB consecutive 128-column blocks of column group
// blockIdx.y. Lane j of a half-wave holds columns 4j..4j+3 of each block.
constexpr int QB = 4;

__global__ void __launch_bounds__(256)
quant_row_blocks_kernel(const float* __restrict__ x, int64_t rows, int64_t ldx, int ncb,
                        uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ scales,
                        int64_t ssr, int64_t ssc) {
  const int lane = threadIdx.x & 31;
  const int64_t row = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
  if (row >= rows) return;
  const int cb0 = blockIdx.y * QB;
  const float* xr = x + row * ldx;
  float4 v[QB];
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    if (cb0 + j < ncb)
      v[j] = *reinterpret_cast<const float4*>(xr + (int64_t)(cb0 + j) * 128 + lane * 4);
    else
      v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float m[QB];
#pragma unroll
  for (int j = 0; j < QB; ++j) m[j] = amax4(v[j], 0.0f);
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) {
#pragma unroll
    for (int j = 0; j < QB; ++j) m[j] = __builtin_fmaxf(m[j], __shfl_xor(m[j], off, 32));
  }
  uint8_t* qr = q + row * ldq;
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    const int cb = cb0 + j;
    if (cb < ncb) {
      const float s = m[j] / kE4M3Max;
      *reinterpret_cast<uint32_t*>(qr + (int64_t)cb * 128 + lane * 4) = pack4(v[j], s);
      if (lane == 0) scales[row * ssr + (int64_t)cb * ssc] = s;
    }
  }
}

// 128x128 blocks. One workgroup per block: lane t holds column chunk t%32
// (4 floats) of rows t/32 + 8 i, i = 0..15, i.e. 64 values in registers. The
// block amax is reduced across the wave with shuffles and across the four
// waves through LDS; then every lane encodes its 64 values.
__global__ void __launch_bounds__(256)
quant_tile_blocks_kernel(const float* __restrict__ x, int64_t rows, int64_t ldx,
                         uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ scales,
                         int64_t ssr, int64_t ssc) {
  __shared__ float wave_max[4];
  const int t = threadIdx.x;
  const int chunk = t & 31;
  const int r_in = t >> 5;
  const int64_t rb = blockIdx.x;
  const int64_t cb = blockIdx.y;
  const int64_t row0 = rb * 128;
  const int64_t col = cb * 128 + chunk * 4;
  float4 v[16];
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t r = row0 + r_in + 8 * i;
    if (r < rows) {
      v[i] = *reinterpret_cast<const float4*>(x + r * ldx + col);
    } else {
      v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    m = amax4(v[i], m);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, off, 64));
  if ((t & 63) == 0) wave_max[t >> 6] = m;
  __syncthreads();
  m = __builtin_fmaxf(__builtin_fmaxf(wave_max[0], wave_max[1]),
                      __builtin_fmaxf(wave_max[2], wave_max[3]));
  const float s = m / kE4M3Max;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t r = row0 + r_in + 8 * i;
    if (r < rows) *reinterpret_cast<uint32_t*>(q + r * ldq + col) = pack4(v[i], s);
  }
  if (t == 0) scales[rb * ssr + cb * ssc] = s;
}

}  // namespace

hipError_t launch_quantize(const float* x, int64_t rows, int64_t cols, int64_t ldx,
                           int block_rows, uint8_t* q, int64_t ldq, float* scales,
                           int64_t s_stride_row, int64_t s_stride_col, hipStream_t stream) {
  const int ncb = (int)(cols / 128);
  if (block_rows == 1) {
    dim3 grid((unsigned)((rows + 7) / 8), (unsigned)((ncb + QB - 1) / QB));
    hipLaunchKernelGGL(quant_row_blocks_kernel, grid, dim3(256), 0, stream, x, rows, ldx, ncb,
                       q, ldq, scales, s_stride_row, s_stride_col);
  } else {
    dim3 grid((unsigned)((rows + 127) / 128), (unsigned)ncb);
    hipLaunchKernelGGL(quant_tile_blocks_kernel, grid, dim3(256), 0, stream, x, rows, ldx, q,
                       ldq, scales, s_stride_row, s_stride_col);
  }
  return hipGetLastError();
}

}  // namespace fp8g
