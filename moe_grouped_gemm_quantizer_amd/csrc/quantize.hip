// Blockwise fp32 (or bf16) -> e4m3 quantisation with one fp32 scale per block.
//
// Method: nxmr §3.1 (block amax; scale = amax / FP8 max; divide to quantise)
// and czchanglian §5.2 (max_val / 448 per block, computed independently).
// Rounding is to nearest, ties to even (nxmr §5.1). Per block:
//   amax = max |x| over the block, NaN skipped
//   s    = amax / 448            (IEEE fp32 division, correctly rounded)
//   q    = e4m3_rne(clamp(x / s, -448, 448))   (fp32 quotient, then e4m3)
// with s == 0 giving signed zeros and NaN elements the NaN code 0x7F|sign.
// The element step is branch-free (selects, not per-lane branches), and the
// e4m3 rounding is the hardware conversion.
//
// Both kernels are HBM-streaming: each element is read once (4 B, or 2 B
// for bf16 input) and its code written once (1 B); a scale adds 4 B per
// block. Loads are 16-byte (bf16: 8-byte) vectors, 32 lanes covering one
// 128-wide block row, and codes leave as one 32-bit store per lane (128
// contiguous bytes per row). A bf16 input is widened to its exact fp32
// value on load, so it quantises exactly as that fp32 value would. The
// launcher gives every workgroup one unit group or block and leaves the
// balancing to the hardware dispatcher; the kernels' unit loops (each wave
// loads its next unit before encoding the current one) only run past the
// launch limit.
//
// fp32 denormals are preserved (the default HIP denormal mode). The quotient
// x / s is always the correctly rounded IEEE one, never a plain reciprocal
// multiply. Within a block s is fixed, so it is formed from y = RN(1/s) (one
// IEEE division per block) by Markstein's correction: q0 = RN(x y),
// r = x - q0 s (exact, by FMA), q = RN(q0 + r y), which equals RN(x / s)
// whenever nothing underflows (Markstein 1990; Muller et al., Handbook of
// Floating-Point Arithmetic, the FMA division theorems). Scales in
// [2^-80, 2^100] keep every residual of a quotient >= 2^-21 normal (smaller
// quotients encode to a signed zero whatever their last bits); a block with
// a smaller or larger scale is first scaled, x and s alike, by an exact
// power of two into that range (e4m3.h gives the argument).

#include <algorithm>
#include <type_traits>
#include <vector>

#include "e4m3.h"
#include "internal.h"

namespace fp8g {
namespace {

using namespace e4m3;

// Four consecutive input values as fp32: fp32 as is, bf16 widened exactly
// (its 16 bits are the top half of the fp32 pattern).
__device__ __forceinline__ float4 load4(const float* p) {
  return *reinterpret_cast<const float4*>(p);
}
__device__ __forceinline__ float4 load4(const uint16_t* p) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                     __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u));
}

// 1x128 blocks. A unit is one row's QB consecutive 128-column blocks, owned
// by a 32-lane half-wave (lane j holds columns 4j..4j+3 of each block). The
// grid is persistent: half-wave h takes units h, h + H, h + 2H, ... (H = all
// half-waves), and loads its next unit before encoding the current one, so
// HBM reads stay in flight while the VALU works. Units are numbered row by
// row, so consecutive half-waves read consecutive 1 KB pieces of one row
// (measured ~10% faster than walking down a column group, although the
// scales they write are then a row count apart). Four blocks per unit
// (64 bytes in flight per lane) against two: 29.8 -> 29.0 us on 4096x8192
// and 4864x7168, 17.1 -> 17.3 us on 8192x2048; two units per half-wave
// (the next one prefetched) measured slower either way.
constexpr int QB = 4;

// (a lane's four columns of block cb exist when cb * 128 + 4 lane < cols:
// cols is a multiple of 16, so the last block may be partial; absent
// columns read as zeros, which leave the amax alone, and are not stored)
template <typename T>
__device__ __forceinline__ void load_unit(const T* __restrict__ x, int64_t ldx, int64_t cols,
                                          int64_t row, int cb0, int lane, float4 (&v)[QB]) {
  const T* xr = x + row * ldx + lane * 4;
#pragma unroll
  for (int j = 0; j < QB; ++j)
    v[j] = ((int64_t)(cb0 + j) * 128 + lane * 4 < cols) ? load4(xr + (int64_t)(cb0 + j) * 128)
                                                        : make_float4(0.f, 0.f, 0.f, 0.f);
}

template <typename T>
__global__ void __launch_bounds__(256)
quant_row_blocks_kernel(const T* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
                        int ncb, uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ scales,
                        int64_t ssr, int64_t ssc) {
  const int lane = threadIdx.x & 31;
  const int64_t H = (int64_t)gridDim.x * 8;
  const int ncg = (ncb + QB - 1) / QB;
  const int64_t units = rows * ncg;
  const int64_t u0 = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
  if (u0 >= units) return;
  // unit u is (row u / ncg, column group u % ncg); stepping u by H moves
  // the pair by (H / ncg, H % ncg) with one carry, so no per-unit division
  const int64_t h_row = H / ncg;
  const int64_t h_cg = H % ncg;
  int64_t row = u0 / ncg;
  int64_t cg = u0 % ncg;
  float4 nxt[QB];
  load_unit(x, ldx, cols, row, (int)cg * QB, lane, nxt);
  while (row < rows) {
    const int cb0 = (int)cg * QB;
    float4 v[QB];
#pragma unroll
    for (int j = 0; j < QB; ++j) v[j] = nxt[j];
    const int64_t cur_row = row;
    row += h_row;
    cg += h_cg;
    if (cg >= ncg) {
      cg -= ncg;
      ++row;
    }
    if (row < rows) load_unit(x, ldx, cols, row, (int)cg * QB, lane, nxt);
    float m[QB];
#pragma unroll
    for (int j = 0; j < QB; ++j) m[j] = amax4(v[j], 0.0f);
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) {
#pragma unroll
      for (int j = 0; j < QB; ++j) m[j] = __builtin_fmaxf(m[j], __shfl_xor(m[j], off, 32));
    }
    uint8_t* qr = q + cur_row * ldq + lane * 4;
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      const int cb = cb0 + j;
      if (cb < ncb) {
        const Divisor d = make_divisor(scale_of(m[j]));
        if ((int64_t)cb * 128 + lane * 4 < cols)
          *reinterpret_cast<uint32_t*>(qr + (int64_t)cb * 128) = encode4(v[j], d);
        if (lane == 0) scales[cur_row * ssr + (int64_t)cb * ssc] = d.s;
      }
    }
  }
}

// 1x128 blocks from bf16 with 16-byte loads: a unit is one row's 2 LPL
// consecutive 128-column blocks, owned by a 32-lane half-wave; for each
// l < LPL, lane j holds columns 8 (j & 15) .. +7 of the unit's block
// 2 l + (j >> 4) (one 16-byte load of eight values, all LPL loads issued
// before any block is reduced), and each block's amax is reduced over its
// 16 lanes. With the fp32 kernels' four values per lane a bf16 load would
// move only 8 bytes, halving the bytes in flight per wave. Used when x is
// 16-byte aligned and ldx % 8 == 0 (else the general kernel); the result is
// the same. Two loads per lane (four blocks per unit) measured fastest:
// 22.3 -> 21.3 us on 4096x8192 and 37.1 -> 34.4 us on 8192x7168 against
// one, equal on 8192x2048; four were slower (24.6, 37.3 us), the grid then
// too small to fill the CUs as evenly.
constexpr int BF16_LPL = 2;
template <int LPL>
__global__ void __launch_bounds__(256)
quant_row_blocks_bf16x8_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                               int64_t ldx, int ncb, uint8_t* __restrict__ q, int64_t ldq,
                               float* __restrict__ scales, int64_t ssr, int64_t ssc) {
  const int lane = threadIdx.x & 31;
  const int l16 = lane & 15;
  const int64_t H = (int64_t)gridDim.x * 8;
  const int ncg = (ncb + 2 * LPL - 1) / (2 * LPL);
  const int64_t units = rows * ncg;
  for (int64_t u = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5); u < units; u += H) {
    const int64_t row = u / ncg;
    const int cb0 = (int)(u - row * ncg) * 2 * LPL + (lane >> 4);
    float4 v0[LPL], v1[LPL];
#pragma unroll
    for (int l = 0; l < LPL; ++l) {
      const int cb = cb0 + 2 * l;
      // (has: uniform over a block's 16 lanes; cols % 16 == 0)
      const bool ok = cb < ncb && (int64_t)cb * 128 + l16 * 8 < cols;
      v0[l] = make_float4(0.f, 0.f, 0.f, 0.f);
      v1[l] = v0[l];
      if (ok) {
        const uint4 w =
            *reinterpret_cast<const uint4*>(x + row * ldx + (int64_t)cb * 128 + l16 * 8);
        v0[l] = make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                            __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u));
        v1[l] = make_float4(__uint_as_float(w.z << 16), __uint_as_float(w.z & 0xFFFF0000u),
                            __uint_as_float(w.w << 16), __uint_as_float(w.w & 0xFFFF0000u));
      }
    }
#pragma unroll
    for (int l = 0; l < LPL; ++l) {
      const int cb = cb0 + 2 * l;
      float m = amax4(v1[l], amax4(v0[l], 0.0f));
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, off, 32));
      if (cb < ncb) {
        const Divisor d = make_divisor(scale_of(m));
        uint8_t* qp = q + row * ldq + (int64_t)cb * 128 + l16 * 8;
        if ((int64_t)cb * 128 + l16 * 8 < cols) {
          *reinterpret_cast<uint32_t*>(qp) = encode4(v0[l], d);
          *reinterpret_cast<uint32_t*>(qp + 4) = encode4(v1[l], d);
        }
        if (l16 == 0) scales[row * ssr + (int64_t)cb * ssc] = d.s;
      }
    }
  }
}

// 128x128 blocks. A workgroup of 256 lanes owns a block at a time: lane t
// holds column chunk t%32 (4 floats) of rows t/32 + 8 i, i = 0..15, i.e. 64
// values in registers. The block amax is reduced across the wave with
// shuffles and across the four waves through LDS, then every lane encodes its
// 64 values. Persistent grid: workgroup w takes blocks w, w + G, ..., with
// two register sets used in turn, so the next block's loads are in flight
// while the current one is reduced and encoded. Row addresses are a
// workgroup-uniform base (row0 + 8 i, block column) plus one per-lane 32-bit
// offset fixed for the whole launch (the launcher checks the strides fit).
struct TileAt {
  int64_t rb, cb;
  bool full;          // all 128 rows exist
  bool col_ok;        // this lane's four columns exist (the last block may be partial)
};
__device__ __forceinline__ TileAt tile_at(int64_t b, int ncb, int64_t rows, int64_t cols,
                                          int chunk) {
  TileAt a;
  a.rb = b / ncb;
  a.cb = b - a.rb * ncb;
  a.full = a.rb * 128 + 128 <= rows;
  a.col_ok = a.cb * 128 + chunk * 4 < cols;
  return a;
}

// The 128x128 kernel reads an fp32 input with the non-temporal cache policy:
// every element is read once, and the streamed lines then stay out of the
// way of the rest (8192x8192: 59.5 -> 54.9 us; 8 x 4096x7168: 206 -> 178
// us; 32 x 7168x2048: 400 -> 380 us). The 1x128 kernel measured slower with
// it (29.1 -> 32.2 us on 4096x8192), and so did the bf16 128x128 kernel on
// an input the Infinity Cache holds (8192x8192: 33.4 -> 37.5 us, though
// 129 -> 118 us on 8 x 4096x7168); both keep ordinary loads.
typedef float f4v_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load4_nt(const float* p) {
  const f4v_t v = __builtin_nontemporal_load(reinterpret_cast<const f4v_t*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 load4_nt(const uint16_t* p) {
  return load4(p);
}

template <typename T>
__device__ __forceinline__ void load_tile(const T* __restrict__ x, int64_t rows, int64_t ldx,
                                          const TileAt& a, uint32_t xo, int r_in,
                                          float4 (&v)[16]) {
  const int64_t row0 = a.rb * 128;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const char* base = reinterpret_cast<const char*>(x + (row0 + 8 * i) * ldx + a.cb * 128);
    if (a.col_ok && (a.full || row0 + r_in + 8 * i < rows))
      v[i] = load4_nt(reinterpret_cast<const T*>(base + xo));
    else
      v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

__device__ __forceinline__ void encode_tile(const float4 (&v)[16], const TileAt& a, int64_t rows,
                                            uint8_t* __restrict__ q, int64_t ldq, uint32_t qo,
                                            int r_in, float* __restrict__ scales, int64_t ssr,
                                            int64_t ssc, float (&wave_max)[2][4], int slot) {
  const int t = threadIdx.x;
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = amax4(v[i], m);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, off, 64));
  // two alternating slots: a fast wave's next write cannot clobber a value
  // a slow wave is still reading from the previous block
  if ((t & 63) == 0) wave_max[slot][t >> 6] = m;
  __syncthreads();
  m = __builtin_fmaxf(__builtin_fmaxf(wave_max[slot][0], wave_max[slot][1]),
                      __builtin_fmaxf(wave_max[slot][2], wave_max[slot][3]));
  const Divisor d = make_divisor(scale_of(m));
  const int64_t row0 = a.rb * 128;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    uint8_t* base = q + (row0 + 8 * i) * ldq + a.cb * 128;
    if (a.col_ok && (a.full || row0 + r_in + 8 * i < rows))
      *reinterpret_cast<uint32_t*>(base + qo) = encode4(v[i], d);
  }
  if (t == 0) scales[a.rb * ssr + a.cb * ssc] = d.s;
}

template <typename T>
__global__ void __launch_bounds__(256)
quant_tile_blocks_kernel(const T* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
                         int ncb, uint8_t* __restrict__ q, int64_t ldq,
                         float* __restrict__ scales, int64_t ssr, int64_t ssc) {
  __shared__ float wave_max[2][4];
  const int t = threadIdx.x;
  const int chunk = t & 31;
  const int r_in = t >> 5;
  const int64_t nrb = (rows + 127) / 128;
  const int64_t blocks = nrb * ncb;
  int64_t b = blockIdx.x;
  if (b >= blocks) return;
  const uint32_t xo = (uint32_t)((int64_t)r_in * ldx + chunk * 4) * (uint32_t)sizeof(T);  // bytes
  const uint32_t qo = (uint32_t)((int64_t)r_in * ldq + chunk * 4);
  const int64_t G = gridDim.x;
  float4 va[16], vb[16];
  TileAt ta = tile_at(b, ncb, rows, cols, chunk);
  load_tile(x, rows, ldx, ta, xo, r_in, va);
  int slot = 0;
  for (;;) {
    const int64_t b1 = b + G;
    const TileAt tb = tile_at(b1, ncb, rows, cols, chunk);
    if (b1 < blocks) load_tile(x, rows, ldx, tb, xo, r_in, vb);
    encode_tile(va, ta, rows, q, ldq, qo, r_in, scales, ssr, ssc, wave_max, slot);
    slot ^= 1;
    if (b1 >= blocks) break;
    const int64_t b2 = b1 + G;
    ta = tile_at(b2, ncb, rows, cols, chunk);
    if (b2 < blocks) load_tile(x, rows, ldx, ta, xo, r_in, va);
    encode_tile(vb, tb, rows, q, ldq, qo, r_in, scales, ssr, ssc, wave_max, slot);
    slot ^= 1;
    if (b2 >= blocks) break;
    b = b2;
  }
}

// 128x128 blocks from bf16 with 16-byte loads: lane t holds columns
// 8 (t & 15) .. +7 of rows (t >> 4) + 16 i, i = 0..7 -- eight 16-byte loads
// of eight values, kept as packed bf16 (32 registers per block) and widened
// exactly when used -- so that each wave load moves 1 KB as in the fp32
// kernel; with the fp32 kernel's four values per lane a bf16 load moves only
// 512 bytes. Otherwise as quant_tile_blocks_kernel: the block amax over the
// wave by shuffles and over the four waves through LDS, the same scale and
// element rule, codes stored 8 bytes per lane (whole 128-byte rows per 16
// lanes). Used when x is 16-byte aligned with ldx % 8 == 0 and q 8-byte
// aligned with ldq % 8 == 0 (else the four-value kernel); the result is the
// same.
__device__ __forceinline__ float4 widen_lo(uint4 w) {
  return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                     __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u));
}
__device__ __forceinline__ float4 widen_hi(uint4 w) {
  return make_float4(__uint_as_float(w.z << 16), __uint_as_float(w.z & 0xFFFF0000u),
                     __uint_as_float(w.w << 16), __uint_as_float(w.w & 0xFFFF0000u));
}
__device__ __forceinline__ TileAt tile_at8(int64_t b, int ncb, int64_t rows, int64_t cols,
                                           int chunk8) {
  TileAt a;
  a.rb = b / ncb;
  a.cb = b - a.rb * ncb;
  a.full = a.rb * 128 + 128 <= rows;
  a.col_ok = a.cb * 128 + chunk8 * 8 < cols;      // (cols % 16 == 0: all eight or none)
  return a;
}
__device__ __forceinline__ void load_tile8(const uint16_t* __restrict__ x, int64_t rows,
                                           int64_t ldx, const TileAt& a, uint32_t xo, int r_in,
                                           uint4 (&w)[8]) {
  const int64_t row0 = a.rb * 128;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const char* base = reinterpret_cast<const char*>(x + (row0 + 16 * i) * ldx + a.cb * 128);
    if (a.col_ok && (a.full || row0 + r_in + 16 * i < rows))
      w[i] = *reinterpret_cast<const uint4*>(base + xo);
    else
      w[i] = make_uint4(0u, 0u, 0u, 0u);
  }
}
__device__ __forceinline__ void encode_tile8(const uint4 (&w)[8], const TileAt& a, int64_t rows,
                                             uint8_t* __restrict__ q, int64_t ldq, uint32_t qo,
                                             int r_in, float* __restrict__ scales, int64_t ssr,
                                             int64_t ssc, float (&wave_max)[2][4], int slot) {
  const int t = threadIdx.x;
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = amax4(widen_hi(w[i]), amax4(widen_lo(w[i]), m));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, off, 64));
  if ((t & 63) == 0) wave_max[slot][t >> 6] = m;
  __syncthreads();
  m = __builtin_fmaxf(__builtin_fmaxf(wave_max[slot][0], wave_max[slot][1]),
                      __builtin_fmaxf(wave_max[slot][2], wave_max[slot][3]));
  const Divisor d = make_divisor(scale_of(m));
  const int64_t row0 = a.rb * 128;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint8_t* base = q + (row0 + 16 * i) * ldq + a.cb * 128;
    if (a.col_ok && (a.full || row0 + r_in + 16 * i < rows))
      *reinterpret_cast<uint2*>(base + qo) =
          make_uint2(encode4(widen_lo(w[i]), d), encode4(widen_hi(w[i]), d));
  }
  if (t == 0) scales[a.rb * ssr + a.cb * ssc] = d.s;
}
__global__ void __launch_bounds__(256)
quant_tile_blocks_bf16x8_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                int64_t ldx, int ncb, uint8_t* __restrict__ q, int64_t ldq,
                                float* __restrict__ scales, int64_t ssr, int64_t ssc) {
  __shared__ float wave_max[2][4];
  const int t = threadIdx.x;
  const int chunk8 = t & 15;
  const int r_in = t >> 4;
  const int64_t nrb = (rows + 127) / 128;
  const int64_t blocks = nrb * ncb;
  int64_t b = blockIdx.x;
  if (b >= blocks) return;
  const uint32_t xo = (uint32_t)((int64_t)r_in * ldx + chunk8 * 8) * 2u;   // bytes
  const uint32_t qo = (uint32_t)((int64_t)r_in * ldq + chunk8 * 8);
  const int64_t G = gridDim.x;
  uint4 wa[8], wb[8];
  TileAt ta = tile_at8(b, ncb, rows, cols, chunk8);
  load_tile8(x, rows, ldx, ta, xo, r_in, wa);
  int slot = 0;
  for (;;) {
    const int64_t b1 = b + G;
    const TileAt tb = tile_at8(b1, ncb, rows, cols, chunk8);
    if (b1 < blocks) load_tile8(x, rows, ldx, tb, xo, r_in, wb);
    encode_tile8(wa, ta, rows, q, ldq, qo, r_in, scales, ssr, ssc, wave_max, slot);
    slot ^= 1;
    if (b1 >= blocks) break;
    const int64_t b2 = b1 + G;
    ta = tile_at8(b2, ncb, rows, cols, chunk8);
    if (b2 < blocks) load_tile8(x, rows, ldx, ta, xo, r_in, wa);
    encode_tile8(wb, tb, rows, q, ldq, qo, r_in, scales, ssr, ssc, wave_max, slot);
    slot ^= 1;
    if (b2 >= blocks) break;
    b = b2;
  }
}

// ---------------------------------------------------------------------------
// Per-tensor quantisation (one scale for the whole matrix, the scaling of the
// gtnt page's Triton kernel): the same element step as the block kernels
// with a single block covering every element. Three passes: the amax
// reduction into *scale (as the bit pattern of a non-negative float, whose
// integer order is its numeric order), the encoding (every workgroup reads
// the amax and forms the same scale), and the replacement of the amax by the
// scale. The column range of a workgroup is blockIdx.x * 1024 .. +1023
// (256 lanes x 4 values), rows blockIdx.y, blockIdx.y + gridDim.y, ...

__global__ void __launch_bounds__(64) tensor_zero_kernel(float* scale) {
  if (threadIdx.x == 0) scale[0] = 0.0f;
}

// m (>= 0, never NaN) into *p as the larger of the two, compared on the
// float's bits (ordered like the values for non-negative floats). The
// workgroups of a launch finish at about the same time and atomics on one
// address are serialised, so the stored value, which only grows during the
// launch, is read first and the atomic skipped when it already holds at
// least m (a stale read costs no more than an atomic that was not needed).
__device__ __forceinline__ void max_into(float* p, float m) {
  unsigned int* u = reinterpret_cast<unsigned int*>(p);
  const unsigned int mb = __float_as_uint(m);
  if (mb > __hip_atomic_load(u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(u, mb);
}

__global__ void __launch_bounds__(256)
tensor_amax_kernel(const float* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
                   float* scale) {
  __shared__ float part[4];
  const int64_t c = (int64_t)blockIdx.x * 1024 + threadIdx.x * 4;
  float m = 0.0f;
  if (c < cols)
    for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) m = amax4(load4(x + r * ldx + c), m);
  for (int o = 32; o >= 1; o >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = __builtin_fmaxf(__builtin_fmaxf(part[0], part[1]), __builtin_fmaxf(part[2], part[3]));
    max_into(scale, m);
  }
}

__global__ void __launch_bounds__(256)
tensor_encode_kernel(const float* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
                     uint8_t* __restrict__ q, int64_t ldq, const float* __restrict__ amax) {
  const Divisor d = make_divisor(scale_of(amax[0]));
  const int64_t c = (int64_t)blockIdx.x * 1024 + threadIdx.x * 4;
  if (c >= cols) return;
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y)
    *reinterpret_cast<uint32_t*>(q + r * ldq + c) = encode4(load4(x + r * ldx + c), d);
}

__global__ void __launch_bounds__(64) tensor_scale_kernel(float* scale) {
  if (threadIdx.x == 0) scale[0] = scale_of(scale[0]);
}

// ---------------------------------------------------------------------------
// Delayed scaling (czchanglian §2.3: a step runs with the scale gathered
// before it): one scale per tensor taken from an amax history, e4m3 or e5m2
// codes, and this step's amax recorded for the steps after it. Two kernels:
// delayed_scale_kernel reads the window (max, NaN skipped), writes
// s = RN(max / FP8 max) (1 when no entry is positive) and clears the entry
// this step's amax goes to; delayed_encode_kernel encodes under s and
// reduces |x| into that entry (max_into, as above).
//
// The element step takes the scale as given, so the data may have outgrown
// it, and an element may be infinite while the scale is finite:
//   y = RN(x / s) (Markstein's correction with the power-of-two prescale of
//   e4m3.h), an infinite x giving an infinite y; s = 0: a signed zero for
//   every non-NaN x; s = inf: x / inf (signed zero, NaN for an infinite x);
//   the quotient of a finite x saturated to the format's largest value
//   (also where it overflowed fp32), infinities kept;
//   codes: e4m3 has no infinity (the conversion gives the NaN code of the
//   infinity's sign), e5m2 encodes it; a NaN y gives 0x7F with x's sign.

template <int FMT>
struct Fp8Fmt;
template <>
struct Fp8Fmt<FMT_E4M3> {
  static constexpr float kMax = 448.0f;        // 7 * 2^6
  static constexpr float kPow2 = 0x1p-6f;
};
template <>
struct Fp8Fmt<FMT_E5M2> {
  static constexpr float kMax = 57344.0f;      // 7 * 2^13
  static constexpr float kPow2 = 0x1p-13f;
};

// RN(amax / kMax): for amax >= 2^-100 it is RN(amax / 7) * kPow2 exactly
// (the division identity of scale_of; the power of two keeps the result
// normal), else the IEEE division.
template <int FMT>
__device__ __forceinline__ float scale_of_fmt(float amax) {
  constexpr float y7 = 1.0f / 7.0f;
  if (amax >= 0x1p-100f && amax <= 0x1.fffffep127f) {
    const float q0 = amax * y7;
    const float r = __builtin_fmaf(-q0, 7.0f, amax);
    return __builtin_fmaf(r, y7, q0) * Fp8Fmt<FMT>::kPow2;
  }
  return amax / Fp8Fmt<FMT>::kMax;
}

// (PLAIN: the scale is neither zero nor infinite and needs no prescale,
// p = 1 -- the usual case, decided once for the whole tensor -- so the
// special-scale selects and the prescale multiply drop out)
template <int FMT, bool PLAIN = false>
__device__ __forceinline__ float given_quotient(float x, const Divisor& d, bool s_inf) {
  const float xp = PLAIN ? x : x * d.p;
  const float q0 = xp * d.r1;
  const float r = __builtin_fmaf(-q0, d.sp, xp);
  float yq = __builtin_copysignf(__builtin_fmaf(r, d.r1, q0), x);
  constexpr float M = Fp8Fmt<FMT>::kMax;
  // a finite element whose quotient overflowed (x p, x r1 or the quotient
  // itself past the fp32 range: only under a scale the data has outgrown)
  // saturates like any other; an infinite one keeps an infinite quotient
  const bool x_fin = __builtin_isfinite(x);
  yq = x_fin ? (__builtin_isfinite(yq) ? yq : __builtin_copysignf(M, x)) : x;
  float y = yq;
  if constexpr (!PLAIN) {
    const float ys = s_inf ? x * 0.0f : ((x != x) ? x : __builtin_copysignf(0.0f, x));
    y = d.special ? ys : yq;
  }
  // (the median would turn a NaN into a bound: NaN and infinities pass)
  return __builtin_isfinite(y) ? __builtin_amdgcn_fmed3f(y, -M, M) : y;
}

template <int FMT, bool PLAIN = false>
__device__ __forceinline__ uint32_t given_encode4(float4 v, const Divisor& d, bool s_inf) {
  const float x[4] = {v.x, v.y, v.z, v.w};
  float y[4];
  // (the bytes of NaN quotients are set, 0x7F with x's sign in either
  // format, rather than taken from the conversion; for e4m3 this measured
  // 39.2-39.8 -> 33.9-34.6 us on 4096x8192 against handing the conversion
  // copysign(inf, x), whose compare-and-selects the compiler had serialised
  // with wait states)
  uint32_t nan_sel = 0, nan_bytes = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    y[e] = given_quotient<FMT, PLAIN>(x[e], d, s_inf);
    const bool nan = y[e] != y[e];
    nan_sel |= nan ? 0xFFu << (8 * e) : 0u;
    nan_bytes |= nan ? (0x7Fu | ((__float_as_uint(x[e]) >> 24) & 0x80u)) << (8 * e) : 0u;
    y[e] = nan ? 0.0f : y[e];
  }
  int w;
  if constexpr (FMT == FMT_E4M3) {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(y[0], y[1], 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(y[2], y[3], w, true);
  }
  return ((uint32_t)w & ~nan_sel) | nan_bytes;
}

// One wave: the window's maximum (NaN skipped), the scale, and the cleared
// entry for this step's amax.
template <int FMT>
__global__ void __launch_bounds__(64)
delayed_scale_kernel(float* __restrict__ history, int hist_len, int slot, float* scale) {
  float m = 0.0f;
  for (int i = threadIdx.x; i < hist_len; i += 64) m = __builtin_fmaxf(m, abs_or_zero(history[i]));
  for (int o = 32; o >= 1; o >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, o));
  if (threadIdx.x == 0) {
    scale[0] = m > 0.0f ? scale_of_fmt<FMT>(m) : 1.0f;
    history[slot] = 0.0f;
  }
}

// Rows blockIdx.y, blockIdx.y + gridDim.y, ... of the column range
// blockIdx.x * 1024 .. +1023, four rows loaded before any is encoded.
template <int FMT, bool PLAIN>
__device__ __forceinline__ float delayed_rows(const float* __restrict__ x, int64_t rows,
                                              int64_t ldx, uint8_t* __restrict__ q, int64_t ldq,
                                              int64_t c, const Divisor& d, bool s_inf) {
  float m = 0.0f;
  int64_t r = blockIdx.y;
  const int64_t step = gridDim.y;
  for (; r + 3 * step < rows; r += 4 * step) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = load4(x + (r + u * step) * ldx + c);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      m = amax4(v[u], m);
      *reinterpret_cast<uint32_t*>(q + (r + u * step) * ldq + c) =
          given_encode4<FMT, PLAIN>(v[u], d, s_inf);
    }
  }
  for (; r < rows; r += step) {
    const float4 v = load4(x + r * ldx + c);
    m = amax4(v, m);
    *reinterpret_cast<uint32_t*>(q + r * ldq + c) = given_encode4<FMT, PLAIN>(v, d, s_inf);
  }
  return m;
}
template <int FMT>
__global__ void __launch_bounds__(256)
delayed_encode_kernel(const float* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
                      uint8_t* __restrict__ q, int64_t ldq, const float* __restrict__ scale,
                      float* __restrict__ amax_out) {
  __shared__ float part[4];
  const float s = scale[0];
  const Divisor d = make_divisor(s);
  const bool s_inf = s == __builtin_inff();
  const int64_t c = (int64_t)blockIdx.x * 1024 + threadIdx.x * 4;
  float m = 0.0f;
  if (c < cols) {
    // (uniform: one scale for the whole tensor)
    if (!d.special && d.p == 1.0f) m = delayed_rows<FMT, true>(x, rows, ldx, q, ldq, c, d, s_inf);
    else m = delayed_rows<FMT, false>(x, rows, ldx, q, ldq, c, d, s_inf);
  }
  for (int o = 32; o >= 1; o >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = __builtin_fmaxf(__builtin_fmaxf(part[0], part[1]), __builtin_fmaxf(part[2], part[3]));
    max_into(amax_out, m);
  }
}

}  // namespace

hipError_t launch_quantize_delayed(const float* x, int64_t rows, int64_t cols, int64_t ldx,
                                   int fmt, float* history, int hist_len, int slot, uint8_t* q,
                                   int64_t ldq, float* scale, hipStream_t stream) {
  const int64_t gx = (cols + 1023) / 1024;
  // about 2048 workgroups (at most one atomic each), at least one row each
  const int64_t gy = std::max<int64_t>(1, std::min<int64_t>(rows, 2048 / gx));
  // (an empty matrix still takes its step: the scale is formed and the
  // entry for this step's amax is cleared, and stays 0)
  if (fmt == FMT_E4M3) {
    hipLaunchKernelGGL(delayed_scale_kernel<FMT_E4M3>, dim3(1), dim3(64), 0, stream, history,
                       hist_len, slot, scale);
    if (rows > 0 && cols > 0)
      hipLaunchKernelGGL(delayed_encode_kernel<FMT_E4M3>, dim3((unsigned)gx, (unsigned)gy),
                         dim3(256), 0, stream, x, rows, cols, ldx, q, ldq, (const float*)scale,
                         history + slot);
  } else {
    hipLaunchKernelGGL(delayed_scale_kernel<FMT_E5M2>, dim3(1), dim3(64), 0, stream, history,
                       hist_len, slot, scale);
    if (rows > 0 && cols > 0)
      hipLaunchKernelGGL(delayed_encode_kernel<FMT_E5M2>, dim3((unsigned)gx, (unsigned)gy),
                         dim3(256), 0, stream, x, rows, cols, ldx, q, ldq, (const float*)scale,
                         history + slot);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_tensor(const float* x, int64_t rows, int64_t cols, int64_t ldx,
                                  uint8_t* q, int64_t ldq, float* scale, hipStream_t stream) {
  const int64_t gx = (cols + 1023) / 1024;
  // about 1024 workgroups for the reduction (at most one atomic each), as many as
  // the rows allow for the encoding
  const int64_t gy_amax = std::max<int64_t>(1, std::min<int64_t>(rows, 1024 / gx));
  const int64_t gy_enc = std::max<int64_t>(1, std::min<int64_t>(rows, 65535));
  hipLaunchKernelGGL(tensor_zero_kernel, dim3(1), dim3(64), 0, stream, scale);
  hipLaunchKernelGGL(tensor_amax_kernel, dim3((unsigned)gx, (unsigned)gy_amax), dim3(256), 0,
                     stream, x, rows, cols, ldx, scale);
  hipLaunchKernelGGL(tensor_encode_kernel, dim3((unsigned)gx, (unsigned)gy_enc), dim3(256), 0,
                     stream, x, rows, cols, ldx, q, ldq, (const float*)scale);
  hipLaunchKernelGGL(tensor_scale_kernel, dim3(1), dim3(64), 0, stream, scale);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_quantize(const T* x, int64_t rows, int64_t cols, int64_t ldx,
                           int block_rows, uint8_t* q, int64_t ldq, float* scales,
                           int64_t s_stride_row, int64_t s_stride_col, hipStream_t stream,
                           int cu_count) {
  const int ncb = (int)((cols + 127) / 128);
  if constexpr (std::is_same<T, uint16_t>::value) {
    if (block_rows == 1 && (uintptr_t)x % 16 == 0 && ldx % 8 == 0) {
      const int64_t units = rows * ((ncb + 2 * BF16_LPL - 1) / (2 * BF16_LPL));
      int64_t grid = (units + 7) / 8;
      if (grid > 0x7FFFFFFF) grid = 0x7FFFFFFF;
      hipLaunchKernelGGL(quant_row_blocks_bf16x8_kernel<BF16_LPL>, dim3((unsigned)grid), dim3(256), 0,
                         stream, x, rows, cols, ldx, ncb, q, ldq, scales, s_stride_row,
                         s_stride_col);
      return hipGetLastError();
    }
  }
  if (block_rows == 1) {
    // One workgroup per 8 units, dispatched by the hardware as residency
    // frees up (the kernel's unit loop only matters past the launch limit):
    // 8-11% faster than a persistent grid of 8 workgroups per CU, which left
    // a part-full last round (27.7 vs 31.0 us on 4096x8192).
    const int64_t units = rows * ((ncb + QB - 1) / QB);
    int64_t grid = (units + 7) / 8;
    const int64_t cap = 0x7FFFFFFF;
    (void)cu_count;
    if (grid > cap) grid = cap;
    hipLaunchKernelGGL(quant_row_blocks_kernel<T>, dim3((unsigned)grid), dim3(256), 0, stream, x,
                       rows, cols, ldx, ncb, q, ldq, scales, s_stride_row, s_stride_col);
  } else {
    // One workgroup per block, dispatched by the hardware (three resident per
    // CU by registers; the block loop with its second register set only
    // runs past the launch limit): 4-11% faster than a persistent grid of
    // three workgroups per CU (59.5 vs 61.7 us on 8192x8192, 394.5 vs 443 us
    // on 32 x 7168x2048). A one-block kernel with half the registers and
    // twice the residency measured slower on the expert weights (215 vs
    // 203.5 us on 8 x 4096x7168).
    const int64_t blocks = ((rows + 127) / 128) * ncb;
    int64_t grid = blocks;
    const int64_t cap = 0x7FFFFFFF;
    if (grid > cap) grid = cap;
    if constexpr (std::is_same<T, uint16_t>::value) {
      if ((uintptr_t)x % 16 == 0 && ldx % 8 == 0 && (uintptr_t)q % 8 == 0 && ldq % 8 == 0) {
        hipLaunchKernelGGL(quant_tile_blocks_bf16x8_kernel, dim3((unsigned)grid), dim3(256), 0,
                           stream, x, rows, cols, ldx, ncb, q, ldq, scales, s_stride_row,
                           s_stride_col);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL(quant_tile_blocks_kernel<T>, dim3((unsigned)grid), dim3(256), 0, stream, x,
                       rows, cols, ldx, ncb, q, ldq, scales, s_stride_row, s_stride_col);
  }
  return hipGetLastError();
}

void quantize_kernels(std::vector<const void*>& out) {
  out.push_back(reinterpret_cast<const void*>(&quant_row_blocks_kernel<float>));
  out.push_back(reinterpret_cast<const void*>(&quant_row_blocks_kernel<uint16_t>));
  out.push_back(reinterpret_cast<const void*>(&quant_row_blocks_bf16x8_kernel<BF16_LPL>));
  out.push_back(reinterpret_cast<const void*>(&quant_tile_blocks_kernel<float>));
  out.push_back(reinterpret_cast<const void*>(&quant_tile_blocks_kernel<uint16_t>));
  out.push_back(reinterpret_cast<const void*>(&quant_tile_blocks_bf16x8_kernel));
  out.push_back(reinterpret_cast<const void*>(&tensor_zero_kernel));
  out.push_back(reinterpret_cast<const void*>(&tensor_amax_kernel));
  out.push_back(reinterpret_cast<const void*>(&tensor_encode_kernel));
  out.push_back(reinterpret_cast<const void*>(&tensor_scale_kernel));
  out.push_back(reinterpret_cast<const void*>(&delayed_scale_kernel<FMT_E4M3>));
  out.push_back(reinterpret_cast<const void*>(&delayed_scale_kernel<FMT_E5M2>));
  out.push_back(reinterpret_cast<const void*>(&delayed_encode_kernel<FMT_E4M3>));
  out.push_back(reinterpret_cast<const void*>(&delayed_encode_kernel<FMT_E5M2>));
}

template hipError_t launch_quantize<float>(const float*, int64_t, int64_t, int64_t, int, uint8_t*,
                                           int64_t, float*, int64_t, int64_t, hipStream_t, int);
template hipError_t launch_quantize<uint16_t>(const uint16_t*, int64_t, int64_t, int64_t, int,
                                              uint8_t*, int64_t, float*, int64_t, int64_t,
                                              hipStream_t, int);

}  // namespace fp8g
