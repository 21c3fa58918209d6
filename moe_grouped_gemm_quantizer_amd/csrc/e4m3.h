// e4m3 encoding shared by the quantiser kernels and the GEMM's fused
// quantising epilogue: the per-block scale and the element rule, so that
// both produce the same bits for the same fp32 values. See quantize.hip for
// the method and the division identities.
#pragma once

#include "internal.h"

namespace fp8g {
namespace e4m3 {

constexpr float kE4M3Max = 448.0f;

// Per-block divisor. The element step needs RN(x / s), the correctly
// rounded IEEE quotient. For s in [2^-80, 2^100] it is formed from the
// block's correctly rounded reciprocal r1 = RN(1/s) by Markstein's
// correction (q0 = RN(x r1), r = x - q0 s exactly by FMA, q = RN(q0 + r r1)),
// which equals RN(x / s) for every quotient that can reach an e4m3 code's
// last bit. Other finite nonzero scales are first brought into that range
// by a power of two p applied to x and s alike (2^100 below 2^-80, 2^-64
// above 2^100), which leaves the quotient unchanged: s p is exact there,
// and so is x p except for |x| < 2^-62 under a huge scale, where the
// quotient is below 2^-162 and encodes to a signed zero either way. A zero
// scale (all-zero block) and an infinite one (a block holding an infinity)
// both need x * 0: a signed zero for finite x and NaN for NaN or infinite x,
// which is what x / inf gives and what a zero block's codes are. The same
// steps give exactly that with r1 = 0 and sp = 1 (q0 = x p * 0, then r = x p,
// then r * 0 + q0, signed like x): x p stays finite for finite x (p = 2^-64
// under an infinite scale; a zero scale's block holds only zeros and NaN),
// so no per-element select is needed.
struct Divisor {
  float s;       // the block scale (what is stored)
  float sp;      // s * p, in [2^-80, 2^100] (1 for a zero or infinite scale)
  float r1;      // RN(1 / sp)
  float p;       // the power of two
  bool special;  // zero or infinite scale (then sp = 1, r1 = 0)
};
// s = RN(amax / 448). 448 = 7 * 2^6, so for amax >= 2^-100 (and finite)
// s = RN(amax / 7) * 2^-6 exactly, and RN(amax / 7) is Markstein's
// correction against the constant RN(1/7); this identity was checked
// against the IEEE division for every fp32 amax in that range. Smaller (or
// infinite) amax take the IEEE division.
__device__ __forceinline__ float scale_of(float amax) {
  constexpr float y7 = 1.0f / 7.0f;
  if (__builtin_expect(amax >= 0x1p-100f && amax <= 0x1.fffffep127f, 1)) {
    const float q0 = amax * y7;
    const float r = __builtin_fmaf(-q0, 7.0f, amax);
    return __builtin_fmaf(r, y7, q0) * 0x1p-6f;
  }
  return amax / kE4M3Max;
}

__device__ __forceinline__ Divisor make_divisor(float s) {
  Divisor d;
  d.s = s;
  d.special = !(s > 0.0f) || s == __builtin_inff();        // (s is never negative or NaN)
  d.p = s < 0x1p-80f ? 0x1p100f : (s > 0x1p100f ? 0x1p-64f : 1.0f);
  d.sp = d.special ? 1.0f : s * d.p;
  d.r1 = d.special ? 0.0f : 1.0f / d.sp;
  return d;
}

// Element step, branch-free: y = RN(x / s) (x * 0 for a zero or infinite
// scale, through r1 = 0), saturated to [-448, 448]. A NaN quotient (x NaN, or inf / inf)
// must give the code 0x7F | sign(x); the hardware conversion turns every NaN
// input into 0xFF but converts an infinity into the NaN code of its own
// sign, so it is handed copysign(inf, x). The sign always comes from x (the
// correction would turn -0 into +0).
__device__ __forceinline__ float quotient(float x, const Divisor& d) {
  const float xp = x * d.p;
  const float q0 = xp * d.r1;
  const float r = __builtin_fmaf(-q0, d.sp, xp);
  const float y = __builtin_copysignf(__builtin_fmaf(r, d.r1, q0), x);
  const float yc = __builtin_amdgcn_fmed3f(y, -kE4M3Max, kE4M3Max);
  const float qnan = __builtin_copysignf(__builtin_inff(), x);
  return (y != y) ? qnan : yc;
}

// Four codes from four values: gfx950's v_cvt_pk_fp8_f32 converts two fp32
// values to OCP e4m3 with round-to-nearest-even (bytes 0,1 then 2,3). Inputs
// are already saturated, so its overflow behaviour never matters; the GPU
// tests check the result bit for bit against the oracle's encoder (every
// e4m3 midpoint neighbourhood, the subnormal range, random patterns).
__device__ __forceinline__ uint32_t encode4(float4 v, const Divisor& d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(quotient(v.x, d), quotient(v.y, d), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(quotient(v.z, d), quotient(v.w, d), w, true);
  return (uint32_t)w;
}

// Running block amax, NaN elements skipped. A maximum with one quiet-NaN
// operand returns the other operand, but a signalling NaN operand may come
// out as a quiet NaN, and the next maximum would then drop everything
// reduced before it; so every |x| is canonicalised first (one v_max_f32 of
// the value with itself, which quiets a signalling NaN), and no maximum ever
// sees a signalling NaN. (Measured: about 2% on the fp32 1x128 kernel,
// against 5% for mapping NaN to 0 by a compare and select.)
__device__ __forceinline__ float abs_or_zero(float x) {
  return __builtin_canonicalizef(__builtin_fabsf(x));
}
__device__ __forceinline__ float amax4(float4 v, float m) {
  m = __builtin_fmaxf(m, abs_or_zero(v.x));
  m = __builtin_fmaxf(m, abs_or_zero(v.y));
  m = __builtin_fmaxf(m, abs_or_zero(v.z));
  m = __builtin_fmaxf(m, abs_or_zero(v.w));
  return m;
}

}  // namespace e4m3
}  // namespace fp8g
