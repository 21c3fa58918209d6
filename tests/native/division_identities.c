/* Exhaustive checks of the two division identities the quantisers rely on,
 * in IEEE single precision with a fused multiply-add (any IEEE 754 machine
 * gives the same bits):
 *
 *  1. scale: for every finite amax >= 2^-100,
 *       RN(amax / 448) == RN(RN(amax * y7) + fma(-RN(amax * y7), 7, amax) * y7) * 2^-6
 *     with y7 = RN(1/7)   (448 = 7 * 2^6; Markstein's correction for the /7);
 *  2. quotient: for a scale s in [2^-80, 2^100] and r1 = RN(1/s),
 *       RN(x / s) == RN(q0 + fma(-q0, s, x) * r1),  q0 = RN(x * r1)
 *     for every positive x whose quotient lies in [2^-21, 449] (the range in
 *     which an e4m3 code can depend on the quotient's last bits; negative x
 *     mirror it, and the kernels take the sign from x);
 *  3. the same for scales outside that range once x and s are both scaled
 *     by the power of two p (2^100 for s < 2^-80, 2^-64 for s > 2^100):
 *     every positive x with x / s in [2^-21, 449] (x subnormal included),
 *     and under huge scales every x below that range must still give a
 *     quotient below 2^-10 (an e4m3 zero).
 *
 * Usage: division_identities [number of random scales]. Prints the number
 * of mismatches and exits 0 only if there are none. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static long check_scale(void) {
  const float y7 = 1.0f / 7.0f;
  long bad = 0;
  for (uint32_t u = f2u(0x1p-100f); u < 0x7f800000u; ++u) {
    const float m = u2f(u);
    const float q0 = m * y7;
    const float q = fmaf(fmaf(-q0, 7.0f, m), y7, q0) * 0x1p-6f;
    if (f2u(q) != f2u(m / 448.0f)) ++bad;
  }
  return bad;
}

static long check_quotient(float s) {
  const float r1 = 1.0f / s;
  long bad = 0;
  const uint32_t lo = f2u(s * 0x1p-21f), hi = f2u(s * 449.0f);
  for (uint32_t u = lo; u <= hi; ++u) {
    const float x = u2f(u);
    const float q0 = x * r1;
    const float q = fmaf(fmaf(-q0, s, x), r1, q0);
    if (f2u(q) != f2u(x / s)) ++bad;
  }
  return bad;
}

static float prescale_of(float s) { return s < 0x1p-80f ? 0x1p100f : (s > 0x1p100f ? 0x1p-64f : 1.0f); }

static long check_quotient_prescaled(float s) {
  const float p = prescale_of(s);
  const float sp = s * p;
  const float r1 = 1.0f / sp;
  long bad = 0;
  uint32_t lo = f2u(s * 0x1p-21f), hi = f2u(s * 449.0f);
  if (lo == 0) lo = 1;
  if (hi > 0x7f7fffffu) hi = 0x7f7fffffu;    /* finite x only (an infinity makes s infinite) */
  for (uint32_t u = lo; u <= hi; ++u) {
    const float x = u2f(u);
    const float xp = x * p;
    const float q0 = xp * r1;
    const float q = fmaf(fmaf(-q0, sp, xp), r1, q0);
    if (f2u(q) != f2u(x / s)) ++bad;
  }
  /* below the range: the prescaled quotient stays an e4m3 zero */
  for (uint32_t u = 1; u < lo; u += 1 + (lo >> 16)) {
    const float x = u2f(u);
    const float xp = x * p;
    const float q0 = xp * r1;
    const float q = fmaf(fmaf(-q0, sp, xp), r1, q0);
    if (!(q < 0x1p-10f)) ++bad;
  }
  return bad;
}

int main(int argc, char** argv) {
  const int n_random = argc > 1 ? atoi(argv[1]) : 4;
  /* the range ends, significands next to 1 and 2, and the 1/448 neighbourhood */
  const uint32_t fixed[] = {0x17800000u, 0x717fffffu, 0x3f800001u, 0x3fffffffu,
                            0x3f7fffffu, 0x3b124925u, 0x3c23d70au, 0x40490fdbu};
  long bad = check_scale();
  printf("scale identity: %ld mismatches\n", bad);
  srand(20241202);
  for (int k = 0; k < (int)(sizeof(fixed) / 4) + n_random; ++k) {
    uint32_t us;
    if (k < (int)(sizeof(fixed) / 4)) {
      us = fixed[k];
    } else {
      us = ((((uint32_t)rand() << 16) ^ (uint32_t)rand()) & 0x007fffffu) |
           ((uint32_t)(47 + rand() % 181) << 23);            /* 2^-80 .. 2^100 */
    }
    const long b = check_quotient(u2f(us));
    printf("quotient identity, s = %08x: %ld mismatches\n", us, b);
    bad += b;
  }
  /* scales outside [2^-80, 2^100]: subnormal ones (down to the smallest),
   * 2^-126, just below 2^-80, just above 2^100, and the largest scale a
   * finite amax gives (RN(FLT_MAX / 448)); then random ones on both sides */
  const uint32_t extreme[] = {0x00000001u, 0x00000abcu, 0x007fffffu, 0x00800000u,
                              0x177fffffu, 0x71800001u, 0x7b000000u};
  const float smax = 0x1.fffffep127f / 448.0f;
  for (int k = 0; k < (int)(sizeof(extreme) / 4) + 1 + 2 * n_random; ++k) {
    uint32_t us;
    if (k < (int)(sizeof(extreme) / 4)) {
      us = extreme[k];
    } else if (k == (int)(sizeof(extreme) / 4)) {
      us = f2u(smax);
    } else {
      const uint32_t mant = (((uint32_t)rand() << 16) ^ (uint32_t)rand()) & 0x007fffffu;
      us = (k & 1) ? (mant | ((uint32_t)(1 + rand() % 46) << 23))          /* 2^-126 .. 2^-81 */
                   : (mant | ((uint32_t)(228 + rand() % 19) << 23));       /* 2^101 .. 2^119 */
      if (u2f(us) > smax) us = f2u(smax);
    }
    const long b = check_quotient_prescaled(u2f(us));
    printf("prescaled quotient identity, s = %08x: %ld mismatches\n", us, b);
    bad += b;
  }
  printf("total mismatches %ld\n", bad);
  return bad == 0 ? 0 : 1;
}
