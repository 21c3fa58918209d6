"""Number formats used by the oracle: FP8 e4m3 and e5m2, bf16 (test infrastructure).

e4m3 follows the OCP 8-bit float definition that the gtnt page names in its
E4M3-vs-E5M2 part: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits, no
infinities, NaN only where exponent and mantissa bits are all ones, largest
finite magnitude 448 (also the e4m3 row of the format table in
czchanglian §2.1). Conversions round to nearest with ties to even, the default
the nxmr page gives for FP8 conversion (§5.1).

e5m2 is the other 8-bit format of the same pages (czchanglian §2.1 table and
the gtnt E4M3-vs-E5M2 part: 5 exponent bits, 2 mantissa bits, largest finite
value 57344, meant for gradients): OCP e5m2 is laid out like IEEE binary16
cut to 8 bits, bias 15, with infinities (exponent all ones, mantissa 0) and
NaNs (exponent all ones, mantissa non-zero).

bf16 (czchanglian §2.1 table: 8 exponent bits, 7 stored mantissa bits) is the
output format; the oracle rounds to it directly from fp64, once.
"""

import numpy as np

E4M3_MAX = 448.0  # largest finite e4m3 magnitude (czchanglian §2.1; gtnt E4M3 vs E5M2)
E4M3_NAN = 0x7F   # exponent 1111 with mantissa 111; 0xFF is its negative twin


def e4m3_decode_table():
    """Real value of each of the 256 e4m3 codes, as float64 (NaN for 0x7F/0xFF).

    Built field by field from the format definition: exponent field 0 gives
    the subnormals m/8 * 2^-6, other exponent fields give (1 + m/8) * 2^(e-7).
    """
    table = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            val = np.nan
        elif e == 0:
            val = (m / 8.0) * 2.0 ** -6
        else:
            val = (1.0 + m / 8.0) * 2.0 ** (e - 7)
        table[code] = sign * val
    return table


_TABLE = e4m3_decode_table()
# Non-negative finite codes 0x00..0x7E in increasing order of value.
_POS = _TABLE[0:0x7F].copy()


def e4m3_encode_rne(y):
    """Encode float32 values as e4m3 codes, round to nearest, ties to even.

    * The nearest representable magnitude is found by comparing distances in
      float64, where every float32 input, every e4m3 value and every midpoint
      between neighbours is exact.
    * A tie goes to the code whose mantissa LSB is 0.
    * The sign bit is kept, also when the magnitude rounds to zero.
    * Magnitudes in (448, 464] round to 448 (464 is the tie between 448 and
      the missing next step 480, and 448 has the even mantissa); magnitudes
      above 464, infinities and NaN give the NaN code with the input's sign.
      This is the non-saturating overflow the czchanglian page warns about
      in §2.1; the quantiser never reaches it (see quantize.py).
    """
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y.astype(np.float64))
    sign = (np.signbit(y).astype(np.uint8) << 7).astype(np.uint8)
    finite = np.isfinite(a)
    a_f = np.where(finite, a, 0.0)
    # idx: the largest code whose value is <= a (clipped to the last finite code)
    idx = np.searchsorted(_POS, a_f, side="right") - 1
    idx = np.clip(idx, 0, 0x7E)
    nxt = np.minimum(idx + 1, 0x7E)
    d_lo = a_f - _POS[idx]
    d_hi = _POS[nxt] - a_f
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (idx % 2 == 1))
    take_hi &= nxt != idx
    code = np.where(take_hi, nxt, idx).astype(np.uint8)
    overflow = (~finite) | (a > 464.0)
    code = np.where(overflow, np.uint8(E4M3_NAN), code).astype(np.uint8)
    return (code | sign).astype(np.uint8)


E5M2_MAX = 57344.0  # largest finite e5m2 magnitude (czchanglian §2.1; gtnt E4M3 vs E5M2)
E5M2_INF = 0x7C     # exponent 11111, mantissa 00
E5M2_NAN = 0x7F     # the NaN code the quantiser writes (mantissa 11), sign from the input


def e5m2_decode_table():
    """Real value of each of the 256 e5m2 codes, as float64.

    Field by field: exponent field 0 gives the subnormals m/4 * 2^-14, fields
    1..30 give (1 + m/4) * 2^(e-15), field 31 gives infinity (m = 0) or NaN.
    """
    table = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 2) & 0x1F
        m = code & 0x3
        if e == 0x1F:
            val = np.inf if m == 0 else np.nan
        elif e == 0:
            val = (m / 4.0) * 2.0 ** -14
        else:
            val = (1.0 + m / 4.0) * 2.0 ** (e - 15)
        table[code] = sign * val
    return table


_TABLE5 = e5m2_decode_table()
_POS5 = _TABLE5[0:0x7C].copy()          # non-negative finite codes 0x00..0x7B, increasing


def e5m2_encode_rne(y):
    """Encode float32 values as e5m2 codes, round to nearest, ties to even.

    The same nearest-value search as e4m3_encode_rne, over the finite e5m2
    values. Magnitudes from 61440 (the tie between 57344 and the next step
    65536, which goes to the even mantissa, i.e. out of range) up, and
    infinities, give the infinity code with the input's sign, as an IEEE
    conversion overflows; NaN gives E5M2_NAN with the input's sign. The
    quantiser saturates first, so it never overflows.
    """
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y.astype(np.float64))
    sign = (np.signbit(y).astype(np.uint8) << 7).astype(np.uint8)
    nan = np.isnan(a)
    a_f = np.where(np.isfinite(a), a, 0.0)
    idx = np.searchsorted(_POS5, a_f, side="right") - 1
    idx = np.clip(idx, 0, 0x7B)
    nxt = np.minimum(idx + 1, 0x7B)
    d_lo = a_f - _POS5[idx]
    d_hi = _POS5[nxt] - a_f
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (idx % 2 == 1))
    take_hi &= nxt != idx
    code = np.where(take_hi, nxt, idx).astype(np.uint8)
    overflow = np.isinf(a) | (a >= 61440.0)
    code = np.where(overflow, np.uint8(E5M2_INF), code)
    code = np.where(nan, np.uint8(E5M2_NAN), code).astype(np.uint8)
    return (code | sign).astype(np.uint8)


FORMATS = {
    # name: (largest finite value, decode table, encoder)
    "e4m3": (E4M3_MAX, _TABLE, e4m3_encode_rne),
    "e5m2": (E5M2_MAX, _TABLE5, e5m2_encode_rne),
}


def bf16_bits_from_f64(v):
    """Round float64 values to bf16 (round to nearest, ties to even) -> uint16 bits.

    Rounded once, straight from float64: normal results keep 8 significant
    bits (frexp + rint), results below 2^-126 are rounded on the subnormal
    grid of spacing 2^-133, results past the largest finite bf16 by half an
    ulp or more become infinity, NaN becomes the quiet NaN 0x7FC0.
    """
    v = np.asarray(v, dtype=np.float64)
    nan = np.isnan(v)
    vv = np.where(nan, 0.0, v)
    mant, ex = np.frexp(vv)                     # vv = mant * 2^ex, |mant| in [0.5, 1)
    normal = np.abs(vv) >= 2.0 ** -126
    r_norm = np.ldexp(np.rint(np.ldexp(mant, 8)), ex - 8)
    r_sub = np.ldexp(np.rint(np.ldexp(vv, 133)), -133)
    r = np.where(normal, r_norm, r_sub)
    bf16_max = (2.0 - 2.0 ** -7) * 2.0 ** 127
    with np.errstate(over="ignore"):
        r = np.where(np.abs(r) > bf16_max, np.copysign(np.inf, r), r)
        bits32 = r.astype(np.float32).view(np.uint32)   # exact: r is a bf16 value
    bits = (bits32 >> 16).astype(np.uint16)
    return np.where(nan, np.uint16(0x7FC0), bits).astype(np.uint16)


def bf16_bits_to_f64(bits):
    """Exact float64 value of bf16 bit patterns."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
