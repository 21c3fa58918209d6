"""Pins of the oracle's number formats against facts that do not come from it.

* the constants the pages print (tests/golden/page_constants.txt);
* closed forms of the OCP e4m3 / e5m2 layouts;
* independent library conversions: torch's float8_e4m3fn and bfloat16
  casts (float32 -> target, round to nearest even, non-saturating);
* exact rational rounding (fractions.Fraction) for fp64 -> bf16.
"""

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import (E4M3_MAX, e4m3_decode_table, e4m3_encode_rne,
                    bf16_bits_from_f64, bf16_bits_to_f64)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _page_constants():
    out = {}
    with open(os.path.join(GOLDEN, "page_constants.txt")) as f:
        for line in f:
            line = line.split("|")[0].strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split()
            out[k] = float(v)
    return out


def test_table_matches_page_constants():
    pc = _page_constants()
    t = e4m3_decode_table()
    finite = t[np.isfinite(t)]
    assert finite.max() == pc["e4m3_max_finite"] == E4M3_MAX
    assert finite.min() == -pc["e4m3_max_finite"]
    # exponent / mantissa widths printed on the pages: 4 + 3 (+ sign) = 8 bits,
    # and the largest finite value is (1 + 6/8) * 2^(15 - 7) with the all-ones
    # exponent and mantissa 111 kept for NaN.
    e, m = int(pc["e4m3_exponent_bits"]), int(pc["e4m3_mantissa_bits"])
    assert 1 + e + m == 8
    assert (1 + 6 / 2 ** m) * 2.0 ** (2 ** e - 1 - 7) == 448.0
    # e5m2 (1-5-2, bias 15, IEEE-style infinities): max (1 + 3/4) * 2^15
    assert (1 + 3 / 4) * 2.0 ** 15 == pc["e5m2_max_finite"]
    assert float(torch.finfo(torch.float8_e5m2).max) == pc["e5m2_max_finite"]
    assert float(np.finfo(np.float16).max) == pc["fp16_max_finite"]
    bf16_max = bf16_bits_to_f64(np.uint16(0x7F7F))
    assert abs(bf16_max - pc["bf16_max_finite_approx"]) / bf16_max < 0.002
    assert pc["scale_divisor"] == E4M3_MAX


def test_table_structure():
    t = e4m3_decode_table()
    nan_codes = [c for c in range(256) if np.isnan(t[c])]
    assert nan_codes == [0x7F, 0xFF]
    assert np.isfinite(t).sum() == 254
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x01] == 2.0 ** -9          # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert t[0x08] == 2.0 ** -6          # smallest normal
    assert t[0x38] == 1.0                # exponent field 7 = bias
    pos = t[0:0x7F]
    assert np.all(np.diff(pos) > 0)      # monotone over 0x00..0x7E
    assert np.all(t[0x80:0xFF] == -pos)  # sign-magnitude mirror
    assert np.signbit(t[0x80]) and not np.signbit(t[0x00])


def test_table_matches_torch_float8():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    t = e4m3_decode_table()
    assert np.array_equal(np.isnan(ref), np.isnan(t))
    ok = ~np.isnan(t)
    assert np.array_equal(ref[ok], t[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(t[ok]))


def _torch_e4m3(y):
    return torch.from_numpy(np.asarray(y, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_roundtrip_all_codes():
    t = e4m3_decode_table()
    for c in range(256):
        if np.isnan(t[c]):
            continue
        assert e4m3_encode_rne(np.float32(t[c])) == c, hex(c)


def test_encode_midpoints_go_to_even():
    t = e4m3_decode_table()
    pos = t[0:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2              # exact in fp64 and fp32
    codes = e4m3_encode_rne(mids.astype(np.float32))
    lo = np.arange(0, 0x7E)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(codes, expect.astype(np.uint8))
    assert np.array_equal(e4m3_encode_rne(-mids.astype(np.float32)), (expect | 0x80).astype(np.uint8))
    # one fp32 ulp either side of each midpoint decides by distance
    up = np.nextafter(mids.astype(np.float32), np.float32(np.inf))
    dn = np.nextafter(mids.astype(np.float32), np.float32(0))
    assert np.array_equal(e4m3_encode_rne(up), (lo + 1).astype(np.uint8))
    assert np.array_equal(e4m3_encode_rne(dn), lo.astype(np.uint8))


def test_encode_overflow_and_specials():
    f = np.float32
    assert e4m3_encode_rne(f(0.0)) == 0x00
    assert e4m3_encode_rne(f(-0.0)) == 0x80
    assert e4m3_encode_rne(f(-(2.0 ** -11))) == 0x80    # rounds to -0, keeps sign
    assert e4m3_encode_rne(f(2.0 ** -10)) == 0x00       # tie between 0 and 2^-9 -> even 0
    assert e4m3_encode_rne(f(3 * 2.0 ** -10)) == 0x02   # tie 2^-9 / 2^-8 -> even 0x02
    assert e4m3_encode_rne(f(3 * 2.0 ** -11)) == 0x01   # 0.75 * 2^-9 -> nearest 2^-9
    assert e4m3_encode_rne(f(448.0)) == 0x7E
    assert e4m3_encode_rne(f(460.0)) == 0x7E
    assert e4m3_encode_rne(f(464.0)) == 0x7E            # tie with the missing 480 -> 448
    assert e4m3_encode_rne(np.nextafter(f(464.0), f(1e9))) == 0x7F
    assert e4m3_encode_rne(f(-1e6)) == 0xFF
    assert e4m3_encode_rne(f(np.inf)) == 0x7F
    assert e4m3_encode_rne(f(-np.inf)) == 0xFF
    assert e4m3_encode_rne(f(np.nan)) == 0x7F


def test_encode_matches_torch_near_every_midpoint():
    t = e4m3_decode_table()
    pos = t[0:0x7F]
    mids = np.concatenate([(pos[:-1] + pos[1:]) / 2, [464.0], pos])
    bits = mids.astype(np.float32).view(np.int32).astype(np.int64)
    off = np.arange(-3000, 3001, dtype=np.int64)
    cand = (bits[:, None] + off[None, :]).ravel()
    cand = cand[(cand >= 0) & (cand < 0x7F800000)]
    y = cand.astype(np.int32).view(np.float32)
    y = np.concatenate([y, -y])
    assert np.array_equal(e4m3_encode_rne(y), _torch_e4m3(y))


def test_encode_matches_torch_random_patterns():
    rng = np.random.default_rng(1234)
    # every fp32 pattern class: uniform over bit patterns up to 480, plus a
    # uniform draw of magnitudes in [0, 470]
    hi = np.float32(480.0).view(np.int32)
    pats = rng.integers(0, int(hi), 2_000_000, dtype=np.int64).astype(np.int32)
    y = pats.view(np.float32)
    y = np.concatenate([y, -y, rng.uniform(-470, 470, 1_000_000).astype(np.float32)])
    assert np.array_equal(e4m3_encode_rne(y), _torch_e4m3(y))


def _bf16_exact(v: Fraction) -> int:
    """Round an exact rational to bf16 (RNE) from first principles."""
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                     # subnormal grid below 2^-126
    ulp = Fraction(2) ** (e - 7)
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * ulp
    if r > (2 - Fraction(1, 128)) * Fraction(2) ** 127:
        return sign | 0x7F80
    bits = int(np.float32(float(r)).view(np.uint32)) >> 16
    return sign | bits


def test_bf16_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(7)
    pats = rng.integers(0, 0x7F800000, 2_000_000, dtype=np.int64).astype(np.uint32)
    y = pats.view(np.float32)
    y = np.concatenate([y, -y, np.float32([0.0, -0.0, 3.3895314e38, 3.40e38, 1e-45, 1.2e-38])])
    ref = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = bf16_bits_from_f64(y.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_direct_from_f64_is_exact_rne():
    rng = np.random.default_rng(11)
    vals = list(rng.standard_normal(400) * 10.0 ** rng.integers(-40, 38, 400))
    # values a hair off a bf16 midpoint: a detour through fp32 would double-round
    for base in (1.0, 3.0, 1e-3, 7e20):
        b = np.float64(base)
        mid = float(bf16_bits_to_f64(bf16_bits_from_f64(b))) * (1 + 2.0 ** -8)
        vals += [mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf),
                 mid * (1 + 2.0 ** -30), mid * (1 - 2.0 ** -30)]
    vals += [2.0 ** -130 * 1.5, 2.0 ** -133 * 0.5, 2.0 ** -133 * 1.5, 3.39e38, 3.4e38, 3.5e38]
    got = bf16_bits_from_f64(np.array(vals))
    for v, g in zip(vals, got):
        assert int(g) == _bf16_exact(Fraction(float(v))), v
