"""Pins of the oracle's e5m2 format, e5m2 quantisation, delayed scaling and
the mixed-format per-tensor GEMM, against facts that do not come from the
oracle: the OCP e5m2 layout in closed form, torch's float8_e5m2 decode and
cast (float32 -> e5m2, round to nearest even), a float32 torch re-derivation
of the quantiser, exact rationals for the GEMM, and special cases that
reduce delayed scaling to the already pinned per-tensor quantiser.

Page facts: e5m2 has 5 exponent and 2 mantissa bits and a largest finite
value of 57344, for gradients and wide-range data (czchanglian §2.1 table;
gtnt E4M3-vs-E5M2 part); delayed scaling runs a step with the scale
gathered before it (czchanglian §2.3).
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import (E5M2_MAX, e5m2_decode_table, e5m2_encode_rne, e4m3_decode_table,
                    quantize_blocks, delayed_scale, tensor_amax, quantize_with_scale,
                    quantize_delayed, gemm_pertensor, bf16_bits_from_f64)

T5 = e5m2_decode_table()
T4 = e4m3_decode_table()


def _torch_e5m2(y):
    return torch.from_numpy(np.asarray(y, np.float32)).to(torch.float8_e5m2).view(torch.uint8).numpy()


# ---------------------------------------------------------------------------
# format


def test_e5m2_table_closed_form():
    assert T5[0x7B] == E5M2_MAX == (1 + 3 / 4) * 2.0 ** 15
    assert T5[0x01] == 2.0 ** -16            # smallest subnormal (1/4 * 2^-14)
    assert T5[0x03] == 3 * 2.0 ** -16        # largest subnormal
    assert T5[0x04] == 2.0 ** -14            # smallest normal
    assert T5[0x3C] == 1.0                   # exponent field 15 = bias
    assert T5[0x7C] == np.inf and T5[0xFC] == -np.inf
    assert [c for c in range(256) if np.isnan(T5[c])] == [0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF]
    pos = T5[0:0x7C]
    assert np.all(np.diff(pos) > 0)
    assert np.all(T5[0x80:0xFC] == -pos)
    # e5m2 is binary16 cut to its top byte: every code's value equals the
    # fp16 value of the pattern code << 8
    f16 = (np.arange(256, dtype=np.uint16) << 8).view(np.float16).astype(np.float64)
    ok = ~np.isnan(T5)
    assert np.array_equal(f16[ok], T5[ok]) and np.array_equal(np.isnan(f16), np.isnan(T5))


def test_e5m2_table_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e5m2).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ref), np.isnan(T5))
    ok = ~np.isnan(T5)
    assert np.array_equal(ref[ok], T5[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(T5[ok]))


def test_e5m2_encode_roundtrip_midpoints_and_specials():
    for c in range(256):
        if not np.isnan(T5[c]):
            assert e5m2_encode_rne(np.float32(T5[c])) == c, hex(c)
    pos = T5[0:0x7C]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    lo = np.arange(0, 0x7B)
    assert np.array_equal(e5m2_encode_rne(mids), np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8))
    f = np.float32
    assert e5m2_encode_rne(f(61440.0)) == 0x7C                 # tie with 65536: even -> inf
    assert e5m2_encode_rne(np.nextafter(f(61440.0), f(0))) == 0x7B
    assert e5m2_encode_rne(f(-np.inf)) == 0xFC
    assert e5m2_encode_rne(f(np.nan)) == 0x7F
    assert e5m2_encode_rne(-f(np.nan)) == 0xFF
    assert e5m2_encode_rne(f(-0.0)) == 0x80
    assert e5m2_encode_rne(f(2.0 ** -17)) == 0x00              # tie 0 / 2^-16 -> even 0


def test_e5m2_encode_matches_torch():
    pos = T5[0:0x7C]
    mids = np.concatenate([(pos[:-1] + pos[1:]) / 2, pos, [61440.0]])
    bits = mids.astype(np.float32).view(np.int32).astype(np.int64)
    off = np.arange(-2000, 2001, dtype=np.int64)
    cand = (bits[:, None] + off[None, :]).ravel()
    cand = cand[(cand >= 0) & (cand < 0x7F800000)]
    y = cand.astype(np.int32).view(np.float32)
    rng = np.random.default_rng(99)
    y = np.concatenate([y, rng.integers(0, 0x7F800000, 1_000_000).astype(np.int32).view(np.float32)])
    y = np.concatenate([y, -y])
    got, ref = e5m2_encode_rne(y), _torch_e5m2(y)
    # torch's cast keeps the finite results and infinities bit for bit
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------------------
# e5m2 block quantisation


def _torch_quantize_e5m2(x, br, bc=128):
    xt = torch.from_numpy(np.ascontiguousarray(x))
    R, C = xt.shape
    q = torch.empty((R, C), dtype=torch.uint8)
    s = torch.empty((-(-R // br), -(-C // bc)), dtype=torch.float32)
    for i in range(s.shape[0]):
        for j in range(s.shape[1]):
            blk = xt[i * br:(i + 1) * br, j * bc:(j + 1) * bc]
            sc = blk.abs().max() / torch.tensor(57344.0, dtype=torch.float32)
            s[i, j] = sc
            y = (blk / sc).clamp(-57344.0, 57344.0)
            q[i * br:(i + 1) * br, j * bc:(j + 1) * bc] = y.to(torch.float8_e5m2).view(torch.uint8)
    return q.numpy(), s.numpy()


@pytest.mark.parametrize("br", [1, 128])
def test_e5m2_blocks_match_torch_rederivation(br):
    rng = np.random.default_rng(11 + br)
    x = (rng.standard_normal((200, 300)) * np.exp(rng.uniform(-8, 8, (200, 1)))).astype(np.float32)
    q, s = quantize_blocks(x, br, fmt="e5m2")
    qt, st = _torch_quantize_e5m2(x, br)
    assert np.array_equal(s.view(np.uint32), st.view(np.uint32))
    assert np.array_equal(q, qt)
    # every block holds +-57344 (its amax element), and no code is infinite
    d = T5[q]
    assert np.all(np.isfinite(d))
    assert np.max(np.abs(d)) == E5M2_MAX


# ---------------------------------------------------------------------------
# delayed scaling


def test_delayed_with_current_amax_is_per_tensor_quantisation():
    """History holding exactly this step's amax: the delayed scale equals the
    per-tensor scale, so the codes equal the per-tensor quantiser's (one block
    covering the whole matrix), which the oracle pins elsewhere."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 384)) * 5).astype(np.float32)
    for fmt in ("e4m3", "e5m2"):
        q_pt, s_pt = quantize_blocks(x, x.shape[0], x.shape[1], fmt=fmt)
        q, s, hist = quantize_delayed(x, [float(np.abs(x).max())], 0, fmt)
        assert np.float32(s).view(np.uint32) == s_pt[0, 0].view(np.uint32)
        assert np.array_equal(q, q_pt)
        assert hist[0] == np.abs(x).max()


def test_delayed_scale_is_window_max_over_fmt_max():
    h = np.array([3.0, 0.0, 7.5, np.nan, 1.0], np.float32)
    assert delayed_scale(h, "e4m3") == np.float32(Fraction(15, 2) / 448)
    assert delayed_scale(h, "e5m2") == np.float32(Fraction(15, 2) / 57344)
    # correctly rounded quotient, checked with exact rationals
    for m in np.random.default_rng(0).uniform(1e-3, 1e3, 200).astype(np.float32):
        exact = Fraction(float(m)) / 448
        s = delayed_scale([m], "e4m3")
        lo, hi = np.nextafter(s, np.float32(0)), np.nextafter(s, np.float32(np.inf))
        assert abs(Fraction(float(s)) - exact) <= abs(Fraction(float(lo)) - exact)
        assert abs(Fraction(float(s)) - exact) <= abs(Fraction(float(hi)) - exact)
    # no positive entry: unit scale
    assert delayed_scale([0.0, 0.0], "e5m2") == 1.0
    assert delayed_scale([np.nan], "e4m3") == 1.0


def test_delayed_unit_scale_is_plain_saturating_cast():
    """Scale 1 (first step): the codes are torch's cast of x clamped to the
    format's range."""
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((32, 256)) * 2000).astype(np.float32)
    q, s, _ = quantize_delayed(x, [0.0], 0, "e5m2")
    assert s == 1.0
    assert np.array_equal(q, _torch_e5m2(np.clip(x, -57344, 57344)))
    q4, _, _ = quantize_delayed(x, [0.0], 0, "e4m3")
    ref4 = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q4, ref4)


def test_delayed_saturates_growth_and_records_amax():
    """The data grew past what last step's scale covers: those elements
    saturate to the largest code; the new history records this step's amax
    in the named entry only."""
    x = np.array([[1.0, -2.0, 40.0, -100.0, np.nan]], np.float32)
    hist = np.array([5.0, 9.0, 10.0], np.float32)
    q, s, new = quantize_delayed(x, hist, 1, "e4m3")
    assert s == np.float32(10.0 / 448)
    assert T4[q[0, 2]] == 448.0 and T4[q[0, 3]] == -448.0
    assert q[0, 4] == 0x7F
    assert np.array_equal(new, np.array([5.0, 100.0, 10.0], np.float32))
    assert tensor_amax(x) == 100.0


def test_finite_data_never_overflows_the_code_range():
    """Under a scale far below what the data needs (history from a much
    smaller tensor) the fp32 quotient itself overflows; finite elements
    still saturate to the largest finite code, only infinite ones give the
    infinity (e5m2) or NaN (e4m3) code."""
    x = np.array([[1.0, -3e30, 2.0 ** -100, np.inf]], np.float32)
    for fmt, top, inf_code in (("e5m2", 0x7B, 0x7C), ("e4m3", 0x7E, 0x7F)):
        q, s, _ = quantize_delayed(x, [2.0 ** -140], 0, fmt)
        assert s < 2.0 ** -126 or s == 0.0
        if s == 0.0:                      # e5m2: 2^-140 / 57344 underflows to 0
            assert list(q[0, :3]) == [0x00, 0x80, 0x00]
        else:
            assert list(q[0, :2]) == [top, 0x80 | top], (fmt, q)
        # (a zero scale gives signed zeros for every non-NaN element)
        assert q[0, 3] == (0x00 if s == 0.0 else inf_code)


def test_quantize_with_scale_specials():
    f = np.float32
    x = np.array([[np.inf, -np.inf, np.nan, -0.0, 1.0]], f)
    q5 = quantize_with_scale(x, f(1.0), "e5m2")
    assert list(q5[0]) == [0x7C, 0xFC, 0x7F, 0x80, 0x3C]      # e5m2 keeps infinities
    q4 = quantize_with_scale(x, f(1.0), "e4m3")
    assert list(q4[0]) == [0x7F, 0xFF, 0x7F, 0x80, 0x38]      # e4m3 has none: NaN code
    qz = quantize_with_scale(x, f(0.0), "e5m2")               # zero scale: signed zeros
    assert list(qz[0]) == [0x00, 0x80, 0x7F, 0x80, 0x00]


# ---------------------------------------------------------------------------
# mixed-format per-tensor GEMM


def _codes(rng, shape, fmt):
    t = T5 if fmt == "e5m2" else T4
    ok = np.flatnonzero(np.isfinite(t))
    return rng.choice(ok, size=shape).astype(np.uint8)


@pytest.mark.parametrize("fa,fb", [("e5m2", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e5m2")])
def test_pertensor_mixed_formats_bruteforce(fa, fb):
    rng = np.random.default_rng(len(fa + fb))
    M, N, K = 3, 4, 160
    qa, qb = _codes(rng, (M, K), fa), _codes(rng, (N, K), fb)
    s_a, s_b = np.float32(0.37), np.float32(1.9e-3)
    bits, _ = gemm_pertensor(qa, s_a, qb, s_b, fa, fb)
    ta, tb = (T5 if fa == "e5m2" else T4), (T5 if fb == "e5m2" else T4)
    for m in range(M):
        for n in range(N):
            acc = sum(Fraction(float(ta[qa[m, k]])) * Fraction(float(tb[qb[n, k]])) for k in range(K))
            v = acc * Fraction(float(s_a)) * Fraction(float(s_b))
            ref = bf16_bits_from_f64(np.float64(float(v)))
            # float(v) rounds to fp64 first; bf16 of that equals bf16 of v
            # unless v sits within 2^-53 of a bf16 midpoint (not the case here)
            assert bits[m, n] == ref, (m, n)


def test_pertensor_e5m2_codes_of_e4m3_values_give_same_product():
    """Values both formats hold (e.g. 1.5 * 2^k for small k): the product is
    the same whichever format carries them."""
    rng = np.random.default_rng(2)
    common = [v for v in T5[np.isfinite(T5)] if v in set(T4[np.isfinite(T4)])]
    vals = rng.choice(common, size=(8, 256))
    valsb = rng.choice(common, size=(16, 256))
    enc4 = lambda v: np.array([np.flatnonzero(T4 == x)[0] for x in v.ravel()], np.uint8).reshape(v.shape)
    enc5 = lambda v: np.array([np.flatnonzero(T5 == x)[0] for x in v.ravel()], np.uint8).reshape(v.shape)
    b44, _ = gemm_pertensor(enc4(vals), 1.0, enc4(valsb), 1.0)
    b55, _ = gemm_pertensor(enc5(vals), 1.0, enc5(valsb), 1.0, "e5m2", "e5m2")
    b54, _ = gemm_pertensor(enc5(vals), 1.0, enc4(valsb), 1.0, "e5m2", "e4m3")
    assert np.array_equal(b44, b55) and np.array_equal(b44, b54)
