"""Pins of the oracle quantiser.

Independent of the oracle: a re-derivation with torch's float32 ops (IEEE
division, abs/amax) and its float8_e4m3fn cast; exact rationals; invariants
the method fixes (the largest code of every block is +-448; exact power-of-two
invariance; dequantisation error bound).
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import quantize_blocks, e4m3_decode_table
from workloads import make_dense

T = e4m3_decode_table()


def _torch_quantize(x, br, bc=128):
    """Library re-derivation: fp32 amax, fp32 division, saturate, torch cast."""
    xt = torch.from_numpy(np.ascontiguousarray(x))
    R, C = xt.shape
    nrb, ncb = -(-R // br), -(-C // bc)
    q = torch.empty((R, C), dtype=torch.uint8)
    s = torch.empty((nrb, ncb), dtype=torch.float32)
    for i in range(nrb):
        for j in range(ncb):
            blk = xt[i * br:(i + 1) * br, j * bc:(j + 1) * bc]
            amax = blk.abs().max()
            sc = amax / torch.tensor(448.0, dtype=torch.float32)
            s[i, j] = sc
            if sc == 0:
                qb = torch.where(torch.signbit(blk), 128, 0).to(torch.uint8)
            else:
                y = (blk / sc).clamp(-448.0, 448.0)
                qb = y.to(torch.float8_e4m3fn).view(torch.uint8)
            q[i * br:(i + 1) * br, j * bc:(j + 1) * bc] = qb
    return q.numpy(), s.numpy()


@pytest.mark.parametrize("br", [1, 128])
def test_quantize_matches_torch_rederivation(br):
    w = make_dense(256, 256, 512, frac=0.01, seed=3)
    for x in (w.a, w.b):
        q, s = quantize_blocks(x, br)
        qt, st = _torch_quantize(x, br)
        assert np.array_equal(s.view(np.uint32), st.view(np.uint32))
        assert np.array_equal(q, qt)


def test_quantize_ragged_blocks_match_torch():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((200, 300)) * 3).astype(np.float32)
    for br in (1, 128):
        q, s = quantize_blocks(x, br)
        qt, st = _torch_quantize(x, br)
        assert s.shape == (-(-200 // br), 3)
        assert np.array_equal(s.view(np.uint32), st.view(np.uint32))
        assert np.array_equal(q, qt)


def test_scale_is_correctly_rounded_quotient():
    rng = np.random.default_rng(9)
    # amax values over many binades, checked with exact rationals
    amax = (rng.uniform(0.5, 1.0, 3000) * 2.0 ** rng.integers(-120, 100, 3000)).astype(np.float32)
    x = np.zeros((3000, 128), np.float32)
    x[:, 17] = amax
    x[:, 40] = -amax * np.float32(0.5)
    _, s = quantize_blocks(x, 1)
    for a, sc in zip(amax, s[:, 0]):
        exact = Fraction(float(a)) / 448
        lo = np.float32(float(exact))                 # candidates around it
        cands = [lo, np.nextafter(lo, np.float32(0)), np.nextafter(lo, np.float32(np.inf))]
        best = min(cands, key=lambda c: (abs(Fraction(float(c)) - exact),
                                         int(np.float32(c).view(np.uint32)) & 1))
        assert sc == best


def test_every_block_reaches_448_and_error_bound():
    w = make_dense(64, 128, 1024, frac=0.01, seed=21)
    for br in (1, 128):
        q, s = quantize_blocks(w.a if br == 1 else w.b, br)
        x = w.a if br == 1 else w.b
        R, C = x.shape
        for i in range(s.shape[0]):
            for j in range(s.shape[1]):
                blk = q[i * br:(i + 1) * br, j * 128:(j + 1) * 128]
                assert np.any((blk & 0x7F) == 0x7E)       # amax/s rounds to 448
        # |x/s - dec(q)| <= half an e4m3 step at dec(q) plus the fp32 quotient rounding
        s_el = np.repeat(np.repeat(s, br, 0), 128, 1)[:R, :C].astype(np.float64)
        ratio = x.astype(np.float64) / s_el
        d = T[q]
        a = np.abs(d)
        # e4m3 step at dec(q): 2^-9 on the subnormal grid, 2^(e-3) in binade e
        step = np.where(a < 2.0 ** -6, 2.0 ** -9,
                        2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3))
        bound = step / 2 + 2.0 ** -23 * np.abs(ratio)
        assert np.all(np.abs(ratio - d) <= bound)


def test_power_of_two_invariance():
    w = make_dense(32, 256, 768, frac=0.01, seed=4)
    for br, x in ((1, w.a), (128, w.b)):
        q0, s0 = quantize_blocks(x, br)
        for j in (-20, -7, 1, 13, 20):
            q1, s1 = quantize_blocks(x * np.float32(2.0 ** j), br)
            assert np.array_equal(q0, q1)
            assert np.array_equal(s1, s0 * np.float32(2.0 ** j))


def test_zero_signed_zero_and_subnormal_blocks():
    x = np.zeros((4, 256), np.float32)
    x[0, :] = 0.0
    x[1, :] = -0.0
    x[2, :128] = np.float32(1e-45) * np.arange(128, dtype=np.float32)   # subnormal amax
    x[2, 128:] = np.float32(-3e-40)
    x[3, :5] = [np.nan, 1.0, -2.0, np.nan, 0.5]
    q, s = quantize_blocks(x, 1)
    assert s[0, 0] == 0 and s[1, 0] == 0
    assert np.all(q[0] == 0x00) and np.all(q[1] == 0x80)
    # row 2 block 0: amax = 127e-45 (subnormal) -> s underflows to a tiny
    # subnormal or zero; codes follow fl32(x/s) saturated, never NaN
    assert not np.any((q[2] & 0x7F) == 0x7F)
    # NaN elements keep NaN codes, the others scale by amax 2.0
    assert q[3, 0] == 0x7F and q[3, 3] == 0x7F
    assert s[3, 0] == np.float32(2.0 / 448.0)
    assert q[3, 2] == 0xFE and T[q[3, 1]] == 224.0


def test_all_nan_and_infinite_blocks():
    x = np.full((1, 128), np.nan, np.float32)
    q, s = quantize_blocks(x, 1)
    assert s[0, 0] == 0 and np.all(q == 0x7F)
    y = np.ones((1, 128), np.float32)
    y[0, 3] = np.inf
    y[0, 4] = -np.inf
    q, s = quantize_blocks(y, 1)
    assert np.isinf(s[0, 0])
    assert q[0, 0] == 0x00 and q[0, 3] == 0x7F and q[0, 4] == 0xFF


def test_amax_skips_quiet_and_signalling_nans():
    """amax is the largest |x| of the block's non-NaN elements whatever kind
    of NaN sits where: checked against a plain Python maximum (math.isnan
    skip) for quiet and signalling NaN patterns at the start, middle and end
    of a block, next to the largest element and away from it."""
    import math
    rng = np.random.default_rng(21)
    nan_patterns = [0x7FC00000, 0xFFC00000, 0x7FBD0000, 0xFF800001, 0x7F800001, 0x7FA00000]
    for trial in range(40):
        x = (rng.standard_normal(128) * 10.0 ** rng.integers(-30, 30)).astype(np.float32)
        xb = x.view(np.uint32).copy()
        for _ in range(int(rng.integers(1, 4))):
            pos = int(rng.choice([0, 64, 127, int(rng.integers(0, 128))]))
            xb[pos] = nan_patterns[int(rng.integers(0, len(nan_patterns)))]
        x = xb.view(np.float32).reshape(1, 128)
        finite_abs = [abs(float(v)) for v in x[0] if not math.isnan(float(v))]
        want = max(finite_abs) if finite_abs else 0.0
        q, s = quantize_blocks(x, 1)
        assert s[0, 0] == np.float32(float(Fraction(want) / 448)), (trial, want, s[0, 0])
        qb, sb = quantize_blocks(np.tile(x, (128, 1)), 128)
        assert sb[0, 0] == s[0, 0]
        # every NaN element gets the NaN code with its own sign
        nan_at = np.isnan(x[0])
        assert np.all((q[0][nan_at] & 0x7F) == 0x7F)
