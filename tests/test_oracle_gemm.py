"""Pins of the oracle GEMM (dense, grouped contiguous, grouped masked).

* exact rational brute force on tiny shapes (fractions.Fraction), rounded to
  bf16 from first principles -- must equal the oracle bit for bit;
* special cases that reduce to a textbook routine: equal (per-tensor) scales
  give s_a * s_b * (A @ B^T) as in the fused-scale epilogue of the gtnt
  page's Triton kernel; unit scales with small-integer codes give an exact
  int64 matrix product;
* exact power-of-two invariance;
* grouped = the concatenation of per-expert dense GEMMs, including the
  2 experts x 8 tokens case czchanglian §5.3 recommends starting from;
* the tolerance admits an fp32-accumulating implementation on every workload
  (sampled rows/experts at the large sizes).
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import (quantize_blocks, gemm_blockscaled, gemm_blockscaled_fp32acc, gemm_pertensor,
                    grouped_contiguous, grouped_masked, tolerance_check,
                    e4m3_decode_table, bf16_bits_from_f64, bf16_bits_to_f64)
from oracle.gemm import gemm_blockscaled_f64
from workloads import make_dense, make_contiguous, make_masked, make_config

T = e4m3_decode_table()


def _bf16_exact(v: Fraction) -> int:
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 7)
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * ulp
    if r > (2 - Fraction(1, 128)) * Fraction(2) ** 127:
        return sign | 0x7F80
    return sign | (int(np.float32(float(r)).view(np.uint32)) >> 16)


def _rand_operands(rng, M, N, K):
    qa = rng.integers(0, 256, (M, K)).astype(np.uint8)
    qb = rng.integers(0, 256, (N, K)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x7E           # no NaN codes
    qb[(qb & 0x7F) == 0x7F] = 0x01
    sa = (rng.uniform(0.5, 2, (M, K // 128)) * 2.0 ** rng.integers(-12, 4, (M, K // 128))).astype(np.float32)
    sb = (rng.uniform(0.5, 2, (N // 128, K // 128)) * 2.0 ** rng.integers(-12, 4, (N // 128, K // 128))).astype(np.float32)
    return qa, sa, qb, sb


@pytest.mark.parametrize("M,K,seed", [(3, 128, 0), (5, 256, 1), (8, 384, 2)])
def test_bruteforce_exact_rational(M, K, seed):
    rng = np.random.default_rng(seed)
    N = 256                                     # two N-blocks with distinct scales
    qa, sa, qb, sb = _rand_operands(rng, M, N, K)
    bits, _ = gemm_blockscaled(qa, sa, qb, sb)
    Fa = [[Fraction(float(T[c])) for c in row] for row in qa]
    cols = list(range(0, 6)) + list(range(125, 133)) + list(range(250, 256))
    Fb = {n: [Fraction(float(T[c])) for c in qb[n]] for n in cols}
    for m in range(M):
        for n in cols:
            tot = Fraction(0)
            for kb in range(K // 128):
                part = sum(Fa[m][k] * Fb[n][k] for k in range(kb * 128, kb * 128 + 128))
                tot += Fraction(float(sa[m, kb])) * Fraction(float(sb[n // 128, kb])) * part
            assert int(bits[m, n]) == _bf16_exact(tot), (m, n)


def test_per_tensor_scales_reduce_to_plain_product():
    rng = np.random.default_rng(3)
    M, N, K = 16, 256, 512
    qa, _, qb, _ = _rand_operands(rng, M, N, K)
    alpha, beta = np.float32(0.0123), np.float32(3.7)
    sa = np.full((M, K // 128), alpha, np.float32)
    sb = np.full((N // 128, K // 128), beta, np.float32)
    D = gemm_blockscaled_f64(qa, sa, qb, sb)
    ref = float(alpha) * float(beta) * (T[qa] @ T[qb].T)
    # the oracle rounds once per K block in float64: allow a few ulps of the
    # largest magnitude the sum passes through
    mag = float(alpha) * float(beta) * (np.abs(T[qa]) @ np.abs(T[qb]).T)
    assert np.all(np.abs(D - ref) <= 2.0 ** -50 * mag)
    assert np.array_equal(bf16_bits_from_f64(D), bf16_bits_from_f64(ref))


def test_unit_scales_small_integers_exact_int64():
    rng = np.random.default_rng(4)
    M, N, K = 24, 128, 384
    ints = np.arange(-16, 17)
    codes = {}
    for c in range(256):
        v = T[c]
        if np.isfinite(v) and v == int(v) and abs(v) <= 16:
            codes.setdefault(int(v), c)
    lut = np.array([codes[int(v)] for v in ints], np.uint8)
    ia = rng.integers(0, len(ints), (M, K))
    ib = rng.integers(0, len(ints), (N, K))
    qa, qb = lut[ia], lut[ib]
    sa = np.ones((M, K // 128), np.float32)
    sb = np.ones((N // 128, K // 128), np.float32)
    D = gemm_blockscaled_f64(qa, sa, qb, sb)
    exact = ints[ia].astype(np.int64) @ ints[ib].astype(np.int64).T
    assert np.array_equal(D, exact.astype(np.float64))


def test_power_of_two_invariance_gemm():
    rng = np.random.default_rng(5)
    qa, sa, qb, sb = _rand_operands(rng, 8, 256, 256)
    b0, d0 = gemm_blockscaled(qa, sa, qb, sb)
    for ja, jb in ((-5, 3), (7, 9), (-11, -2)):
        b1, d1 = gemm_blockscaled(qa, sa * np.float32(2.0 ** ja), qb, sb * np.float32(2.0 ** jb))
        assert np.array_equal(d1, d0 * 2.0 ** (ja + jb))
        assert np.array_equal(bf16_bits_to_f64(b1), bf16_bits_to_f64(b0) * 2.0 ** (ja + jb))


def test_scale_indexing_single_block():
    """Only one K block and one N block carry a nonzero scale: the result is that
    block's plain product times the scales, zero elsewhere (catches a wrong or
    transposed scale index)."""
    rng = np.random.default_rng(6)
    M, N, K = 4, 384, 512
    qa, _, qb, _ = _rand_operands(rng, M, N, K)
    sa = np.zeros((M, 4), np.float32)
    sb = np.zeros((3, 4), np.float32)
    sa[:, 2] = np.float32([1.0, 2.0, 4.0, 0.5])
    sb[1, 2] = np.float32(0.25)
    D = gemm_blockscaled_f64(qa, sa, qb, sb)
    ref = (T[qa][:, 256:384] @ T[qb][:, 256:384].T) * (sa[:, 2:3].astype(np.float64) * 0.25)
    assert np.all(D[:, :128] == 0) and np.all(D[:, 256:] == 0)
    assert np.array_equal(D[:, 128:256], ref[:, 128:256])


def test_two_experts_eight_tokens():
    w = make_contiguous([8, 8], 256, 256, frac=0.01, seed=8)
    assert list(w.offsets) == [0, 128, 256]
    qa, sa = quantize_blocks(w.a, 1)
    qb = np.stack([quantize_blocks(w.b[g], 128)[0] for g in range(2)])
    sb = np.stack([quantize_blocks(w.b[g], 128)[1] for g in range(2)])
    bits, D = grouped_contiguous(qa, sa, qb, sb, w.offsets)
    for g in range(2):
        r0 = int(w.offsets[g])
        ref_bits, _ = gemm_blockscaled(qa[r0:r0 + 8], sa[r0:r0 + 8], qb[g], sb[g])
        assert np.array_equal(bits[r0:r0 + 8], ref_bits)
        assert np.all(D[r0 + 8:r0 + 128] == 0)       # zero padding rows give +0


def test_grouped_contiguous_is_concat_of_dense():
    w = make_contiguous([130, 0, 7, 256], 256, 384, seed=9)
    qa, sa = quantize_blocks(w.a, 1)
    qs = [quantize_blocks(w.b[g], 128) for g in range(4)]
    qb = np.stack([q for q, _ in qs])
    sb = np.stack([s for _, s in qs])
    bits, _ = grouped_contiguous(qa, sa, qb, sb, w.offsets)
    for g in range(4):
        r0, r1 = int(w.offsets[g]), int(w.offsets[g + 1])
        if r1 > r0:
            ref, _ = gemm_blockscaled(qa[r0:r1], sa[r0:r1], qb[g], sb[g])
            assert np.array_equal(bits[r0:r1], ref)


def test_grouped_masked_rows_and_sentinel():
    w = make_masked([0, 1, 255, 256], 256, 128, 256, seed=10)
    G, mm, K = w.a.shape
    qa, sa = quantize_blocks(w.a.reshape(G * mm, K), 1)
    qa = qa.reshape(G, mm, K)
    sa = sa.reshape(G, mm, K // 128)
    qs = [quantize_blocks(w.b[g], 128) for g in range(G)]
    qb = np.stack([q for q, _ in qs])
    sb = np.stack([s for _, s in qs])
    sentinel = np.full((G, mm, 128), 0x7FBF, np.uint16)
    out, _, valid = grouped_masked(qa, sa, qb, sb, w.masked_m, sentinel)
    for g in range(G):
        m = int(w.masked_m[g])
        assert np.all(out[g, m:] == 0x7FBF)
        if m:
            ref, _ = gemm_blockscaled(qa[g, :m], sa[g, :m], qb[g], sb[g])
            assert np.array_equal(out[g, :m], ref)
        assert valid[g].sum() == m


def test_tolerance_rejects_real_errors():
    rng = np.random.default_rng(12)
    ref = bf16_bits_from_f64(rng.standard_normal((64, 64)))
    ok, _, _ = tolerance_check(ref, ref)
    assert ok
    # one bf16 ulp everywhere passes; a 2% error does not
    up = (ref.astype(np.int32) + 1).astype(np.uint16)
    assert tolerance_check(up, ref)[0]
    bad = bf16_bits_from_f64(bf16_bits_to_f64(ref) * 1.02)
    assert not tolerance_check(bad, ref)[0]
    nan = ref.copy()
    nan[3, 3] = 0x7FC0
    assert not tolerance_check(nan, ref)[0]


def _sample_check(qa, sa, qb, sb):
    ref, _ = gemm_blockscaled(qa, sa, qb, sb)
    got = gemm_blockscaled_fp32acc(qa, sa, qb, sb)
    ok, worst, nbad = tolerance_check(got, ref)
    assert ok, (worst, nbad)


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_tolerance_admits_fp32_accumulation(cfg):
    """An fp32-accumulating GEMM must pass the parity bar on every workload.
    Large workloads are sampled: a few rows, one or two experts, 512 columns,
    always the full K (which sets the accumulation error)."""
    w = make_config(cfg) if cfg in (0, 1) else None
    if cfg in (0, 1):
        qa, sa = quantize_blocks(w.a, 1)
        qb, sb = quantize_blocks(w.b, 128)
        _sample_check(qa, sa, qb, sb)
        return
    w = make_config(cfg)
    rng = np.random.default_rng(100 + cfg)
    if w.kind == "dense":
        rows = np.sort(rng.choice(w.M, 24, replace=False))
        qa, sa = quantize_blocks(w.a[rows], 1)
        qb, sb = quantize_blocks(w.b[:512], 128)
        _sample_check(qa, sa, qb, sb)
    elif w.kind == "contiguous":
        for g in (0, w.G - 1):
            r0 = int(w.offsets[g])
            qa, sa = quantize_blocks(w.a[r0:r0 + 16], 1)
            qb, sb = quantize_blocks(w.b[g, :512], 128)
            _sample_check(qa, sa, qb, sb)
    else:
        for g in (0, 9):
            m = int(w.masked_m[g])
            qa, sa = quantize_blocks(w.a[g, :min(m, 16)], 1)
            qb, sb = quantize_blocks(w.b[g, :512], 128)
            _sample_check(qa, sa, qb, sb)


# ---------------------------------------------------------------------------
# per-tensor scaling (gtnt, Triton kernel section): pins for gemm_pertensor


@pytest.mark.parametrize("M,K,seed", [(3, 128, 10), (4, 384, 11), (2, 1000, 12)])
def test_pertensor_bruteforce_exact_rational(M, K, seed):
    """Exact rational sum over all K times the exact scale product, rounded
    to bf16 by hand, equals the oracle bit for bit (K need not be a multiple
    of 128 for this product)."""
    rng = np.random.default_rng(seed)
    N = 5
    qa = rng.integers(0, 256, (M, K)).astype(np.uint8)
    qb = rng.integers(0, 256, (N, K)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x3C
    qb[(qb & 0x7F) == 0x7F] = 0x42
    s_a, s_b = np.float32(0.00371), np.float32(21.5)
    bits, _ = gemm_pertensor(qa, s_a, qb, s_b)
    c = Fraction(float(s_a)) * Fraction(float(s_b))
    for m in range(M):
        for n in range(N):
            tot = sum(Fraction(float(T[x])) * Fraction(float(T[y])) for x, y in zip(qa[m], qb[n]))
            assert int(bits[m, n]) == _bf16_exact(c * tot), (m, n)


def test_pertensor_equals_blockscaled_with_constant_scales():
    """Pin P7(i) from the other side: the block-scaled oracle with every A
    scale equal to s_a and every B scale equal to s_b computes the same value
    (to float64 rounding) as the per-tensor product."""
    rng = np.random.default_rng(13)
    M, N, K = 32, 256, 1024
    qa, _, qb, _ = _rand_operands(rng, M, N, K)
    s_a, s_b = np.float32(0.75), np.float32(0.0019)
    bits_pt, d_pt = gemm_pertensor(qa, s_a, qb, s_b)
    sa = np.full((M, K // 128), s_a, np.float32)
    sb = np.full((N // 128, K // 128), s_b, np.float32)
    d_bs = gemm_blockscaled_f64(qa, sa, qb, sb)
    mag = float(s_a) * float(s_b) * (np.abs(T[qa]) @ np.abs(T[qb]).T)
    assert np.all(np.abs(d_pt - d_bs) <= 2.0 ** -48 * mag)
    ok, worst, _ = tolerance_check(bits_pt, bf16_bits_from_f64(d_bs))
    assert ok and worst <= 2.0 ** -7 * 128


def test_pertensor_unit_scales_small_integers_exact_int64():
    rng = np.random.default_rng(14)
    M, N, K = 9, 40, 777
    small = {int(T[c]): c for c in range(256) if np.isfinite(T[c]) and T[c] == int(T[c])
             and abs(T[c]) <= 12}
    vals = np.array(sorted(small))
    lut = np.array([small[int(v)] for v in vals], np.uint8)
    ia = rng.integers(0, len(vals), (M, K))
    ib = rng.integers(0, len(vals), (N, K))
    _, d = gemm_pertensor(lut[ia], np.float32(1), lut[ib], np.float32(1))
    exact = vals[ia].astype(np.int64) @ vals[ib].astype(np.int64).T
    assert np.array_equal(d, exact.astype(np.float64))


def test_pertensor_quantiser_is_one_block():
    """Per-tensor quantisation is the block rule with one block covering the
    whole matrix: its scale is fl32(amax / 448) of the whole tensor and the
    element holding the amax gets the code of +-448."""
    rng = np.random.default_rng(21)
    x = rng.standard_normal((64, 512)).astype(np.float32)
    x[:, 5] *= np.float32(50.0)                # one outlier channel, in the first K block
    q, s = quantize_blocks(x, x.shape[0], x.shape[1])
    assert s.shape == (1, 1)
    amax = np.max(np.abs(x))
    assert s[0, 0] == np.float32(np.float64(amax) / 448.0)
    assert np.any(q == 0x7E) or np.any(q == 0xFE)
    r, c = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert q[r, c] & 0x7F == 0x7E


# ---------------------------------------------------------------------------
# N and K that are not multiples of 128 (czchanglian §5.1: the library used to
# need the caller to pad; the ragged product is defined as the padded one)


def _rand_ragged(rng, M, N, K):
    kb, nb = -(-K // 128), -(-N // 128)
    qa = rng.integers(0, 256, (M, K)).astype(np.uint8)
    qb = rng.integers(0, 256, (N, K)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x7E
    qb[(qb & 0x7F) == 0x7F] = 0x01
    sa = (rng.uniform(0.5, 2, (M, kb)) * 2.0 ** rng.integers(-12, 4, (M, kb))).astype(np.float32)
    sb = (rng.uniform(0.5, 2, (nb, kb)) * 2.0 ** rng.integers(-12, 4, (nb, kb))).astype(np.float32)
    return qa, sa, qb, sb


@pytest.mark.parametrize("M,N,K,seed", [(3, 144, 176, 0), (4, 48, 16, 1), (2, 272, 400, 2)])
def test_ragged_bruteforce_exact_rational(M, N, K, seed):
    """Ragged N and K against exact rationals, the last K block summing the
    elements that are there with its own scales."""
    rng = np.random.default_rng(seed)
    qa, sa, qb, sb = _rand_ragged(rng, M, N, K)
    bits, _ = gemm_blockscaled(qa, sa, qb, sb)
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for kb in range(-(-K // 128)):
                ks = range(kb * 128, min(K, kb * 128 + 128))
                part = sum(Fraction(float(T[qa[m, k]])) * Fraction(float(T[qb[n, k]])) for k in ks)
                tot += Fraction(float(sa[m, kb])) * Fraction(float(sb[n // 128, kb])) * part
            assert int(bits[m, n]) == _bf16_exact(tot), (m, n)


@pytest.mark.parametrize("M,N,K", [(5, 200, 300), (16, 48, 1040), (129, 400, 144)])
def test_ragged_equals_zero_padded(M, N, K):
    """Quantising ragged fp32 operands and multiplying equals padding them
    with zero columns (and B with zero rows) to multiples of 128, running the
    aligned path, and slicing the padding off: same codes, same scales, same
    output bits."""
    rng = np.random.default_rng(M * 7 + K)
    a = (rng.standard_normal((M, K)) * 3).astype(np.float32)
    b = (rng.standard_normal((N, K)) * 0.5).astype(np.float32)
    Kp, Np = -(-K // 128) * 128, -(-N // 128) * 128
    ap = np.zeros((M, Kp), np.float32)
    ap[:, :K] = a
    bp = np.zeros((Np, Kp), np.float32)
    bp[:N, :K] = b
    qa, sa = quantize_blocks(a, 1)
    qb, sb = quantize_blocks(b, 128)
    qap, sap = quantize_blocks(ap, 1)
    qbp, sbp = quantize_blocks(bp, 128)
    assert np.array_equal(qap[:, :K], qa) and np.all(qap[:, K:] == 0)
    assert np.array_equal(sap.view(np.uint32), sa.view(np.uint32))
    assert np.array_equal(qbp[:N, :K], qb) and np.array_equal(sbp.view(np.uint32), sb.view(np.uint32))
    bits, _ = gemm_blockscaled(qa, sa, qb, sb)
    bitsp, _ = gemm_blockscaled(qap, sap, qbp, sbp)
    assert np.array_equal(bitsp[:, :N], bits)
