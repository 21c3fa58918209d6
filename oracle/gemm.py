"""Block-scaled FP8 GEMM, dense and grouped, in float64 (test infrastructure).

What is computed (operands as the quantiser leaves them):

    D[m][n] = sum over K blocks kb of
              sa[m][kb] * sb[n // 128][kb] * sum_{k in kb} dec(qa[m][k]) * dec(qb[n][k])

then rounded once to bf16. Sources:

* czchanglian §2.3: products are summed in an FP32 accumulator over the whole
  of K and only the write-back goes to the output precision.
* czchanglian §2.2 and nxmr §3.1: the scale is taken into account inside the
  GEMM (dequantise = multiply by the scale); with a scale per 128-wide K
  block this means one multiply per block, applied to the block's partial sum.
* gtnt, Triton kernel and pipeline figure: the epilogue multiplies the
  accumulator by the scales and converts it to bf16 (the per-tensor case).
* nxmr §3.2 and czchanglian §1.2: a grouped GEMM runs every expert's
  product in one launch; each expert is an ordinary GEMM on its own rows
  with its own weights; czchanglian §5.3: experts are identified by group id
  and token offsets, and each expert's rows are contiguous.

The oracle evaluates the sum in float64. The inner block sum is exact there
whatever the order: every product of two e4m3 values is a multiple of 2^-18
below 2^18, so 128 of them stay below 2^25 and need at most 43 bits. The scale
product sa*sb (two 24-bit significands) is exact too. Each promotion rounds in
float64 only, so the result is the exact sum up to ~2^-50 relative, and it is
rounded directly to bf16 (no detour through fp32).

Operand layouts (the math does not depend on them):
  qa [M][K] uint8 codes, sa [M][ceil(K/128)] float32 (row m, block kb)
  qb [N][K] uint8 codes, sb [ceil(N/128)][ceil(K/128)] float32
N and K need not be multiples of 128: a last partial block along K (or of
B's 128 rows) holds the elements that are there.
"""

import numpy as np

from .formats import FORMATS, e4m3_decode_table, bf16_bits_from_f64, bf16_bits_to_f64

KB = 128       # scale block along K
NB = 128       # scale block along N for the weight operand
_TABLE = e4m3_decode_table()


def _cdiv(a, b):
    return -(-a // b)


def _check(qa, sa, qb, sb):
    """N and K need not be multiples of 128: the last block along K (and the
    last 128-row block of B) holds the elements that are there, as the
    quantiser forms it -- the same value as zero-padding both operands to a
    multiple of 128 and slicing the padding off (czchanglian §5.1)."""
    M, K = qa.shape
    N, K2 = qb.shape
    if K != K2 or K < 1 or N < 1:
        raise ValueError("need K == K' >= 1 and N >= 1")
    if sa.shape != (M, _cdiv(K, KB)) or sb.shape != (_cdiv(N, NB), _cdiv(K, KB)):
        raise ValueError("scale shapes do not match the 1x128 / 128x128 blocking")
    return M, N, K


def gemm_blockscaled_f64(qa, sa, qb, sb):
    """Unrounded float64 result of the block-scaled product, shape [M][N]."""
    M, N, K = _check(qa, sa, qb, sb)
    A = _TABLE[qa]                       # exact decode to float64
    B = _TABLE[qb]
    D = np.zeros((M, N), dtype=np.float64)
    sa64 = sa.astype(np.float64)
    sb64 = np.repeat(sb.astype(np.float64), NB, axis=0)[:N]  # [N][ceil(K/128)]
    for kb in range(_cdiv(K, KB)):
        ks = slice(kb * KB, min(K, (kb + 1) * KB))
        P = A[:, ks] @ B[:, ks].T                           # exact block sum
        c = sa64[:, kb][:, None] * sb64[:, kb][None, :]     # exact scale product
        D += c * P
    return D


def gemm_blockscaled(qa, sa, qb, sb):
    """bf16 result (uint16 bits) and the float64 value it was rounded from."""
    D = gemm_blockscaled_f64(qa, sa, qb, sb)
    return bf16_bits_from_f64(D), D


def gemm_pertensor(qa, s_a, qb, s_b, fmt_a="e4m3", fmt_b="e4m3"):
    """Per-tensor-scaled product: one scale per operand.

    D[m][n] = s_a * s_b * sum over all k of dec(qa[m][k]) * dec(qb[n][k]),
    rounded once to bf16. This is the printed Triton kernel's semantics (gtnt,
    Triton kernel section: the dot products are accumulated over every K
    block, then multiplied by scale_a * scale_b and cast to bf16).

    fmt_a / fmt_b name each operand's 8-bit format ("e4m3" or "e5m2"; the
    gradient GEMM of a backward pass takes e5m2 for the gradient operand,
    czchanglian §2.1). With two e4m3 operands the accumulation is exact: every
    product is a multiple of 2^-18 below 2^18, so for K <= 2^17 every partial
    sum fits in 53 bits and the float64 sum is exact in any order. With an
    e5m2 operand the products span 2^-32 .. 2^32, so the float64 sum can
    round: its error is below K * 2^-53 of the sum of |products|, far inside
    any bf16 comparison. The scale product (two 24-bit significands) is exact,
    and the final multiply rounds once in float64.

    qa [M][K], qb [N][K] uint8 codes; s_a, s_b float32 scalars. Returns
    (bf16 bits [M][N], float64 [M][N]).
    """
    qa = np.asarray(qa)
    qb = np.asarray(qb)
    if qa.ndim != 2 or qb.ndim != 2 or qa.shape[1] != qb.shape[1]:
        raise ValueError("need qa [M][K] and qb [N][K] with the same K")
    if qa.shape[1] > 2 ** 17:
        raise ValueError("K above 2^17: outside the range the oracle is stated for")
    P = FORMATS[fmt_a][1][qa] @ FORMATS[fmt_b][1][qb].T
    D = (float(np.float32(s_a)) * float(np.float32(s_b))) * P
    return bf16_bits_from_f64(D), D


def gemm_blockscaled_fp32acc(qa, sa, qb, sb):
    """The same sum with float32 block sums and float32 promotion.

    Not a reference: it models what a float32 accumulator can lose, and is used
    only to check that the parity tolerance admits an fp32-accumulating
    implementation.
    """
    M, N, K = _check(qa, sa, qb, sb)
    A = _TABLE[qa].astype(np.float32)
    B = _TABLE[qb].astype(np.float32)
    D = np.zeros((M, N), dtype=np.float32)
    sb32 = np.repeat(sb.astype(np.float32), NB, axis=0)[:N]
    for kb in range(_cdiv(K, KB)):
        ks = slice(kb * KB, min(K, (kb + 1) * KB))
        P = A[:, ks] @ B[:, ks].T
        c = sa[:, kb].astype(np.float32)[:, None] * sb32[:, kb][None, :]
        D = D + c * P
    return bf16_bits_from_f64(D.astype(np.float64))


def grouped_contiguous(qa, sa, qb, sb, offsets):
    """Grouped GEMM, contiguous layout.

    qa [M_total][K], sa [M_total][K/128]; qb [G][N][K], sb [G][N/128][K/128];
    offsets [G+1] with expert g owning rows offsets[g] .. offsets[g+1]-1.
    Each expert's rows are one ordinary block-scaled GEMM with its own weights.
    Returns (bf16 bits [M_total][N], float64 [M_total][N]).
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    G = qb.shape[0]
    if offsets.shape != (G + 1,) or offsets[0] != 0 or offsets[-1] != qa.shape[0]:
        raise ValueError("offsets must be [G+1] running from 0 to M_total")
    N = qb.shape[1]
    D = np.zeros((qa.shape[0], N), dtype=np.float64)
    for g in range(G):
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        if r1 > r0:
            D[r0:r1] = gemm_blockscaled_f64(qa[r0:r1], sa[r0:r1], qb[g], sb[g])
    return bf16_bits_from_f64(D), D


def grouped_masked(qa, sa, qb, sb, masked_m, d_init):
    """Grouped GEMM, masked layout.

    qa [G][max_m][K], sa [G][max_m][K/128]; qb [G][N][K], sb [G][N/128][K/128];
    masked_m [G]: expert g's valid rows are 0 .. masked_m[g]-1 (clamped to
    [0, max_m]). Rows past the count are not computed and keep the bits of
    d_init (bf16 bits [G][max_m][N]).
    Returns (bf16 bits [G][max_m][N], float64 values of the valid rows, valid
    row mask [G][max_m]).
    """
    G, max_m, _ = qa.shape
    N = qb.shape[1]
    out = np.array(d_init, dtype=np.uint16, copy=True)
    vals = np.zeros((G, max_m, N), dtype=np.float64)
    valid = np.zeros((G, max_m), dtype=bool)
    for g in range(G):
        m = int(min(max(int(masked_m[g]), 0), max_m))
        if m == 0:
            continue
        D = gemm_blockscaled_f64(qa[g, :m], sa[g, :m], qb[g], sb[g])
        out[g, :m] = bf16_bits_from_f64(D)
        vals[g, :m] = D
        valid[g, :m] = True
    return out, vals, valid


def tolerance_check(got_bits, ref_bits):
    """Parity bar for GEMM outputs.

    |got - ref| <= 2^-7 |ref| + 2^-10 rms(ref), elementwise, where ref is the
    oracle's bf16-rounded result and rms is taken over every element passed
    in. Callers pass the output rows that exist: zero padding rows of the
    contiguous layout and the untouched rows of the masked layout are checked
    bit for bit instead, and would only dilute the rms. The first term admits
    a one-ulp bf16 disagreement (a bf16 ulp is at most 2^-7 of the value); the
    second absorbs accumulation error on outputs that cancel to near zero.
    Returns (ok, worst ratio |d| / bound, number of violating elements).
    """
    got = bf16_bits_to_f64(got_bits)
    ref = bf16_bits_to_f64(ref_bits)
    if got.shape != ref.shape:
        raise ValueError("shape mismatch")
    if ref.size == 0:
        return True, 0.0, 0
    rms = float(np.sqrt(np.mean(ref * ref)))
    bound = 2.0 ** -7 * np.abs(ref) + 2.0 ** -10 * rms
    diff = np.abs(got - ref)
    bad = ~(diff <= bound)          # also catches NaN
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, diff / bound, np.where(diff > 0, np.inf, 0.0))
    worst = float(np.nanmax(ratio)) if np.isfinite(ratio).any() or ratio.size else 0.0
    if np.isnan(ratio).any():
        worst = float("inf")
    return (not bad.any()), worst, int(bad.sum())
