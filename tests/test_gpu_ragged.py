"""GPU parity for N and K that are not multiples of 128 (czchanglian §5.1:
the pages pad outside the library and slice the padding off; the library
now takes such shapes itself, for N and K multiples of 16).

The quantisers are bit-exact against the oracle (whose ragged blocks are
pinned to the zero-padded ones); every GEMM layout is checked element by
element against the oracle under |d - ref| <= 2^-7 |ref| + 2^-10 rms(ref),
with shapes that put the partial K block in the first, a middle and the
last K step, partial 128-column blocks at the N edge, both tile
configurations, the small-M kernel and the contiguous split tail."""

import numpy as np
import pytest
import torch

import moe_grouped_gemm_quantizer_amd as fp8g
from oracle import (quantize_blocks, gemm_blockscaled, gemm_pertensor, grouped_contiguous,
                    grouped_masked, tolerance_check, bf16_bits_to_f64)
from workloads import make_dense, make_contiguous, make_masked
from tests.gpu_util import dev, to_dev, to_host, bits, bf16_out, banner

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FBF


def _assert_tol(got, ref, what):
    ok, worst, nbad = tolerance_check(got, ref)
    banner(f"{what}: worst ratio {worst:.4f}")
    assert ok, f"{what}: {nbad} elements out of tolerance"


# ---------------------------------------------------------------------------
# quantisers


@pytest.mark.parametrize("rows,cols", [(5, 16), (33, 144), (300, 1008), (129, 400), (2, 2064)])
@pytest.mark.parametrize("block_rows", [1, 128])
def test_quantise_ragged_columns(rows, cols, block_rows):
    banner(f"quantise {rows}x{cols} blocks {block_rows}x128")
    rng = np.random.default_rng(rows + cols + block_rows)
    x = (rng.standard_normal((rows, cols)) * np.exp(rng.uniform(-3, 3, (rows, 1)))).astype(np.float32)
    qo, so = quantize_blocks(x, block_rows)
    nrb, ncb = so.shape
    for kind in ("fp32", "bf16"):
        if kind == "bf16":
            xb = torch.from_numpy(x).to(torch.bfloat16)
            xo = xb.to(torch.float32).numpy()
            qo, so = quantize_blocks(xo, block_rows)
            xt = xb.to(dev())
        else:
            xt = to_dev(x)
        q = torch.full((rows, cols), 0xAB, dtype=torch.uint8, device=dev())
        s = torch.full((ncb, nrb) if block_rows == 1 else (nrb, ncb), -1.0, dtype=torch.float32,
                       device=dev())
        strides = (1, nrb) if block_rows == 1 else (ncb, 1)
        f = fp8g.fp8_quantize_bf16 if kind == "bf16" else fp8g.fp8_quantize
        f(xt, block_rows, q, s, *strides)
        sh = to_host(s)
        sh = sh.T if block_rows == 1 else sh
        assert np.array_equal(sh.view(np.uint32), so.view(np.uint32)), f"{kind} scales"
        assert np.array_equal(to_host(q), qo), f"{kind} codes"


# ---------------------------------------------------------------------------
# dense and per-tensor


def _dense_case(M, N, K, seed):
    w = make_dense(M, N, K, seed=seed)
    qa, sa = quantize_blocks(w.a, 1)
    qb, sb = quantize_blocks(w.b, 128)
    return qa, sa, qb, sb


# (M, N, K): the partial K block as the only, the second and the last of
# many blocks; partial column blocks of 16 .. 112; the 128-row tiles
# (M <= 128), the 256-row tiles, and the small-M kernel (M <= 32)
DENSE = [(300, 144, 176), (129, 400, 1040), (513, 1040, 2064), (257, 272, 16), (100, 48, 400),
         (64, 656, 8208), (16, 48, 16), (7, 1040, 2064), (32, 272, 400), (1, 16, 144)]


@pytest.mark.parametrize("M,N,K", DENSE)
def test_dense_ragged(M, N, K):
    banner(f"dense ragged {M}x{N}x{K}: {fp8g.fp8g_gemm_kernel_name('dense', M, N, K)}")
    qa, sa, qb, sb = _dense_case(M, N, K, seed=M + N + K)
    ref, _ = gemm_blockscaled(qa, sa, qb, sb)
    d = bf16_out((M, N), fill=SENTINEL)
    fp8g.gemm_fp8_blockscaled(to_dev(qa), to_dev(np.ascontiguousarray(sa.T)), to_dev(qb),
                              to_dev(sb), d)
    _assert_tol(bits(d), ref, f"dense {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(300, 144, 176), (513, 1040, 2064), (40, 400, 1040)])
def test_quant_epilogue_ragged(M, N, K):
    """The quantising epilogue with a partial last column block: codes and
    scales equal the standalone quantiser's on the GEMM's bf16 output."""
    banner(f"quantising epilogue ragged {M}x{N}x{K}")
    qa, sa, qb, sb = _dense_case(M, N, K, seed=3 * M + N)
    ref, _ = gemm_blockscaled(qa, sa, qb, sb)
    nb = -(-N // 128)
    d = bf16_out((M, N), fill=SENTINEL)
    qd = torch.full((M, N), 0xAB, dtype=torch.uint8, device=dev())
    sd = torch.full((nb, M), -1.0, dtype=torch.float32, device=dev())
    fp8g.gemm_fp8_blockscaled_quant(to_dev(qa), to_dev(np.ascontiguousarray(sa.T)), to_dev(qb),
                                    to_dev(sb), d, qd, sd)
    _assert_tol(bits(d), ref, "epilogue bf16")
    q2 = torch.empty_like(qd)
    s2 = torch.empty_like(sd)
    fp8g.fp8_quantize_bf16(d, 1, q2, s2, 1, M)
    assert torch.equal(qd, q2) and torch.equal(sd.view(torch.int32), s2.view(torch.int32))


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e5m2", "e4m3")])
@pytest.mark.parametrize("M,N,K", [(300, 144, 176), (129, 400, 1040), (64, 48, 16)])
def test_pertensor_ragged(fa, fb, M, N, K):
    banner(f"per-tensor ragged {fa} x {fb} {M}x{N}x{K}")
    w = make_dense(M, N, K, seed=M * 5 + K)
    qa, sa = quantize_blocks(w.a, M, K, fmt=fa)
    qb, sb = quantize_blocks(w.b, N, K, fmt=fb)
    ref, _ = gemm_pertensor(qa, sa[0, 0], qb, sb[0, 0], fa, fb)
    d = bf16_out((M, N), fill=SENTINEL)
    fp8g.gemm_fp8_pertensor_fmt(to_dev(qa), fa, to_dev(sa.reshape(1)), to_dev(qb), fb,
                                to_dev(sb.reshape(1)), d)
    _assert_tol(bits(d), ref, f"per-tensor {M}x{N}x{K}")


# ---------------------------------------------------------------------------
# grouped layouts


def _contiguous(counts, N, K, seed, workspace):
    w = make_contiguous(counts, N, K, seed=seed)
    qa, sa = quantize_blocks(w.a, 1)
    qs = [quantize_blocks(w.b[g], 128) for g in range(w.G)]
    qb = np.stack([q for q, _ in qs])
    sb = np.stack([s for _, s in qs])
    d = bf16_out((w.M, N), fill=SENTINEL)
    args = (to_dev(qa), to_dev(np.ascontiguousarray(sa.T)), to_dev(qb), to_dev(sb), d,
            to_dev(w.offsets.astype(np.int32)))
    if workspace:
        n = fp8g.grouped_gemm_fp8_contiguous_workspace_size(w.G, w.M, N, K)
        ws = torch.empty(n, dtype=torch.uint8, device=dev()) if n else None
        fp8g.grouped_gemm_fp8_contiguous_ws(*args, ws)
    else:
        fp8g.grouped_gemm_fp8_contiguous(*args)
    ref, _ = grouped_contiguous(qa, sa, qb, sb, w.offsets)
    tok = np.zeros(w.M, bool)
    for g in range(w.G):
        tok[int(w.offsets[g]):int(w.offsets[g]) + int(w.counts[g])] = True
    got = bits(d)
    return got, ref, tok


@pytest.mark.parametrize("counts,N,K", [([130, 0, 7, 256], 144, 400), ([8, 8], 48, 16),
                                        ([9000, 4500, 2600, 2200], 1040, 2064)])
@pytest.mark.parametrize("entry", ["plain", "workspace"])
def test_contiguous_ragged(counts, N, K, entry):
    """Including a shape whose last round of tiles runs as K pieces (with a
    workspace), the partial K block then falling in the last piece."""
    banner(f"contiguous ragged G={len(counts)} N={N} K={K} {entry}")
    got, ref, tok = _contiguous(counts, N, K, seed=N + K, workspace=entry == "workspace")
    _assert_tol(got[tok], ref[tok], f"contiguous ragged {entry}")
    assert np.all(got[~tok] == 0), "padding rows not +0"


@pytest.mark.parametrize("counts,max_m,N,K,em", [([0, 1, 255, 256], 256, 144, 400, 200),
                                                  ([3, 0, 77], 100, 48, 16, 50),
                                                  ([129, 128, 0, 200, 5], 200, 400, 1040, 64)])
def test_masked_ragged(counts, max_m, N, K, em):
    banner(f"masked ragged G={len(counts)} max_m={max_m} N={N} K={K}")
    w = make_masked(counts, max_m, N, K, seed=max_m + N)
    G = len(counts)
    qa, sa = quantize_blocks(w.a.reshape(G * max_m, K), 1)
    qs = [quantize_blocks(w.b[g], 128) for g in range(G)]
    qb = np.stack([q for q, _ in qs])
    sb = np.stack([s for _, s in qs])
    d = bf16_out((G, max_m, N), fill=SENTINEL)
    fp8g.grouped_gemm_fp8_masked(to_dev(qa.reshape(G, max_m, K)), to_dev(np.ascontiguousarray(sa.T)),
                                 to_dev(qb), to_dev(sb), d, to_dev(np.asarray(counts, np.int32)),
                                 expected_m=em)
    got = bits(d)
    sentinel = np.full((G, max_m, N), SENTINEL, np.uint16)
    K128 = -(-K // 128)
    ref, _, valid = grouped_masked(qa.reshape(G, max_m, K), sa.reshape(G, max_m, K128), qb, sb,
                                   np.asarray(counts), sentinel)
    assert np.array_equal(got[~valid], ref[~valid]), "rows past the counts changed"
    _assert_tol(got[valid], ref[valid], f"masked ragged G={G}")
