"""GPU parity on seeded random shapes, every element against the oracle.

Thirty cases drawn from one seed: dense (M 1..700), contiguous (1..6
experts, 0..400 tokens each, with and without a split-tail workspace) and
masked (1..6 experts, max_m 1..300, counts 0..max_m, a random expected_m)
GEMMs, N and K multiples of 16 (so partial 128-column blocks and partial
last K blocks of every size turn up, K from a single partial block to 2240),
which between them take the small-M kernel, both tile configurations and
the shape-generic and ragged-K instantiations. Operands are
quantised by the oracle; the outputs must lie within
|d - ref| <= 2^-7 |ref| + 2^-10 rms(ref) of the oracle's fp64 result,
padding rows of the contiguous layout must be +0, and masked rows past
their expert's count must keep the sentinel. Three more contiguous cases
are sized to have a split tail (280-320 tiles of 256x256 on 256 CUs, 16 K
blocks cut into 4 pieces) with a ragged K, so that the partial last K
block falls in the last piece. Each case prints its shape before it
runs."""

import numpy as np
import pytest
import torch

import moe_grouped_gemm_quantizer_amd as fp8g
from oracle import quantize_blocks, gemm_blockscaled, grouped_contiguous, grouped_masked, \
    tolerance_check
from workloads import make_dense, make_contiguous, make_masked
from tests.gpu_util import dev, to_dev, bits, bf16_out, banner

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FBF


def _cases():
    rng = np.random.default_rng(20261203)
    out = []
    for i in range(30):
        kind = ("dense", "contiguous", "masked")[i % 3]
        N = 16 * int(rng.integers(1, 71))
        K = 16 * int(rng.integers(1, 141))
        if kind == "dense":
            M = int(rng.integers(1, 33)) if rng.random() < 0.3 else int(rng.integers(1, 701))
            out.append((i, kind, dict(M=M, N=N, K=K)))
        elif kind == "contiguous":
            G = int(rng.integers(1, 7))
            counts = [int(c) for c in rng.integers(0, 401, G)]
            out.append((i, kind, dict(counts=counts, N=N, K=K, ws=bool(rng.random() < 0.5))))
        else:
            G = int(rng.integers(1, 7))
            max_m = int(rng.integers(1, 301))
            counts = [int(c) for c in rng.integers(0, max_m + 1, G)]
            em = int(rng.integers(1, max_m + 1))
            out.append((i, kind, dict(counts=counts, max_m=max_m, N=N, K=K, em=em)))
    return out


CASES = _cases()


def _assert_tol(got, ref, what):
    ok, worst, nbad = tolerance_check(got, ref)
    banner(f"{what}: worst ratio {worst:.4f}")
    assert ok, f"{what}: {nbad} elements out of tolerance"


SPLIT_CASES = [(100, "contiguous", dict(counts=[2000, 3000, 1500, 2300], N=2048, K=2032, ws=True)),
               (101, "contiguous", dict(counts=[4100, 900, 3000], N=2048, K=2000, ws=True)),
               (102, "contiguous", dict(counts=[1000] * 9, N=2048, K=1968, ws=True))]


@pytest.mark.parametrize("case", CASES + SPLIT_CASES,
                         ids=[f"{c[0]}-{c[1]}" for c in CASES + SPLIT_CASES])
def test_random_shape(case):
    i, kind, p = case
    banner(f"random case {i}: {kind} {p}")
    if kind == "dense":
        M, N, K = p["M"], p["N"], p["K"]
        w = make_dense(M, N, K, seed=1000 + i)
        qa, sa = quantize_blocks(w.a, 1)
        qb, sb = quantize_blocks(w.b, 128)
        d = bf16_out((M, N), fill=SENTINEL)
        fp8g.gemm_fp8_blockscaled(to_dev(qa), to_dev(np.ascontiguousarray(sa.T)), to_dev(qb),
                                  to_dev(sb), d)
        ref, _ = gemm_blockscaled(qa, sa, qb, sb)
        _assert_tol(bits(d), ref, f"case {i} dense {M}x{N}x{K}")
    elif kind == "contiguous":
        counts, N, K = p["counts"], p["N"], p["K"]
        w = make_contiguous(counts, N, K, seed=1000 + i)
        if w.M == 0:
            return
        qa, sa = quantize_blocks(w.a, 1)
        qs = [quantize_blocks(w.b[g], 128) for g in range(w.G)]
        qb = np.stack([q for q, _ in qs])
        sb = np.stack([s for _, s in qs])
        d = bf16_out((w.M, N), fill=SENTINEL)
        args = (to_dev(qa), to_dev(np.ascontiguousarray(sa.T)), to_dev(qb), to_dev(sb), d,
                to_dev(w.offsets.astype(np.int32)))
        if p["ws"]:
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
        if tok.any():
            _assert_tol(got[tok], ref[tok], f"case {i} contiguous")
        assert np.all(got[~tok] == 0), "padding rows not +0"
    else:
        counts, max_m, N, K, em = p["counts"], p["max_m"], p["N"], p["K"], p["em"]
        G = len(counts)
        w = make_masked(counts, max_m, N, K, seed=1000 + i)
        qa, sa = quantize_blocks(w.a.reshape(G * max_m, K), 1)
        qs = [quantize_blocks(w.b[g], 128) for g in range(G)]
        qb = np.stack([q for q, _ in qs])
        sb = np.stack([s for _, s in qs])
        d = bf16_out((G, max_m, N), fill=SENTINEL)
        fp8g.grouped_gemm_fp8_masked(to_dev(qa.reshape(G, max_m, K)),
                                     to_dev(np.ascontiguousarray(sa.T)), to_dev(qb), to_dev(sb), d,
                                     to_dev(np.asarray(counts, np.int32)), expected_m=em)
        K128 = -(-K // 128)
        sentinel = np.full((G, max_m, N), SENTINEL, np.uint16)
        ref, _, valid = grouped_masked(qa.reshape(G, max_m, K), sa.reshape(G, max_m, K128), qb, sb,
                                       np.asarray(counts), sentinel)
        got = bits(d)
        assert np.array_equal(got[~valid], ref[~valid]), "rows past the counts changed"
        if valid.any():
            _assert_tol(got[valid], ref[valid], f"case {i} masked")
