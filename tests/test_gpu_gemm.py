"""GPU GEMM parity (dense, grouped contiguous, grouped masked) against the oracle.

Operands are quantised by the oracle (bit-exact with the GPU quantiser, which
test_gpu_quantize pins) and uploaded; the GPU result must satisfy
|d - ref| <= 2^-7 |ref| + 2^-10 rms(ref) elementwise, ref being the oracle's
bf16 result and rms taken over the output rows that exist (dense: all rows;
contiguous: token rows, the zero padding rows are checked to be exactly +0
instead; masked: valid rows, the others must keep their sentinel bits).
Large workloads are checked on sampled rows / experts that the oracle computes
independently (rows and experts do not interact).
"""

import numpy as np
import pytest
import torch

import moe_grouped_gemm_quantizer_amd as fp8g
from oracle import (quantize_blocks, gemm_blockscaled, grouped_contiguous, grouped_masked,
                    tolerance_check)
from workloads import make_config, make_dense, make_contiguous, make_masked
from tests.gpu_util import (dev, to_dev, to_host, bits, bf16_out, quantize_a, quantize_b,
                            banner)

pytestmark = pytest.mark.gpu


def _oracle_operands_dense(w):
    qa, sa = quantize_blocks(w.a, 1)
    qb, sb = quantize_blocks(w.b, 128)
    return qa, sa, qb, sb


def _run_dense(qa, sa, qb, sb):
    M, K = qa.shape
    N = qb.shape[0]
    d = bf16_out((M, N), fill=0x7FBF)
    fp8g.gemm_fp8_blockscaled(to_dev(qa), to_dev(sa.T), to_dev(qb), to_dev(sb), d)
    return bits(d)


def _assert_tol(got, ref, what):
    ok, worst, nbad = tolerance_check(got, ref)
    assert ok, f"{what}: {nbad} elements out of tolerance, worst ratio {worst:.3g}"


@pytest.mark.parametrize("M,N,K", [(128, 256, 512), (1, 128, 128), (7, 256, 256),
                                   (100, 384, 384), (129, 128, 640), (300, 512, 1024),
                                   (257, 640, 256), (16, 1024, 2048), (17, 384, 1280),
                                   (32, 256, 640), (5, 256, 8960), (33, 128, 256)])
def test_dense_shapes(M, N, K):
    banner(f"dense {M}x{N}x{K}")
    w = make_dense(M, N, K, seed=M + N + K)
    qa, sa, qb, sb = _oracle_operands_dense(w)
    got = _run_dense(qa, sa, qb, sb)
    ref, _ = gemm_blockscaled(qa, sa, qb, sb)
    _assert_tol(got, ref, f"dense {M}x{N}x{K}")


def test_config0_end_to_end_gpu_quantiser():
    w = make_config(0)
    banner("cfg0 end to end: GPU quantise -> GPU GEMM")
    qa_d, sa_d = quantize_a(w.a)
    qb_d, sb_d = quantize_b(w.b)
    d = bf16_out((w.M, w.N))
    fp8g.gemm_fp8_blockscaled(qa_d, sa_d, qb_d, sb_d, d)
    ref, _ = gemm_blockscaled(*_oracle_operands_dense(w))
    _assert_tol(bits(d), ref, "cfg0 e2e")


def test_config1_small_m_full():
    w = make_config(1)
    banner("cfg1 16x4096x7168 full")
    qa, sa, qb, sb = _oracle_operands_dense(w)
    got = _run_dense(qa, sa, qb, sb)
    ref, _ = gemm_blockscaled(qa, sa, qb, sb)
    _assert_tol(got, ref, "cfg1")


def test_config2_dense_large_sampled_rows():
    w = make_config(2)
    banner("cfg2 4096x8192x8192, GPU quantise + GEMM, 48 sampled rows checked")
    qa_d, sa_d = quantize_a(w.a)
    qb_d, sb_d = quantize_b(w.b)
    d = bf16_out((w.M, w.N))
    fp8g.gemm_fp8_blockscaled(qa_d, sa_d, qb_d, sb_d, d)
    got = bits(d)
    rng = np.random.default_rng(2024)
    rows = np.sort(np.concatenate([[0, 127, 128, 4095], rng.choice(4096, 44, replace=False)]))
    rows = np.unique(rows)
    qa, sa = quantize_blocks(w.a[rows], 1)
    qb = to_host(qb_d)
    sb = to_host(sb_d)
    ref, _ = gemm_blockscaled(qa, sa, qb, sb)
    _assert_tol(got[rows], ref, "cfg2 sampled rows")
    # determinism: a second run is bitwise identical
    d2 = bf16_out((w.M, w.N))
    fp8g.gemm_fp8_blockscaled(qa_d, sa_d, qb_d, sb_d, d2)
    assert torch.equal(d, d2)


def test_power_of_two_scales_exact_on_gpu():
    w = make_dense(256, 512, 1024, seed=5)
    qa, sa, qb, sb = _oracle_operands_dense(w)
    g0 = _run_dense(qa, sa, qb, sb)
    g1 = _run_dense(qa, sa * np.float32(2.0 ** -3), qb, sb * np.float32(2.0 ** 5))
    v0 = (g0.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    v1 = (g1.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(v1, v0 * 4.0)


def _contiguous_case(counts, N, K, seed):
    w = make_contiguous(counts, N, K, seed=seed)
    qa, sa = quantize_blocks(w.a, 1)
    qs = [quantize_blocks(w.b[g], 128) for g in range(w.G)]
    qb = np.stack([q for q, _ in qs])
    sb = np.stack([s for _, s in qs])
    d = bf16_out((w.M, N), fill=0x7FBF)
    fp8g.grouped_gemm_fp8_contiguous(to_dev(qa), to_dev(sa.T), to_dev(qb), to_dev(sb), d,
                                     to_dev(w.offsets.astype(np.int32)))
    return w, qa, sa, qb, sb, bits(d)


@pytest.mark.parametrize("counts", [[8, 8], [130, 0, 7, 256], [0, 0, 300], [1], [500, 1, 0]])
def test_contiguous_small(counts):
    banner(f"contiguous counts={counts}")
    w, qa, sa, qb, sb, got = _contiguous_case(counts, 256, 384, seed=len(counts))
    ref, _ = grouped_contiguous(qa, sa, qb, sb, w.offsets)
    # token rows within tolerance (rms over token rows); padding rows exactly +0
    tok = np.zeros(w.M, bool)
    for g in range(w.G):
        r0 = int(w.offsets[g])
        tok[r0:r0 + int(w.counts[g])] = True
    _assert_tol(got[tok], ref[tok], f"contiguous {counts}")
    assert np.all(got[~tok] == 0) and np.all(ref[~tok] == 0)


# (tile counts on 256 CUs: 256-row tiles enumerated per expert / 128x256 tiles)
@pytest.mark.parametrize("counts,N,K", [
    ([9000, 4500, 2600, 2200], 1024, 2048),   # 74 x 4 = 296 tiles: 40 left, 4 pieces / 584: 72 left, 2
    ([12000, 6000, 3000, 3000], 640, 1024),   # 95 x 3 = 285, last block 128 columns: 29 left, 2 pieces
    ([10000, 6000, 3000], 384, 1024),         # 76 x 2 = 152: one round / 300: 44 left, 2 pieces
    ([5000, 1, 0, 4200], 768, 1024),          # less than one round either way
    ([4000, 2000, 300], 256, 1024)])
@pytest.mark.parametrize("cfg", ["default", "mid"])
def test_contiguous_split_tail_full(counts, N, K, cfg, monkeypatch):
    """Contiguous shapes whose last round of tiles would run at most half
    full: the leftover tiles are cut into K pieces and summed in a separate
    reduction (planned on the device for the default 256-row tiles, on the
    host for 128x256 tiles, forced with FP8G_FORCE_CFG=mid). Every output
    element is checked."""
    if cfg == "mid":
        monkeypatch.setenv("FP8G_FORCE_CFG", "mid")
    banner(f"contiguous split tail counts={counts} N={N} K={K} cfg={cfg}")
    w, qa, sa, qb, sb, got = _contiguous_case(counts, N, K, seed=N + K)
    ref, _ = grouped_contiguous(qa, sa, qb, sb, w.offsets)
    tok = np.zeros(w.M, bool)
    for g in range(w.G):
        r0 = int(w.offsets[g])
        tok[r0:r0 + int(w.counts[g])] = True
    _assert_tol(got[tok], ref[tok], f"contiguous split tail {counts} {cfg}")
    assert np.all(got[~tok] == 0) and np.all(ref[~tok] == 0)


def test_contiguous_split_workspace_two_streams():
    """Two contiguous calls that both split their tail share the per-device
    workspace; issued back to back on two streams, each must still match its
    own oracle (the second waits for the first one's reduction)."""
    banner("contiguous split tail on two streams")
    cases = []
    for seed, counts in ((1, [9000, 4500, 2600, 2200]), (2, [7000, 7000, 2000, 2400])):
        w = make_contiguous(counts, 1024, 2048, seed=seed)
        qa, sa = quantize_blocks(w.a, 1)
        qs = [quantize_blocks(w.b[g], 128) for g in range(w.G)]
        qb = np.stack([q for q, _ in qs])
        sb = np.stack([x for _, x in qs])
        dev_args = (to_dev(qa), to_dev(np.ascontiguousarray(sa.T)), to_dev(qb), to_dev(sb))
        d = bf16_out((w.M, 1024), fill=0x7FBF)
        cases.append((w, qa, sa, qb, sb, dev_args, d, to_dev(w.offsets.astype(np.int32))))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for (w, qa, sa, qb, sb, dev_args, d, offs), st in zip(cases, streams):
        with torch.cuda.stream(st):
            fp8g.grouped_gemm_fp8_contiguous(*dev_args, d, offs)
    torch.cuda.synchronize()
    for w, qa, sa, qb, sb, dev_args, d, offs in cases:
        got = bits(d)
        ref, _ = grouped_contiguous(qa, sa, qb, sb, w.offsets)
        tok = np.zeros(w.M, bool)
        for g in range(w.G):
            r0 = int(w.offsets[g])
            tok[r0:r0 + int(w.counts[g])] = True
        _assert_tol(got[tok], ref[tok], f"two streams {w.counts.tolist()}")
        assert np.all(got[~tok] == 0)


def test_contiguous_more_than_1024_experts():
    """More experts than the per-expert metadata holds: the contiguous call
    falls back to 128-row tiles over the global row grid."""
    counts = [0] * 1025
    counts[0], counts[7], counts[500], counts[1024] = 5, 128, 130, 1
    banner("contiguous G=1025")
    w, qa, sa, qb, sb, got = _contiguous_case(counts, 128, 256, seed=3)
    ref, _ = grouped_contiguous(qa, sa, qb, sb, w.offsets)
    tok = np.zeros(w.M, bool)
    for g in range(w.G):
        r0 = int(w.offsets[g])
        tok[r0:r0 + int(w.counts[g])] = True
    _assert_tol(got[tok], ref[tok], "contiguous G=1025")
    assert np.all(got[~tok] == 0)


def test_config3_contiguous_sampled():
    w = make_config(3)
    G, N, K = w.b.shape
    banner(f"cfg3 contiguous G={G} M_total={w.M} N={N} K={K}")
    qa_d, sa_d = quantize_a(w.a)
    b2 = torch.from_numpy(w.b.reshape(G * N, K)).to(dev())
    qb_d, sb_d = quantize_b(b2)
    del b2
    d = bf16_out((w.M, N), fill=0x7FBF)
    fp8g.grouped_gemm_fp8_contiguous(qa_d, sa_d, qb_d.view(G, N, K),
                                     sb_d.view(G, N // 128, K // 128), d,
                                     to_dev(w.offsets.astype(np.int32)))
    got = bits(d)
    qb = to_host(qb_d).reshape(G, N, K)
    sb = to_host(sb_d).reshape(G, N // 128, K // 128)
    rng = np.random.default_rng(33)
    checked = 0
    for g in range(G):
        r0, r1 = int(w.offsets[g]), int(w.offsets[g + 1])
        c = int(w.counts[g])
        rows = np.unique(np.concatenate([[r0, r0 + c - 1],
                                         r0 + rng.choice(c, min(c, 5), replace=False)]))
        qa, sa = quantize_blocks(w.a[rows], 1)
        ref, _ = gemm_blockscaled(qa, sa, qb[g], sb[g])
        _assert_tol(got[rows], ref, f"cfg3 expert {g}")
        assert np.all(got[r0 + c:r1] == 0)          # zero padding rows -> +0
        checked += len(rows)
    assert checked > 8 * 3


def _masked_inputs(w):
    G, mm, K = w.a.shape
    qa, sa = quantize_blocks(w.a.reshape(G * mm, K), 1)
    qs = [quantize_blocks(w.b[g], 128) for g in range(G)]
    return qa.reshape(G, mm, K), sa, np.stack([q for q, _ in qs]), np.stack([s for _, s in qs])


@pytest.mark.parametrize("counts,max_m", [([0, 1, 255, 256], 256), ([3, 0, 77], 100),
                                          ([129, 128, 0, 200, 5], 200)])
def test_masked_small(counts, max_m):
    banner(f"masked counts={counts} max_m={max_m}")
    w = make_masked(counts, max_m, 256, 384, seed=max_m)
    G, mm, K = w.a.shape
    N = 256
    qa, sa, qb, sb = _masked_inputs(w)
    d = bf16_out((G, mm, N), fill=0x7FBF)
    fp8g.grouped_gemm_fp8_masked(to_dev(qa), to_dev(sa.T), to_dev(qb), to_dev(sb), d,
                                 to_dev(np.asarray(counts, np.int32)), expected_m=max_m // 2)
    got = bits(d)
    sentinel = np.full((G, mm, N), 0x7FBF, np.uint16)
    ref, _, valid = grouped_masked(qa, sa.reshape(G, mm, K // 128), qb, sb, w.masked_m, sentinel)
    assert np.array_equal(got[~valid], ref[~valid])          # untouched rows keep the sentinel
    _assert_tol(got[valid], ref[valid], f"masked {counts}")


@pytest.mark.parametrize("counts,max_m,N", [
    ([600, 0, 257, 513, 1, 16, 17, 255], 600, 512),          # several 256-row blocks per expert
    (list(np.random.default_rng(5).integers(0, 257, 64)), 256, 2048),   # 2 rounds of tiles, ties
    ([256] * 3 + [0] * 5 + [33] * 4 + [240, 241, 15, 16], 256, 768)])    # equal counts
def test_masked_large_tiles(counts, max_m, N):
    """256-row tiles (expected_m above 128): per-16-row skipping, experts
    scheduled largest first, alternate rounds walked backwards."""
    counts = [int(c) for c in counts]
    banner(f"masked large tiles G={len(counts)} max_m={max_m} N={N}")
    w = make_masked(counts, max_m, N, 256, seed=len(counts))
    G, mm, K = w.a.shape
    qa, sa, qb, sb = _masked_inputs(w)
    d = bf16_out((G, mm, N), fill=0x7FBF)
    fp8g.grouped_gemm_fp8_masked(to_dev(qa), to_dev(sa.T), to_dev(qb), to_dev(sb), d,
                                 to_dev(np.asarray(counts, np.int32)), expected_m=max_m)
    got = bits(d)
    sentinel = np.full((G, mm, N), 0x7FBF, np.uint16)
    ref, _, valid = grouped_masked(qa, sa.reshape(G, mm, K // 128), qb, sb, w.masked_m, sentinel)
    assert np.array_equal(got[~valid], ref[~valid])          # untouched rows keep the sentinel
    _assert_tol(got[valid], ref[valid], f"masked large tiles G={G}")


def test_config4_masked_sampled():
    w = make_config(4)
    G, N, K = w.b.shape
    mm = w.M
    banner(f"cfg4 masked G={G} max_m={mm} N={N} K={K}")
    qa_d, sa_d = quantize_a(w.a.reshape(G * mm, K))
    b2 = torch.from_numpy(w.b.reshape(G * N, K)).to(dev())
    qb_d, sb_d = quantize_b(b2)
    del b2
    d = bf16_out((G, mm, N), fill=0x7FBF)
    fp8g.grouped_gemm_fp8_masked(qa_d.view(G, mm, K), sa_d, qb_d.view(G, N, K),
                                 sb_d.view(G, N // 128, K // 128), d,
                                 to_dev(w.masked_m.astype(np.int32)), expected_m=135)
    got = bits(d)
    # every row past its expert's count still holds the sentinel
    for g in range(G):
        assert np.all(got[g, int(w.masked_m[g]):] == 0x7FBF), g
    # sampled experts: empty, tiny, just above one block, the largest
    qb = to_host(qb_d).reshape(G, N, K)
    sb = to_host(sb_d).reshape(G, N // 128, K // 128)
    for g in (23, 7, 12, 14):
        m = int(w.masked_m[g])
        if m == 0:
            continue
        qa, sa = quantize_blocks(w.a[g, :m], 1)
        ref, _ = gemm_blockscaled(qa, sa, qb[g], sb[g])
        _assert_tol(got[g, :m], ref, f"cfg4 expert {g}")
