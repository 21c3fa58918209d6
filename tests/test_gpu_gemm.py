"""GPU GEMM parity (dense, grouped contiguous, grouped masked) against the oracle.

Every expected value comes from oracle/ alone: the operands are quantised by
the oracle (tests/oracle_ops.py), uploaded, multiplied by the library, and
every output element is compared with the oracle's bf16 result under

    |d - ref| <= 2^-7 |ref| + 2^-10 rms(ref)

with rms taken over the output rows that exist (dense: all rows; contiguous:
token rows, the zero padding rows are checked to be exactly +0 instead;
masked: valid rows, the others must keep their sentinel bits). The worst
ratio |d - ref| / bound is printed for each case. The GPU quantiser is pinned
bit-exact by test_gpu_quantize; the end-to-end tests here chain the two.
"""

import numpy as np
import pytest
import torch

import moe_grouped_gemm_quantizer_amd as fp8g
from oracle import (quantize_blocks, gemm_blockscaled, gemm_blockscaled_fp32acc,
                    grouped_contiguous, grouped_masked, tolerance_check, e4m3_decode_table,
                    bf16_bits_from_f64, bf16_bits_to_f64)
from workloads import make_config, make_dense, make_contiguous, make_masked
from tests import oracle_ops
from tests.gpu_util import (dev, to_dev, to_host, bits, bf16_out, quantize_a, quantize_b,
                            banner)

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FBF


def _oracle_operands_dense(w):
    qa, sa = quantize_blocks(w.a, 1)
    qb, sb = quantize_blocks(w.b, 128)
    return qa, sa, qb, sb


def _run_dense(qa, sa, qb, sb):
    M, K = qa.shape
    N = qb.shape[0]
    d = bf16_out((M, N), fill=SENTINEL)
    fp8g.gemm_fp8_blockscaled(to_dev(qa), to_dev(sa.T), to_dev(qb), to_dev(sb), d)
    return bits(d)


def _ulp_distance(got, ref):
    """Distance in bf16 ulps between bit patterns (sign-magnitude mapped onto
    a monotone integer line; +0 and -0 coincide)."""
    def ordinal(b):
        b = np.asarray(b, np.uint16).astype(np.int64)
        return np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(ordinal(got) - ordinal(ref))


def _assert_tol(got, ref, what):
    ok, worst, nbad = tolerance_check(got, ref)
    u = _ulp_distance(got, ref)
    # (outputs far below the rms, where blocks cancel, are held by the bound's
    # absolute term; their ulp distance says little, so it is split off)
    r = bf16_bits_to_f64(ref)
    big = np.abs(r) >= np.sqrt(np.mean(r * r)) / 16 if r.size else r.astype(bool)
    ub = u[big]
    banner(f"{what}: {got.size} elements, worst |d - ref| / bound = {worst:.4f}; bf16 ulps from "
           f"the oracle: 0 for {np.count_nonzero(u == 0)}, 1 for {np.count_nonzero(u == 1)}, "
           f"more for {np.count_nonzero(u > 1)}; where |ref| >= rms/16 ({ub.size} elements): "
           f"max {int(ub.max()) if ub.size else 0} ulp, {np.count_nonzero(ub > 1)} above 1")
    assert ok, f"{what}: {nbad} elements out of tolerance, worst ratio {worst:.3g}"
    return worst


def _token_rows(w):
    tok = np.zeros(w.M, bool)
    for g in range(w.G):
        r0 = int(w.offsets[g])
        tok[r0:r0 + int(w.counts[g])] = True
    return tok


def _contiguous_ws(G, M, N, K):
    n = fp8g.grouped_gemm_fp8_contiguous_workspace_size(G, M, N, K)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=dev()) if n else None


# ---------------------------------------------------------------------------
# dense


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


def test_config2_dense_full():
    """4096x8192x8192, the launch configuration the bench times: every output
    element against the oracle, operands quantised by the oracle; a second
    run must be bitwise identical."""
    w = oracle_ops.workload(2)
    banner("cfg2 4096x8192x8192: oracle operands, every element")
    qa, sa, qb, sb = oracle_ops.operands(2)
    ref = oracle_ops.reference(2)
    args = (to_dev(qa), to_dev(sa.T), to_dev(qb), to_dev(sb))
    d = bf16_out((w.M, w.N), fill=SENTINEL)
    fp8g.gemm_fp8_blockscaled(*args, d)
    _assert_tol(bits(d), ref, "cfg2 all elements")
    d2 = bf16_out((w.M, w.N), fill=0)
    fp8g.gemm_fp8_blockscaled(*args, d2)
    assert torch.equal(d, d2), "cfg2: two runs differ"


def test_config2_end_to_end_gpu_quantiser():
    """GPU quantise -> GPU GEMM on the full 4096x8192x8192 workload: the GPU
    codes and scales equal the oracle's bit for bit, so the GEMM result must
    equal the one from oracle operands bit for bit (the kernel is
    deterministic), which is itself checked against the oracle above."""
    w = oracle_ops.workload(2)
    banner("cfg2 end to end: GPU quantise -> GPU GEMM, bitwise against oracle operands")
    qa, sa, qb, sb = oracle_ops.operands(2)
    qa_d, sa_d = quantize_a(w.a)
    qb_d, sb_d = quantize_b(w.b)
    assert np.array_equal(to_host(qa_d), qa) and np.array_equal(to_host(qb_d), qb)
    assert np.array_equal(to_host(sa_d).view(np.uint32), np.ascontiguousarray(sa.T).view(np.uint32))
    assert np.array_equal(to_host(sb_d).view(np.uint32), sb.view(np.uint32))
    d = bf16_out((w.M, w.N))
    fp8g.gemm_fp8_blockscaled(qa_d, sa_d, qb_d, sb_d, d)
    got = bits(d)
    ref = oracle_ops.reference(2)
    _assert_tol(got, ref, "cfg2 e2e")


def test_power_of_two_scales_exact_on_gpu():
    w = make_dense(256, 512, 1024, seed=5)
    qa, sa, qb, sb = _oracle_operands_dense(w)
    g0 = _run_dense(qa, sa, qb, sb)
    g1 = _run_dense(qa, sa * np.float32(2.0 ** -3), qb, sb * np.float32(2.0 ** 5))
    v0 = (g0.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    v1 = (g1.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(v1, v0 * 4.0)


def _accumulate_bf16(qa, sa, qb, sb):
    """A deliberately wrong model (bf16 accumulator): the exact block sums,
    promoted into an accumulator rounded to bf16 after every block. Used
    only to show that the cancelling case below separates fp32 promotion
    from a low-precision one."""
    t = e4m3_decode_table()
    A, B = t[qa], t[qb]
    M, K = qa.shape
    N = qb.shape[0]
    acc = np.zeros((M, N))
    sbn = np.repeat(sb.astype(np.float64), 128, axis=0)
    for kb in range(K // 128):
        ks = slice(kb * 128, kb * 128 + 128)
        P = A[:, ks] @ B[:, ks].T
        c = sa[:, kb].astype(np.float64)[:, None] * sbn[:, kb][None, :]
        acc = (bf16_bits_from_f64(acc + c * P).astype(np.uint32) << 16).view(np.float32)
        acc = acc.astype(np.float64)
    return bf16_bits_from_f64(acc)


def test_nan_codes_propagate():
    """An e4m3 NaN code (0x7F or 0xFF) in an operand makes every output that
    sums over it NaN, which the bf16 rounding (formats.bf16_bits_from_f64)
    writes as 0x7FC0 whatever the sign: one NaN code in A row 3 and one in B
    row 17 turn all of output row 3 and column 17 into 0x7FC0, bit for bit
    with the oracle, and leave every other output within tolerance. Ragged
    N and K (multiples of 16) included."""
    for (M, N, K) in ((64, 256, 512), (40, 144, 400)):
        w = make_dense(M, N, K, seed=7)
        qa, sa, qb, sb = _oracle_operands_dense(w)
        qa = qa.copy()
        qb = qb.copy()
        qa[3, 100] = 0x7F                   # positive NaN code
        qb[17, K - 5] = 0xFF                # negative NaN code, in the last K block
        ref, _ = gemm_blockscaled(qa, sa, qb, sb)
        nan_ref = ref == 0x7FC0
        assert nan_ref[3, :].all() and nan_ref[:, 17].all()
        assert nan_ref.sum() == N + M - 1
        got = _run_dense(qa, sa, qb, sb)
        banner(f"NaN codes {M}x{N}x{K}: {int((got == 0x7FC0).sum())} NaN outputs, expected {N + M - 1}")
        assert np.array_equal(got[nan_ref], ref[nan_ref])
        _assert_tol(got[~nan_ref], ref[~nan_ref], f"NaN codes {M}x{N}x{K}, other outputs")


def test_cancelling_blocks():
    """K blocks whose promoted partial sums alternate in sign and nearly
    cancel: every A row repeats one positive 128-vector in each K block, and
    block kb of every B row is (-1)^kb times one positive vector plus a small
    per-block perturbation. The result is about 2^5 .. 2^9 times smaller
    than the partial sums, so the error of the accumulator (czchanglian §2.3:
    fp32 over all of K) is magnified by that much. The fp32-promotion model
    of the oracle passes, a bf16 accumulator fails, and the GPU must pass."""
    M, N, K = 64, 256, 2048
    rng = np.random.default_rng(99)
    nkb = K // 128
    x = np.abs(rng.standard_normal((M, 128))).astype(np.float32) + 0.1
    a = np.tile(x, (1, nkb))
    z = np.abs(rng.standard_normal((N, 128))).astype(np.float32) + 0.1
    b = np.empty((N, K), np.float32)
    for kb in range(nkb):
        delta = 0.02 * rng.standard_normal((N, 128)).astype(np.float32)
        b[:, kb * 128:(kb + 1) * 128] = (-1.0) ** kb * (z + delta)
    qa, sa = quantize_blocks(a, 1)
    qb, sb = quantize_blocks(b, 128)
    ref, ref64 = gemm_blockscaled(qa, sa, qb, sb)
    # size of the partial sums against the result
    t = e4m3_decode_table()
    P0 = (t[qa[:, :128]] @ t[qb[:, :128]].T) * sa[:, :1].astype(np.float64) * float(sb[0, 0])
    cancel = np.median(np.abs(P0) / np.maximum(np.abs(ref64), 1e-30))
    banner(f"cancelling blocks: median |partial| / |result| = {cancel:.1f}")
    assert cancel > 32
    assert tolerance_check(gemm_blockscaled_fp32acc(qa, sa, qb, sb), ref)[0]
    assert not tolerance_check(_accumulate_bf16(qa, sa, qb, sb), ref)[0]
    got = _run_dense(qa, sa, qb, sb)
    _assert_tol(got, ref, "cancelling blocks (GPU)")


# ---------------------------------------------------------------------------
# contiguous


def _contiguous_case(counts, N, K, seed, workspace=False):
    w = make_contiguous(counts, N, K, seed=seed)
    qa, sa = quantize_blocks(w.a, 1)
    qs = [quantize_blocks(w.b[g], 128) for g in range(w.G)]
    qb = np.stack([q for q, _ in qs])
    sb = np.stack([s for _, s in qs])
    d = bf16_out((w.M, N), fill=SENTINEL)
    args = (to_dev(qa), to_dev(sa.T), to_dev(qb), to_dev(sb), d,
            to_dev(w.offsets.astype(np.int32)))
    if workspace:
        fp8g.grouped_gemm_fp8_contiguous_ws(*args, _contiguous_ws(w.G, w.M, N, K))
    else:
        fp8g.grouped_gemm_fp8_contiguous(*args)
    return w, qa, sa, qb, sb, bits(d)


def _check_contiguous(w, got, ref, what):
    tok = _token_rows(w)
    _assert_tol(got[tok], ref[tok], what)
    assert np.all(got[~tok] == 0) and np.all(ref[~tok] == 0), f"{what}: padding rows not +0"


@pytest.mark.parametrize("counts", [[8, 8], [130, 0, 7, 256], [0, 0, 300], [1], [500, 1, 0]])
def test_contiguous_small(counts):
    banner(f"contiguous counts={counts}")
    w, qa, sa, qb, sb, got = _contiguous_case(counts, 256, 384, seed=len(counts))
    ref, _ = grouped_contiguous(qa, sa, qb, sb, w.offsets)
    _check_contiguous(w, got, ref, f"contiguous {counts}")


# (tile counts on 256 CUs, 256-row tiles enumerated per expert / 128x256 tiles)
@pytest.mark.parametrize("counts,N,K", [
    ([9000, 4500, 2600, 2200], 1024, 2048),   # 74 x 4 = 296 tiles: 40 left, 4 pieces
    ([12000, 6000, 3000, 3000], 640, 1024),   # 95 x 3 = 285, last block 128 columns: 2 pieces
    ([10000, 6000, 3000], 384, 1024),         # 76 x 2 = 152: one round
    ([5000, 1, 0, 4200], 768, 1024),          # less than one round
    ([4000, 2000, 300], 256, 1024),
    ([9000, 4500, 2600, 2200] + [0] * 1021, 1024, 2048)])  # 1025 experts: 128x256 tiles,
                                                           # 584 tiles, 72 left, 2 pieces
@pytest.mark.parametrize("entry", ["plain", "workspace"])
def test_contiguous_split_tail_full(counts, N, K, entry):
    """Contiguous shapes whose last round of tiles would run at most half
    full. With a workspace the leftover tiles are cut into K pieces and
    summed by a separate reduction (planned on the device for 256-row tiles,
    on the host for the 128x256 tiles of more than 1024 experts); without
    one every tile runs whole. Every output element is checked."""
    banner(f"contiguous split tail G={len(counts)} N={N} K={K} {entry}")
    w, qa, sa, qb, sb, got = _contiguous_case(counts, N, K, seed=N + K,
                                              workspace=entry == "workspace")
    ref, _ = grouped_contiguous(qa, sa, qb, sb, w.offsets)
    _check_contiguous(w, got, ref, f"contiguous split tail G={w.G} {entry}")


def test_contiguous_workspace_two_streams():
    """Two contiguous calls that both split their tail, on two streams with
    a workspace each, issued back to back: each must match its own oracle."""
    banner("contiguous split tail on two streams, one workspace each")
    cases = []
    for seed, counts in ((1, [9000, 4500, 2600, 2200]), (2, [7000, 7000, 2000, 2400])):
        w = make_contiguous(counts, 1024, 2048, seed=seed)
        qa, sa = quantize_blocks(w.a, 1)
        qs = [quantize_blocks(w.b[g], 128) for g in range(w.G)]
        qb = np.stack([q for q, _ in qs])
        sb = np.stack([x for _, x in qs])
        dev_args = (to_dev(qa), to_dev(np.ascontiguousarray(sa.T)), to_dev(qb), to_dev(sb))
        d = bf16_out((w.M, 1024), fill=SENTINEL)
        ws = _contiguous_ws(w.G, w.M, 1024, 2048)
        assert ws is not None
        cases.append((w, qa, sa, qb, sb, dev_args, d, to_dev(w.offsets.astype(np.int32)), ws))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for (w, qa, sa, qb, sb, dev_args, d, offs, ws), st in zip(cases, streams):
        with torch.cuda.stream(st):
            fp8g.grouped_gemm_fp8_contiguous_ws(*dev_args, d, offs, ws)
    torch.cuda.synchronize()
    for w, qa, sa, qb, sb, dev_args, d, offs, ws in cases:
        ref, _ = grouped_contiguous(qa, sa, qb, sb, w.offsets)
        _check_contiguous(w, bits(d), ref, f"two streams {w.counts.tolist()}")


def test_contiguous_more_than_1024_experts():
    """More experts than the per-expert metadata holds: the contiguous call
    falls back to 128-row tiles over the global row grid."""
    counts = [0] * 1025
    counts[0], counts[7], counts[500], counts[1024] = 5, 128, 130, 1
    banner("contiguous G=1025")
    w, qa, sa, qb, sb, got = _contiguous_case(counts, 128, 256, seed=3)
    ref, _ = grouped_contiguous(qa, sa, qb, sb, w.offsets)
    _check_contiguous(w, got, ref, "contiguous G=1025")


@pytest.mark.parametrize("entry", ["workspace", "plain"])
def test_config3_contiguous_full(entry):
    """8 experts, 4096 Zipf-routed tokens padded to 4608 rows, N=4096
    K=7168, as the bench times it (with a workspace) and through the plain
    call: every token row against the oracle, padding rows exactly +0, and
    a second run bitwise identical."""
    w = oracle_ops.workload(3)
    G, N, K = w.G, w.N, w.K
    banner(f"cfg3 contiguous G={G} M_total={w.M} N={N} K={K} ({entry}): every element")
    qa, sa, qb, sb = oracle_ops.operands(3)
    ref = oracle_ops.reference(3)
    args = (to_dev(qa), to_dev(sa.T), to_dev(qb.reshape(G, N, K)),
            to_dev(sb.reshape(G, N // 128, K // 128)))
    offs = to_dev(w.offsets.astype(np.int32))
    ws = _contiguous_ws(G, w.M, N, K) if entry == "workspace" else None
    outs = []
    for fill in (SENTINEL, 0):
        d = bf16_out((w.M, N), fill=fill)
        if entry == "workspace":
            fp8g.grouped_gemm_fp8_contiguous_ws(*args, d, offs, ws)
        else:
            fp8g.grouped_gemm_fp8_contiguous(*args, d, offs)
        outs.append(d)
    _check_contiguous(w, bits(outs[0]), ref, f"cfg3 {entry}")
    assert torch.equal(outs[0], outs[1]), "cfg3: two runs differ"


def test_grouped_equals_dense_bitwise():
    """Oracle pin P5 on the GPU: each expert of a grouped call equals a dense
    call on that expert's rows and weights, bit for bit (every tile
    configuration applies the same per-element MFMA and promotion sequence;
    no split here). Contiguous: the expert's padded rows as one dense
    matrix; masked: the expert's whole slab, valid rows compared."""
    N, K = 512, 1024
    counts = [200, 129, 333, 64, 1, 0]
    banner(f"grouped == dense bitwise, counts={counts}")
    w = make_contiguous(counts, N, K, seed=55)
    qa, sa = quantize_blocks(w.a, 1)
    qs = [quantize_blocks(w.b[g], 128) for g in range(w.G)]
    qb = np.stack([q for q, _ in qs])
    sb = np.stack([s for _, s in qs])
    d = bf16_out((w.M, N), fill=SENTINEL)
    fp8g.grouped_gemm_fp8_contiguous(to_dev(qa), to_dev(sa.T), to_dev(qb), to_dev(sb), d,
                                     to_dev(w.offsets.astype(np.int32)))
    got = bits(d)
    for g in range(w.G):
        r0, r1 = int(w.offsets[g]), int(w.offsets[g + 1])
        if r1 > r0:
            dense = _run_dense(qa[r0:r1], sa[r0:r1], qb[g], sb[g])
            assert np.array_equal(got[r0:r1], dense), f"contiguous expert {g}"
    mm = 256
    wm = make_masked(counts, mm, N, K, seed=56)
    G = wm.G
    qam, sam = quantize_blocks(wm.a.reshape(G * mm, K), 1)
    qsm = [quantize_blocks(wm.b[g], 128) for g in range(G)]
    qbm = np.stack([q for q, _ in qsm])
    sbm = np.stack([s for _, s in qsm])
    dm = bf16_out((G, mm, N), fill=SENTINEL)
    fp8g.grouped_gemm_fp8_masked(to_dev(qam.reshape(G, mm, K)), to_dev(sam.T), to_dev(qbm),
                                 to_dev(sbm), dm, to_dev(np.asarray(counts, np.int32)))
    gotm = bits(dm)
    for g in range(G):
        m = counts[g]
        if m:
            dense = _run_dense(qam[g * mm:(g + 1) * mm], sam[g * mm:(g + 1) * mm], qbm[g], sbm[g])
            assert np.array_equal(gotm[g, :m], dense[:m]), f"masked expert {g}"


# ---------------------------------------------------------------------------
# masked


def _masked_inputs(w):
    G, mm, K = w.a.shape
    qa, sa = quantize_blocks(w.a.reshape(G * mm, K), 1)
    qs = [quantize_blocks(w.b[g], 128) for g in range(G)]
    return qa.reshape(G, mm, K), sa, np.stack([q for q, _ in qs]), np.stack([s for _, s in qs])


def _run_masked(qa, sa, qb, sb, counts, expected_m):
    G, mm, K = qa.shape
    N = qb.shape[1]
    d = bf16_out((G, mm, N), fill=SENTINEL)
    fp8g.grouped_gemm_fp8_masked(to_dev(qa), to_dev(sa.T), to_dev(qb), to_dev(sb), d,
                                 to_dev(np.asarray(counts, np.int32)), expected_m=expected_m)
    return bits(d)


def _check_masked(qa, sa, qb, sb, counts, got, what):
    G, mm, K = qa.shape
    N = qb.shape[1]
    sentinel = np.full((G, mm, N), SENTINEL, np.uint16)
    ref, _, valid = grouped_masked(qa, sa.reshape(G, mm, K // 128), qb, sb,
                                   np.asarray(counts), sentinel)
    assert np.array_equal(got[~valid], ref[~valid]), f"{what}: untouched rows changed"
    _assert_tol(got[valid], ref[valid], what)


@pytest.mark.parametrize("counts,max_m", [([0, 1, 255, 256], 256), ([3, 0, 77], 100),
                                          ([129, 128, 0, 200, 5], 200)])
def test_masked_small(counts, max_m):
    banner(f"masked counts={counts} max_m={max_m}")
    w = make_masked(counts, max_m, 256, 384, seed=max_m)
    qa, sa, qb, sb = _masked_inputs(w)
    got = _run_masked(qa, sa, qb, sb, counts, max_m // 2)
    _check_masked(qa, sa, qb, sb, counts, got, f"masked {counts}")


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
    qa, sa, qb, sb = _masked_inputs(w)
    got = _run_masked(qa, sa, qb, sb, counts, max_m)
    _check_masked(qa, sa, qb, sb, counts, got, f"masked large tiles G={len(counts)}")


def test_masked_counts_are_clamped():
    """masked_m values outside [0, max_m] are clamped by the kernel: a
    negative count computes nothing, one above max_m computes the whole slab
    (the oracle clamps the same way)."""
    counts = [-3, 300, 0, 77, 256, -1000000, 1 << 30]
    max_m = 256
    banner(f"masked clamping counts={counts}")
    w = make_masked([0] * len(counts), max_m, 256, 512, seed=17)
    qa, sa, qb, sb = _masked_inputs(w)
    for em in (0, 64):
        got = _run_masked(qa, sa, qb, sb, counts, em)
        _check_masked(qa, sa, qb, sb, counts, got, f"masked clamping expected_m={em}")


def test_masked_expected_m_hint_never_changes_bits():
    """expected_m only picks the tile configuration: results are bitwise
    identical whatever the hint."""
    counts = [int(c) for c in np.random.default_rng(8).integers(0, 257, 12)]
    banner(f"masked expected_m invariance counts={counts}")
    w = make_masked(counts, 256, 512, 1024, seed=8)
    qa, sa, qb, sb = _masked_inputs(w)
    outs = [_run_masked(qa, sa, qb, sb, counts, em) for em in (0, 1, 100, 129, 256, 1 << 20)]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    _check_masked(qa, sa, qb, sb, counts, outs[0], "masked expected_m invariance")


def test_config4_masked_full():
    """32 experts x 256-row slabs, N=7168 K=2048, as the bench times it: every
    valid row of all 31 active experts against the oracle, every other row
    keeps the sentinel, and a second run is bitwise identical."""
    w = oracle_ops.workload(4)
    G, N, K, mm = w.G, w.N, w.K, w.M
    banner(f"cfg4 masked G={G} max_m={mm} N={N} K={K}: every element")
    qa, sa, qb, sb = oracle_ops.operands(4)
    ref = oracle_ops.reference(4)
    args = (to_dev(qa.reshape(G, mm, K)), to_dev(sa.T), to_dev(qb.reshape(G, N, K)),
            to_dev(sb.reshape(G, N // 128, K // 128)))
    meta = to_dev(w.masked_m.astype(np.int32))
    em = int(np.mean(w.masked_m))
    outs = []
    for _ in range(2):
        d = bf16_out((G, mm, N), fill=SENTINEL)
        fp8g.grouped_gemm_fp8_masked(*args, d, meta, expected_m=em)
        outs.append(d)
    got = bits(outs[0])
    valid = np.zeros((G, mm), bool)
    for g in range(G):
        valid[g, :int(w.masked_m[g])] = True
    assert int(np.sum(w.masked_m > 0)) == 31
    assert np.all(got[~valid] == SENTINEL), "cfg4: rows past the counts were written"
    _assert_tol(got[valid], ref[valid], "cfg4 all valid rows")
    assert torch.equal(outs[0], outs[1]), "cfg4: two runs differ"
