"""GPU parity of the per-tensor-scaled path (gtnt, Triton kernel section):
fp8_quantize_tensor bit-exact against the oracle's quantiser with one block
covering the whole matrix, and gemm_fp8_pertensor against the oracle's
gemm_pertensor under |d - ref| <= 2^-7 |ref| + 2^-10 rms(ref), every output
element, on small and ragged-M shapes and on the 4096x8192x8192 workload
the gtnt page times."""

import numpy as np
import pytest
import torch

import moe_grouped_gemm_quantizer_amd as fp8g
from oracle import quantize_blocks, gemm_pertensor, tolerance_check
from workloads import make_dense
from tests import oracle_ops
from tests.gpu_util import dev, to_dev, to_host, bits, bf16_out, banner

pytestmark = pytest.mark.gpu


def _quantize_tensor(x):
    xt = x if isinstance(x, torch.Tensor) else to_dev(np.asarray(x, np.float32))
    q = torch.empty(xt.shape, dtype=torch.uint8, device=dev())
    s = torch.full((1,), -1.0, dtype=torch.float32, device=dev())
    fp8g.fp8_quantize_tensor(xt, q, s)
    return q, s


def _check_quant(x, what):
    q, s = _quantize_tensor(x)
    qo, so = quantize_blocks(x, x.shape[0], x.shape[1])
    assert np.array_equal(to_host(s).view(np.uint32), so.reshape(1).view(np.uint32)), what
    qh = to_host(q)
    bad = np.argwhere(qh != qo)[:5]
    assert np.array_equal(qh, qo), f"{what}: {int((qh != qo).sum())} codes differ, e.g. {bad.tolist()}"


@pytest.mark.parametrize("rows,cols", [(1, 4), (3, 1000), (64, 4096), (257, 1028), (2048, 12)])
def test_quantize_tensor_shapes(rows, cols):
    banner(f"quantize per tensor {rows}x{cols}")
    rng = np.random.default_rng(rows * 7 + cols)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x[rng.integers(0, rows), rng.integers(0, cols)] *= np.float32(1e3)
    _check_quant(x, f"{rows}x{cols}")


def test_quantize_tensor_special_values():
    """All-zero tensor (s = 0, signed-zero codes), NaN elements (skipped by
    the amax, coded 0x7F with their sign), subnormal amax, negative zeros."""
    z = np.zeros((16, 64), np.float32)
    z[3, 5] = -0.0
    _check_quant(z, "zeros")
    rng = np.random.default_rng(5)
    x = rng.standard_normal((32, 256)).astype(np.float32)
    x[0, 0] = np.nan
    x[7, 9] = -np.nan
    _check_quant(x, "nan elements")
    tiny = (rng.standard_normal((8, 128)) * 1e-42).astype(np.float32)
    _check_quant(tiny, "subnormal amax")


def test_quantize_tensor_full_workload():
    w = oracle_ops.workload(2)
    banner("quantize per tensor: A 4096x8192 and B 8192x8192")
    qa, s_a, qb, s_b = oracle_ops.pertensor_operands(2)
    for x, qo, so, what in ((w.a, qa, s_a, "A"), (w.b, qb, s_b, "B")):
        q, s = _quantize_tensor(x)
        assert to_host(s).view(np.uint32)[0] == np.float32(so).view(np.uint32), what
        assert np.array_equal(to_host(q), qo), what
        del q, s


@pytest.mark.parametrize("M,N,K", [(128, 256, 512), (1, 128, 128), (100, 384, 384),
                                   (300, 512, 1024), (257, 640, 2048), (33, 128, 256)])
def test_gemm_pertensor_shapes(M, N, K):
    banner(f"gemm per tensor {M}x{N}x{K}")
    w = make_dense(M, N, K, seed=M + 3 * N + K)
    qa, sa = quantize_blocks(w.a, M, K)
    qb, sb = quantize_blocks(w.b, N, K)
    d = bf16_out((M, N), fill=0x7FBF)
    fp8g.gemm_fp8_pertensor(to_dev(qa), to_dev(sa.reshape(1)), to_dev(qb), to_dev(sb.reshape(1)), d)
    ref, _ = gemm_pertensor(qa, sa[0, 0], qb, sb[0, 0])
    ok, worst, nbad = tolerance_check(bits(d), ref)
    banner(f"gemm per tensor {M}x{N}x{K}: worst ratio {worst:.4f}")
    assert ok, f"{nbad} elements out of tolerance (worst {worst:.3g})"


def test_gemm_pertensor_full_workload():
    """4096x8192x8192 (the gtnt H100 table's shape): every element against
    the oracle; then GPU quantise -> GPU GEMM must give the same bits."""
    w = oracle_ops.workload(2)
    banner("gemm per tensor 4096x8192x8192: every element")
    qa, s_a, qb, s_b = oracle_ops.pertensor_operands(2)
    ref = oracle_ops.pertensor_reference(2)
    d = bf16_out((w.M, w.N), fill=0x7FBF)
    fp8g.gemm_fp8_pertensor(to_dev(qa), to_dev(np.float32([s_a])), to_dev(qb),
                            to_dev(np.float32([s_b])), d)
    got = bits(d)
    ok, worst, nbad = tolerance_check(got, ref)
    banner(f"gemm per tensor full: worst |d - ref| / bound = {worst:.4f}")
    assert ok, f"{nbad} elements out of tolerance (worst {worst:.3g})"
    qa_d, sa_d = _quantize_tensor(w.a)
    qb_d, sb_d = _quantize_tensor(w.b)
    d2 = bf16_out((w.M, w.N), fill=0)
    fp8g.gemm_fp8_pertensor(qa_d, sa_d, qb_d, sb_d, d2)
    assert torch.equal(d, d2), "GPU-quantised operands give different bits"
