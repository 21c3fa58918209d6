"""The GEMM with the quantiser fused into its epilogue (the producer of the
next layer's activations writes them already quantised, nxmr §3.1):
gemm_fp8_blockscaled_quant against the oracle.

* Its bf16 result is the block-scaled GEMM's: within the parity tolerance of
  the oracle, and bitwise equal to gemm_fp8_blockscaled for M > 32 (same
  tile configuration and per-element arithmetic).
* Its codes and scales are the 1x128 quantisation of that bf16 result: on
  every 128-column block whose 128 bf16 values equal the oracle's result
  they equal the oracle quantiser applied to the oracle's result, bit for
  bit; on every block they equal the standalone GPU quantiser (pinned bit
  for bit to the oracle by test_gpu_quantize) applied to the fused kernel's
  own bf16 output.
"""

import numpy as np
import pytest
import torch

import moe_grouped_gemm_quantizer_amd as fp8g
from oracle import quantize_blocks, gemm_blockscaled, tolerance_check, bf16_bits_to_f64
from workloads import make_dense
from tests import oracle_ops
from tests.gpu_util import dev, to_dev, to_host, bits, bf16_out, banner

pytestmark = pytest.mark.gpu


def _fused(qa, sa, qb, sb, with_d=True):
    M, K = qa.shape
    N = qb.shape[0]
    args = (to_dev(qa), to_dev(np.ascontiguousarray(sa.T)), to_dev(qb), to_dev(sb))
    d = bf16_out((M, N), fill=0x7FBF) if with_d else None
    qd = torch.full((M, N), 0xAB, dtype=torch.uint8, device=dev())
    sd = torch.full((N // 128, M), -1.0, dtype=torch.float32, device=dev())
    fp8g.gemm_fp8_blockscaled_quant(*args, d, qd, sd)
    return args, d, qd, sd


def _check(qa, sa, qb, sb, ref, what):
    M, K = qa.shape
    N = qb.shape[0]
    args, d, qd, sd = _fused(qa, sa, qb, sb)
    got = bits(d)
    ok, worst, nbad = tolerance_check(got, ref)
    banner(f"{what}: fused bf16 worst ratio {worst:.4f}")
    assert ok, f"{what}: {nbad} elements out of tolerance"
    if M > 32:
        dp = bf16_out((M, N), fill=0)
        fp8g.gemm_fp8_blockscaled(*args, dp)
        assert torch.equal(d, dp), f"{what}: fused bf16 result differs from the plain GEMM"
    # codes/scales == the standalone quantiser on the fused kernel's own bf16 output
    q2 = torch.empty((M, N), dtype=torch.uint8, device=dev())
    s2 = torch.empty((N // 128, M), dtype=torch.float32, device=dev())
    fp8g.fp8_quantize_bf16(d, 1, q2, s2, 1, M)
    assert torch.equal(qd, q2), f"{what}: fused codes differ from the quantiser"
    assert torch.equal(sd.view(torch.int32), s2.view(torch.int32)), f"{what}: fused scales differ"
    # direct oracle check on the blocks whose bf16 values equal the oracle's
    ref_f32 = bf16_bits_to_f64(ref).astype(np.float32)
    oq, osc = oracle_ops.quantize_rows(ref_f32, 1)
    same = np.all((got == ref).reshape(M, N // 128, 128), axis=2)           # [M][N/128]
    qh = to_host(qd).reshape(M, N // 128, 128)
    assert np.array_equal(qh[same], oq.reshape(M, N // 128, 128)[same]), f"{what}: codes vs oracle"
    sh = to_host(sd).T                                                        # [M][N/128]
    assert np.array_equal(sh[same].view(np.uint32), osc[same].view(np.uint32)), f"{what}: scales"
    banner(f"{what}: {int(same.sum())} of {same.size} blocks checked against the oracle directly")
    # without the bf16 output the codes and scales are the same
    _, _, qd_n, sd_n = _fused(qa, sa, qb, sb, with_d=False)
    assert torch.equal(qd_n, qd) and torch.equal(sd_n.view(torch.int32), sd.view(torch.int32))


@pytest.mark.parametrize("M,N,K", [(300, 512, 1024), (129, 256, 640), (16, 384, 256),
                                   (1, 128, 128), (512, 1024, 2048)])
def test_fused_quant_shapes(M, N, K):
    banner(f"fused quantising epilogue {M}x{N}x{K}")
    w = make_dense(M, N, K, seed=M * 3 + N + K)
    qa, sa = quantize_blocks(w.a, 1)
    qb, sb = quantize_blocks(w.b, 128)
    ref, _ = gemm_blockscaled(qa, sa, qb, sb)
    _check(qa, sa, qb, sb, ref, f"{M}x{N}x{K}")


def test_fused_quant_full_workload():
    banner("fused quantising epilogue 4096x8192x8192")
    qa, sa, qb, sb = oracle_ops.operands(2)
    _check(qa, sa, qb, sb, oracle_ops.reference(2), "4096x8192x8192")
