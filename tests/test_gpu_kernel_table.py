"""The kernel table on the GPU (nxmr §2.3, done ahead of time): warm-up,
and the shape-specialised kernels against the generic ones.

Every hot shape is the shape of a full-size parity test (test_gpu_gemm,
test_gpu_pertensor, test_gpu_fused_quant), so those tests check the
specialised kernels against the oracle element by element. Here the same
calls run again with the specialisations switched off, and the generic
kernels must give the same bits, so the generic path is covered at the
same sizes. Operands are quantised on the GPU (the property compares two
GPU kernels on identical inputs; nothing here needs the oracle)."""

import numpy as np
import pytest
import torch

import moe_grouped_gemm_quantizer_amd as fp8g
from tests import oracle_ops
from tests.gpu_util import dev, to_dev, bf16_out, quantize_a, quantize_b, banner

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FBF


def _both(call, what):
    """Run call() with the specialisations on, then off; return both outputs."""
    assert "specialised" in what, what
    outs = []
    try:
        for spec in (True, False):
            fp8g.fp8g_set_shape_specialisation(spec)
            outs.append(call())
    finally:
        fp8g.fp8g_set_shape_specialisation(True)
    torch.cuda.synchronize()
    return outs


def _assert_same(outs, what):
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                           b.view(torch.int32) if b.dtype == torch.float32 else b), \
            f"{what}: specialised and generic kernels differ"


def test_warmup_loads_every_kernel():
    banner("fp8g_warmup twice")
    fp8g.fp8g_warmup()
    fp8g.fp8g_warmup()


def _dense_operands(cfg):
    w = oracle_ops.workload(cfg)
    qa, sa = quantize_a(w.a)
    qb, sb = quantize_b(w.b)
    return w, qa, sa, qb, sb


def test_dense_specialised_equals_generic():
    w, qa, sa, qb, sb = _dense_operands(2)
    M, N, K = w.M, w.N, w.K
    what = fp8g.fp8g_gemm_kernel_name("dense", M, N, K)
    banner(f"dense {M}x{N}x{K}: {what} vs generic")

    def call():
        d = bf16_out((M, N), fill=SENTINEL)
        fp8g.gemm_fp8_blockscaled(qa, sa, qb, sb, d)
        return (d,)
    _assert_same(_both(call, what), "dense")

    pqa = torch.empty_like(qa)
    pqb = torch.empty_like(qb)
    psa = torch.empty(1, dtype=torch.float32, device=dev())
    psb = torch.empty(1, dtype=torch.float32, device=dev())
    fp8g.fp8_quantize_tensor(to_dev(w.a), pqa, psa)
    fp8g.fp8_quantize_tensor(to_dev(w.b), pqb, psb)
    whatp = fp8g.fp8g_gemm_kernel_name("pertensor", M, N, K)
    banner(f"per-tensor: {whatp} vs generic")

    def callp():
        d = bf16_out((M, N), fill=SENTINEL)
        fp8g.gemm_fp8_pertensor(pqa, psa, pqb, psb, d)
        return (d,)
    _assert_same(_both(callp, whatp), "per-tensor")


def test_small_m_specialised_equals_generic():
    w, qa, sa, qb, sb = _dense_operands(1)
    M, N, K = w.M, w.N, w.K
    what = fp8g.fp8g_gemm_kernel_name("dense", M, N, K)
    banner(f"small-M {M}x{N}x{K}: {what} vs generic")

    def call():
        d = bf16_out((M, N), fill=SENTINEL)
        fp8g.gemm_fp8_blockscaled(qa, sa, qb, sb, d)
        return (d,)
    _assert_same(_both(call, what), "small-M")


@pytest.mark.parametrize("entry", ["workspace", "plain"])
def test_contiguous_specialised_equals_generic(entry):
    w = oracle_ops.workload(3)
    G, N, K = w.G, w.N, w.K
    qa, sa = quantize_a(w.a)
    qb, sb = quantize_b(w.b.reshape(G * N, K))
    qb, sb = qb.view(G, N, K), sb.view(G, N // 128, K // 128)
    offs = to_dev(w.offsets.astype(np.int32))
    n = fp8g.grouped_gemm_fp8_contiguous_workspace_size(G, w.M, N, K)
    ws = torch.empty(n, dtype=torch.uint8, device=dev()) if (n and entry == "workspace") else None
    what = fp8g.fp8g_gemm_kernel_name("contiguous", w.M, N, K, G=G)
    banner(f"contiguous G={G} M_total={w.M} N={N} K={K} ({entry}): {what} vs generic")

    def call():
        d = bf16_out((w.M, N), fill=SENTINEL)
        if ws is not None:
            fp8g.grouped_gemm_fp8_contiguous_ws(qa, sa, qb, sb, d, offs, ws)
        else:
            fp8g.grouped_gemm_fp8_contiguous(qa, sa, qb, sb, d, offs)
        return (d,)
    _assert_same(_both(call, what), f"contiguous ({entry})")


def test_masked_specialised_equals_generic():
    w = oracle_ops.workload(4)
    G, N, K, mm = w.G, w.N, w.K, w.M
    qa, sa = quantize_a(w.a.reshape(G * mm, K))
    qb, sb = quantize_b(w.b.reshape(G * N, K))
    meta = to_dev(w.masked_m.astype(np.int32))
    em = int(np.mean(w.masked_m))
    what = fp8g.fp8g_gemm_kernel_name("masked", mm, N, K, G=G, expected_m=em)
    banner(f"masked G={G} max_m={mm} N={N} K={K}: {what} vs generic")

    def call():
        d = bf16_out((G, mm, N), fill=SENTINEL)
        fp8g.grouped_gemm_fp8_masked(qa.view(G, mm, K), sa, qb.view(G, N, K),
                                     sb.view(G, N // 128, K // 128), d, meta, expected_m=em)
        return (d,)
    _assert_same(_both(call, what), "masked")
