"""The allocation-free contiguous entry point against the workspace one.

grouped_gemm_fp8_contiguous_noalloc runs the same kernels as
grouped_gemm_fp8_contiguous_ws, with the library's fixed scratch array in
place of a caller workspace. Called twice in a row (the second call smaller,
so the scratch holds the first call's leftovers), each result must equal the
workspace call's bit for bit, and the workspace call is itself checked
against the oracle.
"""

import ctypes

import numpy as np
import pytest
import torch

import moe_grouped_gemm_quantizer_amd as fp8g
from moe_grouped_gemm_quantizer_amd import _lib
from oracle import quantize_blocks, grouped_contiguous, tolerance_check
from workloads import make_contiguous
from tests.gpu_util import dev, to_dev, bits, bf16_out, banner

pytestmark = pytest.mark.gpu


def _noalloc():
    lib = _lib.load()
    f = lib.grouped_gemm_fp8_contiguous_noalloc
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    f.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, vp]
    f.restype = ctypes.c_int
    return f


def _case(counts, N, K, seed):
    w = make_contiguous(counts, N, K, seed=seed)
    qa, sa = quantize_blocks(w.a, 1)
    qs = [quantize_blocks(w.b[g], 128) for g in range(w.G)]
    qb = np.stack([q for q, _ in qs])
    sb = np.stack([s for _, s in qs])
    args = (to_dev(qa), to_dev(np.ascontiguousarray(sa.T)), to_dev(qb), to_dev(sb))
    return w, (qa, sa, qb, sb), args, to_dev(w.offsets.astype(np.int32))


@pytest.mark.parametrize("first,second", [
    (([9000, 4500, 2600, 2200], 1024, 2048), ([5000, 1000, 2600], 768, 1024)),
    (([12000, 6000, 3000, 3000], 640, 1024), ([8, 8], 256, 384))])
def test_noalloc_matches_workspace_call(first, second):
    f = _noalloc()
    stream = torch.cuda.current_stream().cuda_stream
    for i, (counts, N, K) in enumerate((first, second)):
        banner(f"noalloc call {i}: G={len(counts)} N={N} K={K}")
        w, ops, (a, sa, b, sb), offs = _case(counts, N, K, seed=N + K + i)
        n = fp8g.grouped_gemm_fp8_contiguous_workspace_size(w.G, w.M, N, K)
        ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev()) if n else None
        d_ws = bf16_out((w.M, N), fill=0x7FBF)
        fp8g.grouped_gemm_fp8_contiguous_ws(a, sa, b, sb, d_ws, offs, ws)
        d_na = bf16_out((w.M, N), fill=0x7FBF)
        st = f(a.data_ptr(), sa.data_ptr(), b.data_ptr(), sb.data_ptr(), d_na.data_ptr(),
               offs.data_ptr(), w.G, w.M, N, K, stream)
        assert st == 0, fp8g.status_string(st)
        torch.cuda.synchronize()
        assert torch.equal(d_ws, d_na), f"call {i}: noalloc result differs from the workspace call"
        ref, _ = grouped_contiguous(*ops, w.offsets)
        tok = np.zeros(w.M, bool)
        for g in range(w.G):
            tok[int(w.offsets[g]):int(w.offsets[g]) + int(w.counts[g])] = True
        got = bits(d_na)
        ok, worst, nbad = tolerance_check(got[tok], ref[tok])
        assert ok, f"call {i}: {nbad} elements out of tolerance (worst {worst:.3g})"
        assert np.all(got[~tok] == 0)
