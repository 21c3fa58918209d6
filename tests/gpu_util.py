"""Helpers for the GPU parity tests: device transfer and layout plumbing.

Nothing here computes any part of the method; the GPU side goes through the C
ABI (via the package binding) and the expected values come from oracle/.
"""

import numpy as np
import torch

import moe_grouped_gemm_quantizer_amd as fp8g


def dev():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU (gfx950)")
    return torch.device("cuda:0")


def to_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev())


def to_host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def quantize_a(x, rows=None):
    """GPU 1x128 quantisation of a [rows][K] fp32 matrix -> (q [rows][K],
    sa [K/128][rows]) device tensors (the GEMM's A layout)."""
    xt = x if isinstance(x, torch.Tensor) else to_dev(np.asarray(x, np.float32))
    R, K = xt.shape
    q = torch.empty((R, K), dtype=torch.uint8, device=dev())
    s = torch.empty((K // 128, R), dtype=torch.float32, device=dev())
    fp8g.fp8_quantize(xt, 1, q, s, 1, R)
    return q, s


def quantize_b(x):
    """GPU 128x128 quantisation of a [rows][K] fp32 matrix (rows a multiple of
    128; stacked experts pass [G*N][K]) -> (q, sb [rows/128][K/128])."""
    xt = x if isinstance(x, torch.Tensor) else to_dev(np.asarray(x, np.float32))
    R, K = xt.shape
    q = torch.empty((R, K), dtype=torch.uint8, device=dev())
    s = torch.empty((-(-R // 128), K // 128), dtype=torch.float32, device=dev())
    fp8g.fp8_quantize(xt, 128, q, s, K // 128, 1)
    return q, s


def bf16_out(shape, fill=None):
    t = torch.empty(shape, dtype=torch.int16, device=dev())
    if fill is not None:
        t.fill_(int(np.uint16(fill).view(np.int16)))
    return t


def bits(t):
    return to_host(t).view(np.uint16)


def banner(msg):
    print(f"[gpu-test] {msg}", flush=True)
