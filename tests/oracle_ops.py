"""Oracle results for the full-size workloads, computed once per test session.

Pure NumPy on the host: only oracle/ functions compute anything, unchanged.
Large inputs are cut along pieces the method treats independently (128-row
bands of quantiser blocks, bands of GEMM output rows, experts) and the
pieces run on a thread pool, since NumPy releases the GIL inside its array
kernels. Nothing here touches the GPU or the library, so every expected
value the GPU tests compare against comes from the oracle alone.
"""

import functools
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from oracle import quantize_blocks, gemm_blockscaled
from workloads import make_config


def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _pool_map(fn, items):
    with ThreadPoolExecutor(_threads()) as ex:
        return list(ex.map(fn, items))


def quantize_rows(x, block_rows, band=None):
    """oracle quantize_blocks over a [rows][K] matrix, band by band.

    A band is a multiple of block_rows rows, so every scale block lies in
    exactly one band and the result equals one call on the whole matrix.
    Returns (codes [rows][K], scales [ceil(rows/block_rows)][K/128])."""
    rows, K = x.shape
    if band is None:
        band = max(block_rows, (4 << 20) // max(K, 1) // block_rows * block_rows)
    starts = list(range(0, rows, band))
    parts = _pool_map(lambda r0: quantize_blocks(x[r0:r0 + band], block_rows), starts)
    return (np.concatenate([q for q, _ in parts], axis=0),
            np.concatenate([s for _, s in parts], axis=0))


def gemm_rows(qa, sa, qb, sb, band=None):
    """oracle gemm_blockscaled over bands of output rows (rows are independent).
    qa [M][K], sa [M][K/128]; returns bf16 bits [M][N]. A few wide bands: each
    band decodes all of qb again, and the products run on BLAS threads."""
    M = qa.shape[0]
    if band is None:
        band = max(256, -(-M // 4))
    starts = list(range(0, M, band))
    parts = _pool_map(lambda r0: gemm_blockscaled(qa[r0:r0 + band], sa[r0:r0 + band], qb, sb)[0],
                      starts)
    return np.concatenate(parts, axis=0)


@functools.lru_cache(maxsize=None)
def workload(cfg):
    return make_config(cfg)


@functools.lru_cache(maxsize=None)
def operands(cfg):
    """Oracle-quantised operands of workload `cfg` in the oracle's layouts:
    qa [rows][K] with sa [rows][K/128] (rows = M, M_total or G*max_m), and
    qb [G*N][K] with sb [G*N/128][K/128] (experts stacked)."""
    w = workload(cfg)
    K = w.K
    qa, sa = quantize_rows(w.a.reshape(-1, K), 1)
    qb, sb = quantize_rows(w.b.reshape(-1, K), 128)
    return qa, sa, qb, sb


@functools.lru_cache(maxsize=None)
def reference(cfg):
    """Oracle bf16 result of workload `cfg`, every output element.

    dense: [M][N]; contiguous: [M_total][N] (padding rows are +0);
    masked: [G][max_m][N] with only rows < masked_m[g] meaningful (the rest
    are 0 here and are checked against the sentinel instead)."""
    w = workload(cfg)
    qa, sa, qb, sb = operands(cfg)
    K, N = w.K, w.N
    if w.kind == "dense":
        return gemm_rows(qa, sa, qb, sb)
    kb, nb = K // 128, N // 128
    qbg = qb.reshape(w.G, N, K)
    sbg = sb.reshape(w.G, nb, kb)
    if w.kind == "contiguous":
        out = np.zeros((w.M, N), np.uint16)
        for g in range(w.G):
            r0, c = int(w.offsets[g]), int(w.counts[g])
            if c:
                out[r0:r0 + c] = gemm_rows(qa[r0:r0 + c], sa[r0:r0 + c], qbg[g], sbg[g])
        return out
    G, mm = w.G, w.M
    out = np.zeros((G, mm, N), np.uint16)
    active = [g for g in range(G) if int(w.masked_m[g]) > 0]

    def one(g):
        m = int(w.masked_m[g])
        r0 = g * mm
        return gemm_blockscaled(qa[r0:r0 + m], sa[r0:r0 + m], qbg[g], sbg[g])[0]

    for g, r in zip(active, _pool_map(one, active)):
        out[g, :int(w.masked_m[g])] = r
    return out


@functools.lru_cache(maxsize=None)
def pertensor_operands(cfg):
    """Workload `cfg`'s A and B quantised per tensor by the oracle (one block
    covering each whole matrix): (qa, s_a, qb, s_b) with float32 scalars."""
    w = workload(cfg)
    K = w.K
    a2, b2 = w.a.reshape(-1, K), w.b.reshape(-1, K)
    qa, sa = quantize_blocks(a2, a2.shape[0], a2.shape[1])
    qb, sb = quantize_blocks(b2, b2.shape[0], b2.shape[1])
    return qa, sa[0, 0], qb, sb[0, 0]


@functools.lru_cache(maxsize=None)
def pertensor_reference(cfg):
    """Oracle bf16 result of the per-tensor-scaled product of workload cfg."""
    from oracle import gemm_pertensor
    qa, s_a, qb, s_b = pertensor_operands(cfg)
    M = qa.shape[0]
    band = max(256, -(-M // 4))
    parts = _pool_map(lambda r0: gemm_pertensor(qa[r0:r0 + band], s_a, qb, s_b)[0],
                      list(range(0, M, band)))
    return np.concatenate(parts, axis=0)
