"""GPU parity of the e5m2 / delayed-scaling path (czchanglian §2.1 and §2.3;
gtnt E4M3-vs-E5M2 part): fp8_quantize_delayed bit for bit against the
oracle's quantize_delayed (codes, the scale used, the updated history), over
several steps of a rotating history, special values and every fp32 pattern
near the e5m2 and e4m3 rounding boundaries; gemm_fp8_pertensor_fmt with
e5m2 operands against the oracle's gemm_pertensor under
|d - ref| <= 2^-7 |ref| + 2^-10 rms(ref), every output element, on small
and ragged shapes and on 4096x8192x8192 with an e5m2 A."""

import numpy as np
import pytest
import torch

import moe_grouped_gemm_quantizer_amd as fp8g
from oracle import (quantize_delayed, quantize_with_scale, quantize_blocks, gemm_pertensor,
                    tolerance_check, e5m2_decode_table, e4m3_decode_table)
from workloads import make_dense
from tests import oracle_ops
from tests.gpu_util import dev, to_dev, to_host, bits, bf16_out, banner

pytestmark = pytest.mark.gpu


def _gpu_step(x, fmt, hist_dev, slot):
    xt = x if isinstance(x, torch.Tensor) else to_dev(np.asarray(x, np.float32))
    q = torch.full(xt.shape, 0xAB, dtype=torch.uint8, device=dev())
    s = torch.full((1,), -1.0, dtype=torch.float32, device=dev())
    fp8g.fp8_quantize_delayed(xt, fmt, hist_dev, slot, q, s)
    return to_host(q), to_host(s)[0]


def _check_step(x, fmt, hist, slot, what):
    hist = np.asarray(hist, np.float32)
    hd = to_dev(hist.copy())
    q, s = _gpu_step(x, fmt, hd, slot)
    qo, so, ho = quantize_delayed(x, hist, slot, fmt)
    assert np.float32(s).view(np.uint32) == np.float32(so).view(np.uint32), f"{what}: scale {s} vs {so}"
    bad = np.argwhere(q != qo)[:5]
    assert np.array_equal(q, qo), f"{what}: {int((q != qo).sum())} codes differ, e.g. {bad.tolist()}"
    hg = to_host(hd)
    assert np.array_equal(hg.view(np.uint32), ho.view(np.uint32)), f"{what}: history {hg} vs {ho}"


def _data(rows, cols, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, cols)) * 3).astype(np.float32)
    if cols > 8:
        x[:, rng.integers(0, cols, max(1, cols // 100))] *= 50
    return x


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("rows,cols", [(1, 4), (3, 1000), (64, 4096), (257, 1028), (2048, 12)])
def test_delayed_step_shapes(fmt, rows, cols):
    banner(f"delayed {fmt} {rows}x{cols}")
    x = _data(rows, cols, rows * 7 + cols)
    amax = float(np.abs(x).max())
    histories = {
        "first step (no history)": ([0.0, 0.0], 1),
        "current amax (per tensor)": ([amax], 0),
        "window max above": ([amax * 0.5, amax * 4.0, 0.0], 2),
        "data outgrew the scale": ([amax / 20.0], 0),
        "subnormal scale": ([1e-40], 0),
        "huge scale": ([3e38, 1.0], 1),
    }
    for name, (h, slot) in histories.items():
        _check_step(x, fmt, h, slot, f"{fmt} {rows}x{cols} {name}")


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_delayed_special_values(fmt):
    banner(f"delayed {fmt} special values")
    x = np.zeros((4, 16), np.float32)
    x[0, :8] = [np.inf, -np.inf, np.nan, -np.nan, -0.0, 0.0, 1e-45, -3e-42]
    x[1, :] = np.float32(2.0) ** np.arange(-20, 12, 2)
    x[2, :] = -x[1, :]
    x[3, :] = np.linspace(-70000, 70000, 16)
    for h, slot in (([1.0], 0), ([57344.0], 0), ([448.0], 0), ([np.inf], 0), ([2.0 ** -140], 0),
                    ([np.nan, 5.0], 0), ([0.0], 0)):
        _check_step(x, fmt, h, slot, f"{fmt} specials, history {h}")
    z = np.zeros((3, 8), np.float32)
    _check_step(z, fmt, [2.0], 0, f"{fmt} all-zero data")


def test_delayed_rotating_history_over_steps():
    """Five steps of a three-entry history, the slot rotating as a training
    loop would rotate it; every step against the oracle's step on the
    oracle's own history."""
    rng = np.random.default_rng(21)
    hist = np.zeros(3, np.float32)
    hd = to_dev(hist.copy())
    for step in range(5):
        x = (rng.standard_normal((128, 512)) * (1.5 ** step)).astype(np.float32)
        slot = step % 3
        q, s = _gpu_step(x, "e5m2", hd, slot)
        qo, so, hist = quantize_delayed(x, hist, slot, "e5m2")
        banner(f"step {step}: scale {s}")
        assert np.float32(s).view(np.uint32) == np.float32(so).view(np.uint32), step
        assert np.array_equal(q, qo), step
        assert np.array_equal(to_host(hd).view(np.uint32), hist.view(np.uint32)), step


def _near_boundaries(table, lo_code, hi_code, width):
    pos = table[lo_code:hi_code + 1]
    pts = np.concatenate([(pos[:-1] + pos[1:]) / 2, pos])
    b = pts.astype(np.float32).view(np.int32).astype(np.int64)
    off = np.arange(-width, width + 1, dtype=np.int64)
    c = (b[:, None] + off[None, :]).ravel()
    c = c[(c >= 0) & (c < 0x7F800000)]
    y = c.astype(np.int32).view(np.float32)
    return np.concatenate([y, -y])


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_encoder_near_every_boundary(fmt):
    """Scale exactly 1 (history = [FP8 max]): the codes are the encoder's on
    the raw values; every fp32 pattern within 400 ulps of every code value and
    midpoint, every pattern of the format's subnormal range, and values
    beyond the largest code (saturation)."""
    if fmt == "e5m2":
        t, top, fmax = e5m2_decode_table(), 0x7B, 57344.0
        sub = np.arange(np.float32(2.0 ** -18).view(np.int32), np.float32(2.0 ** -13).view(np.int32),
                        dtype=np.int64)
    else:
        t, top, fmax = e4m3_decode_table(), 0x7E, 448.0
        sub = np.arange(np.float32(2.0 ** -11).view(np.int32), np.float32(2.0 ** -5).view(np.int32),
                        dtype=np.int64)
    y = np.concatenate([_near_boundaries(t, 0, top, 400),
                        sub.astype(np.int32).view(np.float32),
                        np.float32([fmax * 1.01, fmax * 2, 1e30, -fmax * 1.5])])
    n = (len(y) + 3) // 4 * 4
    y = np.concatenate([y, np.zeros(n - len(y), np.float32)])
    x = y.reshape(-1, 4096 if n % 4096 == 0 else 4)
    banner(f"{fmt} encoder: {x.size} values")
    hd = to_dev(np.float32([fmax]))
    q, s = _gpu_step(x, fmt, hd, 0)
    assert s == 1.0
    qo = quantize_with_scale(x, np.float32(1.0), fmt)
    bad = np.argwhere(q != qo)[:5]
    assert np.array_equal(q, qo), f"{int((q != qo).sum())} differ, e.g. {[(x[tuple(i)], q[tuple(i)], qo[tuple(i)]) for i in bad]}"


# ---------------------------------------------------------------------------
# GEMM with e5m2 operands


def _pt_operands(w, fa, fb):
    qa, sa = quantize_blocks(w.a, w.a.shape[0], w.a.shape[1], fmt=fa)
    qb, sb = quantize_blocks(w.b, w.b.shape[0], w.b.shape[1], fmt=fb)
    return qa, sa[0, 0], qb, sb[0, 0]


def _run_fmt(qa, fa, s_a, qb, fb, s_b):
    M, N = qa.shape[0], qb.shape[0]
    d = bf16_out((M, N), fill=0x7FBF)
    fp8g.gemm_fp8_pertensor_fmt(to_dev(qa), fa, to_dev(np.float32([s_a])), to_dev(qb), fb,
                                to_dev(np.float32([s_b])), d)
    return bits(d)


@pytest.mark.parametrize("fa,fb", [("e5m2", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e5m2"),
                                   ("e4m3", "e4m3")])
@pytest.mark.parametrize("M,N,K", [(300, 512, 1024), (129, 256, 640), (16, 384, 256), (1, 128, 128)])
def test_pertensor_fmt_shapes(fa, fb, M, N, K):
    banner(f"per-tensor {fa} x {fb} {M}x{N}x{K}")
    w = make_dense(M, N, K, seed=M + 2 * N + 3 * K)
    qa, s_a, qb, s_b = _pt_operands(w, fa, fb)
    ref, _ = gemm_pertensor(qa, s_a, qb, s_b, fa, fb)
    got = _run_fmt(qa, fa, s_a, qb, fb, s_b)
    ok, worst, nbad = tolerance_check(got, ref)
    banner(f"worst ratio {worst:.4f}")
    assert ok, f"{nbad} elements out of tolerance"


def test_pertensor_e5m2_gradient_full_workload():
    """4096x8192x8192 with A in e5m2 (a gradient) and B in e4m3, both
    quantised on the GPU by the delayed quantiser with the history holding
    each operand's current amax (the per-tensor special case), every output
    element against the oracle."""
    w = oracle_ops.workload(2)
    banner("per-tensor e5m2 x e4m3 4096x8192x8192 end to end")
    ha = to_dev(np.float32([np.abs(w.a).max()]))
    hb = to_dev(np.float32([np.abs(w.b).max()]))
    qa_d = torch.empty(w.a.shape, dtype=torch.uint8, device=dev())
    qb_d = torch.empty(w.b.shape, dtype=torch.uint8, device=dev())
    sa_d = torch.empty(1, dtype=torch.float32, device=dev())
    sb_d = torch.empty(1, dtype=torch.float32, device=dev())
    fp8g.fp8_quantize_delayed(to_dev(w.a), "e5m2", ha, 0, qa_d, sa_d)
    fp8g.fp8_quantize_delayed(to_dev(w.b), "e4m3", hb, 0, qb_d, sb_d)
    qa, s_a, qb, s_b = _pt_operands(w, "e5m2", "e4m3")
    assert np.array_equal(to_host(qa_d), qa) and np.array_equal(to_host(qb_d), qb)
    assert to_host(sa_d)[0] == s_a and to_host(sb_d)[0] == s_b
    d = bf16_out((w.M, w.N), fill=0x7FBF)
    fp8g.gemm_fp8_pertensor_fmt(qa_d, "e5m2", sa_d, qb_d, "e4m3", sb_d, d)
    band = 1024
    ref = np.concatenate([gemm_pertensor(qa[r:r + band], s_a, qb, s_b, "e5m2", "e4m3")[0]
                          for r in range(0, w.M, band)])
    ok, worst, nbad = tolerance_check(bits(d), ref)
    banner(f"worst ratio {worst:.4f}")
    assert ok, f"{nbad} elements out of tolerance"
