#!/usr/bin/env python3
"""Benchmark of the FP8 block-scaled GEMM path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
  1. quantise A (fp32 [M][K]) to e4m3 with 1x128 per-token scales,
  2. quantise B (fp32 [N][K]) to e4m3 with 128x128 block scales,
  3. the block-scaled GEMM D = A.B^T with fp32 promotion per K block, bf16 out.
Default workload: dense M=4096 N=8192 K=8192 (the shape the gtnt page times
on H100), inputs seeded and synthetic (N(0,1) with 0.5% outlier K-columns x50),
resident in HBM before timing. value = 2*M*N*K / (time of one step) in TFLOPS.

Printed: one JSON line with the step throughput, a roofline object for the
dominant kernel (the GEMM, timed with HIP events on the stream it runs on), and
the CPU oracle timed on a bounded sample of the same workload.

Before the W counted warm-up steps, untimed steps run for --prewarm-s seconds
so that clocks have settled (the pages' benchmark hygiene: warm up, then
time the steady state).

Before timing, sampled output rows are checked against a float32 product of
the dequantised operands computed with plain torch ops on the GPU (--no-check
skips it); the oracle runs only for the CPU baseline (--no-cpu-baseline skips
it).

Other workloads (--workload small_m | contiguous | masked) run the same way on
the other shapes of the method. The decode-shaped small_m GEMM is timed with
its weight codes rotated over copies larger than the Infinity Cache (cold,
the HBM roofline's figure) and reported warm beside it. --calibrate-copy runs
a plain device copy of a known size (for scaling hardware byte counters).
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np

FP8_PEAK_TFLOPS = 5000.0      # MI355X dense FP8 MFMA (published)
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E (published)
GEMM_SOURCE = os.path.join(ROOT, "moe_grouped_gemm_quantizer_amd", "csrc", "gemm.hip")

# HBM bytes per GEMM launch from hardware counters (FETCH_SIZE + WRITE_SIZE,
# scaled by the same counters' reading for a plain copy of known size), keyed
# by gemm_code_digest() of the GEMM source they were taken on: a changed
# kernel reports null until the counters are taken again.
MEASURED_TRAFFIC = {
    # rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE, KiB per dispatch (mean of 6), scaled by a
    # 1 GiB copy's readings (read 1048576 KiB shows as FETCH_SIZE 524304 -> x 2.0; write
    # 1048576 KiB shows as WRITE_SIZE 1048576 -> x 1.0). The contiguous call is two
    # dispatches (GEMM with K pieces, then their reduction): both are counted.
    "ba9779c5321fd479d368e9d913f5d073357c71eaa05fecfaca1d5d0c46040dfb": {
        "dense_4096x8192x8192":
            int(((198936.9) * 2.0 + (66436.1) * 1.0) * 1024),
        "dense_16x4096x7168":
            int(((14881.0) * 2.0 + (128.0) * 1.0) * 1024),
        "moe_contiguous_G8_T4096_N4096_K7168":
            int(((191630.8 + 24610.2) * 2.0 + (80228.9 + 6144.0) * 1.0) * 1024),
        "moe_masked_G32_maxm256_N7168_K2048":
            int(((230285.3) * 2.0 + (60659.2) * 1.0) * 1024),
    },
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="dense",
                   choices=["dense", "small_m", "contiguous", "masked"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-check", action="store_true", help="skip the parity spot check")
    p.add_argument("--calibrate-copy", action="store_true")
    p.add_argument("--prewarm-s", type=float, default=1.0,
                   help="seconds of untimed steps before the warmup steps, so that the "
                        "GPU clocks have settled (steady-state throughput is reported)")
    return p.parse_args()


def cfg_index(workload):
    return {"dense": 2, "small_m": 1, "contiguous": 3, "masked": 4}[workload]


class Path:
    """Device buffers and the launch sequence of one step."""

    def __init__(self, w, torch, fp8g):
        self.w, self.torch, self.fp8g = w, torch, fp8g
        dev = torch.device("cuda:0")
        K = w.K
        a2 = w.a.reshape(-1, K)
        self.rows_a = a2.shape[0]
        self.xa = torch.from_numpy(np.ascontiguousarray(a2)).to(dev)
        b2 = w.b.reshape(-1, K)
        self.rows_b = b2.shape[0]
        self.xb = torch.from_numpy(np.ascontiguousarray(b2)).to(dev)
        self.qa = torch.empty((self.rows_a, K), dtype=torch.uint8, device=dev)
        self.sa = torch.empty((K // 128, self.rows_a), dtype=torch.float32, device=dev)
        self.qb = torch.empty((self.rows_b, K), dtype=torch.uint8, device=dev)
        self.sb = torch.empty((self.rows_b // 128, K // 128), dtype=torch.float32, device=dev)
        if w.kind == "masked":
            self.d = torch.empty((w.G, w.M, w.N), dtype=torch.int16, device=dev)
            self.meta = torch.from_numpy(w.masked_m.astype(np.int32)).to(dev)
        else:
            self.d = torch.empty((self.rows_a, w.N), dtype=torch.int16, device=dev)
            self.meta = (torch.from_numpy(w.offsets.astype(np.int32)).to(dev)
                         if w.kind == "contiguous" else None)

    def quant_a(self):
        self.fp8g.fp8_quantize(self.xa, 1, self.qa, self.sa, 1, self.rows_a)

    def quant_b(self):
        self.fp8g.fp8_quantize(self.xb, 128, self.qb, self.sb, self.w.K // 128, 1)

    def gemm(self):
        w, f = self.w, self.fp8g
        K, N = w.K, w.N
        if w.kind == "dense":
            f.gemm_fp8_blockscaled(self.qa, self.sa, self.qb, self.sb, self.d)
        elif w.kind == "contiguous":
            f.grouped_gemm_fp8_contiguous(self.qa, self.sa, self.qb.view(w.G, N, K),
                                          self.sb.view(w.G, N // 128, K // 128), self.d,
                                          self.meta)
        else:
            f.grouped_gemm_fp8_masked(self.qa.view(w.G, w.M, K), self.sa,
                                      self.qb.view(w.G, N, K),
                                      self.sb.view(w.G, N // 128, K // 128), self.d, self.meta,
                                      expected_m=int(np.mean(w.masked_m)))

    KERNELS = ("quantize_a", "quantize_b", "gemm")

    def step(self):
        self.quant_a()
        self.quant_b()
        self.gemm()


def algorithmic(w):
    """Algorithmic flops and bytes of each kernel of one step."""
    K, N = w.K, w.N
    rows_a = w.a.reshape(-1, K).shape[0]
    rows_b = w.b.reshape(-1, K).shape[0]
    if w.kind == "dense":
        m_eff = w.M
    else:
        m_eff = int(np.sum(w.counts))              # valid rows
    G = w.G
    flops = 2.0 * m_eff * N * K
    # quantisers: 4 B read + 1 B written per element, 4 B per scale
    qa_bytes = rows_a * K * 5 + rows_a * (K // 128) * 4
    qb_bytes = rows_b * K * 5 + (rows_b // 128) * (K // 128) * 4
    # GEMM: fp8 A rows read once, fp8 B of the experts that have rows read once,
    # scales, bf16 output of the rows computed
    if w.kind == "dense":
        b_rows = N
        a_rows = w.M
    elif w.kind == "contiguous":
        b_rows = N * int(np.sum(w.counts > 0))
        a_rows = w.M                                # padded rows are read and written
    else:
        b_rows = N * int(np.sum(w.masked_m > 0))
        a_rows = m_eff
    gemm_bytes = (a_rows * K + b_rows * K + a_rows * (K // 128) * 4
                  + (b_rows // 128) * (K // 128) * 4 + a_rows * N * 2)
    return {"flops": flops, "quantize_a": qa_bytes, "quantize_b": qb_bytes, "gemm": gemm_bytes}


def cpu_baseline(w):
    """The oracle, untouched, on a bounded sample of the same workload."""
    from oracle import quantize_blocks, gemm_blockscaled
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = 1
    K = w.K
    if w.kind == "dense":
        ms, ns = min(w.M, 2048), min(w.N, 2048)
        xa, xb = w.a[:ms], w.b[:ns]
        full_a, full_b = w.M, w.N
        flop_scale = (w.M * w.N) / (ms * ns)
        sample = f"A rows 0..{ms - 1}, B rows 0..{ns - 1} (full K)"
    else:
        # one expert's share: its valid rows and the first 2048 rows of its weights
        g = int(np.argmax(w.counts))
        if w.kind == "masked":
            xa = w.a[g, :int(w.masked_m[g])]
        else:
            r0 = int(w.offsets[g])
            xa = w.a[r0:r0 + int(w.counts[g])]
        ms = xa.shape[0]
        ns = min(w.N, 2048)
        xb = w.b[g, :ns]
        full_a = w.a.reshape(-1, K).shape[0]
        full_b = w.b.reshape(-1, K).shape[0]
        flop_scale = (np.sum(w.counts) * w.N) / (ms * ns)
        sample = f"expert {g}: {ms} valid rows, weight rows 0..{ns - 1} (full K)"
    t0 = time.perf_counter()
    qa, sa = quantize_blocks(xa, 1)
    t1 = time.perf_counter()
    qb, sb = quantize_blocks(xb, 128)
    t2 = time.perf_counter()
    gemm_blockscaled(qa, sa, qb, sb)
    t3 = time.perf_counter()
    # extrapolate each leg to the full step by its own size ratio
    est = ((t1 - t0) * full_a / xa.shape[0] + (t2 - t1) * full_b / xb.shape[0]
           + (t3 - t2) * flop_scale)
    flops = algorithmic(w)["flops"]
    return {"value": flops / est / 1e12, "unit": "TFLOPS", "cores": int(cores), "kind": "oracle",
            "sample": f"{sample}; measured {t3 - t0:.1f} s (quantise A {t1 - t0:.2f} s, "
                      f"quantise B {t2 - t1:.2f} s, GEMM {t3 - t2:.2f} s), each leg scaled to "
                      f"the full step: {est:.1f} s per step"}


def gemm_code_digest(path=GEMM_SOURCE):
    """sha256 of the GEMM source with comments and whitespace removed: any
    change to the code changes it, an edit of a comment does not."""
    import hashlib
    import re
    text = open(path, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    text = re.sub(r"\s+", "", text)
    return hashlib.sha256(text.encode("utf-8")).hexdigest()


def measured_traffic(workload):
    try:
        digest = gemm_code_digest()
    except OSError:
        return None
    return MEASURED_TRAFFIC.get(digest, {}).get(workload)


def spot_check(path, w):
    """Sanity check of sampled GEMM rows before timing, on the GPU with plain
    torch float32 ops (parity proper is the test suite's job): the codes and
    scales are dequantised, multiplied in float32, and the library's bf16
    rows must lie within |d - ref| <= 2^-7 |ref| + 2^-10 rms(ref)."""
    torch = path.torch
    torch.cuda.synchronize()
    K, N = w.K, w.N
    kb = K // 128

    def dequant_rows(q, s_rows):
        # q: uint8 [r][K] codes, s_rows: float32 [r][K/128] scales of those rows
        x = q.view(torch.float8_e4m3fn).to(torch.float32).view(q.shape[0], kb, 128)
        return (x * s_rows.unsqueeze(-1)).view(q.shape[0], K)

    def dequant_b(q, s_blocks):
        # q: uint8 [n][K], s_blocks: float32 [n/128][K/128]
        x = q.view(torch.float8_e4m3fn).to(torch.float32).view(q.shape[0] // 128, 128, kb, 128)
        return (x * s_blocks.view(q.shape[0] // 128, 1, kb, 1)).view(q.shape[0], K)

    qb = path.qb.view(-1, N, K)
    sb = path.sb.view(-1, N // 128, kb)
    if w.kind == "dense":
        rows = torch.tensor([0, w.M // 3, w.M - 1], device=path.qa.device)
        g = 0
        got = path.d[rows]
    else:
        g = int(np.argmax(w.counts))
        r0 = g * w.M if w.kind == "masked" else int(w.offsets[g])
        rows = torch.arange(r0, r0 + 3, device=path.qa.device)
        got = path.d.view(-1, N)[rows]
    a = dequant_rows(path.qa[rows], path.sa[:, rows].t().contiguous())
    b = dequant_b(qb[g], sb[g])
    ref = a @ b.t().contiguous()
    got = got.view(torch.bfloat16).to(torch.float32)
    rms = torch.sqrt(torch.mean(ref * ref))
    bad = (got - ref).abs() > (2.0 ** -7) * ref.abs() + (2.0 ** -10) * rms
    if not torch.isfinite(got).all() or bool(bad.any()):
        raise SystemExit(f"parity spot check failed: {int(bad.sum())} elements out of tolerance")
    return True


def calibrate_copy(args):
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    print(json.dumps({"copy_bytes": n, "read_bytes": n, "write_bytes": n,
                      "ms": dt * 1e3, "GBs": 2 * n / dt / 1e9}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "the library runs on one GPU (no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        return calibrate_copy(args)

    import torch
    import moe_grouped_gemm_quantizer_amd as fp8g
    from workloads import make_config

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    fp8g.load()
    t0 = time.perf_counter()
    w = make_config(cfg_index(args.workload))
    print(f"[bench] workload {w.name}: generated in {time.perf_counter() - t0:.1f} s",
          file=sys.stderr, flush=True)
    path = Path(w, torch, fp8g)
    alg = algorithmic(w)

    # parity spot check first: it keeps the GPU idle while the host computes,
    # and the shader clock needs 10-20 ms of load to recover from an idle gap
    path.step()
    torch.cuda.synchronize()
    if not args.no_check:
        spot_check(path, w)
        print("[bench] parity spot check ok", file=sys.stderr, flush=True)
    # pre-warm with the same back-to-back launches as the timed region (a sync
    # after every step would leave idle gaps and run at a different clock)
    t_pre = time.perf_counter()
    while time.perf_counter() - t_pre < args.prewarm_s:
        for _ in range(16):
            path.step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        path.step()
    torch.cuda.synchronize()

    # Timed region: K whole steps launched back to back, HIP events only at
    # its two ends. (An event between two kernels costs a ~10 us bubble on
    # the stream, and enough of them lower the shader clock: per-launch
    # events would time a different machine state than the one measured.)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        path.step()
    e1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    gpu_ms_per_step = e0.elapsed_time(e1) / args.steps
    # Per-kernel average launch duration: each kernel launched K times back
    # to back on the same stream, HIP events at the ends of its run.
    per_kernel = {}
    for name, fn in zip(Path.KERNELS, (path.quant_a, path.quant_b, path.gemm)):
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        per_kernel[name] = e0.elapsed_time(e1) / args.steps
    # Decode-shaped GEMM: its 29 MB of weights stay in the 256 MB Infinity
    # Cache from one launch to the next, so the figure above is the warm one.
    # The cold one rotates over enough copies of the weight codes (> 256 MB)
    # that each launch reads its weights from HBM; it is the one the HBM
    # roofline is taken on.
    warm_gemm_ms = None
    if w.kind == "dense" and w.M <= 32:
        ncopy = max(10, -(-300 * 2**20 // path.qb.numel()))
        copies = [path.qb.clone() for _ in range(ncopy)]
        reps = max(args.steps, 2 * ncopy)
        for q in copies:
            fp8g.gemm_fp8_blockscaled(path.qa, path.sa, q, path.sb, path.d)
        torch.cuda.synchronize()
        e0.record()
        for i in range(reps):
            fp8g.gemm_fp8_blockscaled(path.qa, path.sa, copies[i % ncopy], path.sb, path.d)
        e1.record()
        torch.cuda.synchronize()
        warm_gemm_ms = per_kernel["gemm"]
        per_kernel["gemm"] = e0.elapsed_time(e1) / reps
        del copies
    print(f"[bench] per-kernel ms: {per_kernel}; step ms (events) {gpu_ms_per_step:.4f}",
          file=sys.stderr, flush=True)

    gemm_s = per_kernel["gemm"] / 1e3
    achieved_tf = alg["flops"] / gemm_s / 1e12
    traffic = measured_traffic(w.name)
    if w.kind == "masked" or w.M <= 32:
        # low arithmetic intensity (decode-shaped): the HBM roofline bounds it
        achieved_gbs = alg["gemm"] / gemm_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
                "traffic": traffic}
    else:
        roof = {"bound": "mfma", "achieved": round(achieved_tf, 1), "peak": FP8_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved_tf / FP8_PEAK_TFLOPS, 4),
                "traffic": traffic}
    kernels = {}
    for name in Path.KERNELS:
        sec = per_kernel[name] / 1e3
        ent = {"avg_us": round(per_kernel[name] * 1e3, 2),
               "alg_GBs": round(alg[name] / sec / 1e9, 1)}
        ent["hbm_frac"] = round(ent["alg_GBs"] / HBM_PEAK_GBS, 4)
        if name == "gemm":
            ent["TFLOPS"] = round(achieved_tf, 1)
            ent["fp8_peak_frac"] = round(achieved_tf / FP8_PEAK_TFLOPS, 4)
            if warm_gemm_ms is not None:
                ent["weights"] = "cold (rotated over copies larger than the Infinity Cache)"
                ent["warm_avg_us"] = round(warm_gemm_ms * 1e3, 2)
                ent["warm_alg_GBs"] = round(alg[name] / (warm_gemm_ms / 1e3) / 1e9, 1)
        kernels[name] = ent

    value = alg["flops"] / (ms_per_step / 1e3) / 1e12
    out = {
        "metric": "FP8 block-scaled GEMM TFLOPS + % FP8 MFMA peak (dense 4096x8192x8192, MoE)",
        "value": round(value, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "prewarm_s": args.prewarm_s,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 x fp8e4m3 -> f32 accumulate, bf16 out",
        "data": "synthetic (seeded N(0,1) with x50 outlier K-columns)",
        "config": {"workload": w.name, "M": int(w.M), "N": int(w.N), "K": int(w.K),
                   "G": int(w.G), "valid_rows": int(w.valid_rows()),
                   "step": "quantize A 1x128 + quantize B 128x128 + block-scaled GEMM"},
        "roofline": roof,
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
