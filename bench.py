#!/usr/bin/env python3
"""Benchmark of the FP8 block-scaled GEMM path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
  1. quantise A (fp32 [M][K]) to e4m3 with 1x128 per-token scales,
  2. quantise B (fp32 [N][K]) to e4m3 with 128x128 block scales,
  3. the block-scaled GEMM D = A.B^T with fp32 promotion per K block, bf16 out.
Headline workload: dense M=4096 N=8192 K=8192 (the shape the gtnt page times
on H100), inputs seeded and synthetic (N(0,1) with 0.5% outlier K-columns
x50), resident in HBM before timing. value = 2*M*N*K / (time of one step) in
TFLOPS.

The same JSON line carries, under "kernels", every kernel of the path timed
on its own: the step's three kernels, and the GEMM on the other shapes of the
method -- the MoE contiguous layout (8 experts, 4096 Zipf-routed tokens,
N=4096 K=7168), the MoE masked layout (32 experts x 256 rows, N=7168
K=2048) and the decode-shaped small-M GEMM (16x4096x7168, weights rotated
over copies larger than the Infinity Cache) -- each with its roofline
fraction (FP8 MFMA or HBM), average / median / min over repetitions, and the
hardware-counter HBM traffic where it was taken on the current code.

Timing follows the pages' benchmark hygiene (czchanglian §4.3: warm up, fixed
conditions, know the clock): untimed steps for --prewarm-s seconds so the
clocks settle, W counted warm-up steps, then exactly K timed steps launched
back to back between HIP events (no event between launches: each costs a
bubble that lowers the shader clock). Per-kernel figures come from R
repetitions of K back-to-back launches of that kernel alone. The shader
clock the chip holds under each GEMM is read on the device (fp8g_clock_probe
between launches) and reported.

Before timing, sampled output rows of every GEMM are checked against a
float32 product of the dequantised operands computed with plain torch ops on
the GPU (--no-check skips it; parity proper is the test suite's job). The
oracle runs only in the cpu_baseline leg (--no-cpu-baseline skips it), on a
bounded sample of the headline workload with BLAS pinned to the cores this
process may use.
"""

import argparse
import atexit
import json
import os
import re
import shutil
import statistics
import subprocess
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np

FP8_PEAK_TFLOPS = 5000.0      # MI355X dense FP8 MFMA (published)
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E (published)
GEMM_SOURCES = [os.path.join(ROOT, "moe_grouped_gemm_quantizer_amd", "csrc", f)
                for f in ("gemm.hip", "gemm_index.h", "e4m3.h")]
METRIC = "FP8 block-scaled GEMM TFLOPS + % FP8 MFMA peak (dense 4096x8192x8192, MoE)"

# HBM bytes per GEMM launch from hardware counters (FETCH_SIZE + WRITE_SIZE,
# scaled by the same counters' reading for a plain copy of known size), keyed
# by gemm_code_digest() of the GEMM sources they were taken on: a changed
# kernel reports null until the counters are taken again.
MEASURED_TRAFFIC = {
    # rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE, KiB per dispatch (mean over the
    # dispatches of the shape-specialised kernel, 53 per run; 76 for small-M),
    # scaled by a 1 GiB copy's readings (read 1048576 KiB shows as FETCH_SIZE
    # 524300 -> x 2.0; write 1048576 KiB shows as WRITE_SIZE 1048576 -> x 1.0).
    # The contiguous call is two dispatches (GEMM with K pieces, then their
    # reduction): both are counted.
    "03784b71ff2f01853d0e8ecb44c2f2c4ffd71c329686b122001c65e2c659cf7e": {
        "dense_4096x8192x8192":
            int(((198838.3) * 2.0 + (65562.5) * 1.0) * 1024),
        "dense_16x4096x7168":
            int(((14875.0) * 2.0 + (128.0) * 1.0) * 1024),
        "moe_contiguous_G8_T4096_N4096_K7168":
            int(((188154.5 + 24608.6) * 2.0 + (79955.2 + 6144.0) * 1.0) * 1024),
        "moe_masked_G32_maxm256_N7168_K2048":
            int(((229910.2) * 2.0 + (60548.0) * 1.0) * 1024),
    },
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--reps", type=int, default=5, help="repetitions of each per-kernel timing")
    p.add_argument("--workload", default="dense",
                   choices=["dense", "small_m", "contiguous", "masked"],
                   help="the workload of the timed steps (default: the headline dense shape)")
    p.add_argument("--only", action="store_true",
                   help="time only the --workload path (no other kernels in the line)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-check", action="store_true", help="skip the parity spot checks")
    p.add_argument("--calibrate-copy", action="store_true")
    p.add_argument("--no-warmup-call", action="store_true",
                   help="skip fp8g_warmup, so that the first step pays for loading the "
                        "kernels (to measure the first-call latency without it)")
    p.add_argument("--prewarm-s", type=float, default=1.0,
                   help="seconds of untimed steps before the warmup steps, so that the "
                        "GPU clocks have settled (steady-state throughput is reported)")
    return p.parse_args()


CFG_INDEX = {"dense": 2, "small_m": 1, "contiguous": 3, "masked": 4}


class Path:
    """Device buffers and the launch sequence of one step on one workload."""

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
        self.ws = None
        if w.kind == "masked":
            self.d = torch.empty((w.G, w.M, w.N), dtype=torch.int16, device=dev)
            self.meta = torch.from_numpy(w.masked_m.astype(np.int32)).to(dev)
        else:
            self.d = torch.empty((self.rows_a, w.N), dtype=torch.int16, device=dev)
            self.meta = None
            if w.kind == "contiguous":
                self.meta = torch.from_numpy(w.offsets.astype(np.int32)).to(dev)
                n = fp8g.grouped_gemm_fp8_contiguous_workspace_size(w.G, w.M, w.N, K)
                if n:
                    self.ws = torch.empty(n, dtype=torch.uint8, device=dev)
        self.qb_gemm = self.qb          # the weight codes the GEMM reads (rotated for cold runs)

    def quant_a(self):
        self.fp8g.fp8_quantize(self.xa, 1, self.qa, self.sa, 1, self.rows_a)

    def quant_b(self):
        self.fp8g.fp8_quantize(self.xb, 128, self.qb, self.sb, self.w.K // 128, 1)

    def gemm(self):
        w, f = self.w, self.fp8g
        K, N = w.K, w.N
        if w.kind == "dense":
            f.gemm_fp8_blockscaled(self.qa, self.sa, self.qb_gemm, self.sb, self.d)
        elif w.kind == "contiguous":
            f.grouped_gemm_fp8_contiguous_ws(self.qa, self.sa, self.qb.view(w.G, N, K),
                                             self.sb.view(w.G, N // 128, K // 128), self.d,
                                             self.meta, self.ws)
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

    def free_inputs(self):
        """Drop the fp32 inputs once the codes exist (GEMM-only timing)."""
        self.xa = self.xb = None


def algorithmic(w):
    """Algorithmic flops and bytes of each kernel of one step."""
    K, N = w.K, w.N
    rows_a = w.a.reshape(-1, K).shape[0]
    rows_b = w.b.reshape(-1, K).shape[0]
    m_eff = w.M if w.kind == "dense" else int(np.sum(w.counts))   # valid rows
    flops = 2.0 * m_eff * N * K
    # quantisers: 4 B read + 1 B written per element, 4 B per scale
    qa_bytes = rows_a * K * 5 + rows_a * (K // 128) * 4
    qb_bytes = rows_b * K * 5 + (rows_b // 128) * (K // 128) * 4
    # GEMM: fp8 A rows read once, fp8 B of the experts that have rows read once,
    # scales, bf16 output of the rows computed
    if w.kind == "dense":
        b_rows, a_rows = N, w.M
    elif w.kind == "contiguous":
        b_rows = N * int(np.sum(w.counts > 0))
        a_rows = w.M                                # padded rows are read and written
    else:
        b_rows = N * int(np.sum(w.masked_m > 0))
        a_rows = m_eff
    gemm_bytes = (a_rows * K + b_rows * K + a_rows * (K // 128) * 4
                  + (b_rows // 128) * (K // 128) * 4 + a_rows * N * 2)
    return {"flops": flops, "quantize_a": qa_bytes, "quantize_b": qb_bytes, "gemm": gemm_bytes}


def host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w):
    """The oracle, untouched, on a bounded sample of the headline workload:
    the first half of A's rows (full K) against all of B. BLAS runs on every
    core this process may use; the rest of the oracle is single-threaded
    NumPy."""
    from oracle import quantize_blocks, gemm_blockscaled
    cores = host_cores()
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=cores, user_api="blas")
    except Exception:
        limiter = None
    K = w.K
    ms = w.M // 2 if w.kind == "dense" else w.a.reshape(-1, K).shape[0]
    xa = w.a.reshape(-1, K)[:ms]
    xb = w.b.reshape(-1, K) if w.kind == "dense" else w.b[0]
    t0 = time.perf_counter()
    qa, sa = quantize_blocks(xa, 1)
    qb, sb = quantize_blocks(xb, 128)
    t1 = time.perf_counter()
    gemm_blockscaled(qa, sa, qb, sb)
    t2 = time.perf_counter()
    if limiter is not None:
        limiter.unregister()
    flops = 2.0 * ms * xb.shape[0] * K
    return {"value": flops / (t2 - t0) / 1e12, "unit": "TFLOPS", "cores": int(cores),
            "kind": "oracle",
            "sample": f"A rows 0..{ms - 1} against all {xb.shape[0]} B rows, full K={K} "
                      f"({flops / 1e9:.0f} GFLOP): quantise A and B {t1 - t0:.1f} s, GEMM "
                      f"{t2 - t1:.1f} s; CPU {cpu_model()}"}


def gemm_code_digest(paths=GEMM_SOURCES):
    """sha256 of the GEMM sources with comments and whitespace removed: any
    change to the code changes it, an edit of a comment does not."""
    import hashlib
    import re
    h = hashlib.sha256()
    for path in paths:
        text = open(path, encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        text = re.sub(r"\s+", "", text)
        h.update(text.encode("utf-8"))
    return h.hexdigest()


def measured_traffic(workload):
    try:
        digest = gemm_code_digest()
    except OSError:
        return None
    return MEASURED_TRAFFIC.get(digest, {}).get(workload)


def spot_check(path, w, d=None):
    """Sanity check of sampled GEMM rows, on the GPU with plain torch float32
    ops: the codes and scales are dequantised, multiplied in float32, and the
    library's bf16 rows (of d, by default the step's output) must lie within
    |d - ref| <= 2^-7 |ref| + 2^-10 rms."""
    torch = path.torch
    d = path.d if d is None else d
    torch.cuda.synchronize()
    K, N = w.K, w.N
    kb = K // 128

    def dequant_rows(q, s_rows):
        x = q.view(torch.float8_e4m3fn).to(torch.float32).view(q.shape[0], kb, 128)
        return (x * s_rows.unsqueeze(-1)).view(q.shape[0], K)

    def dequant_b(q, s_blocks):
        x = q.view(torch.float8_e4m3fn).to(torch.float32).view(q.shape[0] // 128, 128, kb, 128)
        return (x * s_blocks.view(q.shape[0] // 128, 1, kb, 1)).view(q.shape[0], K)

    qb = path.qb_gemm.view(-1, N, K)
    sb = path.sb.view(-1, N // 128, kb)
    if w.kind == "dense":
        rows = torch.tensor([0, w.M // 3, w.M - 1], device=path.qa.device)
        g = 0
        got = d[rows]
    else:
        g = int(np.argmax(w.counts))
        r0 = g * w.M if w.kind == "masked" else int(w.offsets[g])
        rows = torch.arange(r0, r0 + 3, device=path.qa.device)
        got = d.view(-1, N)[rows]
    a = dequant_rows(path.qa[rows], path.sa[:, rows].t().contiguous())
    b = dequant_b(qb[g], sb[g])
    ref = a @ b.t().contiguous()
    got = got.view(torch.bfloat16).to(torch.float32)
    rms = torch.sqrt(torch.mean(ref * ref))
    bad = (got - ref).abs() > (2.0 ** -7) * ref.abs() + (2.0 ** -10) * rms
    if not torch.isfinite(got).all() or bool(bad.any()):
        raise SystemExit(f"parity spot check failed on {w.name}: "
                         f"{int(bad.sum())} elements out of tolerance")


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


# GPU clock and power from rocm-smi while the steps run. A child process,
# started before this process touches the GPU, calls rocm-smi in a loop and
# appends each reading (with the wall-clock interval it was taken in) to a
# file; the bench keeps the readings taken during its pre-warm and timed
# steps (the same back-to-back launches; the timed region alone is too short
# for rocm-smi's ~0.3 s per reading). Not started under a profiler, whose
# preloaded library would bring up the GPU in every child process.
SMI_LOOP = r"""
import json, os, subprocess, sys, time
exe, path = sys.argv[1], sys.argv[2]
parent, start = os.getppid(), time.time()
with open(path, "a") as f:
    # (ends with the bench: when its parent is gone, or after an hour)
    while os.getppid() == parent and time.time() - start < 3600:
        t0 = time.time()
        try:
            out = subprocess.run([exe, "--showpower", "--showclocks", "--showuse", "--json"],
                                 capture_output=True, text=True, timeout=10).stdout
        except Exception:
            out = ""
        f.write(json.dumps({"t0": t0, "t1": time.time(), "out": out}) + "\n")
        f.flush()
        time.sleep(0.05)
"""


class SmiMonitor:
    def __init__(self):
        self.proc, self.path, self.reason = None, None, None
        if any(k.startswith("ROCPROF") for k in os.environ) or \
                "rocprof" in os.environ.get("LD_PRELOAD", ""):
            self.reason = "not sampled under a profiler"
            return
        exe = shutil.which("rocm-smi") or "/opt/rocm/bin/rocm-smi"
        if not os.access(exe, os.X_OK):
            self.reason = "rocm-smi not found"
            return
        fd, self.path = tempfile.mkstemp(prefix="bench_smi_", suffix=".jsonl")
        os.close(fd)
        try:
            self.proc = subprocess.Popen([sys.executable, "-c", SMI_LOOP, exe, self.path],
                                         stdin=subprocess.DEVNULL, stdout=subprocess.DEVNULL,
                                         stderr=subprocess.DEVNULL, start_new_session=True)
        except OSError as e:
            self.reason = f"rocm-smi sampler not started: {e}"
        atexit.register(self.stop)

    def stop(self):
        if self.proc is not None and self.proc.poll() is None:
            self.proc.terminate()
            try:
                self.proc.wait(timeout=5)
            except subprocess.TimeoutExpired:
                self.proc.kill()
                self.proc.wait()

    def summary(self, t_start, t_end):
        """Readings that overlap [t_start, t_end] (wall clock) of the busiest card."""
        self.stop()
        if self.proc is None:
            return {"tool": "rocm-smi", "samples": 0, "reason": self.reason}
        per_card = {}
        with open(self.path) as f:
            for line in f:
                try:
                    r = json.loads(line)
                except ValueError:
                    continue
                if r["t1"] < t_start or r["t0"] > t_end or not r["out"].strip():
                    continue
                try:
                    cards = json.loads(r["out"])
                except ValueError:
                    continue
                for card, vals in cards.items():
                    if not isinstance(vals, dict):
                        continue
                    e = {}
                    for k, v in vals.items():
                        if "Power (W)" in k:
                            try:
                                e["power_w"] = float(v)
                            except (TypeError, ValueError):
                                pass
                        elif k.startswith("sclk clock speed"):
                            m = re.search(r"(\d+)\s*Mhz", str(v), re.I)
                            if m:
                                e["sclk_mhz"] = float(m.group(1))
                        elif k.startswith("GPU use"):
                            try:
                                e["use_pct"] = float(v)
                            except (TypeError, ValueError):
                                pass
                    per_card.setdefault(card, []).append(e)
        os.unlink(self.path)
        if not per_card:
            return {"tool": "rocm-smi", "samples": 0, "reason": "no reading in the window"}

        def mean_of(rows, key):
            v = [x[key] for x in rows if key in x]
            return (round(statistics.fmean(v), 1), round(max(v), 1)) if v else (None, None)
        card = max(per_card, key=lambda c: (mean_of(per_card[c], "use_pct")[0] or 0.0))
        rows = per_card[card]
        p_mean, p_max = mean_of(rows, "power_w")
        c_mean, c_max = mean_of(rows, "sclk_mhz")
        out = {"tool": "rocm-smi", "card": card, "samples": len(rows),
               "window": "pre-warm and timed steps (back-to-back launches)",
               "use_pct_mean": mean_of(rows, "use_pct")[0],
               "power_w_mean": p_mean, "power_w_max": p_max,
               "sclk_mhz_mean": c_mean, "sclk_mhz_max": c_max}
        if p_mean is None:
            out["power_note"] = "rocm-smi reports no power reading for this GPU"
        return out


def prewarm(torch, fn, seconds):
    t = time.perf_counter()
    while time.perf_counter() - t < seconds:
        for _ in range(16):
            fn()
        torch.cuda.synchronize()


def time_kernel(torch, fn, launches, reps):
    """R repetitions of `launches` back-to-back launches of fn, HIP events at
    the ends of each repetition (on the current stream, the one the library
    launches on). Returns the per-launch ms of each repetition."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for r in range(reps):
        for _ in range(launches):
            fn()
        ev[r + 1].record()
    torch.cuda.synchronize()
    return [ev[r].elapsed_time(ev[r + 1]) / launches for r in range(reps)]


def held_clock_ghz(torch, fp8g, fn, n=8):
    """Shader clock while fn runs back to back: fn, probe, fn, probe, ...
    (each probe reads the clock the chip holds under that load)."""
    out = torch.zeros((n, 2), dtype=torch.int64, device="cuda")
    for _ in range(4):
        fn()
    for i in range(n):
        for _ in range(3):
            fn()
        fp8g.fp8g_clock_probe(out[i], 2000)
    torch.cuda.synchronize()
    o = out.cpu().numpy().astype(np.float64)
    ghz = o[:, 0] / o[:, 1] * 0.1
    return round(float(np.median(ghz)), 3)


def summarise(ms_list):
    return {"avg_us": round(statistics.fmean(ms_list) * 1e3, 2),
            "median_us": round(statistics.median(ms_list) * 1e3, 2),
            "min_us": round(min(ms_list) * 1e3, 2)}


def gemm_entry(w, alg, ms_list, clock, extra=None):
    """One kernels entry for a GEMM: times, roofline fraction (HBM for the
    decode-shaped and masked shapes, FP8 MFMA otherwise), counter traffic."""
    ent = summarise(ms_list)
    sec = ent["avg_us"] / 1e6
    tf = alg["flops"] / sec / 1e12
    gbs = alg["gemm"] / sec / 1e9
    ent.update({"workload": w.name, "TFLOPS": round(tf, 1),
                "fp8_peak_frac": round(tf / FP8_PEAK_TFLOPS, 4),
                "alg_GBs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                "bound": "hbm" if (w.kind == "masked" or w.M <= 32) else "mfma",
                "alg_flops": alg["flops"], "alg_bytes": alg["gemm"],
                "traffic": measured_traffic(w.name), "held_clock_ghz": clock})
    if extra:
        ent.update(extra)
    return ent


def roofline_of(ent):
    if ent["bound"] == "hbm":
        return {"bound": "hbm", "achieved": ent["alg_GBs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": ent["hbm_frac"], "traffic": ent["traffic"]}
    return {"bound": "mfma", "achieved": ent["TFLOPS"], "peak": FP8_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": ent["fp8_peak_frac"], "traffic": ent["traffic"]}


def add_generic_time(torch, fp8g, fn, launches, args, ent):
    """The same GEMM with the shape-specialised kernels switched off (the
    kernel table's generic kernels; the results are bit-identical)."""
    try:
        fp8g.fp8g_set_shape_specialisation(False)
        prewarm(torch, fn, min(args.prewarm_s, 0.3))
        ent["generic_kernel_avg_us"] = summarise(time_kernel(torch, fn, launches, args.reps))["avg_us"]
    finally:
        fp8g.fp8g_set_shape_specialisation(True)


def gemm_only(torch, fp8g, w, args, log):
    """Set up one workload (GPU quantisation), then time its GEMM alone."""
    t0 = time.perf_counter()
    path = Path(w, torch, fp8g)
    path.quant_a()
    path.quant_b()
    path.free_inputs()
    path.gemm()
    torch.cuda.synchronize()
    if not args.no_check:
        spot_check(path, w)
    alg = algorithmic(w)
    extra = None
    fn = path.gemm
    launches = max(args.steps, 20)
    if w.kind == "dense" and w.M <= 32:
        # decode shape: 29 MB of weights would stay in the 256 MB Infinity
        # Cache; the headline (cold) figure rotates over copies larger than it
        prewarm(torch, fn, min(args.prewarm_s, 0.3))
        warm = time_kernel(torch, fn, launches, args.reps)
        ncopy = max(10, -(-300 * 2**20 // path.qb.numel()))
        copies = [path.qb.clone() for _ in range(ncopy)]
        state = {"i": 0}

        def cold():
            path.qb_gemm = copies[state["i"] % ncopy]
            state["i"] += 1
            path.gemm()
        fn = cold
        launches = max(launches, 2 * ncopy)
        extra = {"weights": f"cold (rotated over {ncopy} copies, > Infinity Cache)",
                 "warm": summarise(warm)}
    prewarm(torch, fn, min(args.prewarm_s, 0.3))
    ms = time_kernel(torch, fn, launches, args.reps)
    clock = held_clock_ghz(torch, fp8g, fn)
    ent = gemm_entry(w, alg, ms, clock, extra)
    add_generic_time(torch, fp8g, fn, launches, args, ent)
    log(f"{w.name}: {ent['avg_us']} us (median {ent['median_us']}, min {ent['min_us']}), "
        f"{ent['TFLOPS']} TFLOPS, {ent['alg_GBs']} GB/s, clock {clock} GHz, "
        f"set up in {time.perf_counter() - t0:.1f} s")
    del path
    torch.cuda.empty_cache()
    return ent


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the library "
              "and this benchmark run on a single GPU, there is no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        return calibrate_copy(args)
    smi = SmiMonitor()                # (before this process touches the GPU)

    import torch
    import moe_grouped_gemm_quantizer_amd as fp8g
    from workloads import make_config

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    fp8g.load()
    t0 = time.perf_counter()
    w = make_config(CFG_INDEX[args.workload])
    log(f"workload {w.name}: generated in {time.perf_counter() - t0:.1f} s")
    torch.zeros(1, device="cuda:0")
    torch.cuda.synchronize()          # (the HIP runtime is up before anything is timed)
    # First-call latency (nxmr §2.3: warm the kernels up before the first
    # request): fp8g_warmup loads every kernel's code object onto the GPU;
    # without it the first step pays for that itself.
    first_call = {"warmup_call": not args.no_warmup_call}
    if not args.no_warmup_call:
        t0 = time.perf_counter()
        fp8g.fp8g_warmup()
        first_call["warmup_ms"] = round((time.perf_counter() - t0) * 1e3, 3)
    path = Path(w, torch, fp8g)
    alg = algorithmic(w)
    torch.cuda.synchronize()
    for key in ("first_step_ms", "second_step_ms"):
        t0 = time.perf_counter()
        path.step()
        torch.cuda.synchronize()
        first_call[key] = round((time.perf_counter() - t0) * 1e3, 3)
    log(f"first call: {first_call}")

    # parity spot check first: it keeps the GPU idle while the host computes,
    # and the shader clock needs 10-20 ms of load to recover from an idle gap
    if not args.no_check:
        spot_check(path, w)
        log("parity spot check ok")
    # pre-warm with the same back-to-back launches as the timed region
    smi_t0 = time.time()
    prewarm(torch, path.step, args.prewarm_s)
    for _ in range(args.warmup):
        path.step()
    torch.cuda.synchronize()

    # Timed region: K whole steps launched back to back, HIP events only at
    # its two ends.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        path.step()
    e1.record()
    torch.cuda.synchronize()
    smi_t1 = time.time()
    timed_d = path.d.clone() if not args.no_check else None   # (checked below)
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    gpu_ms_per_step = e0.elapsed_time(e1) / args.steps
    log(f"{args.steps} steps: {ms_per_step:.4f} ms per step (host clock), "
        f"{gpu_ms_per_step:.4f} ms (events)")

    # Each kernel of the step alone: R repetitions of K back-to-back launches.
    kernels = {}
    launches = max(args.steps, 20)
    for name, fn in (("quantize_a", path.quant_a), ("quantize_b", path.quant_b)):
        ms = time_kernel(torch, fn, launches, args.reps)
        ent = summarise(ms)
        gbs = alg[name] / (ent["avg_us"] / 1e6) / 1e9
        ent.update({"alg_bytes": alg[name], "alg_GBs": round(gbs, 1),
                    "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "bound": "hbm"})
        kernels[name] = ent
    # The per-tensor-scaled GEMM on the same inputs (gtnt, Triton kernel
    # section): quantised with one scale per operand, MFMA accumulation over
    # all of K, one epilogue multiply. Beside the block-scaled GEMM it gives
    # the cost of the per-block promotion.
    pt = None
    if w.kind == "dense" and w.M > 32 and not args.only:
        dev = torch.device("cuda:0")
        pqa = torch.empty_like(path.qa)
        pqb = torch.empty_like(path.qb)
        psa = torch.empty(1, dtype=torch.float32, device=dev)
        psb = torch.empty(1, dtype=torch.float32, device=dev)
        pd = torch.empty_like(path.d)
        fp8g.fp8_quantize_tensor(path.xa, pqa, psa)
        fp8g.fp8_quantize_tensor(path.xb, pqb, psb)
        qt_ms = time_kernel(torch, lambda: fp8g.fp8_quantize_tensor(path.xa, pqa, psa),
                            launches, args.reps)
        # delayed scaling (czchanglian §2.3) with e5m2 codes for A, as a
        # gradient would be quantised: one pass, the scale from the history
        eqa = torch.empty_like(path.qa)
        esa = torch.empty(1, dtype=torch.float32, device=dev)
        hist = torch.full((16,), float(np.abs(w.a).max()), dtype=torch.float32, device=dev)
        fp8g.fp8_quantize_delayed(path.xa, "e5m2", hist, 0, eqa, esa)
        dq_ms = time_kernel(torch, lambda: fp8g.fp8_quantize_delayed(path.xa, "e5m2", hist, 0, eqa, esa),
                            launches, args.reps)
        pt = (pqa, psa, pqb, psb, pd, qt_ms, eqa, esa, dq_ms)
    path.free_inputs()
    torch.cuda.empty_cache()
    main_gemm = None
    if w.kind == "dense" and w.M <= 32:
        main_gemm = gemm_only(torch, fp8g, w, args, log)
    else:
        prewarm(torch, path.gemm, min(args.prewarm_s, 0.3))
        ms = time_kernel(torch, path.gemm, launches, args.reps)
        clock = held_clock_ghz(torch, fp8g, path.gemm)
        main_gemm = gemm_entry(w, alg, ms, clock)
        add_generic_time(torch, fp8g, path.gemm, launches, args, main_gemm)
        log(f"{w.name} GEMM: {main_gemm['avg_us']} us (median {main_gemm['median_us']}, "
            f"min {main_gemm['min_us']}), {main_gemm['TFLOPS']} TFLOPS, clock {clock} GHz")
    kernels["gemm"] = main_gemm
    if pt is not None:
        pqa, psa, pqb, psb, pd, qt_ms, eqa, esa, dq_ms = pt
        ent = summarise(dq_ms)
        gbs = alg["quantize_a"] / (ent["avg_us"] / 1e6) / 1e9
        ent.update({"alg_bytes": alg["quantize_a"], "alg_GBs": round(gbs, 1),
                    "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "bound": "hbm",
                    "note": "A per tensor, delayed scaling (scale from a 16-entry amax "
                            "history), e5m2 codes: one pass"})
        kernels["quantize_delayed_a_e5m2"] = ent
        ent = summarise(qt_ms)
        gbs = alg["quantize_a"] / (ent["avg_us"] / 1e6) / 1e9
        ent.update({"alg_bytes": alg["quantize_a"], "alg_GBs": round(gbs, 1),
                    "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "bound": "hbm",
                    "note": "A per tensor: amax pass + encode pass (reads A twice)"})
        kernels["quantize_tensor_a"] = ent

        def pt_gemm():
            fp8g.gemm_fp8_pertensor(pqa, psa, pqb, psb, pd)
        pt_gemm()
        torch.cuda.synchronize()
        if not args.no_check:
            # sampled rows against a float32 product of the dequantised codes
            rows = torch.tensor([0, w.M // 2, w.M - 1], device=pqa.device)
            a = pqa[rows].view(torch.float8_e4m3fn).to(torch.float32) * psa
            b = pqb.view(torch.float8_e4m3fn).to(torch.float32) * psb
            ref = a @ b.t().contiguous()
            got = pd[rows].view(torch.bfloat16).to(torch.float32)
            rms = torch.sqrt(torch.mean(ref * ref))
            if bool(((got - ref).abs() > 2.0 ** -7 * ref.abs() + 2.0 ** -10 * rms).any()):
                raise SystemExit("parity spot check failed on the per-tensor GEMM")
        prewarm(torch, pt_gemm, min(args.prewarm_s, 0.3))
        ms = time_kernel(torch, pt_gemm, launches, args.reps)
        clock = held_clock_ghz(torch, fp8g, pt_gemm)
        ent = gemm_entry(w, alg, ms, clock)
        ent["workload"] = w.name + "_pertensor"
        ent["traffic"] = measured_traffic(w.name + "_pertensor")
        ent["promotion_cost"] = round(main_gemm["avg_us"] / ent["avg_us"], 3)
        kernels["gemm_pertensor"] = ent
        log(f"per-tensor GEMM: {ent['avg_us']} us, {ent['TFLOPS']} TFLOPS, clock {clock} GHz; "
            f"block-scaled / per-tensor time = {ent['promotion_cost']}")

        def e5_gemm():
            fp8g.gemm_fp8_pertensor_fmt(eqa, "e5m2", esa, pqb, "e4m3", psb, pd)
        e5_gemm()
        prewarm(torch, e5_gemm, min(args.prewarm_s, 0.3))
        ms = time_kernel(torch, e5_gemm, launches, args.reps)
        ent = gemm_entry(w, alg, ms, held_clock_ghz(torch, fp8g, e5_gemm))
        ent["workload"] = w.name + "_pertensor_e5m2_x_e4m3"
        ent["traffic"] = measured_traffic(ent["workload"])
        kernels["gemm_pertensor_e5m2"] = ent
        log(f"per-tensor e5m2 x e4m3 GEMM: {ent['avg_us']} us, {ent['TFLOPS']} TFLOPS")
        del pt, pqa, pqb, pd, eqa
    # The GEMM with the 1x128 quantiser of its output fused into the epilogue
    # (nxmr section 3.1: the producer writes the next layer's activations
    # already quantised) against the GEMM followed by the standalone
    # quantiser on its bf16 output.
    if w.kind == "dense" and w.M > 32 and not args.only:
        dev = torch.device("cuda:0")
        fqd = torch.empty((w.M, w.N), dtype=torch.uint8, device=dev)
        fsd = torch.empty((w.N // 128, w.M), dtype=torch.float32, device=dev)
        uqd, usd = torch.empty_like(fqd), torch.empty_like(fsd)

        def fused():
            fp8g.gemm_fp8_blockscaled_quant(path.qa, path.sa, path.qb, path.sb, path.d, fqd, fsd)

        def fused_noout():
            fp8g.gemm_fp8_blockscaled_quant(path.qa, path.sa, path.qb, path.sb, None, fqd, fsd)

        def unfused():
            path.gemm()
            fp8g.fp8_quantize_bf16(path.d, 1, uqd, usd, 1, w.M)
        fused()
        unfused()
        torch.cuda.synchronize()
        if not args.no_check and not (torch.equal(fqd, uqd) and torch.equal(fsd, usd)):
            raise SystemExit("fused quantising epilogue differs from GEMM + quantiser")
        ent = {}
        for nm, fn in (("fused", fused), ("fused_no_bf16", fused_noout), ("gemm_then_quantize", unfused)):
            prewarm(torch, fn, min(args.prewarm_s, 0.3))
            ent[nm + "_us"] = summarise(time_kernel(torch, fn, launches, args.reps))["avg_us"]
        ent["note"] = ("output of the 4096x8192x8192 GEMM quantised 1x128 for the next GEMM: "
                       "in the epilogue vs a separate quantiser pass over the bf16 result")
        kernels["gemm_quant_epilogue"] = ent
        log(f"quantising epilogue: fused {ent['fused_us']} us, without bf16 out "
            f"{ent['fused_no_bf16_us']} us, GEMM then quantiser {ent['gemm_then_quantize_us']} us")
        del fqd, fsd, uqd, usd
    # the last timed step's output, checked now that this workload's timing
    # is done (a host check right after the timed region would idle the GPU
    # before the per-kernel timings); the operands are unchanged since
    parity_timed = None
    if timed_d is not None:
        spot_check(path, w, timed_d)
        log("parity spot check of the timed steps' output ok")
        parity_timed = True
        del timed_d
    del path
    torch.cuda.empty_cache()

    # The GEMM on the method's other shapes (MoE contiguous and masked, the
    # decode-shaped small M), each set up and timed on its own.
    if not args.only:
        for key, wl in (("gemm_contiguous", "contiguous"), ("gemm_masked", "masked"),
                        ("gemm_small_m", "small_m")):
            if wl == args.workload:
                continue
            tg = time.perf_counter()
            wo = make_config(CFG_INDEX[wl])
            log(f"workload {wo.name}: generated in {time.perf_counter() - tg:.1f} s")
            kernels[key] = gemm_only(torch, fp8g, wo, args, log)
            del wo

    value = alg["flops"] / (ms_per_step / 1e3) / 1e12
    out = {
        "metric": METRIC,
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
        "roofline": roofline_of(main_gemm),
        "held_clock_ghz": main_gemm["held_clock_ghz"],
        "smi": smi.summary(smi_t0, smi_t1),
        "first_call": first_call,
        "kernels": kernels,
    }
    if parity_timed:
        out["parity_rechecked_on_timed_output"] = True
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
