"""Host logic of bench.py that runs without a GPU.

* The rocm-smi sampler: a stand-in rocm-smi (a script printing the JSON
  shape rocm-smi gives: per card, a power entry, "sclk clock speed:" as
  "(NNNNMhz)", "GPU use (%)") is sampled by the same child process the
  bench starts; the summary keeps the busiest card's readings inside the
  window, reports missing power as absent, stops the child and removes its
  file; under a profiler (a ROCPROF* variable set) nothing is started.
* The stored counter traffic is keyed by a digest of the GEMM sources with
  comments and whitespace removed: a comment edit keeps the key, a code
  edit changes it (the bench then reports no traffic until the counters
  are taken again).
"""

import os
import stat
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FAKE_SMI = """#!{python}
import json
print(json.dumps({{
    "card0": {{"Current Socket Graphics Package Power (W)": "{p0}", "sclk clock speed:": "(2100Mhz)",
              "GPU use (%)": "100"}},
    "card1": {{"Current Socket Graphics Package Power (W)": "150.0", "sclk clock speed:": "(132Mhz)",
              "GPU use (%)": "0"}},
}}))
"""


def _fake_smi(tmp_path, p0="1000.0"):
    d = tmp_path / "bin"
    d.mkdir()
    exe = d / "rocm-smi"
    exe.write_text(FAKE_SMI.format(python=sys.executable, p0=p0))
    exe.chmod(exe.stat().st_mode | stat.S_IEXEC)
    return str(d)


def test_smi_sampler_summary(tmp_path, monkeypatch):
    monkeypatch.setenv("PATH", _fake_smi(tmp_path) + os.pathsep + os.environ["PATH"])
    for k in [k for k in os.environ if k.startswith("ROCPROF")]:
        monkeypatch.delenv(k)
    mon = bench.SmiMonitor()
    assert mon.proc is not None, mon.reason
    t0 = time.time()
    time.sleep(1.0)
    out = mon.summary(t0, time.time())
    assert out["card"] == "card0"                  # the busy card
    assert out["samples"] >= 1
    assert out["power_w_mean"] == 1000.0 and out["power_w_max"] == 1000.0
    assert out["sclk_mhz_mean"] == 2100.0 and out["use_pct_mean"] == 100.0
    assert "power_note" not in out
    assert mon.proc.poll() is not None              # the sampler has stopped
    assert not os.path.exists(mon.path)             # and its file is gone


def test_smi_sampler_missing_power(tmp_path, monkeypatch):
    monkeypatch.setenv("PATH", _fake_smi(tmp_path, p0="N/A") + os.pathsep + os.environ["PATH"])
    for k in [k for k in os.environ if k.startswith("ROCPROF")]:
        monkeypatch.delenv(k)
    mon = bench.SmiMonitor()
    t0 = time.time()
    time.sleep(0.8)
    out = mon.summary(t0, time.time())
    assert out["power_w_mean"] is None and "power_note" in out
    assert out["sclk_mhz_mean"] == 2100.0


def test_smi_sampler_window_outside(tmp_path, monkeypatch):
    monkeypatch.setenv("PATH", _fake_smi(tmp_path) + os.pathsep + os.environ["PATH"])
    for k in [k for k in os.environ if k.startswith("ROCPROF")]:
        monkeypatch.delenv(k)
    mon = bench.SmiMonitor()
    time.sleep(0.5)
    out = mon.summary(0.0, 1.0)                     # a window long before the run
    assert out["samples"] == 0


def test_smi_sampler_not_under_profiler(monkeypatch):
    monkeypatch.setenv("ROCPROF_OUTPUT_PATH", "/tmp")
    mon = bench.SmiMonitor()
    assert mon.proc is None
    assert mon.summary(0.0, 1.0)["samples"] == 0


def test_traffic_digest_ignores_comments(tmp_path):
    src = "int f(int x) {\n  // the argument, doubled\n  return 2 * x;  /* twice */\n}\n"
    a = tmp_path / "a.hip"
    a.write_text(src)
    b = tmp_path / "b.hip"
    b.write_text(src.replace("// the argument, doubled", "// doubled").replace("  return", "    return"))
    c = tmp_path / "c.hip"
    c.write_text(src.replace("2 * x", "3 * x"))
    da, db, dc = (bench.gemm_code_digest([str(p)]) for p in (a, b, c))
    assert da == db
    assert da != dc

