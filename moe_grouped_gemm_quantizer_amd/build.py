"""Build libfp8gemm.so in-tree with hipcc for gfx950.

Run as `python -m moe_grouped_gemm_quantizer_amd.build` (or call build()).
The library is written next to this file so that it travels with the tree.
"""

import glob
import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
LIB_NAME = "libfp8gemm.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 anywhere in the device code.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(glob.glob(os.path.join(PKG_DIR, "csrc", "*.hip")))


def build(verbose=False, extra_flags=()):
    out_tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, *HIP_FLAGS, *extra_flags, "-I", os.path.join(ROOT, "include"),
           "-o", out_tmp, *sources()]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    os.replace(out_tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
