"""Host build of the persistent GEMM's index arithmetic with bounds checks.

The tile scheduling, tile decoding and copy planning of the GEMM kernel
live in csrc/gemm_index.h as functions that compile for host and device.
tests/native/gemm_index_check.cpp compiles that header with the host C++
compiler and walks every workgroup, tile, K block, copy wave and lane of
283 launches (dense and per-tensor, contiguous with and without a split
tail, masked with empty, full and clamped experts, both tile shapes,
ragged N and K, grids of 36 to 256 workgroups), checking that every copy
source and scale read stays inside its buffer and every copy lands inside
its tile's region of the LDS stage, that every stored element
lies inside D and is stored exactly once (split tiles: each K block
covered once by the pieces), and that every slot walk ends. Contiguous
group offsets that break the layout's contract (decreasing, negative, past
the rows, not multiples of 128) are checked for bounds alone: the kernel
clamps them, and which rows it then stores is unspecified. The small-M
(split-K) kernel's loads are walked too, for every instantiated row-tile
count and blocks per wave, aligned and ragged K: every 16-byte half inside
its row, rows and scale reads inside their buffers, every byte of K loaded
exactly once by a half that is kept, and every half replaced by zeros
wholly past K. The LDS stage layout is checked as well: every copy lands
its 16-byte chunk at the swizzled slot the fragment reads use, and the
zeroing of a partial last K block writes every past-K chunk of every row
once and no chunk inside K. No GPU is used; the operands are fake
addresses.
"""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "moe_grouped_gemm_quantizer_amd", "csrc")
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs a host C++ compiler and the HIP headers")
def test_gemm_index_arithmetic_in_bounds(tmp_path):
    exe = tmp_path / "gemm_index_check"
    subprocess.run(["g++", "-std=c++17", "-O2", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE,
                    "-I", CSRC, "-o", str(exe),
                    os.path.join(HERE, "native", "gemm_index_check.cpp")],
                   check=True, capture_output=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "violations 0" in res.stdout
    assert "(split tail: 0)" not in res.stdout      # split tails are exercised
    assert "small-M cases 0," not in res.stdout
