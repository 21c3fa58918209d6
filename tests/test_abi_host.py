"""The C ABI library on the host (no GPU needed).

Checks that libfp8gemm.so loads, exports every function include/fp8gemm.h
declares, and rejects invalid arguments with the documented status before it
touches the device (every call here fails validation, so nothing reaches HIP).
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8gemm.h")

from moe_grouped_gemm_quantizer_amd import _lib


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*"
                                 r"([A-Za-z_][A-Za-z0-9_]*)\s*\(", text, flags=re.M)))


STATUS = dict(OK=0, NULL=1, SHAPE=2, ALIGN=3, STRIDE=4, DEVICE=5, LAUNCH=6, UNSUPPORTED=7)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from moe_grouped_gemm_quantizer_amd.build import build
        build()
    return _lib.load()


def test_header_declares_the_four_entry_points():
    fns = _declared_functions()
    for name in ("fp8_quantize", "gemm_fp8_blockscaled", "grouped_gemm_fp8_contiguous",
                 "grouped_gemm_fp8_masked", "fp8g_status_string", "fp8g_abi_version"):
        assert name in fns, fns


def test_library_exports_every_declared_function(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert set(_lib.ENTRY_POINTS) <= set(_declared_functions())


def test_status_strings_and_version(lib):
    assert lib.fp8g_abi_version() == 1
    for code in range(8):
        assert lib.fp8g_status_string(code)
    assert lib.fp8g_status_string(0) == b"ok"
    assert lib.fp8g_status_string(99) == b"unknown status"


# fake, well-aligned addresses: validation fails before anything uses them
P = 0x100000
P2 = 0x200000


def test_quantize_validation(lib):
    f = lib.fp8_quantize
    assert f(P, 4, 256, 256, 2, P2, 256, P, 1, 4, None) == STATUS["SHAPE"]        # block_rows
    assert f(P, -1, 256, 256, 1, P2, 256, P, 1, 4, None) == STATUS["SHAPE"]
    assert f(P, 0, 256, 256, 1, P2, 256, P, 1, 4, None) == STATUS["OK"]           # no-op
    assert f(P, 4, 200, 256, 1, P2, 256, P, 1, 4, None) == STATUS["SHAPE"]        # cols % 128
    assert f(None, 4, 256, 256, 1, P2, 256, P, 1, 4, None) == STATUS["NULL"]
    assert f(P, 4, 256, 256, 1, None, 256, P, 1, 4, None) == STATUS["NULL"]
    assert f(P, 4, 256, 256, 1, P2, 256, None, 1, 4, None) == STATUS["NULL"]
    assert f(P, 4, 256, 128, 1, P2, 256, P, 1, 4, None) == STATUS["STRIDE"]       # ldx < cols
    assert f(P, 4, 256, 256, 1, P2, 256, P, 0, 4, None) == STATUS["STRIDE"]
    assert f(P + 4, 4, 256, 256, 1, P2, 256, P, 1, 4, None) == STATUS["ALIGN"]
    assert f(P, 4, 256, 258, 1, P2, 256, P, 1, 4, None) == STATUS["ALIGN"]       # ldx % 4
    assert f(P, 4, 256, 256, 1, P2 + 1, 256, P, 1, 4, None) == STATUS["ALIGN"]
    # 128x128 blocks: row strides past the kernel's 32-bit in-block offsets
    assert f(P, 4, 256, (1 << 26) + 4, 128, P2, 256, P, 2, 1, None) == STATUS["UNSUPPORTED"]
    assert f(P, 4, 256, 256, 128, P2, (1 << 28) + 4, P, 2, 1, None) == STATUS["UNSUPPORTED"]


def test_quantize_bf16_validation(lib):
    f = lib.fp8_quantize_bf16
    assert f(P, 4, 256, 256, 2, P2, 256, P, 1, 4, None) == STATUS["SHAPE"]        # block_rows
    assert f(P, 0, 256, 256, 1, P2, 256, P, 1, 4, None) == STATUS["OK"]           # no-op
    assert f(P, 4, 200, 256, 1, P2, 256, P, 1, 4, None) == STATUS["SHAPE"]        # cols % 128
    assert f(None, 4, 256, 256, 1, P2, 256, P, 1, 4, None) == STATUS["NULL"]
    assert f(P, 4, 256, 128, 1, P2, 256, P, 1, 4, None) == STATUS["STRIDE"]       # ldx < cols
    # bf16 rows are read 8 bytes (4 values) at a time
    assert f(P + 4, 4, 256, 256, 1, P2, 256, P, 1, 4, None) == STATUS["ALIGN"]
    assert f(P, 4, 256, 258, 1, P2, 256, P, 1, 4, None) == STATUS["ALIGN"]       # ldx % 4
    assert f(P, 4, 256, (1 << 26) + 4, 128, P2, 256, P, 2, 1, None) == STATUS["UNSUPPORTED"]


def test_gemm_validation(lib):
    f = lib.gemm_fp8_blockscaled
    assert f(P, P, P, P, P2, 16, 200, 256, None) == STATUS["SHAPE"]      # N % 128
    assert f(P, P, P, P, P2, 16, 256, 100, None) == STATUS["SHAPE"]      # K % 128
    assert f(P, P, P, P, P2, -1, 256, 256, None) == STATUS["SHAPE"]
    assert f(P, P, P, P, P2, 0, 256, 256, None) == STATUS["OK"]
    assert f(None, P, P, P, P2, 16, 256, 256, None) == STATUS["NULL"]
    assert f(P, P, P, P, None, 16, 256, 256, None) == STATUS["NULL"]
    assert f(P + 8, P, P, P, P2, 16, 256, 256, None) == STATUS["ALIGN"]
    assert f(P, P, P, P, P2 + 2, 16, 256, 256, None) == STATUS["ALIGN"]


def test_grouped_validation(lib):
    c = lib.grouped_gemm_fp8_contiguous
    assert c(P, P, P, P, P2, P, 2, 200, 256, 256, None) == STATUS["SHAPE"]   # M_total % 128
    assert c(P, P, P, P, P2, P, -1, 256, 256, 256, None) == STATUS["SHAPE"]
    assert c(P, P, P, P, P2, P, 0, 256, 256, 256, None) == STATUS["OK"]
    assert c(P, P, P, P, P2, None, 2, 256, 256, 256, None) == STATUS["NULL"]
    assert c(P, P, P, P, P2, P + 2, 2, 256, 256, 256, None) == STATUS["ALIGN"]
    m = lib.grouped_gemm_fp8_masked
    assert m(P, P, P, P, P2, P, 2, 256, 200, 256, 0, None) == STATUS["SHAPE"]
    assert m(P, P, P, P, P2, P, 2, -5, 256, 256, 0, None) == STATUS["SHAPE"]
    assert m(P, P, P, P, P2, P, 2, 0, 256, 256, 0, None) == STATUS["OK"]
    assert m(P, P, P, P, P2, None, 2, 256, 256, 256, 0, None) == STATUS["NULL"]
    assert m(P, P, P, P, P2, P, 5000, 256, 256, 256, 0, None) == STATUS["UNSUPPORTED"]


def test_python_binding_fails_loudly_without_library(tmp_path):
    saved = _lib._lib
    _lib._lib = None
    try:
        with pytest.raises(RuntimeError):
            _lib.load(str(tmp_path / "missing.so"))
    finally:
        _lib._lib = saved
