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


STATUS = dict(OK=0, NULL=1, SHAPE=2, ALIGN=3, STRIDE=4, DEVICE=5, LAUNCH=6, UNSUPPORTED=7,
              WORKSPACE=8)


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
    assert lib.fp8g_abi_version() == 3
    for code in range(9):
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
    fq = lib.gemm_fp8_blockscaled_quant
    assert fq(P, P, P, P, None, P2, P, 16, 200, 256, None) == STATUS["SHAPE"]
    assert fq(P, P, P, P, None, P2, P, 0, 256, 256, None) == STATUS["OK"]
    assert fq(P, P, P, P, None, None, P, 16, 256, 256, None) == STATUS["NULL"]
    assert fq(P, P, P, P, None, P2, None, 16, 256, 256, None) == STATUS["NULL"]
    assert fq(P, P, P, P, P2 + 2, P2, P, 16, 256, 256, None) == STATUS["ALIGN"]
    assert fq(P, P, P, P, None, P2 + 1, P, 16, 256, 256, None) == STATUS["ALIGN"]
    pt = lib.gemm_fp8_pertensor
    assert pt(P, P, P, P, P2, 16, 200, 256, None) == STATUS["SHAPE"]
    assert pt(P, None, P, P, P2, 16, 256, 256, None) == STATUS["NULL"]
    qt = lib.fp8_quantize_tensor
    assert qt(P, 4, 6, 8, P2, 8, P, None) == STATUS["SHAPE"]           # cols % 4
    assert qt(P, 0, 8, 8, P2, 8, P, None) == STATUS["OK"]
    assert qt(P, 4, 8, 4, P2, 8, P, None) == STATUS["STRIDE"]
    assert qt(P + 4, 4, 8, 8, P2, 8, P, None) == STATUS["ALIGN"]
    assert qt(P, 4, 8, 8, P2, 8, None, None) == STATUS["NULL"]
    # operand rows are addressed with 32-bit offsets: 255 * K + 112 < 2^32 needs K <= 2^24
    assert f(P, P, P, P, P2, 16, 256, (1 << 24) + 128, None) == STATUS["UNSUPPORTED"]
    assert f(P, P, P, P, P2, 0, 256, (1 << 24) + 128, None) == STATUS["UNSUPPORTED"]


def test_grouped_validation(lib):
    c = lib.grouped_gemm_fp8_contiguous
    assert c(P, P, P, P, P2, P, 2, 200, 256, 256, None) == STATUS["SHAPE"]   # M_total % 128
    assert c(P, P, P, P, P2, P, -1, 256, 256, 256, None) == STATUS["SHAPE"]
    assert c(P, P, P, P, P2, P, 0, 256, 256, 256, None) == STATUS["OK"]
    assert c(P, P, P, P, P2, None, 2, 256, 256, 256, None) == STATUS["NULL"]
    assert c(P, P, P, P, P2, P + 2, 2, 256, 256, 256, None) == STATUS["ALIGN"]
    assert c(P, P, P, P, P2, P, 2, 256, 256, (1 << 24) + 128, None) == STATUS["UNSUPPORTED"]
    w = lib.grouped_gemm_fp8_contiguous_ws
    assert w(P, P, P, P, P2, P, 2, 200, 256, 256, None, 0, None) == STATUS["SHAPE"]
    assert w(P, P, P, P, P2, P, 0, 256, 256, 256, P, 1 << 20, None) == STATUS["OK"]
    assert w(P, P, P, P, P2, None, 2, 256, 256, 256, P, 1 << 20, None) == STATUS["NULL"]
    assert w(P, P, P, P, P2, P, 2, 256, 256, 256, None, 64, None) == STATUS["NULL"]
    assert w(P, P, P, P, P2, P, 2, 256, 256, 256, P + 64, 1 << 20, None) == STATUS["ALIGN"]
    n = lib.grouped_gemm_fp8_contiguous_noalloc
    assert n(P, P, P, P, P2, P, 2, 200, 256, 256, None) == STATUS["SHAPE"]
    assert n(P, P, P, P, P2, P, 0, 256, 256, 256, None) == STATUS["OK"]
    assert n(P, P, P, P, P2, None, 2, 256, 256, 256, None) == STATUS["NULL"]
    assert n(P, P, P, P, P2, P + 2, 2, 256, 256, 256, None) == STATUS["ALIGN"]
    assert n(P, P, P, P, P2, P, 2, 256, 256, (1 << 24) + 128, None) == STATUS["UNSUPPORTED"]
    size = ctypes.c_size_t(7)
    q = lib.grouped_gemm_fp8_contiguous_workspace_size
    assert q(2, 200, 256, 256, ctypes.byref(size)) == STATUS["SHAPE"] and size.value == 0
    assert q(0, 256, 256, 256, ctypes.byref(size)) == STATUS["OK"] and size.value == 0
    assert q(2, 256, 256, 256, None) == STATUS["NULL"]
    m = lib.grouped_gemm_fp8_masked
    assert m(P, P, P, P, P2, P, 2, 256, 200, 256, 0, None) == STATUS["SHAPE"]
    assert m(P, P, P, P, P2, P, 2, -5, 256, 256, 0, None) == STATUS["SHAPE"]
    assert m(P, P, P, P, P2, P, 2, 0, 256, 256, 0, None) == STATUS["OK"]
    assert m(P, P, P, P, P2, None, 2, 256, 256, 256, 0, None) == STATUS["NULL"]
    assert m(P, P, P, P, P2, P, 5000, 256, 256, 256, 0, None) == STATUS["UNSUPPORTED"]
    assert m(P, P, P, P, P2, P, 2, (1 << 30) + 1, 256, 256, 0, None) == STATUS["UNSUPPORTED"]
    assert m(P, P, P, P, P2, P + 1, 2, 256, 256, 256, 0, None) == STATUS["ALIGN"]


def test_e5m2_and_delayed_validation(lib):
    g = lib.gemm_fp8_pertensor_fmt
    assert g(P, 2, P, P, 0, P, P2, 16, 256, 256, None) == STATUS["UNSUPPORTED"]
    assert g(P, 0, P, P, -1, P, P2, 16, 256, 256, None) == STATUS["UNSUPPORTED"]
    assert g(P, 1, P, P, 1, P, P2, 16, 200, 256, None) == STATUS["SHAPE"]
    assert g(P, 1, None, P, 1, P, P2, 16, 256, 256, None) == STATUS["NULL"]
    assert g(P, 1, P, P, 1, P, P2, 0, 256, 256, None) == STATUS["OK"]
    q = lib.fp8_quantize_delayed
    H = P2 + 0x1000
    assert q(P, 4, 8, 8, 2, H, 4, 0, P2, 8, P, None) == STATUS["UNSUPPORTED"]
    assert q(P, 4, 8, 8, 1, H, 0, 0, P2, 8, P, None) == STATUS["SHAPE"]        # empty history
    assert q(P, 4, 8, 8, 1, H, 65537, 0, P2, 8, P, None) == STATUS["SHAPE"]
    assert q(P, 4, 8, 8, 1, H, 4, 4, P2, 8, P, None) == STATUS["SHAPE"]        # slot out of range
    assert q(P, 4, 8, 8, 1, H, 4, -1, P2, 8, P, None) == STATUS["SHAPE"]
    assert q(P, 4, 6, 8, 1, H, 4, 0, P2, 8, P, None) == STATUS["SHAPE"]        # cols % 4
    assert q(P, -1, 8, 8, 1, H, 4, 0, P2, 8, P, None) == STATUS["SHAPE"]
    assert q(P, 4, 8, 8, 1, None, 4, 0, P2, 8, P, None) == STATUS["NULL"]
    assert q(P, 4, 8, 8, 1, H, 4, 0, P2, 8, None, None) == STATUS["NULL"]
    assert q(None, 4, 8, 8, 1, H, 4, 0, P2, 8, P, None) == STATUS["NULL"]
    assert q(P, 4, 8, 4, 1, H, 4, 0, P2, 8, P, None) == STATUS["STRIDE"]
    assert q(P + 4, 4, 8, 8, 1, H, 4, 0, P2, 8, P, None) == STATUS["ALIGN"]
    assert q(P, 4, 8, 8, 1, H + 2, 4, 0, P2, 8, P, None) == STATUS["ALIGN"]


def test_clock_probe_validation(lib):
    f = lib.fp8g_clock_probe
    assert f(None, 100, None) == STATUS["NULL"]
    assert f(P + 4, 100, None) == STATUS["ALIGN"]
    assert f(P, 0, None) == STATUS["SHAPE"]
    assert f(P, 1000001, None) == STATUS["SHAPE"]


def test_kernel_table_selection(lib):
    """The kernel table (nxmr §2.3, ahead of time): the hot shapes select
    their shape-specialised kernels, other shapes the generic ones, and the
    process-wide switch turns the specialisations off. Selection is host
    logic: no device is needed to ask which kernel a shape would run."""
    import moe_grouped_gemm_quantizer_amd as fp8g
    name = fp8g.fp8g_gemm_kernel_name
    assert name("dense", 4096, 8192, 8192) == \
        "persistent 256x256, dense, specialised N8192 K8192"
    assert name("dense", 4096, 8192, 8192, quant=True) == \
        "persistent 256x256 quantising epilogue, dense, generic"
    assert name("pertensor", 4096, 8192, 8192).endswith("specialised N8192 K8192")
    assert name("dense", 4096, 8192, 4096).endswith("generic")
    assert name("dense", 100, 8192, 8192) == "persistent 128x256, dense, generic"
    assert name("contiguous", 4608, 4096, 7168, G=8).endswith("specialised N4096 K7168")
    assert name("contiguous", 4608, 4096, 7168, G=2000).startswith("persistent 128x256")
    assert name("masked", 256, 7168, 2048, G=32, expected_m=134).endswith(
        "specialised N7168 K2048")
    assert name("masked", 256, 7168, 2048, G=32, expected_m=64) == \
        "persistent 128x256, masked, generic"
    assert name("dense", 16, 4096, 7168) == \
        "small-M split-K, 1 row tile(s), 7 K blocks per wave, specialised K7168"
    assert name("dense", 32, 4096, 7168).startswith("small-M split-K, 2 row tile(s)")
    try:
        fp8g.fp8g_set_shape_specialisation(False)
        assert name("dense", 4096, 8192, 8192).endswith("generic")
        assert name("dense", 16, 4096, 7168).endswith("generic")
    finally:
        fp8g.fp8g_set_shape_specialisation(True)
    assert name("dense", 4096, 8192, 8192).endswith("specialised N8192 K8192")
    f = lib.fp8g_gemm_kernel_name
    buf = ctypes.create_string_buffer(16)
    assert f(0, 4096, 8192, 8192, 1, 0, 0, None, 16) == STATUS["NULL"]
    assert f(0, 4096, 8192, 8192, 1, 0, 0, buf, 0) == STATUS["SHAPE"]
    assert f(4, 4096, 8192, 8192, 1, 0, 0, buf, 16) == STATUS["SHAPE"]
    assert f(0, -1, 8192, 8192, 1, 0, 0, buf, 16) == STATUS["SHAPE"]
    assert f(0, 16, 8192, 100, 1, 0, 0, buf, 16) == STATUS["SHAPE"]
    assert f(1, 16, 8192, 8192, 1, 0, 1, buf, 16) == STATUS["UNSUPPORTED"]
    assert f(0, 4096, 8192, 8192, 1, 0, 0, buf, 16) == STATUS["OK"]
    assert buf.value == b"persistent 256x"            # truncated like snprintf


def test_warmup_without_device(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present (covered by the GPU tests)")
    assert lib.fp8g_warmup() == STATUS["DEVICE"]


def test_python_binding_fails_loudly_without_library(tmp_path):
    saved = _lib._lib
    _lib._lib = None
    try:
        with pytest.raises(RuntimeError):
            _lib.load(str(tmp_path / "missing.so"))
    finally:
        _lib._lib = saved


def test_python_wrapper_rejects_mismatched_scales_and_dtypes():
    """The wrappers check shapes and element types before anything reaches
    the library (nxmr §5.1: per-row scales given for a 128x128 blocking is
    a named bug); CPU tensors are enough, the checks come first."""
    import torch
    import moe_grouped_gemm_quantizer_amd as fp8g
    M, N, K = 16, 256, 512
    a = torch.zeros((M, K), dtype=torch.uint8)
    b = torch.zeros((N, K), dtype=torch.uint8)
    sa = torch.zeros((K // 128, M), dtype=torch.float32)
    sb = torch.zeros((N // 128, K // 128), dtype=torch.float32)
    d = torch.zeros((M, N), dtype=torch.int16)
    with pytest.raises(ValueError, match="sb must be"):          # per-row scales for B
        fp8g.gemm_fp8_blockscaled(a, sa, b, torch.zeros((N, K // 128)), d)
    with pytest.raises(ValueError, match="sa must be"):          # transposed A scales
        fp8g.gemm_fp8_blockscaled(a, sa.t().contiguous(), b, sb, d)
    with pytest.raises(ValueError, match="float32"):
        fp8g.gemm_fp8_blockscaled(a, sa.double(), b, sb, d)
    with pytest.raises(ValueError, match="e4m3 codes"):
        fp8g.gemm_fp8_blockscaled(a.to(torch.int16), sa, b, sb, d)
    with pytest.raises(ValueError, match="bf16"):
        fp8g.gemm_fp8_blockscaled(a, sa, b, sb, d.float())
    G = 2
    bg = torch.zeros((G, N, K), dtype=torch.uint8)
    sbg = torch.zeros((G, N // 128, K // 128), dtype=torch.float32)
    offs = torch.tensor([0, 0, M], dtype=torch.int32)
    with pytest.raises(ValueError, match="int32"):
        fp8g.grouped_gemm_fp8_contiguous(a, sa, bg, sbg, d, offs.long())
    with pytest.raises(ValueError, match="sb must be"):
        fp8g.grouped_gemm_fp8_contiguous(a, sa, bg, sb, d, offs)
    am = torch.zeros((G, 8, K), dtype=torch.uint8)
    sam = torch.zeros((K // 128, G * 8), dtype=torch.float32)
    dm = torch.zeros((G, 8, N), dtype=torch.int16)
    with pytest.raises(ValueError, match="int32"):
        fp8g.grouped_gemm_fp8_masked(am, sam, bg, sbg, dm, torch.zeros(G, dtype=torch.int64))
    with pytest.raises(ValueError, match="sa must be"):
        fp8g.grouped_gemm_fp8_masked(am, sam[:, :8], bg, sbg, dm, torch.zeros(G, dtype=torch.int32))
