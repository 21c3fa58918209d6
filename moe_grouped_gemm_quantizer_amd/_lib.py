"""ctypes binding of libfp8gemm.so (argument marshalling only).

Each function has the name of the C entry point it calls, takes torch tensors
that already live on the current GPU, passes their device pointers, sizes and
the current torch stream, and raises on a non-zero status. No arithmetic of the
method happens here, and there is no fallback: if the library cannot be
loaded, every call raises.
"""

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libfp8gemm.so")

ENTRY_POINTS = ("fp8_quantize", "fp8_quantize_bf16", "fp8_quantize_tensor", "gemm_fp8_blockscaled",
                "gemm_fp8_pertensor", "gemm_fp8_pertensor_fmt", "fp8_quantize_delayed",
                "gemm_fp8_blockscaled_quant",
                "grouped_gemm_fp8_contiguous", "grouped_gemm_fp8_contiguous_workspace_size",
                "grouped_gemm_fp8_contiguous_ws", "grouped_gemm_fp8_contiguous_noalloc",
                "grouped_gemm_fp8_masked", "fp8g_clock_probe", "fp8g_warmup",
                "fp8g_set_shape_specialisation", "fp8g_gemm_kernel_name",
                "fp8g_status_string", "fp8g_abi_version")

_c_i64 = ctypes.c_int64
_c_int = ctypes.c_int
_c_vp = ctypes.c_void_p
_c_sz = ctypes.c_size_t

_SIGS = {
    "fp8_quantize": [_c_vp, _c_i64, _c_i64, _c_i64, _c_int, _c_vp, _c_i64, _c_vp, _c_i64, _c_i64, _c_vp],
    "fp8_quantize_bf16": [_c_vp, _c_i64, _c_i64, _c_i64, _c_int, _c_vp, _c_i64, _c_vp, _c_i64, _c_i64,
                          _c_vp],
    "fp8_quantize_tensor": [_c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_i64, _c_vp, _c_vp],
    "gemm_fp8_blockscaled": [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_vp],
    "gemm_fp8_pertensor": [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_vp],
    "gemm_fp8_pertensor_fmt": [_c_vp, _c_int, _c_vp, _c_vp, _c_int, _c_vp, _c_vp, _c_i64, _c_i64,
                               _c_i64, _c_vp],
    "fp8_quantize_delayed": [_c_vp, _c_i64, _c_i64, _c_i64, _c_int, _c_vp, _c_int, _c_int, _c_vp,
                             _c_i64, _c_vp, _c_vp],
    "gemm_fp8_blockscaled_quant": [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64,
                                   _c_i64, _c_vp],
    "grouped_gemm_fp8_contiguous": [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_int, _c_i64,
                                    _c_i64, _c_i64, _c_vp],
    "grouped_gemm_fp8_contiguous_workspace_size": [_c_int, _c_i64, _c_i64, _c_i64,
                                                   ctypes.POINTER(_c_sz)],
    "grouped_gemm_fp8_contiguous_ws": [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_int, _c_i64,
                                       _c_i64, _c_i64, _c_vp, _c_sz, _c_vp],
    "grouped_gemm_fp8_contiguous_noalloc": [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_int,
                                            _c_i64, _c_i64, _c_i64, _c_vp],
    "grouped_gemm_fp8_masked": [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_int, _c_i64,
                                _c_i64, _c_i64, _c_int, _c_vp],
    "fp8g_clock_probe": [_c_vp, _c_int, _c_vp],
    "fp8g_warmup": [],
    "fp8g_set_shape_specialisation": [_c_int],
    "fp8g_gemm_kernel_name": [_c_int, _c_i64, _c_i64, _c_i64, _c_int, _c_int, _c_int,
                              ctypes.c_char_p, _c_sz],
}

LAYOUTS = {"dense": 0, "contiguous": 1, "masked": 2, "pertensor": 3}
FORMATS = {"e4m3": 0, "e5m2": 1}

_lib = None


class Fp8GemmError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: status {status} ({status_string(status)})")


def load(path=LIB_PATH):
    """Load the shared library (once) and declare every entry point."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m moe_grouped_gemm_quantizer_amd.build`")
    lib = ctypes.CDLL(path)
    for name, args in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.fp8g_status_string.argtypes = [ctypes.c_int]
    lib.fp8g_status_string.restype = ctypes.c_char_p
    lib.fp8g_abi_version.argtypes = []
    lib.fp8g_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status):
    return load().fp8g_status_string(int(status)).decode()


def fp8g_abi_version():
    return load().fp8g_abi_version()


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _nb(n):
    """128-wide blocks covering n (the last may be partial)."""
    return -(-int(n) // 128)


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _check(status, what):
    if status != 0:
        raise Fp8GemmError(status, what)


def _dev(*ts):
    for t in ts:
        _need(t.is_cuda, "tensors must live on the GPU")
        _need(t.is_contiguous(), "tensors must be contiguous")


def _gemm_dtypes(a, sa, b, sb, d, meta=None):
    """The C calls read raw bytes: a wrong element type would be misread, not
    converted, so it is refused here."""
    import torch
    codes = (torch.uint8, torch.float8_e4m3fn)
    _need(a.dtype in codes and b.dtype in codes, "a and b must be e4m3 codes (uint8 or float8_e4m3fn)")
    _need(sa.dtype == torch.float32 and sb.dtype == torch.float32, "sa and sb must be float32")
    _need(d.dtype in (torch.int16, torch.bfloat16, torch.uint16),
          "d must hold bf16 values (bfloat16, or int16/uint16 bit patterns)")
    if meta is not None:
        _need(meta.dtype == torch.int32, "group metadata must be int32")


def fp8_quantize(x, block_rows, q, scales, s_stride_row, s_stride_col, stream=None):
    """x float32 [rows][cols] -> q uint8 [rows][cols], scales float32 (strided).

    block_rows 1: A operand, call with s_stride_row=1, s_stride_col=rows.
    block_rows 128: B operand, s_stride_row=cols//128, s_stride_col=1.
    """
    import torch
    _need(x.dim() == 2 and q.dim() == 2 and x.shape == q.shape, "x and q must be same-shape 2-D")
    _need(x.dtype == torch.float32 and q.dtype == torch.uint8 and scales.dtype == torch.float32,
          "x float32, q uint8, scales float32")
    _dev(x, q, scales)
    rows, cols = x.shape
    nrb = -(-rows // block_rows)
    ncb = -(-cols // 128)
    if rows and cols:
        need = (nrb - 1) * s_stride_row + (ncb - 1) * s_stride_col + 1
        _need(scales.numel() >= need, "scales tensor too small for the blocking")
    st = load().fp8_quantize(_ptr(x), rows, cols, cols, int(block_rows), _ptr(q), cols,
                             _ptr(scales), int(s_stride_row), int(s_stride_col), _stream(stream))
    _check(st, "fp8_quantize")


def fp8_quantize_bf16(x, block_rows, q, scales, s_stride_row, s_stride_col, stream=None):
    """x bfloat16 (or int16 bit patterns) [rows][cols] -> q uint8, scales float32;
    arguments and result as for fp8_quantize on x's exact float32 values."""
    import torch
    _need(x.dim() == 2 and q.dim() == 2 and x.shape == q.shape, "x and q must be same-shape 2-D")
    _need(x.dtype in (torch.bfloat16, torch.int16) and q.dtype == torch.uint8
          and scales.dtype == torch.float32, "x bfloat16, q uint8, scales float32")
    _dev(x, q, scales)
    rows, cols = x.shape
    nrb = -(-rows // block_rows)
    ncb = -(-cols // 128)
    if rows and cols:
        need = (nrb - 1) * s_stride_row + (ncb - 1) * s_stride_col + 1
        _need(scales.numel() >= need, "scales tensor too small for the blocking")
    st = load().fp8_quantize_bf16(_ptr(x), rows, cols, cols, int(block_rows), _ptr(q), cols,
                                  _ptr(scales), int(s_stride_row), int(s_stride_col),
                                  _stream(stream))
    _check(st, "fp8_quantize_bf16")


def gemm_fp8_blockscaled_quant(a, sa, b, sb, d, qd, sd, stream=None):
    """gemm_fp8_blockscaled with the result also quantised 1x128 for the next
    GEMM: qd uint8 [M][N] codes, sd float32 [N/128][M] scales; d bf16 [M][N]
    or None."""
    import torch
    M, K = a.shape
    N = b.shape[0]
    _need(b.shape[1] == K, "a and b disagree on K")
    _need(tuple(sa.shape) == (_nb(K), M), "sa must be [ceil(K/128)][M] (1x128 per-token scales)")
    _need(tuple(sb.shape) == (_nb(N), _nb(K)), "sb must be [ceil(N/128)][ceil(K/128)] (128x128 block scales)")
    _need(tuple(qd.shape) == (M, N) and qd.dtype == torch.uint8, "qd must be uint8 [M][N]")
    _need(tuple(sd.shape) == (_nb(N), M) and sd.dtype == torch.float32, "sd must be float32 [ceil(N/128)][M]")
    dd = d if d is not None else torch.empty(0, dtype=torch.int16)
    _gemm_dtypes(a, sa, b, sb, dd)
    if d is not None:
        _need(tuple(d.shape) == (M, N), "d must be [M][N]")
        _dev(d)
    _dev(a, sa, b, sb, qd, sd)
    st = load().gemm_fp8_blockscaled_quant(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(d), _ptr(qd),
                                           _ptr(sd), M, N, K, _stream(stream))
    _check(st, "gemm_fp8_blockscaled_quant")


def fp8_quantize_tensor(x, q, scale, stream=None):
    """x float32 [rows][cols] -> q uint8 [rows][cols] with one scale: scale
    is a float32 device tensor of one element (receives amax / 448)."""
    import torch
    _need(x.dim() == 2 and q.dim() == 2 and x.shape == q.shape, "x and q must be same-shape 2-D")
    _need(x.dtype == torch.float32 and q.dtype == torch.uint8 and scale.dtype == torch.float32
          and scale.numel() == 1, "x float32, q uint8, scale float32 [1]")
    _dev(x, q, scale)
    rows, cols = x.shape
    st = load().fp8_quantize_tensor(_ptr(x), rows, cols, cols, _ptr(q), cols, _ptr(scale),
                                    _stream(stream))
    _check(st, "fp8_quantize_tensor")


def gemm_fp8_pertensor(a, scale_a, b, scale_b, d, stream=None):
    """a uint8 [M][K], scale_a float32 [1], b uint8 [N][K], scale_b float32 [1],
    d bf16 (int16/bfloat16) [M][N]."""
    import torch
    M, K = a.shape
    N = b.shape[0]
    _need(b.shape[1] == K, "a and b disagree on K")
    _need(scale_a.numel() == 1 and scale_b.numel() == 1, "per-tensor scales are one float each")
    _need(tuple(d.shape) == (M, N), "d must be [M][N]")
    _gemm_dtypes(a, scale_a, b, scale_b, d)
    _dev(a, scale_a, b, scale_b, d)
    st = load().gemm_fp8_pertensor(_ptr(a), _ptr(scale_a), _ptr(b), _ptr(scale_b), _ptr(d), M, N,
                                   K, _stream(stream))
    _check(st, "gemm_fp8_pertensor")


def _fmt(name):
    _need(name in FORMATS, f"format must be one of {sorted(FORMATS)}")
    return FORMATS[name]


def _codes_dtype_ok(t, fmt):
    import torch
    ok = (torch.uint8, torch.float8_e4m3fn) if fmt == "e4m3" else (torch.uint8, torch.float8_e5m2)
    return t.dtype in ok


def gemm_fp8_pertensor_fmt(a, fmt_a, scale_a, b, fmt_b, scale_b, d, stream=None):
    """gemm_fp8_pertensor with each operand's format: fmt_a, fmt_b 'e4m3' or
    'e5m2' (codes as uint8, or torch's float8 dtype of that format)."""
    import torch
    fa, fb = _fmt(fmt_a), _fmt(fmt_b)
    M, K = a.shape
    N = b.shape[0]
    _need(b.shape[1] == K, "a and b disagree on K")
    _need(scale_a.numel() == 1 and scale_b.numel() == 1, "per-tensor scales are one float each")
    _need(tuple(d.shape) == (M, N), "d must be [M][N]")
    _need(_codes_dtype_ok(a, fmt_a) and _codes_dtype_ok(b, fmt_b),
          "a and b must be codes of their formats (uint8 or the matching float8 dtype)")
    _need(scale_a.dtype == torch.float32 and scale_b.dtype == torch.float32,
          "scales must be float32")
    _need(d.dtype in (torch.int16, torch.bfloat16, torch.uint16),
          "d must hold bf16 values (bfloat16, or int16/uint16 bit patterns)")
    _dev(a, scale_a, b, scale_b, d)
    st = load().gemm_fp8_pertensor_fmt(_ptr(a), fa, _ptr(scale_a), _ptr(b), fb, _ptr(scale_b),
                                       _ptr(d), M, N, K, _stream(stream))
    _check(st, "gemm_fp8_pertensor_fmt")


def fp8_quantize_delayed(x, fmt, amax_history, slot, q, scale, stream=None):
    """One delayed-scaling step: x float32 [rows][cols] -> q uint8 codes in
    fmt ('e4m3' or 'e5m2') under the scale taken from amax_history (float32
    device tensor, read and written; entry `slot` receives this step's amax);
    scale: float32 device tensor of one element (receives the scale used)."""
    import torch
    f = _fmt(fmt)
    _need(x.dim() == 2 and q.dim() == 2 and x.shape == q.shape, "x and q must be same-shape 2-D")
    _need(x.dtype == torch.float32 and q.dtype == torch.uint8 and scale.dtype == torch.float32
          and scale.numel() == 1 and amax_history.dtype == torch.float32
          and amax_history.dim() == 1, "x float32, q uint8, scale float32 [1], history float32 [H]")
    _dev(x, q, scale, amax_history)
    rows, cols = x.shape
    st = load().fp8_quantize_delayed(_ptr(x), rows, cols, cols, f, _ptr(amax_history),
                                     amax_history.numel(), int(slot), _ptr(q), cols, _ptr(scale),
                                     _stream(stream))
    _check(st, "fp8_quantize_delayed")


def gemm_fp8_blockscaled(a, sa, b, sb, d, stream=None):
    """a uint8 [M][K], sa float32 [K/128][M], b uint8 [N][K], sb float32
    [N/128][K/128], d bf16 (int16/bfloat16) [M][N]."""
    M, K = a.shape
    N = b.shape[0]
    _need(b.shape[1] == K, "a and b disagree on K")
    _need(tuple(sa.shape) == (_nb(K), M), "sa must be [ceil(K/128)][M] (1x128 per-token scales)")
    _need(tuple(sb.shape) == (_nb(N), _nb(K)), "sb must be [ceil(N/128)][ceil(K/128)] (128x128 block scales)")
    _need(tuple(d.shape) == (M, N), "d must be [M][N]")
    _gemm_dtypes(a, sa, b, sb, d)
    _dev(a, sa, b, sb, d)
    st = load().gemm_fp8_blockscaled(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(d), M, N, K,
                                     _stream(stream))
    _check(st, "gemm_fp8_blockscaled")


def _contiguous_args(a, sa, b, sb, d, group_offsets):
    M, K = a.shape
    G, N, K2 = b.shape
    _need(K2 == K, "a and b disagree on K")
    _need(tuple(sa.shape) == (_nb(K), M), "sa must be [ceil(K/128)][M_total]")
    _need(tuple(sb.shape) == (G, _nb(N), _nb(K)), "sb must be [G][ceil(N/128)][ceil(K/128)]")
    _need(tuple(d.shape) == (M, N), "d must be [M_total][N]")
    _need(group_offsets.numel() == G + 1, "group_offsets must be int32 [G+1]")
    _gemm_dtypes(a, sa, b, sb, d, group_offsets)
    _dev(a, sa, b, sb, d, group_offsets)
    return (_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(d), _ptr(group_offsets), G, M, N, K)


def grouped_gemm_fp8_contiguous(a, sa, b, sb, d, group_offsets, stream=None):
    """a uint8 [M_total][K], sa [K/128][M_total], b uint8 [G][N][K],
    sb [G][N/128][K/128], d [M_total][N], group_offsets int32 [G+1] (device)."""
    st = load().grouped_gemm_fp8_contiguous(*_contiguous_args(a, sa, b, sb, d, group_offsets),
                                            _stream(stream))
    _check(st, "grouped_gemm_fp8_contiguous")


def grouped_gemm_fp8_contiguous_workspace_size(G, M_total, N, K):
    """Bytes of workspace grouped_gemm_fp8_contiguous_ws can use (0: none)."""
    out = ctypes.c_size_t(0)
    st = load().grouped_gemm_fp8_contiguous_workspace_size(int(G), int(M_total), int(N), int(K),
                                                           ctypes.byref(out))
    _check(st, "grouped_gemm_fp8_contiguous_workspace_size")
    return int(out.value)


def grouped_gemm_fp8_contiguous_ws(a, sa, b, sb, d, group_offsets, workspace, stream=None):
    """grouped_gemm_fp8_contiguous with a caller-owned workspace (a contiguous
    device tensor of at least grouped_gemm_fp8_contiguous_workspace_size
    bytes, or None)."""
    if workspace is None:
        wp, wb = None, 0
    else:
        _dev(workspace)
        wp, wb = _ptr(workspace), workspace.numel() * workspace.element_size()
    st = load().grouped_gemm_fp8_contiguous_ws(*_contiguous_args(a, sa, b, sb, d, group_offsets),
                                               wp, wb, _stream(stream))
    _check(st, "grouped_gemm_fp8_contiguous_ws")


def grouped_gemm_fp8_contiguous_noalloc(a, sa, b, sb, d, group_offsets, stream=None):
    """grouped_gemm_fp8_contiguous_ws with the library's fixed scratch array
    as the workspace (no allocation; calls on one GPU must not overlap)."""
    st = load().grouped_gemm_fp8_contiguous_noalloc(
        *_contiguous_args(a, sa, b, sb, d, group_offsets), _stream(stream))
    _check(st, "grouped_gemm_fp8_contiguous_noalloc")


def grouped_gemm_fp8_masked(a, sa, b, sb, d, masked_m, expected_m=0, stream=None):
    """a uint8 [G][max_m][K], sa [K/128][G*max_m], b uint8 [G][N][K],
    sb [G][N/128][K/128], d [G][max_m][N], masked_m int32 [G] (device)."""
    import torch
    G, max_m, K = a.shape
    G2, N, K2 = b.shape
    _need(G2 == G and K2 == K, "a and b disagree on G or K")
    _need(tuple(sa.shape) == (_nb(K), G * max_m), "sa must be [ceil(K/128)][G*max_m]")
    _need(tuple(sb.shape) == (G, _nb(N), _nb(K)), "sb must be [G][ceil(N/128)][ceil(K/128)]")
    _need(tuple(d.shape) == (G, max_m, N), "d must be [G][max_m][N]")
    _need(masked_m.numel() == G, "masked_m must be int32 [G]")
    _gemm_dtypes(a, sa, b, sb, d, masked_m)
    _dev(a, sa, b, sb, d, masked_m)
    st = load().grouped_gemm_fp8_masked(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(d),
                                        _ptr(masked_m), G, max_m, N, K, int(expected_m),
                                        _stream(stream))
    _check(st, "grouped_gemm_fp8_masked")


def fp8g_clock_probe(out, ticks=2000, stream=None):
    """Enqueue the clock probe: out is a device int64 tensor of >= 2 elements;
    afterwards out[0] / out[1] * 1e8 is the shader clock in Hz."""
    import torch
    _need(out.dtype == torch.int64 and out.numel() >= 2, "out must be int64 with 2 elements")
    _dev(out)
    _check(load().fp8g_clock_probe(_ptr(out), int(ticks), _stream(stream)), "fp8g_clock_probe")


def fp8g_warmup():
    """Load every kernel's code object onto the current device (host-side,
    synchronous; launches and allocates nothing)."""
    _check(load().fp8g_warmup(), "fp8g_warmup")


def fp8g_set_shape_specialisation(enable):
    """Switch the shape-specialised kernels on (default) or off process-wide;
    results are bit-identical either way."""
    _check(load().fp8g_set_shape_specialisation(1 if enable else 0),
           "fp8g_set_shape_specialisation")


def fp8g_gemm_kernel_name(layout, rows, N, K, G=1, expected_m=0, quant=False):
    """The kernel a GEMM call of this shape launches. layout: 'dense',
    'contiguous', 'masked' or 'pertensor'; rows: M, M_total or max_m."""
    _need(layout in LAYOUTS, f"layout must be one of {sorted(LAYOUTS)}")
    buf = ctypes.create_string_buffer(256)
    _check(load().fp8g_gemm_kernel_name(LAYOUTS[layout], int(rows), int(N), int(K), int(G),
                                        int(expected_m), 1 if quant else 0, buf, len(buf)),
           "fp8g_gemm_kernel_name")
    return buf.value.decode()
