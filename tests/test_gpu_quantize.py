"""GPU quantiser parity: e4m3 codes and fp32 scales bit-exact against the oracle."""

import ctypes

import numpy as np
import pytest
import torch

import moe_grouped_gemm_quantizer_amd as fp8g
from oracle import quantize_blocks, e4m3_encode_rne, e4m3_decode_table
from workloads import make_config, make_dense
from tests import oracle_ops
from tests.gpu_util import quantize_a, quantize_b, to_dev, to_host, banner

pytestmark = pytest.mark.gpu


def _mismatch(got, ref, x=None):
    idx = np.argwhere(got != ref)[:8]
    items = []
    for i in idx:
        t = tuple(int(v) for v in i)
        xv = "" if x is None else f" x={x[t]!r}"
        items.append(f"{t}: got {int(got[t]):#04x} want {int(ref[t]):#04x}{xv}")
    return f"{int((got != ref).sum())} mismatches; " + "; ".join(items)


def _check_a(x, q, s):
    qo, so = quantize_blocks(x, 1)
    qg = to_host(q)
    assert np.array_equal(qg, qo), _mismatch(qg, qo, x)
    assert np.array_equal(to_host(s).view(np.uint32), so.T.copy().view(np.uint32))


def _check_b_rows(x, q, s, block_rows_idx):
    """Compare the given 128-row block rows of a B quantisation."""
    qh, sh = to_host(q), to_host(s)
    for rb in block_rows_idx:
        r0 = rb * 128
        qo, so = quantize_blocks(x[r0:r0 + 128], 128)
        assert np.array_equal(qh[r0:r0 + 128], qo), rb
        assert np.array_equal(sh[rb].view(np.uint32), so[0].view(np.uint32)), rb


@pytest.mark.parametrize("cfg", [0, 1])
def test_small_configs_bit_exact(cfg):
    w = make_config(cfg)
    banner(f"quantize cfg{cfg} A{w.a.shape} B{w.b.shape}")
    q, s = quantize_a(w.a)
    _check_a(w.a, q, s)
    q, s = quantize_b(w.b)
    _check_b_rows(w.b, q, s, range(w.b.shape[0] // 128))


def _check_full(cfg):
    """GPU 1x128 quantisation of the whole A and 128x128 quantisation of the
    whole B (experts stacked) of workload cfg, every code and scale compared
    with the oracle's bit for bit."""
    w = oracle_ops.workload(cfg)
    K = w.K
    qa, sa, qb, sb = oracle_ops.operands(cfg)
    a2 = w.a.reshape(-1, K)
    banner(f"quantize cfg{cfg} A{a2.shape} and B{w.b.reshape(-1, K).shape}: every block")
    q, s = quantize_a(a2)
    qh = to_host(q)
    assert np.array_equal(qh, qa), _mismatch(qh, qa, a2)
    assert np.array_equal(to_host(s).view(np.uint32), np.ascontiguousarray(sa.T).view(np.uint32))
    del q, s
    b2 = torch.from_numpy(w.b.reshape(-1, K)).to("cuda")
    q, s = quantize_b(b2)
    del b2
    qh = to_host(q)
    assert np.array_equal(qh, qb), _mismatch(qh, qb)
    assert np.array_equal(to_host(s).view(np.uint32), sb.view(np.uint32))
    del q, s
    torch.cuda.empty_cache()


def test_dense_large_bit_exact():
    _check_full(2)


@pytest.mark.parametrize("cfg", [3, 4])
def test_moe_configs_bit_exact(cfg):
    _check_full(cfg)


def test_encoder_on_arbitrary_fp32_patterns():
    """A block whose amax is exactly 448 has scale 1.0, so the codes are the
    RNE encoding of the raw values: exercise every e4m3 midpoint
    neighbourhood and random fp32 patterns through the GPU kernel."""
    t = e4m3_decode_table()
    pos = t[0:0x7F]
    mids = np.concatenate([(pos[:-1] + pos[1:]) / 2, pos])
    bits = mids.astype(np.float32).view(np.int32).astype(np.int64)
    off = np.arange(-512, 512, dtype=np.int64)
    cand = (bits[:, None] + off[None, :]).ravel()
    cand = cand[(cand >= 0) & (cand <= np.float32(448.0).view(np.int32))]
    vals = cand.astype(np.int32).view(np.float32)
    rng = np.random.default_rng(77)
    rnd = rng.integers(0, int(np.float32(448.0).view(np.int32)) + 1, 4_000_000).astype(np.int32)
    vals = np.concatenate([vals, -vals, rnd.view(np.float32), -rnd.view(np.float32)])
    n = -(-vals.size // 127)
    x = np.zeros((n, 128), np.float32)
    x[:, 0] = 448.0                        # amax 448 -> s = 1
    flat = np.zeros(n * 127, np.float32)
    flat[:vals.size] = vals
    x[:, 1:] = flat.reshape(n, 127)
    q, s = quantize_a(x)
    assert np.all(to_host(s) == 1.0)
    got = to_host(q)[:, 1:].reshape(-1)[:vals.size]
    assert np.array_equal(got, e4m3_encode_rne(vals))


def _codes_through_kernel(vals):
    """Encode raw fp32 values through the 1x128 kernel: each row holds 448
    (so its scale is exactly 1.0) and 127 of the values."""
    n = -(-vals.size // 127)
    x = np.zeros((n, 128), np.float32)
    x[:, 0] = 448.0
    flat = np.zeros(n * 127, np.float32)
    flat[:vals.size] = vals
    x[:, 1:] = flat.reshape(n, 127)
    q, s = quantize_a(x)
    assert np.all(to_host(s) == 1.0)
    return to_host(q)[:, 1:].reshape(-1)[:vals.size]


def test_encoder_exhaustive_subnormal_range_and_top_binade():
    """Every fp32 value in [2^-12, 2^-5] (the e4m3 subnormal grid and the
    first normal binades, where the rounding grid changes) and in [256, 448]
    (the top binade up to the largest code), through the kernel."""
    for lo, hi in ((2.0 ** -12, 2.0 ** -5), (256.0, 448.0)):
        b0 = int(np.float32(lo).view(np.uint32))
        b1 = int(np.float32(hi).view(np.uint32))
        banner(f"exhaustive encode [{lo}, {hi}]: {b1 - b0 + 1} values")
        vals = np.arange(b0, b1 + 1, dtype=np.uint32).view(np.float32)
        got = _codes_through_kernel(vals)
        assert np.array_equal(got, e4m3_encode_rne(vals))
        got = _codes_through_kernel(-vals[::97])
        assert np.array_equal(got, e4m3_encode_rne(-vals[::97]))


def test_encoder_fp32_denormals_and_zeros():
    vals = np.concatenate([np.arange(0, 1 << 20, 7, dtype=np.uint32),
                           np.array([0, 1, 2, 0x7FFFFF], np.uint32)]).view(np.float32)
    vals = np.concatenate([vals, -vals])
    got = _codes_through_kernel(vals)
    assert np.array_equal(got, e4m3_encode_rne(vals))     # all signed zeros


def test_edge_blocks():
    x = np.zeros((19, 384), np.float32)
    x[1] = -0.0
    x[2, :128] = np.float32(1e-45) * np.arange(128, dtype=np.float32)
    x[2, 128:] = np.float32(-3e-40)
    x[3, :5] = [np.nan, 1.0, -2.0, -np.nan, 0.5]
    x[4, 128:256] = np.nan
    x[5, :3] = [np.inf, -np.inf, 7.0]
    x[6, 256:] = np.float32(2.0 ** -130)                          # subnormal, all equal
    x[7] = np.linspace(-1e-3, 1e-3, 384, dtype=np.float32)
    rng = np.random.default_rng(3)
    x[8:] = rng.standard_normal((11, 384)).astype(np.float32) * np.float32(1e30)
    banner("quantize edge blocks 1x128 and 128x128 with 19 ragged rows")
    q, s = quantize_a(x)
    _check_a(x, q, s)
    # 128x128 with a partial last block row: rows = 19
    q, s = quantize_b(x)
    qo, so = quantize_blocks(x, 128)
    qg = to_host(q)
    assert np.array_equal(qg, qo), _mismatch(qg, qo, x)
    assert np.array_equal(to_host(s).view(np.uint32), so.view(np.uint32))


def test_ragged_rows_many_blocks():
    w = make_dense(1000, 300 + 84, 640, seed=31)      # rows not a multiple of 8 or 128
    banner("quantize 1000x640 and 384x640 ragged")
    q, s = quantize_a(w.a)
    _check_a(w.a, q, s)
    q, s = quantize_b(w.b)
    qo, so = quantize_blocks(w.b, 128)
    assert np.array_equal(to_host(q), qo)
    assert np.array_equal(to_host(s).view(np.uint32), so.view(np.uint32))


def test_power_of_two_invariance_gpu():
    w = make_config(0)
    q0, s0 = quantize_a(w.a)
    q1, s1 = quantize_a(w.a * np.float32(2.0 ** -9))
    assert torch.equal(q0, q1)
    assert torch.equal(s1, s0 * 2.0 ** -9)


def _near_midpoint_blocks(n_blocks, rng):
    """n_blocks blocks of 128 values: element 0 is the block amax (scales
    spread over ~1e-30 .. 1e35, inside and outside [2^-80, 2^100]); the rest
    sit within a few fp32 ulps of fl32(m * s) for e4m3 values and midpoints m,
    both signs, plus signed zeros: quotients that land next to rounding
    boundaries, so that an inexact quotient would change a code."""
    t = e4m3_decode_table()
    pos = t[0:0x7F].astype(np.float64)
    grid = np.concatenate([(pos[:-1] + pos[1:]) / 2, pos[1:]])       # midpoints and values
    exps = rng.uniform(-30, 35, n_blocks)
    amax = (10.0 ** exps * rng.uniform(1.0, 9.99, n_blocks)).astype(np.float32)
    s = amax / np.float32(448.0)                                       # IEEE fp32, as the method
    m = rng.choice(grid, (n_blocks, 127))
    base = (m * s[:, None].astype(np.float64)).astype(np.float32)
    bits = base.view(np.int32).astype(np.int64) + rng.integers(-3, 4, (n_blocks, 127))
    x = bits.astype(np.int32).view(np.float32)
    x = np.where(rng.random((n_blocks, 127)) < 0.5, -x, x)
    x[:, :2] = [np.float32(-0.0), np.float32(0.0)]
    x = np.clip(x, -amax[:, None], amax[:, None])                      # keep amax the block max
    return np.concatenate([amax[:, None], x], axis=1).astype(np.float32)


def test_quotient_near_rounding_boundaries():
    """Bit-exact codes for quotients next to e4m3 rounding boundaries under
    arbitrary (non power of two) scales, through both kernels."""
    rng = np.random.default_rng(2024)
    a = _near_midpoint_blocks(8192, rng)                # 8192 rows of one 1x128 block
    banner("quantize 8192 near-boundary 1x128 blocks")
    q, s = quantize_a(a)
    _check_a(a, q, s)
    # 128x128: 48 blocks (384 x 2048); each block's rows come from 128
    # near-boundary rows sharing one scale (rescaled to that block's amax)
    nb_r, nb_c = 3, 16
    b = np.zeros((nb_r * 128, nb_c * 128), np.float32)
    for i in range(nb_r):
        for j in range(nb_c):
            blk = _near_midpoint_blocks(128, rng)
            amax = blk[0, 0]
            sc = amax / np.float32(448.0)
            # every row: the block's own scale, so re-derive the values from row 0's amax
            m = blk[:, 1:].astype(np.float64) / (blk[:, :1].astype(np.float64) / 448.0)
            vals = (m * np.float64(sc)).astype(np.float32)
            vals = np.clip(vals, -amax, amax)
            blk = np.concatenate([np.full((128, 1), amax, np.float32), vals], axis=1)
            b[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128] = blk
    banner("quantize 48 near-boundary 128x128 blocks")
    q, s = quantize_b(b)
    qo, so = quantize_blocks(b, 128)
    qg = to_host(q)
    assert np.array_equal(qg, qo), _mismatch(qg, qo, b)
    assert np.array_equal(to_host(s).view(np.uint32), so.view(np.uint32))


def _bf16_case(x_bf16, block_rows):
    """Quantise a bfloat16 tensor on the GPU; check against the oracle on the
    inputs' exact float32 values (every bf16 value is an fp32 value)."""
    rows, cols = x_bf16.shape
    x32 = x_bf16.float().numpy()
    xd = x_bf16.cuda()
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    if block_rows == 1:
        s = torch.empty((cols // 128, rows), dtype=torch.float32, device="cuda")
        fp8g.fp8_quantize_bf16(xd, 1, q, s, 1, rows)
        qo, so = quantize_blocks(x32, 1)
        so = so.T.copy()
    else:
        s = torch.empty((-(-rows // 128), cols // 128), dtype=torch.float32, device="cuda")
        fp8g.fp8_quantize_bf16(xd, 128, q, s, cols // 128, 1)
        qo, so = quantize_blocks(x32, 128)
    qg = to_host(q)
    assert np.array_equal(qg, qo), _mismatch(qg, qo, x32)
    assert np.array_equal(to_host(s).view(np.uint32), so.view(np.uint32))


@pytest.mark.parametrize("block_rows", [1, 128])
@pytest.mark.parametrize("rows,cols", [(300, 512), (128, 7168), (1, 128)])
def test_bf16_input_bit_exact(block_rows, rows, cols):
    """fp8_quantize_bf16 equals the fp32 quantiser on the widened values:
    generator data with outlier columns, rounded to bf16 (ragged row blocks)."""
    banner(f"quantize bf16 {rows}x{cols} block_rows={block_rows}")
    w = make_dense(rows, 128, cols, seed=rows + cols)
    _bf16_case(torch.from_numpy(w.a).to(torch.bfloat16), block_rows)


@pytest.mark.parametrize("block_rows", [1, 128])
@pytest.mark.parametrize("view", ["offset", "stride"])
def test_bf16_input_unaligned_views(block_rows, view):
    """bf16 inputs the 16-byte-load kernels cannot take (x only 8-byte
    aligned, or a row stride that is not a multiple of 8 elements) go to the
    four-value kernels; the result is the same, bit for bit with the oracle."""
    rows, cols = 300, 512
    banner(f"quantize bf16 {view} view {rows}x{cols} block_rows={block_rows}")
    w = make_dense(rows, 128, cols, seed=77)
    xb = torch.from_numpy(w.a).to(torch.bfloat16)
    if view == "offset":
        # contiguous, but 8 bytes past a 16-byte boundary
        buf = torch.zeros(rows * cols + 4, dtype=torch.bfloat16, device="cuda")
        x = buf[4:].view(rows, cols)
        ldx = cols
    else:
        # 16-byte aligned rows of cols + 4 elements (through the C ABI: the
        # Python binding takes contiguous tensors)
        buf = torch.zeros((rows, cols + 4), dtype=torch.bfloat16, device="cuda")
        x = buf[:, :cols]
        ldx = cols + 4
    x.copy_(xb.cuda())
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    if block_rows == 1:
        s = torch.empty((cols // 128, rows), dtype=torch.float32, device="cuda")
        ssr, ssc = 1, rows
        qo, so = quantize_blocks(xb.float().numpy(), 1)
        so = so.T.copy()
    else:
        s = torch.empty((-(-rows // 128), cols // 128), dtype=torch.float32, device="cuda")
        ssr, ssc = cols // 128, 1
        qo, so = quantize_blocks(xb.float().numpy(), 128)
    lib = fp8g._lib.load()
    st = lib.fp8_quantize_bf16(ctypes.c_void_p(x.data_ptr()), rows, cols, ldx, block_rows,
                               ctypes.c_void_p(q.data_ptr()), cols, ctypes.c_void_p(s.data_ptr()),
                               ssr, ssc, None)
    assert st == 0
    torch.cuda.synchronize()
    assert np.array_equal(to_host(q), qo)
    assert np.array_equal(to_host(s).view(np.uint32), so.view(np.uint32))


@pytest.mark.parametrize("block_rows", [1, 128])
def test_bf16_input_every_pattern(block_rows):
    """All 65536 bf16 bit patterns (NaNs, infinities, subnormals, signed
    zeros), shuffled into 128-wide blocks."""
    banner(f"quantize bf16 every pattern block_rows={block_rows}")
    bits = np.random.default_rng(11).permutation(np.arange(65536, dtype=np.uint32)).astype(np.uint16)
    x = torch.from_numpy(bits.view(np.int16).reshape(256, 256)).view(torch.bfloat16)
    _bf16_case(x, block_rows)


@pytest.mark.parametrize("block_rows", [1, 128])
def test_signalling_nans_after_large_values(block_rows):
    """fp32 blocks whose largest |x| comes before a signalling (or quiet) NaN
    in every lane's order: the amax must still be the largest non-NaN |x|."""
    banner(f"quantize fp32 signalling NaNs block_rows={block_rows}")
    rng = np.random.default_rng(31)
    x = (rng.standard_normal((256, 512)) * 1e20).astype(np.float32)
    xb = x.view(np.uint32)
    for r in range(0, 256, 3):
        c0 = int(rng.integers(0, 4)) * 128
        big = c0 + int(rng.integers(0, 64))
        xb[r, big] = np.float32(3.0e37).view(np.uint32)
        for pos in (big + 1, big + 4, c0 + 127):
            xb[r, pos] = [0x7FBD0000, 0xFF800001, 0x7FC00000][pos % 3]
    x = xb.view(np.float32)
    xd = torch.from_numpy(x).cuda()
    q = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
    if block_rows == 1:
        s = torch.empty((4, 256), dtype=torch.float32, device="cuda")
        fp8g.fp8_quantize(xd, 1, q, s, 1, 256)
        qo, so = quantize_blocks(x, 1)
        so = so.T.copy()
    else:
        s = torch.empty((2, 4), dtype=torch.float32, device="cuda")
        fp8g.fp8_quantize(xd, 128, q, s, 4, 1)
        qo, so = quantize_blocks(x, 128)
    qg = to_host(q)
    assert np.array_equal(qg, qo), _mismatch(qg, qo, x)
    assert np.array_equal(to_host(s).view(np.uint32), so.view(np.uint32))
