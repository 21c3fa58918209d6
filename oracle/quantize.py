"""Block quantisation to e4m3 with one fp32 scale per block (test infrastructure).

The method, as the pages state it:

* nxmr §3.1: cut the matrix into blocks, take each block's largest absolute
  value amax, set the block's scale to amax divided by the largest FP8 value;
  quantising divides each element by the scale, dequantising multiplies back.
* czchanglian §5.2: the e4m3 limit is about 448, so the scale starts as
  max_val / 448, computed independently for every tensor (here: block).
* czchanglian §2.2: activations are grouped per token, weights per channel,
  optionally with K cut into blocks; nxmr §5.1: blocks of 128x128, and the
  scale tensor's shape has to match the blocking.

Readings taken where the pages leave a step open:

* The scale is the dequantisation multiplier, x ~ s * dec(q).
* s = fl32(amax / 448): an IEEE fp32 division, rounded to nearest even. It is
  computed here as a float64 quotient rounded once to float32, which equals
  the correctly rounded float32 quotient because 53 >= 2*24 + 2.
* The element step divides (it does not multiply by a reciprocal):
  y = fl32(x / s), again rounded once from float64, then e4m3 RNE. That is two
  roundings, exactly as the step reads.
* amax skips NaN (IEEE maxNum); a block with no non-NaN element has amax 0.
* amax == 0, or an amax so small that s underflows to 0: s = 0 and every
  non-NaN element gets a signed zero code.
* Quotients of finite elements are saturated to [-448, 448] before encoding.
  For a normal s the quotient never exceeds 448 by more than one fp32 ulp,
  which rounds to 448 anyway, so saturation changes nothing there; it only
  keeps a block whose s is an fp32 subnormal (too coarse to give amax/s ~ 448)
  from producing NaN codes out of finite data.
* A NaN element gets the NaN code 0x7F with its own sign bit; so does an
  infinite element of a block whose scale is infinite (inf / inf).
* No flush to zero anywhere: subnormal fp32 inputs, scales and quotients, and
  e4m3 subnormal codes are all kept.
* A last partial block (rows or columns not a multiple of the block size)
  takes the elements that are there.
"""

import numpy as np

from .formats import FORMATS

BLOCK_COLS = 128  # the K extent of every scale block (czchanglian §2.2; nxmr §5.1)


def _ceil_div(a, b):
    return -(-a // b)


def quantize_blocks(x, block_rows, block_cols=BLOCK_COLS, chunk_rows=None, fmt="e4m3"):
    """Quantise a 2-D float32 matrix in blocks of block_rows x block_cols.

    block_rows = 1 gives the per-token 1x128 scales used for the activation
    operand A; block_rows = 128 gives the 128x128 block scales of the weight
    operand B. fmt "e5m2" applies the same rules with 57344 in place of 448.

    Returns (q, s): q uint8 [rows][cols] e4m3 codes, s float32
    [ceil(rows/block_rows)][ceil(cols/block_cols)] with s[i][j] the scale of
    block (i, j).
    """
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("x must be 2-D")
    rows, cols = x.shape
    nrb = _ceil_div(rows, block_rows)
    ncb = _ceil_div(cols, block_cols)
    q = np.empty((rows, cols), dtype=np.uint8)
    s = np.empty((nrb, ncb), dtype=np.float32)
    if chunk_rows is None:
        # bound the float64 temporaries to roughly 64 MiB each
        chunk_rows = max(block_rows, (8 << 20) // max(cols, 1) // block_rows * block_rows)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        qc, sc = _quantize_chunk(x[r0:r1], block_rows, block_cols, fmt)
        q[r0:r1] = qc
        s[r0 // block_rows:r0 // block_rows + sc.shape[0]] = sc
    return q, s


def _block_amax(xp, nrb, br, ncb, bc):
    # amax skips every NaN element, quiet or signalling: NaNs are set to 0,
    # which cannot raise a maximum of absolute values. (np.fmax turns a
    # signalling NaN into a quiet NaN result, which would restart a
    # reduction part-way through a block.)
    ax = np.abs(xp)
    ax = np.where(np.isnan(ax), np.float32(0.0), ax)
    blocks = ax.reshape(nrb, br, ncb, bc)
    return blocks.max(axis=3).max(axis=1).astype(np.float32)


def _encode_with_scale(x, s_el, fmt):
    """Element step: y = fl32(x / s), saturated, encoded (see the readings)."""
    fmax, _, encode = FORMATS[fmt]
    xd = x.astype(np.float64)
    sd = s_el.astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        y = (xd / np.where(sd == 0.0, 1.0, sd)).astype(np.float32)
    # finite elements saturate, also where the fp32 quotient overflowed
    # (possible only under a scale the data has outgrown: delayed scaling)
    fin = np.isfinite(x) & ~np.isnan(y)
    y = np.where(fin, np.clip(y, -fmax, fmax), y).astype(np.float32)
    code = encode(y)
    sign = (np.signbit(x).astype(np.uint8) << 7).astype(np.uint8)
    nan_x = np.isnan(x)
    nan_code = (np.uint8(0x7F) | sign).astype(np.uint8)
    code = np.where(np.isnan(y) | nan_x, nan_code, code)
    return np.where((sd == 0.0) & ~nan_x, sign, code).astype(np.uint8)


def _quantize_chunk(x, br, bc, fmt):
    rows, cols = x.shape
    nrb = _ceil_div(rows, br)
    ncb = _ceil_div(cols, bc)
    # Pad with NaN, which the amax skips, so every block has the full shape.
    xp = np.full((nrb * br, ncb * bc), np.nan, dtype=np.float32)
    xp[:rows, :cols] = x
    amax = _block_amax(xp, nrb, br, ncb, bc)

    # scale: correctly rounded fp32 quotient amax / (448 or 57344)
    s = (amax.astype(np.float64) / FORMATS[fmt][0]).astype(np.float32)

    # per-element scale, broadcast back to the element grid
    s_el = np.repeat(np.repeat(s, br, axis=0), bc, axis=1)[:rows, :cols]
    return _encode_with_scale(x, s_el, fmt), s


# ---------------------------------------------------------------------------
# Delayed scaling (czchanglian §2.3): the scale a step quantises with comes
# from statistics gathered earlier -- the page describes running today's
# computation with the scale computed last time, which saves the separate
# statistics pass, since in training the distribution changes slowly. The
# readings taken:
#
# * one scale per tensor (the granularity a step-to-step statistic has);
# * the statistic is a window of the last H amax values (an amax history;
#   H = 1 is exactly "last time's"), and the scale is max(window) / FP8 max,
#   a correctly rounded fp32 quotient as in the block quantiser;
# * a window with no positive entry (the first step) gives the scale 1;
# * the current data may exceed what the scale covers: the quotient of every
#   finite element saturates to the format's largest value, as in the block
#   quantiser, also where the fp32 quotient itself overflowed (so finite
#   data never gives an infinity or NaN code); an infinite element keeps an
#   infinite quotient;
# * the step's own amax (NaN skipped) is recorded into the window, in the
#   entry the caller names, after the scale has been taken from it.


def delayed_scale(history, fmt="e4m3"):
    """fp32 scale from an amax history: max(history) / FP8 max, or 1 when no
    entry is positive."""
    h = np.asarray(history, dtype=np.float32)
    h = np.where(np.isnan(h), np.float32(0.0), h)
    m = float(h.max()) if h.size else 0.0
    if not m > 0.0:
        return np.float32(1.0)
    return np.float32(np.float64(np.float32(m)) / FORMATS[fmt][0])


def tensor_amax(x):
    """max |x| over a matrix, NaN skipped (0 for an empty or all-NaN one)."""
    x = np.asarray(x, dtype=np.float32)
    if x.size == 0:
        return np.float32(0.0)
    return _block_amax(x, 1, x.shape[0], 1, x.shape[1])[0, 0]


def quantize_with_scale(x, s, fmt="e4m3"):
    """Codes of x under one given fp32 scale s (the element step above)."""
    x = np.asarray(x, dtype=np.float32)
    return _encode_with_scale(x, np.full(x.shape, np.float32(s), np.float32), fmt)


def quantize_delayed(x, history, slot, fmt="e4m3"):
    """One step of delayed scaling on a 2-D float32 matrix.

    Returns (codes, scale used, new history): the scale comes from the
    history as it was before this step; the new history is the old one with
    entry `slot` replaced by this step's amax."""
    s = delayed_scale(history, fmt)
    q = quantize_with_scale(x, s, fmt)
    new = np.array(history, dtype=np.float32, copy=True)
    new[slot] = tensor_amax(x)
    return q, s, new
