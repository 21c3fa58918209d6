"""The five synthetic workloads and their generator.

Recipe (one numpy Generator, default_rng(seed), per workload; draw order:
routing structure, outlier columns, A, B):

* Values: float32 standard normal.
* Outlier channels: one set S of round(f*K) (at least 1) K-columns drawn
  without replacement; A[..., S] and B[..., S] are both multiplied by 50.
  f = 1% for the 128x256x512, 16x4096x7168 and both MoE workloads, 0.5% for
  the 4096x8192x8192 one. This models the outlier channel that spoils a
  per-tensor scale (czchanglian §2.2).
* Contiguous MoE: 8 experts, 4096 tokens routed top-1 with probability of the
  expert of rank r proportional to r^-1.2 (multinomial draw of the counts);
  each expert's rows are contiguous and padded with zero rows up to a multiple
  of 128 (czchanglian §5.1 pads outside the library; §5.3 wants each expert's
  rows contiguous and movable in blocks).
* Masked MoE: 32 experts with a 256-row slab each, valid counts drawn
  uniformly from {0..256}; every slab row (valid or not) holds generator data.
* The dense 4096x8192x8192 shape is the one the gtnt page times on H100.
"""

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

OUTLIER_GAIN = 50.0


@dataclass
class Workload:
    name: str
    kind: str                      # "dense" | "contiguous" | "masked"
    M: int                         # dense: rows; contiguous: padded total rows; masked: max_m
    N: int
    K: int
    G: int
    a: np.ndarray                  # float32: dense/contiguous [M][K]; masked [G][max_m][K]
    b: np.ndarray                  # float32: dense [N][K]; grouped [G][N][K]
    outlier_cols: np.ndarray
    counts: Optional[np.ndarray] = None        # per-expert valid rows (grouped)
    offsets: Optional[np.ndarray] = None       # contiguous: [G+1] padded row offsets
    masked_m: Optional[np.ndarray] = None      # masked: [G]
    meta: dict = field(default_factory=dict)

    def valid_rows(self):
        if self.kind == "dense":
            return self.M
        return int(np.sum(self.counts))


def pad_to(x, mult):
    return -(-int(x) // mult) * mult


def zipf_counts(rng, tokens, experts, s):
    r = np.arange(1, experts + 1, dtype=np.float64)
    p = r ** -s
    p /= p.sum()
    return rng.multinomial(tokens, p).astype(np.int64)


def _outliers(rng, K, frac):
    n = max(1, int(round(frac * K)))
    return np.sort(rng.choice(K, size=n, replace=False))


def make_dense(M, N, K, frac=0.01, seed=0, name=None):
    rng = np.random.default_rng(seed)
    S = _outliers(rng, K, frac)
    a = rng.standard_normal((M, K), dtype=np.float32)
    b = rng.standard_normal((N, K), dtype=np.float32)
    a[:, S] *= np.float32(OUTLIER_GAIN)
    b[:, S] *= np.float32(OUTLIER_GAIN)
    return Workload(name or f"dense_{M}x{N}x{K}", "dense", M, N, K, 1, a, b, S)


def make_contiguous(counts, N, K, frac=0.01, seed=0, rng=None, name=None, tokens=None):
    """Contiguous grouped layout from given per-expert counts (or routed counts
    drawn by the caller's rng). Tokens of expert g occupy padded rows
    offsets[g] .. offsets[g] + counts[g] - 1; padding rows are zero."""
    if rng is None:
        rng = np.random.default_rng(seed)
    counts = np.asarray(counts, dtype=np.int64)
    G = counts.shape[0]
    padded = np.array([pad_to(c, 128) for c in counts], dtype=np.int64)
    offsets = np.zeros(G + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(padded)
    M_total = int(offsets[-1])
    S = _outliers(rng, K, frac)
    T = int(counts.sum())
    tok = rng.standard_normal((T, K), dtype=np.float32)
    b = rng.standard_normal((G, N, K), dtype=np.float32)
    tok[:, S] *= np.float32(OUTLIER_GAIN)
    b[:, :, S] *= np.float32(OUTLIER_GAIN)
    a = np.zeros((M_total, K), dtype=np.float32)
    t0 = 0
    for g in range(G):
        c = int(counts[g])
        a[offsets[g]:offsets[g] + c] = tok[t0:t0 + c]
        t0 += c
    del tok
    return Workload(name or f"contiguous_G{G}_N{N}_K{K}", "contiguous", M_total, N, K, G,
                    a, b, S, counts=counts, offsets=offsets)


def make_masked(masked_m, max_m, N, K, frac=0.01, seed=0, rng=None, name=None):
    if rng is None:
        rng = np.random.default_rng(seed)
    masked_m = np.asarray(masked_m, dtype=np.int64)
    G = masked_m.shape[0]
    S = _outliers(rng, K, frac)
    a = rng.standard_normal((G, max_m, K), dtype=np.float32)
    b = rng.standard_normal((G, N, K), dtype=np.float32)
    a[:, :, S] *= np.float32(OUTLIER_GAIN)
    b[:, :, S] *= np.float32(OUTLIER_GAIN)
    return Workload(name or f"masked_G{G}_maxm{max_m}_N{N}_K{K}", "masked", max_m, N, K, G,
                    a, b, S, counts=np.minimum(masked_m, max_m), masked_m=masked_m)


# name, builder -- index order matches the five workloads of the method
WORKLOAD_NAMES = [
    "dense_128x256x512",
    "dense_16x4096x7168",
    "dense_4096x8192x8192",
    "moe_contiguous_G8_T4096_N4096_K7168",
    "moe_masked_G32_maxm256_N7168_K2048",
]


def make_config(i, seed=0):
    """Build workload i (0..4) with the recipe in the module docstring."""
    if i == 0:
        return make_dense(128, 256, 512, frac=0.01, seed=seed, name=WORKLOAD_NAMES[0])
    if i == 1:
        return make_dense(16, 4096, 7168, frac=0.01, seed=seed, name=WORKLOAD_NAMES[1])
    if i == 2:
        return make_dense(4096, 8192, 8192, frac=0.005, seed=seed, name=WORKLOAD_NAMES[2])
    if i == 3:
        rng = np.random.default_rng(seed)
        counts = zipf_counts(rng, 4096, 8, 1.2)
        return make_contiguous(counts, 4096, 7168, frac=0.01, rng=rng, name=WORKLOAD_NAMES[3])
    if i == 4:
        rng = np.random.default_rng(seed)
        masked_m = rng.integers(0, 257, 32).astype(np.int64)
        return make_masked(masked_m, 256, 7168, 2048, frac=0.01, rng=rng, name=WORKLOAD_NAMES[4])
    raise ValueError(f"no workload {i}")
