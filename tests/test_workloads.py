"""The seeded synthetic workloads: structure and recipe (CPU only)."""

import os

import numpy as np

from workloads import make_config, make_contiguous, zipf_counts, WORKLOAD_NAMES

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# Routing structure of the two MoE workloads at seed 0 (numpy 2.2 Generator).
# These are inputs, not expected outputs: the test only guards against a
# change of the generator stream.
ZIPF_COUNTS_SEED0 = [1796, 753, 466, 321, 255, 211, 161, 133]
MASKED_M_SEED0 = [218, 163, 131, 69, 79, 10, 19, 4, 45, 209, 166, 234, 129, 155, 249, 187,
                  162, 139, 143, 240, 71, 209, 172, 0, 101, 220, 142, 8, 196, 187, 217, 45]


def test_structure_seed0():
    rng = np.random.default_rng(0)
    assert zipf_counts(rng, 4096, 8, 1.2).tolist() == ZIPF_COUNTS_SEED0
    rng = np.random.default_rng(0)
    assert rng.integers(0, 257, 32).tolist() == MASKED_M_SEED0
    assert sum(MASKED_M_SEED0) == 4319


def test_small_configs_shapes_and_outliers():
    w0 = make_config(0)
    assert (w0.M, w0.N, w0.K) == (128, 256, 512)
    assert w0.a.dtype == np.float32 and w0.a.shape == (128, 512) and w0.b.shape == (256, 512)
    assert len(w0.outlier_cols) == 5
    # outlier columns carry the x50 gain: their rms is ~50x the others'
    S = w0.outlier_cols
    rest = np.setdiff1d(np.arange(512), S)
    ratio = np.sqrt(np.mean(w0.a[:, S] ** 2)) / np.sqrt(np.mean(w0.a[:, rest] ** 2))
    assert 35 < ratio < 70
    w1 = make_config(1)
    assert (w1.M, w1.N, w1.K) == (16, 4096, 7168) and len(w1.outlier_cols) == 72
    # same seed -> same data
    assert np.array_equal(make_config(0).a, w0.a)


def test_contiguous_padding_layout():
    w = make_contiguous([3, 0, 129], 128, 256, seed=1)
    assert w.offsets.tolist() == [0, 128, 128, 384]
    assert np.all(w.a[3:128] == 0) and np.all(w.a[128 + 129:] == 0)
    assert np.all(np.any(w.a[:3] != 0, axis=1))
    assert w.valid_rows() == 132


def test_config_names():
    assert len(WORKLOAD_NAMES) == 5
