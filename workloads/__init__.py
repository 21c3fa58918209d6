"""Seeded synthetic inputs shared by the oracle checks and the GPU path.

Holds no arithmetic of the method (no scaling, no quantisation, no products):
only random draws, shapes and the MoE routing structure.
"""

from .gen import (WORKLOAD_NAMES, Workload, make_config, make_dense, make_contiguous,
                  make_masked, zipf_counts, pad_to)

__all__ = ["WORKLOAD_NAMES", "Workload", "make_config", "make_dense", "make_contiguous",
           "make_masked", "zipf_counts", "pad_to"]
