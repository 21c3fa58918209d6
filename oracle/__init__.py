"""CPU oracle for the FP8 block-scaled GEMM path -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously correct NumPy implementation of what
the GPU path computes. It exists to check the GPU path, never to stand in for
it: only the tests, the smoke check of the package entry file and the CPU
baseline leg of the benchmark may import it. The product library never calls
it, and it shares no code, table or helper with the HIP sources.

Sources (the three pages the method is described on):

* [czchanglian] m.czchanglian.com/news/60438 -- an essay taking DeepGEMM apart:
  FP8 formats (§2.1 table), fine-grained scaling (§2.2), FP32 accumulation
  (§2.3), padding (§5.1), scale initialisation (§5.2), MoE grouping (§5.3).
* [gtnt] www.gtnt.cn/news/117510, "生产级 FP8 GEMM 算子对齐与 Tensor Core 峰值利用率调优":
  the E4M3/E5M2 comparison, the fused-scale Triton kernel and the H100 table.
* [nxmr] www.nxmr.cn/news/131680 -- an explainer of DeepGEMM: block
  quantisation (§3.1), grouped GEMM (§3.2), the API (§4.2), rounding (§5.1).

Modules:
  formats   -- e4m3 and e5m2 decode tables and RNE encoders, fp64 -> bf16 RNE.
  quantize  -- per-block amax / scale / codes (1x128 and 128x128), and
               delayed (amax-history) per-tensor scaling.
  gemm      -- block-scaled GEMM, grouped contiguous and masked, the
               per-tensor-scaled GEMM (e4m3 / e5m2 operands), tolerance.

Every function is pinned by the CPU tests (tests/test_oracle_*.py) to facts
that do not come from the oracle itself: the pages' printed constants, closed
forms, exact rational brute force, and independent library conversions.
"""

from .formats import (E4M3_MAX, E5M2_MAX, e4m3_decode_table, e4m3_encode_rne,
                      e5m2_decode_table, e5m2_encode_rne, bf16_bits_from_f64, bf16_bits_to_f64)
from .quantize import (quantize_blocks, delayed_scale, tensor_amax, quantize_with_scale,
                       quantize_delayed)
from .gemm import (gemm_blockscaled, gemm_blockscaled_fp32acc, gemm_pertensor,
                   grouped_contiguous, grouped_masked, tolerance_check)

__all__ = [
    "E4M3_MAX", "E5M2_MAX", "e4m3_decode_table", "e4m3_encode_rne", "e5m2_decode_table",
    "e5m2_encode_rne", "bf16_bits_from_f64", "bf16_bits_to_f64", "quantize_blocks",
    "delayed_scale", "tensor_amax", "quantize_with_scale", "quantize_delayed", "gemm_blockscaled",
    "gemm_blockscaled_fp32acc", "gemm_pertensor", "grouped_contiguous", "grouped_masked",
    "tolerance_check",
]
