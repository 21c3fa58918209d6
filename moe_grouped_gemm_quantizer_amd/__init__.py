"""MI355X-native FP8 block-scaled GEMM (dense and grouped MoE).

The compute lives in libfp8gemm.so (HIP kernels for gfx950, C ABI declared in
include/fp8gemm.h); this package only marshals torch tensors into those
calls. Build the library with `python -m moe_grouped_gemm_quantizer_amd.build`.
"""

from ._lib import (fp8_quantize, fp8_quantize_bf16, fp8_quantize_tensor, gemm_fp8_blockscaled,
                   gemm_fp8_pertensor, gemm_fp8_blockscaled_quant, grouped_gemm_fp8_contiguous,
                   grouped_gemm_fp8_contiguous_workspace_size, grouped_gemm_fp8_contiguous_ws,
                   grouped_gemm_fp8_contiguous_noalloc,
                   grouped_gemm_fp8_masked, gemm_fp8_pertensor_fmt, fp8_quantize_delayed,
                   fp8g_clock_probe, fp8g_warmup,
                   fp8g_set_shape_specialisation, fp8g_gemm_kernel_name, fp8g_abi_version,
                   status_string, load,
                   Fp8GemmError, LIB_PATH, ENTRY_POINTS)

__all__ = ["fp8_quantize", "fp8_quantize_bf16", "fp8_quantize_tensor", "gemm_fp8_blockscaled",
           "gemm_fp8_pertensor", "gemm_fp8_blockscaled_quant", "grouped_gemm_fp8_contiguous",
           "grouped_gemm_fp8_contiguous_workspace_size", "grouped_gemm_fp8_contiguous_ws",
           "grouped_gemm_fp8_contiguous_noalloc",
           "grouped_gemm_fp8_masked", "gemm_fp8_pertensor_fmt", "fp8_quantize_delayed",
           "fp8g_clock_probe", "fp8g_warmup",
           "fp8g_set_shape_specialisation", "fp8g_gemm_kernel_name", "fp8g_abi_version",
           "status_string", "load",
           "Fp8GemmError", "LIB_PATH", "ENTRY_POINTS"]
