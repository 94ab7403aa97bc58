"""FP8 E4M3 amax / quantize / scaled GEMM for AMD MI355X (gfx950).

The compute path is the HIP library ``libfp8amax.so`` (C ABI in include/fp8amax.h);
the functions below are its Python binding under the same names.  Build the library
with ``python -m fp8_quantized_gemm_amax_amd.build``.
"""

from .binding import (Fp8Error, fp8_amax, fp8_quantize_per_tensor, fp8_quantize_per_token_group,
                      fp8_gemm_scaled_tensorwise, fp8_gemm_scaled_blockwise, fp8_debug_cast_f32,
                      fp8_quantize_per_token_group_ue8m0, fp8_gemm_scaled_blockwise_ue8m0,
                      e8m0_row_bytes, fp8_quantize_static, fp8_delayed_scaling_update, fp8_quantize_delayed,
                      DelayedScaling, fp8_quantize_rowwise, fp8_gemm_scaled_rowwise,
                      fp8_gemm_grouped_blockwise, fp8_gemm_grouped_blockwise_ue8m0,
                      fp8_debug_byte_mix, fp8_debug_gemm_plan, fp8_gemv_dynamic, lib, LIB_PATH)

__all__ = ["Fp8Error", "fp8_amax", "fp8_quantize_per_tensor", "fp8_quantize_per_token_group",
           "fp8_gemm_scaled_tensorwise", "fp8_gemm_scaled_blockwise", "fp8_debug_cast_f32",
           "fp8_quantize_per_token_group_ue8m0", "fp8_gemm_scaled_blockwise_ue8m0", "e8m0_row_bytes",
           "fp8_quantize_static", "fp8_delayed_scaling_update", "fp8_quantize_delayed",
           "DelayedScaling", "fp8_quantize_rowwise", "fp8_gemm_scaled_rowwise",
           "fp8_gemm_grouped_blockwise", "fp8_gemm_grouped_blockwise_ue8m0",
           "fp8_debug_byte_mix", "fp8_debug_gemm_plan", "fp8_gemv_dynamic", "lib", "LIB_PATH"]
