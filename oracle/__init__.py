"""CPU oracle for the FP8 E4M3 amax / scale / cast / scaled-GEMM path.

THIS PACKAGE IS TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or call it.  The product
path (the HIP library and its Python binding) never imports it and shares no
code, table or helper with it.

It is a plain, slow, obviously correct restatement of what the pages define:

* ``e4m3``  - the OCP "e4m3fn" 8-bit float (1 sign, 4 exponent, 3 mantissa bits,
  no infinities, largest finite value 448): decoding from the bit fields, and a
  saturating round-to-nearest-even encoder that searches by value.
  Sources: "Что такое FP8 инференс на H100 (Transformer Engine)?" §2 (E4M3 for
  inference) and §3 step 3 (448 is the E4M3 maximum); §5 (range -448..448);
  "FP8混合精度推理" §2 (4 exponent bits, 3 mantissa bits).
* ``quant`` - amax (largest magnitude) per tensor, per 1x128 token group and per
  128x128 weight block; scale = amax / 448 in float32; x / scale rounded to
  e4m3.  Sources: the Transformer Engine page §3 steps 2-4 and its pseudocode;
  "FP8 chi tiết" (Transformers fine-grained FP8 page), opening bullets.
* ``gemm``  - the FP8 x FP8 product accumulated exactly in float64, multiplied by
  scale_A * scale_B per tensor or per 128-wide K slab, and the north-star
  tolerance check.  Sources: the Transformer Engine page §3 steps 5-6 and its
  pseudocode; "FP8 chi tiết", opening bullets.

* ``ue8m0`` - power-of-two block scales stored as e8m0fnu bytes: the smallest
  power of two not below amax / 448, the cast with it, and the blockwise product
  with the decoded scales.  Source: "FP8 chi tiết", section on the UE8M0 scale
  format.

* ``rowwise`` - per-channel scaling: one scale per row (per output channel of the
  weights, per token of the activations), the cast with it, and the product with
  sa[m] * sb[n].  Source: the Transformer Engine page §5 (per-channel scaling of the
  weights) with §3 steps 2-6.

* ``grouped`` - the mixture-of-experts grouped blockwise product: contiguous segments of
  the routed activations, each multiplied by its expert's weight (float32 or UE8M0 block
  scales).  Source: "FP8 chi tiết", its section on MoE experts (grouped_mm / batched_mm,
  DeepGEMM expert kernels) with the opening bullets' block scaling.

* ``delayed`` - static scaling (a scale fixed in advance; saturation) and the
  delayed-scaling amax history (max over the window, times 2^margin, every
  `interval` steps).  Source: the task page's DelayedScaling recipe and calibration
  step.

Every function here is pinned by ``tests/test_oracle_*.py`` against facts the
pages print (tests/golden), closed forms, brute force over all 256 codes, exact
rational arithmetic and library special cases.  No function is "parity
unpinned".

Readings of points the pages leave open are listed in each function's
docstring (zero amax -> scale 1, NaN -> 0x7F, saturation at 448, fp32 IEEE
division, operand layout C = A @ B^T).
"""

from .e4m3 import (E4M3_MAX, decode_e4m3, positive_values, encode_e4m3,
                   nonneg_breakpoints)
from .quant import (input_to_f32, amax_per_tensor, amax_groups, scale_from_amax,
                    quantize_per_tensor, quantize_groups, quantize_with_scale)
from .gemm import (gemm_tensorwise_ref, gemm_blockwise_ref, bound_tensorwise,
                   bound_blockwise, output_ulp, check_gemm)
from .ue8m0 import (e8m0_decode, e8m0_from_amax, quantize_groups_ue8m0,
                    gemm_blockwise_ue8m0_ref, bound_blockwise_ue8m0)
from .delayed import quantize_static, delayed_scale_from_history, delayed_step
from .rowwise import amax_rows, quantize_rowwise, gemm_rowwise_ref, bound_rowwise
from .grouped import (offsets_from_sizes, gemm_grouped_blockwise_ref, bound_grouped_blockwise,
                      gemm_grouped_blockwise_ue8m0_ref, bound_grouped_blockwise_ue8m0)

__all__ = [
    "E4M3_MAX", "decode_e4m3", "positive_values", "encode_e4m3", "nonneg_breakpoints",
    "input_to_f32", "amax_per_tensor", "amax_groups", "scale_from_amax",
    "quantize_per_tensor", "quantize_groups", "quantize_with_scale",
    "gemm_tensorwise_ref", "gemm_blockwise_ref", "bound_tensorwise", "bound_blockwise",
    "output_ulp", "check_gemm",
    "e8m0_decode", "e8m0_from_amax", "quantize_groups_ue8m0", "gemm_blockwise_ue8m0_ref",
    "bound_blockwise_ue8m0", "quantize_static", "delayed_scale_from_history", "delayed_step",
    "amax_rows", "quantize_rowwise", "gemm_rowwise_ref", "bound_rowwise",
    "offsets_from_sizes", "gemm_grouped_blockwise_ref", "bound_grouped_blockwise",
    "gemm_grouped_blockwise_ue8m0_ref", "bound_grouped_blockwise_ue8m0",
]
