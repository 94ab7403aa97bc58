"""UE8M0 (power-of-two) block scales on the CPU.  Test infrastructure only.

Source: "FP8 chi tiết" (Transformers fine-grained FP8 page), section "Định dạng
thang đo UE8M0" (the UE8M0 scale format): DeepSeek-V4-style checkpoints keep the
FP8 weight scales as packed float8_e8m0fnu bytes instead of float32, mark them
with scale_fmt="ue8m0", and the FP8 kernels read that format directly.  The
blocks and groups are those of the same page's opening bullets (128x128 weight
blocks, 1x128 per-token activation groups).

The e8m0fnu byte is an unsigned 8-bit exponent: code c stands for 2^(c - 127);
code 255 is NaN; there is no sign, zero or infinity.

Readings where the page is silent:
* a block's scale is the smallest power of two not below amax / 448, so that no
  |x| / scale exceeds the e4m3 maximum (rounding the exponent up; rounding down
  would saturate the largest elements).  The exponent is exact:
  e = min{ e integer : 448 * 2^e >= amax };
* e is clamped to the byte's finite range [-127, 127]; an all-zero block
  (amax = 0) gets 2^0, code 127, as the float32 scales use 1.0 there;
* a NaN or infinite amax gives code 255 (NaN), since e8m0 has no infinity;
* the codes are q = e4m3(x / 2^e) with the float32 division and the encoder of
  the float32-scale path (dividing by a power of two is exact unless the
  quotient falls below 2^-126, where e4m3 rounds to zero anyway);
* activation groups use the same format as weight blocks, and the product is the
  blockwise one with the decoded scales.
"""

import math

import numpy as np

from .e4m3 import E4M3_MAX
from .quant import input_to_f32, amax_groups, quantize_with_scale
from .gemm import gemm_blockwise_ref, bound_blockwise

E8M0_NAN = 255
E8M0_BIAS = 127


def e8m0_decode(codes):
    """Float64 value 2^(c - 127) of e8m0fnu codes; code 255 is NaN."""
    c = np.asarray(codes, dtype=np.uint8)
    out = np.ldexp(1.0, c.astype(np.int64) - E8M0_BIAS)
    return np.where(c == E8M0_NAN, np.nan, out)


def _exponent_for(amax):
    """Smallest integer e with 448 * 2^e >= amax, for a finite amax > 0 (exact)."""
    a = float(amax)
    e = math.floor(math.log2(a / E4M3_MAX)) - 2          # an estimate below the answer
    while math.ldexp(float(E4M3_MAX), e) < a:            # exact comparisons of floats
        e += 1
    return e


def e8m0_from_amax(amax):
    """UE8M0 scale code of each amax (float32 array): the smallest power of two
    not below amax / 448, clamped to 2^-127 .. 2^127; amax 0 -> code 127;
    NaN or infinite amax -> code 255."""
    a = np.asarray(amax, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint8)
    flat_a, flat_o = a.reshape(-1), out.reshape(-1)
    for i, v in enumerate(flat_a):
        if not np.isfinite(v):
            flat_o[i] = E8M0_NAN
        elif v == 0:
            flat_o[i] = E8M0_BIAS
        else:
            e = min(max(_exponent_for(v), -E8M0_BIAS), E8M0_BIAS)
            flat_o[i] = e + E8M0_BIAS
    return out


def quantize_groups_ue8m0(bits, dtype, group_rows, group_cols):
    """Blocks of group_rows x group_cols (1 x 128 per-token groups or 128 x 128
    weight blocks) with UE8M0 scales.

    Returns (q uint8 [R, C], codes uint8 [ceil(R/gr), ceil(C/gc)]).
    """
    x32 = input_to_f32(bits, dtype)
    R, C = x32.shape
    codes = e8m0_from_amax(amax_groups(x32, group_rows, group_cols))
    scales = e8m0_decode(codes).astype(np.float32)        # powers of two (or NaN): exact
    per_elem = np.repeat(np.repeat(scales, group_rows, axis=0), group_cols, axis=1)[:R, :C]
    return quantize_with_scale(x32, per_elem), codes


def gemm_blockwise_ue8m0_ref(qa, ea, qb, eb, nblock=None):
    """C64[m, n] = sum_g 2^(ea[m,g]-127) * 2^(eb[n//128,g]-127) * (sum_{k in slab g} dec(qa) dec(qb)):
    the blockwise product with the decoded UE8M0 scales (exact in float64)."""
    sa = e8m0_decode(ea).astype(np.float32)
    sb = e8m0_decode(eb).astype(np.float32)
    return gemm_blockwise_ref(qa, sa, qb, sb, nblock=nblock)


def bound_blockwise_ue8m0(qa, ea, qb, eb, nblock=None):
    """Magnitude term of the UE8M0 blockwise product (|.| everywhere)."""
    sa = e8m0_decode(ea).astype(np.float32)
    sb = e8m0_decode(eb).astype(np.float32)
    return bound_blockwise(qa, sa, qb, sb, nblock=nblock)
