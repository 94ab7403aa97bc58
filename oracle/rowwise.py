"""Per-channel ("rowwise") scaling on the CPU.  Test infrastructure only.

Source: the Transformer Engine page ("Что такое FP8 инференс на H100 (Transformer
Engine)?") §5, which lists per-channel scaling of the weights beside per-tensor scaling
as a way to limit the accuracy loss; the scale of each channel follows §3 steps 2-4
(amax, amax / 448, divide and round), the product §3 steps 5-6 (wide accumulator, then
the scales, then the 16-bit output).

Readings where the page is silent:
* a weight channel is an output channel: one row n of W [N, K], with its amax over the
  K input channels;
* the activations are scaled the same way per token: one row m of A [M, K] (the page
  does not say; a single per-tensor activation scale is the special case of equal
  entries, and per token is what a serving step computes for free when it quantizes
  each token's row);
* amax 0 -> scale 1, NaN propagates to the row's scale (as in the per-tensor path);
* C[m, n] = (sum_k dec(qa[m, k]) * dec(qb[n, k])) * sa[m] * sb[n].
"""

import numpy as np

from .e4m3 import decode_e4m3
from .quant import input_to_f32, scale_from_amax, quantize_with_scale


def amax_rows(x32):
    """Largest |x| of each row of a 2-D float32 tensor (NaN if the row has one; 0 if empty)."""
    x32 = np.asarray(x32, dtype=np.float32)
    R, C = x32.shape
    if C == 0:
        return np.zeros(R, dtype=np.float32)
    a = np.abs(x32)
    m = a.max(axis=1).astype(np.float32)
    return np.where(np.isnan(a).any(axis=1), np.float32(np.nan), m).astype(np.float32)


def quantize_rowwise(bits, dtype):
    """One scale per row: (q uint8 [R, C], scales float32 [R])."""
    x32 = input_to_f32(bits, dtype)
    scales = scale_from_amax(amax_rows(x32))
    return quantize_with_scale(x32, scales[:, None]), scales.astype(np.float32)


def gemm_rowwise_ref(qa, sa, qb, sb):
    """C64[m, n] = (sum_k dec(qa[m,k]) dec(qb[n,k])) * (sa[m] * sb[n]), float64.

    The unscaled sum is exact (see the gemm module); sa[m] * sb[n] of two float32 values
    is exact in float64, so the result carries one rounding."""
    da = decode_e4m3(np.asarray(qa, dtype=np.uint8))
    db = decode_e4m3(np.asarray(qb, dtype=np.uint8))
    sa64 = np.asarray(sa, dtype=np.float32).astype(np.float64)
    sb64 = np.asarray(sb, dtype=np.float32).astype(np.float64)
    return (da @ db.T) * (sa64[:, None] * sb64[None, :])


def bound_rowwise(qa, sa, qb, sb):
    """Magnitude term sum_k |dec(qa) sa[m]| |dec(qb) sb[n]|."""
    da = np.abs(decode_e4m3(np.asarray(qa, dtype=np.uint8)))
    db = np.abs(decode_e4m3(np.asarray(qb, dtype=np.uint8)))
    sa64 = np.abs(np.asarray(sa, dtype=np.float32).astype(np.float64))
    sb64 = np.abs(np.asarray(sb, dtype=np.float32).astype(np.float64))
    return (da @ db.T) * (sa64[:, None] * sb64[None, :])
