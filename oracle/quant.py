"""amax, scale and quantize (cast) on the CPU.  Test infrastructure only.

Steps, as the Transformer Engine page ("Что такое FP8 инференс на H100
(Transformer Engine)?") lays them out in §3 and in its pseudocode:
  step 2: take the largest magnitude (amax) of the tensor before the GEMM;
  step 3: scale = amax / max_fp8 with max_fp8 = 448 for E4M3;
  step 4: divide the tensor by the scale and round to FP8.
"FP8 chi tiết" (Transformers fine-grained FP8 page), opening bullets, applies
the same steps per 128x128 weight block and per token to groups of 128
consecutive input channels.

Readings where the pages are silent:
* scales are float32 (the Transformer Engine page §8 says scales are stored,
  usually in float32); amax / 448 and x / scale are single IEEE float32
  divisions, round to nearest even, with subnormals kept;
* an all-zero tensor, group or block (amax = 0) gets scale 1.0 instead of 0;
* amax propagates NaN; a NaN amax or scale is the canonical quiet NaN 0x7FC00000 (so
  results are comparable bit for bit); an infinite amax gives an infinite scale;
* groups and blocks at a ragged edge cover only the elements that exist.
"""

import numpy as np

from .e4m3 import E4M3_MAX, encode_e4m3


def input_to_f32(bits, dtype):
    """Exact float32 value of bf16 ("bf16") or fp16 ("f16") bit patterns (uint16)."""
    b = np.asarray(bits, dtype=np.uint16)
    if dtype == "bf16":
        return (b.astype(np.uint32) << 16).view(np.float32)
    if dtype == "f16":
        return b.view(np.float16).astype(np.float32)
    raise ValueError(f"unknown input dtype {dtype!r}")


def amax_per_tensor(x32):
    """Largest |x| over the whole tensor (NaN if any element is NaN; 0 if empty)."""
    x32 = np.asarray(x32, dtype=np.float32)
    if x32.size == 0:
        return np.float32(0.0)
    m = np.float32(np.max(np.abs(x32)))
    return np.float32(np.nan) if np.isnan(m) else m


def amax_groups(x32, group_rows, group_cols):
    """Largest |x| per block of group_rows x group_cols elements of a 2-D tensor.

    The result has ceil(R/group_rows) x ceil(C/group_cols) entries; blocks on a
    ragged edge take the max over the elements that exist (padding with zeros
    changes no max of magnitudes).
    """
    x32 = np.asarray(x32, dtype=np.float32)
    R, C = x32.shape
    gr = -(-R // group_rows)
    gc = -(-C // group_cols)
    if gr == 0 or gc == 0:
        return np.zeros((gr, gc), dtype=np.float32)
    pad = np.zeros((gr * group_rows, gc * group_cols), dtype=np.float32)
    pad[:R, :C] = np.abs(x32)
    blocks = pad.reshape(gr, group_rows, gc, group_cols)
    m = blocks.max(axis=(1, 3)).astype(np.float32)
    return np.where(np.isnan(m), np.float32(np.nan), m).astype(np.float32)


def scale_from_amax(amax):
    """scale = amax / 448 in float32 (Transformer Engine page §3 step 3); amax 0 -> 1.0."""
    a = np.asarray(amax, dtype=np.float32)
    s = a / np.float32(E4M3_MAX)
    s = np.where(np.isnan(s), np.float32(np.nan), s)
    return np.where(a == 0, np.float32(1.0), s).astype(np.float32)


def quantize_with_scale(x32, scale):
    """q = e4m3(x / scale): one float32 division per element, then the
    saturating round-to-nearest-even encode (§3 step 4).  ``scale`` broadcasts."""
    x32 = np.asarray(x32, dtype=np.float32)
    q32 = x32 / np.asarray(scale, dtype=np.float32)
    return encode_e4m3(q32.astype(np.float32))


def quantize_per_tensor(bits, dtype):
    """One scale for the whole tensor.  Returns (q uint8 like bits, scale float32)."""
    x32 = input_to_f32(bits, dtype)
    scale = scale_from_amax(amax_per_tensor(x32))
    return quantize_with_scale(x32, scale), np.float32(scale)


def quantize_groups(bits, dtype, group_rows, group_cols):
    """Blockwise scales: group_rows=1, group_cols=128 is the per-token 1x128
    activation grouping; group_rows=group_cols=128 is the 128x128 weight block
    ("FP8 chi tiết", opening bullets).

    Returns (q uint8 [R, C], scales float32 [ceil(R/gr), ceil(C/gc)]).
    """
    x32 = input_to_f32(bits, dtype)
    R, C = x32.shape
    scales = scale_from_amax(amax_groups(x32, group_rows, group_cols))
    per_elem = np.repeat(np.repeat(scales, group_rows, axis=0), group_cols, axis=1)[:R, :C]
    return quantize_with_scale(x32, per_elem), scales
