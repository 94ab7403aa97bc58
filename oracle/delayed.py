"""Static and delayed per-tensor scaling on the CPU.  Test infrastructure only.

Sources: the task page's FP8 recipe (Transformer Engine DelayedScaling with margin 0,
interval 4, E4M3) and its calibration step, which runs batches to collect the tensors'
amax before FP8 inference; the fine-grained FP8 page's note that static activation
quantization exists beside the dynamic one.

Readings where the pages are silent (the recipe is named, its internals are not):
* static scaling casts with a scale fixed in advance: q = e4m3(x / scale), one float32
  division per element; elements with |x| > 448 * scale saturate to +-448;
* delayed scaling keeps a history of the last L amaxes (most recent first).  Each step
  pushes the step's amax; after every `interval`-th step the scale becomes
  max(history) * 2^margin / 448 in float32 (max(history) = 0 -> 1; a NaN amax in the
  window gives the canonical NaN scale), and between those steps the scale is unchanged.
  The scale convention is the one of the dynamic path (x is divided by it), so the
  margin multiplies it by 2^margin;
* a step's amax is the largest |x| of the tensor the step quantized (NaN propagates).
"""

import numpy as np

from .e4m3 import E4M3_MAX
from .quant import input_to_f32, amax_per_tensor, quantize_with_scale


def quantize_static(bits, dtype, scale):
    """Static scaling: (q uint8 like bits, amax float32 of the tensor) for a given scale."""
    x32 = input_to_f32(bits, dtype)
    return quantize_with_scale(x32, np.float32(scale)), amax_per_tensor(x32)


def delayed_scale_from_history(history, margin):
    """max(history) * 2^margin / 448 in float32; 0 -> 1; NaN -> canonical NaN."""
    h = np.asarray(history, dtype=np.float32)
    m = np.float32(np.max(h)) if h.size else np.float32(0.0)
    if np.any(np.isnan(h)):
        return np.float32(np.nan)
    if m == 0:
        return np.float32(1.0)
    return np.float32(np.float32(m * np.float32(2.0 ** margin)) / np.float32(E4M3_MAX))


def delayed_step(history, step, scale, amax, interval, margin):
    """One step of delayed scaling.  history: float32 [L] (most recent first), step:
    steps done so far, scale: the current scale, amax: this step's amax.  Returns the new
    (history, step, scale)."""
    h = np.asarray(history, dtype=np.float32).copy()
    if h.size:
        h[1:] = h[:-1].copy()
        h[0] = np.float32(amax)
    step += 1
    if step % interval == 0:
        scale = delayed_scale_from_history(h, margin)
    return h, step, np.float32(scale)
