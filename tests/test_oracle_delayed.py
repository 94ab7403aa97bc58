"""Pins for the oracle's static and delayed per-tensor scaling (CPU only).

References used: the dynamic per-tensor quantizer (static scaling with the tensor's own
amax/448 must reproduce it), brute-force nearest e4m3 search in exact rationals for the
saturating cast, and step sequences worked out by hand for the delayed-scaling history.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.delayed import quantize_static, delayed_scale_from_history, delayed_step


def bf16(a):
    return (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_static_with_own_amax_equals_dynamic():
    rng = np.random.default_rng(1)
    bits = bf16(rng.standard_t(4, (37, 300)))
    q_dyn, s_dyn = oracle.quantize_per_tensor(bits, "bf16")
    q, amax = quantize_static(bits, "bf16", s_dyn)
    np.testing.assert_array_equal(q, q_dyn)
    assert amax == oracle.amax_per_tensor(oracle.input_to_f32(bits, "bf16"))


def test_static_saturates_and_rounds_like_brute_force():
    """A scale four times too small: every element above 448 * scale saturates to the
    code of +-448; the others are the nearest e4m3 value (ties to the even code)."""
    rng = np.random.default_rng(2)
    bits = bf16(rng.standard_normal((3, 70)) * 10)
    x32 = oracle.input_to_f32(bits, "bf16")
    scale = np.float32(np.max(np.abs(x32)) / np.float32(448) / np.float32(4))
    q, _ = quantize_static(bits, "bf16", scale)
    mags = [Fraction(float(v)) for v in oracle.positive_values()]
    nsat = 0
    for (r, c), v in np.ndenumerate(x32):
        t = Fraction(float(np.float32(v) / scale))          # the float32 quotient
        if abs(t) >= 448:
            want = 0x7E
            nsat += 1
        else:
            want = min(range(127), key=lambda i: (abs(mags[i] - abs(t)), i & 1))
        want |= 0x80 if v < 0 else 0
        assert int(q[r, c]) == want, (r, c)
    assert nsat > 0


def test_static_amax_brute_force_and_nan():
    bits = bf16([[0.5, -3.0, 2.0], [1.0, -0.25, 2.5]])
    _, amax = quantize_static(bits, "bf16", np.float32(1.0))
    assert amax == np.float32(3.0)
    bits[1, 1] = 0x7FC0
    q, amax = quantize_static(bits, "bf16", np.float32(1.0))
    assert np.isnan(amax) and (q[1, 1] & 0x7F) == 0x7F


def test_scale_from_history_closed_forms():
    assert delayed_scale_from_history([448.0, 1.0], 0) == np.float32(1.0)
    assert delayed_scale_from_history([7.0, 3.0, 0.5], 0) == np.float32(2.0 ** -6)     # 7 / (7 * 64)
    assert delayed_scale_from_history([7.0, 3.0, 0.5], 2) == np.float32(2.0 ** -4)
    assert delayed_scale_from_history([0.0, 0.0], 3) == np.float32(1.0)                # empty window
    assert np.isnan(delayed_scale_from_history([1.0, np.nan], 0))


@pytest.mark.parametrize("margin,after4,after8", [(0, 1.0, 2.0 ** -6), (1, 2.0, 2.0 ** -5)])
def test_delayed_sequence_by_hand(margin, after4, after8):
    """History of 3, interval 4.  Steps 1-3 keep the initial scale; step 4 sees
    [3, 448, 2] -> 448 * 2^margin / 448; steps 5-7 keep it; step 8 sees [0.25, 0.5, 7]
    -> 7 * 2^margin / 448."""
    h, step, scale = np.zeros(3, np.float32), 0, np.float32(0.75)
    amaxes = [1, 2, 448, 3, 5, 7, 0.5, 0.25]
    scales = []
    for a in amaxes:
        h, step, scale = delayed_step(h, step, scale, np.float32(a), 4, margin)
        scales.append(float(scale))
    assert scales[:3] == [0.75, 0.75, 0.75]
    assert scales[3] == after4
    assert scales[4:7] == [after4] * 3
    assert scales[7] == after8
    np.testing.assert_array_equal(h, np.array([0.25, 0.5, 7], np.float32))
    assert step == 8


def test_delayed_nan_leaves_the_window():
    """A NaN amax makes the scale NaN at the next update and stops doing so once it has
    been pushed out of the history (length 2, interval 1)."""
    h, step, scale = np.zeros(2, np.float32), 0, np.float32(1.0)
    out = []
    for a in [448.0, np.nan, 224.0, 112.0]:
        h, step, scale = delayed_step(h, step, scale, np.float32(a), 1, 0)
        out.append(float(scale))
    assert out[0] == 1.0 and np.isnan(out[1]) and np.isnan(out[2]) and out[3] == 0.5
