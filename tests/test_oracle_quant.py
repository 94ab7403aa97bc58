"""Pins for the oracle's input conversion, amax, scale and quantize (CPU only).

References used: torch's bf16/fp16 -> fp32 conversions (library), pure-Python
loops on small inputs (brute force), exact rational arithmetic with
fractions.Fraction, the numbers the pages print, and invariants that follow
from scale = amax / 448.
"""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from conftest import golden_facts

ALL16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def f32_nearest(fr):
    """Round a Fraction to the nearest float32 (ties to even), by brute force on
    the float32 neighbours of its float64 approximation."""
    approx = np.float32(float(fr))
    cands = {approx, np.nextafter(approx, np.float32(np.inf)), np.nextafter(approx, np.float32(-np.inf))}
    best = None
    for c in cands:
        if not np.isfinite(c):
            continue
        d = abs(Fraction(float(c)) - fr)
        key = (d, int(np.float32(c).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def e4m3_nearest(fr, negative):
    """Nearest e4m3 code to the rational |fr| (ties to even code), saturating."""
    a = abs(fr)
    if a >= 448:
        return 0xFE if negative else 0x7E
    best = None
    for c in range(0x7F):
        d = abs(Fraction(float(oracle.decode_e4m3(np.uint8(c)))) - a)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1] | (0x80 if negative else 0)


# ---------------------------------------------------------------- conversion

def test_input_conversion_all_patterns_vs_torch():
    for dt, tdt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
        ours = oracle.input_to_f32(ALL16, dt)
        ref = torch.from_numpy(ALL16.view(np.int16).copy()).view(tdt).float().numpy()
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(ours), nan)
        assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _agrees_to_printed_digits(value, printed, digits):
    """|value - printed| is below one unit in the last printed significant digit."""
    unit = 10.0 ** (np.floor(np.log10(abs(printed))) - (digits - 1))
    return abs(float(value) - printed) < unit


def test_input_ranges_match_pages_table():
    g = golden_facts()
    f16 = oracle.input_to_f32(ALL16, "f16")
    pos = f16[np.isfinite(f16) & (f16 > 0)]
    # the table prints the smallest positive (subnormal) and the largest finite fp16 value
    assert _agrees_to_printed_digits(pos.min(), g["fp16_range"][0], 2)
    assert _agrees_to_printed_digits(pos.max(), g["fp16_range"][1], 2)
    # bf16: the smallest normal and the largest finite value
    b16 = oracle.input_to_f32(ALL16, "bf16")
    normal = b16[np.isfinite(b16) & (b16 >= np.float32(2.0 ** -126))]
    assert _agrees_to_printed_digits(normal.min(), g["bf16_range"][0], 3)
    assert _agrees_to_printed_digits(normal.max(), g["bf16_range"][1], 2)


# ---------------------------------------------------------------- amax

def brute_amax(vals):
    m = 0.0
    for v in vals:
        if math.isnan(v):
            return math.nan
        m = max(m, abs(v))
    return m


def test_amax_per_tensor_brute_force():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(777) * 3).astype(np.float32)
    assert oracle.amax_per_tensor(x) == brute_amax(x.tolist())
    x[5] = -1e20
    assert oracle.amax_per_tensor(x) == np.float32(1e20)
    x[9] = np.inf
    assert oracle.amax_per_tensor(x) == np.inf
    x[11] = np.nan
    assert np.isnan(oracle.amax_per_tensor(x))
    assert oracle.amax_per_tensor(np.zeros((0, 5), np.float32)) == 0


def test_amax_all_bf16_patterns():
    x = oracle.input_to_f32(ALL16, "bf16")
    assert np.isnan(oracle.amax_per_tensor(x))
    fin = x[np.isfinite(x)]
    assert oracle.amax_per_tensor(fin) == np.float32(3.3895313892515355e38)   # bf16 max finite
    noninf = x[~np.isnan(x)]
    assert oracle.amax_per_tensor(noninf) == np.inf


@pytest.mark.parametrize("shape,gr,gc", [((3, 300), 1, 128), ((130, 260), 128, 128),
                                         ((5, 128), 1, 128), ((1, 7), 1, 128), ((129, 129), 128, 128)])
def test_amax_groups_brute_force(shape, gr, gc):
    rng = np.random.default_rng(sum(shape))
    x = rng.standard_normal(shape).astype(np.float32) * np.exp2(rng.integers(-20, 20, shape)).astype(np.float32)
    got = oracle.amax_groups(x, gr, gc)
    R, C = shape
    assert got.shape == (-(-R // gr), -(-C // gc))
    for bi in range(got.shape[0]):
        for bj in range(got.shape[1]):
            vals = [float(x[i, j]) for i in range(bi * gr, min(R, (bi + 1) * gr))
                    for j in range(bj * gc, min(C, (bj + 1) * gc))]
            assert got[bi, bj] == np.float32(brute_amax(vals))


# ---------------------------------------------------------------- scale

def test_scale_closed_forms():
    g = golden_facts()
    assert oracle.scale_from_amax(np.float32(g["e4m3_max"][0])) == 1.0
    for k in range(-100, 101):
        assert oracle.scale_from_amax(np.float32(448.0 * 2.0 ** k)) == np.float32(2.0 ** k)
    assert oracle.scale_from_amax(np.float32(0)) == 1.0          # all-zero reading
    assert np.isnan(oracle.scale_from_amax(np.float32(np.nan)))
    assert oracle.scale_from_amax(np.float32(np.inf)) == np.inf


def test_scale_is_correctly_rounded_division():
    rng = np.random.default_rng(3)
    samples = [np.float32(v) for v in oracle.input_to_f32(rng.integers(1, 0x7F80, 400).astype(np.uint16), "bf16")]
    samples += [np.float32(v) for v in oracle.input_to_f32(rng.integers(1, 0x7C00, 400).astype(np.uint16), "f16")]
    samples += [np.float32(2.0 ** -133), np.float32(3 * 2.0 ** -133), np.float32(2.0 ** -126), np.float32(2.0 ** -24)]
    for a in samples:
        want = f32_nearest(Fraction(float(a)) / 448)
        got = oracle.scale_from_amax(a)
        assert got.view(np.uint32) == want.view(np.uint32), (a, got, want)
    # subnormal scale survives: smallest bf16 subnormal / 448 = 146.29 * 2^-149 -> 146 * 2^-149
    assert oracle.scale_from_amax(np.float32(2.0 ** -133)).view(np.uint32) == 146


# ---------------------------------------------------------------- quantize

def test_quantize_matches_rational_definition():
    """q = e4m3(RN32(x / s)) with s = RN32(amax / 448), checked with Fractions."""
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 0x7F80, (4, 64)).astype(np.uint16) | (rng.integers(0, 2, (4, 64)) << 15).astype(np.uint16)
    q, s = oracle.quantize_per_tensor(bits, "bf16")
    x = oracle.input_to_f32(bits, "bf16")
    amax = max(abs(float(v)) for v in x.ravel())
    s_want = f32_nearest(Fraction(amax) / 448)
    assert s.view(np.uint32) == s_want.view(np.uint32)
    for xv, qv in zip(x.ravel(), q.ravel()):
        quot = f32_nearest(Fraction(float(xv)) / Fraction(float(s_want)))
        want = e4m3_nearest(Fraction(float(quot)), math.copysign(1.0, float(xv)) < 0)
        assert qv == want, (xv, qv, want)


def test_quantize_amax_element_maps_to_448():
    rng = np.random.default_rng(5)
    for dt in ("bf16", "f16"):
        bits = rng.integers(0, 0x7B00, (8, 256)).astype(np.uint16)
        x = oracle.input_to_f32(bits, dt)
        i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
        q, s = oracle.quantize_per_tensor(bits, dt)
        assert q[i] == 0x7E
        neg = bits.copy()
        neg[i] |= 0x8000
        qn, _ = oracle.quantize_per_tensor(neg, dt)
        assert qn[i] == 0xFE


def test_quantize_power_of_two_invariance():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((16, 256)).astype(np.float32)
    from fp8_quantized_gemm_amax_amd.workloads import to_bf16_bits
    bits = to_bf16_bits(x)
    q0, s0 = oracle.quantize_groups(bits, "bf16", 1, 128)
    for j in (-30, -3, 5, 40):
        xs = oracle.input_to_f32(bits, "bf16") * np.float32(2.0 ** j)     # exact in bf16
        q1, s1 = oracle.quantize_groups(to_bf16_bits(xs), "bf16", 1, 128)
        assert np.array_equal(q0, q1)
        assert np.array_equal(s1, (s0 * np.float32(2.0 ** j)).astype(np.float32))


def test_quantize_dequant_error_bound():
    rng = np.random.default_rng(8)
    from fp8_quantized_gemm_amax_amd.workloads import to_bf16_bits
    bits = to_bf16_bits(rng.standard_t(4, (64, 512)))
    q, s = oracle.quantize_groups(bits, "bf16", 1, 128)
    x = oracle.input_to_f32(bits, "bf16").astype(np.float64)
    se = np.repeat(s.astype(np.float64), 128, axis=1)
    deq = oracle.decode_e4m3(q) * se
    # half an e4m3 spacing at |x/s| (2^-4 relative for normals, 2^-10 absolute for subnormals),
    # widened by one float32 rounding of the quotient
    t = np.abs(x / se)
    spacing = np.where(t >= 2.0 ** -6, np.exp2(np.floor(np.log2(np.maximum(t, 2.0 ** -6))) - 3), 2.0 ** -9)
    assert np.all(np.abs(deq - x) <= (0.5 * spacing * (1 + 2.0 ** -20) + t * 2.0 ** -23) * se)


def test_quantize_zero_and_special_groups():
    bits = np.zeros((2, 256), np.uint16)
    bits[0, 128:] = 0x8000                  # -0.0 in the second group of row 0
    bits[1, 3] = 0x7FC0                     # NaN in group 0 of row 1
    bits[1, 130] = 0x7F80                   # +inf in group 1 of row 1
    bits[1, 131] = 0x3F80                   # 1.0 next to it
    bits[1, 132] = 0xFF80                   # -inf
    q, s = oracle.quantize_groups(bits, "bf16", 1, 128)
    assert s[0, 0] == 1.0 and s[0, 1] == 1.0
    assert np.all(q[0, :128] == 0x00) and np.all(q[0, 128:] == 0x80)
    assert np.isnan(s[1, 0]) and np.all(q[1, :128] == 0x7F)
    assert s[1, 1] == np.inf
    assert q[1, 130] == 0x7F and q[1, 132] == 0x7F      # inf / inf
    assert q[1, 131] == 0x00                            # 1 / inf = +0
    assert np.all(q[1, 133:] == 0x00)


def test_quantize_groups_vs_brute_force_ragged():
    rng = np.random.default_rng(9)
    for (R, C, gr) in [(3, 200, 1), (130, 136, 128)]:
        bits = rng.integers(0, 0x4400, (R, C)).astype(np.uint16) | (rng.integers(0, 2, (R, C)) << 15).astype(np.uint16)
        q, s = oracle.quantize_groups(bits, "bf16", gr, 128)
        x = oracle.input_to_f32(bits, "bf16")
        for bi in range(s.shape[0]):
            for bj in range(s.shape[1]):
                rows = range(bi * gr, min(R, (bi + 1) * gr))
                cols = range(bj * 128, min(C, (bj + 1) * 128))
                am = brute_amax([float(x[i, j]) for i in rows for j in cols])
                sw = np.float32(1.0) if am == 0 else f32_nearest(Fraction(am) / 448)
                assert s[bi, bj].view(np.uint32) == sw.view(np.uint32)
        # spot-check codes of a few elements against the rational definition
        for _ in range(200):
            i, j = rng.integers(0, R), rng.integers(0, C)
            sv = s[i // gr, j // 128]
            quot = f32_nearest(Fraction(float(x[i, j])) / Fraction(float(sv)))
            assert q[i, j] == e4m3_nearest(Fraction(float(quot)), bool(np.signbit(x[i, j])))


def test_quantize_with_scale_saturates():
    x = np.array([1.0, 500.0, -1000.0, 0.001], np.float32)
    q = oracle.quantize_with_scale(x, np.float32(1.0))
    assert list(q) == [0x38, 0x7E, 0xFE, oracle.encode_e4m3(np.float32(0.001))]


def test_nan_results_are_canonical():
    x = np.array([[1.0, np.float32(np.nan), 2.0]], np.float32)
    x[0, 1] = np.array([0x7FC12345], np.uint32).view(np.float32)[0]      # NaN with a payload
    assert oracle.amax_per_tensor(x).view(np.uint32) == 0x7FC00000
    assert oracle.amax_groups(x, 1, 128).view(np.uint32)[0, 0] == 0x7FC00000
    assert oracle.scale_from_amax(np.float32(np.nan)).view(np.uint32) == 0x7FC00000

