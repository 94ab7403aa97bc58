"""Pins for the oracle's e4m3fn decoder and encoder (CPU only).

Every check compares the oracle with something other than itself: numbers the
pages print (tests/golden/pages_facts.txt), torch's own float8_e4m3fn dtype,
or closed-form facts about the code space.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from conftest import golden_facts

ALL = np.arange(256, dtype=np.uint8)


def torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).float().numpy()


def torch_encode(v32):
    """torch's CPU cast (round to nearest even, non-saturating above 464)."""
    return torch.from_numpy(np.asarray(v32, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_matches_pages_facts():
    g = golden_facts()
    dec = oracle.decode_e4m3(ALL)
    finite = dec[np.isfinite(dec)]
    assert finite.max() == g["e4m3_max"][0] == oracle.E4M3_MAX
    assert finite.min() == g["e4m3_range"][0] and finite.max() == g["e4m3_range"][1]
    # 2^(exponent bits) binades of 2^(mantissa bits) codes each, per sign
    e_bits, m_bits = int(g["e4m3_exponent_bits"][0]), int(g["e4m3_mantissa_bits"][0])
    assert 2 * (2 ** e_bits) * (2 ** m_bits) == 256
    # largest finite = (2 - 2*2^-m) * 2^(2^e - 1 - bias) with bias 2^(e-1)-1 and the top code NaN
    bias = 2 ** (e_bits - 1) - 1
    assert (2 - 2 * 2.0 ** -m_bits) * 2.0 ** (2 ** e_bits - 1 - bias) == 448


def test_decode_all_codes_vs_torch():
    ours = oracle.decode_e4m3(ALL)
    ref = torch_decode(ALL).astype(np.float64)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))


def test_decode_special_codes():
    d = oracle.decode_e4m3(ALL)
    assert d[0x00] == 0 and not np.signbit(d[0x00])
    assert d[0x80] == 0 and np.signbit(d[0x80])
    assert d[0x01] == 2.0 ** -9            # smallest subnormal
    assert d[0x07] == 7 * 2.0 ** -9         # largest subnormal
    assert d[0x08] == 2.0 ** -6             # smallest normal
    assert d[0x38] == 1.0
    assert d[0x7E] == 448 and d[0xFE] == -448
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF])
    assert int(np.isnan(d).sum()) == 2      # "fn": no infinities, one NaN per sign
    pos = oracle.positive_values()
    assert len(pos) == 127 and np.all(np.diff(pos) > 0)
    assert np.array_equal(d[0x80:0xFF], -pos)


def test_encode_round_trip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.decode_e4m3(codes).astype(np.float32)
    assert np.array_equal(oracle.encode_e4m3(vals), codes)


def test_encode_midpoints_ties_to_even_and_neighbours():
    pos = oracle.positive_values()
    lo, hi = pos[:-1], pos[1:]
    mid = ((lo + hi) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)   # midpoints are exact in fp32
    codes_lo = np.arange(0, 126)
    even = np.where(codes_lo % 2 == 0, codes_lo, codes_lo + 1)
    assert np.array_equal(oracle.encode_e4m3(mid), even.astype(np.uint8))
    assert np.array_equal(oracle.encode_e4m3(-mid), (even | 0x80).astype(np.uint8))
    up = np.nextafter(mid, np.float32(np.inf))
    dn = np.nextafter(mid, np.float32(0))
    assert np.array_equal(oracle.encode_e4m3(up), (codes_lo + 1).astype(np.uint8))
    assert np.array_equal(oracle.encode_e4m3(dn), codes_lo.astype(np.uint8))
    # subnormal edge cases: 2^-10 is the tie between 0 and 2^-9 -> 0; 3*2^-10 -> code 2
    assert oracle.encode_e4m3(np.float32(2.0 ** -10)) == 0x00
    assert oracle.encode_e4m3(np.float32(3 * 2.0 ** -10)) == 0x02
    assert oracle.encode_e4m3(np.float32(-2.0 ** -10)) == 0x80


def test_encode_saturation_nan_and_zero():
    big = np.array([448, 449, 463.99, 464, 465, 480, 1e4, 3.4e38, np.inf], dtype=np.float32)
    assert np.all(oracle.encode_e4m3(big) == 0x7E)
    assert np.all(oracle.encode_e4m3(-big) == 0xFE)
    nan = np.array([np.nan, -np.nan], dtype=np.float32)
    assert np.all(oracle.encode_e4m3(nan) == 0x7F)
    z = np.array([0.0, -0.0, 1e-30, -1e-30, 2.0 ** -149, -(2.0 ** -149)], dtype=np.float32)
    assert list(oracle.encode_e4m3(z)) == [0x00, 0x80, 0x00, 0x80, 0x00, 0x80]


def test_encode_vs_torch_dense_sample():
    # every 61st non-negative fp32 pattern up to 464 (torch saturates to NaN above), both signs
    pats = np.arange(0, 0x43E80000, 61, dtype=np.uint32)
    v = pats.view(np.float32)
    v = np.concatenate([v, -v])
    assert np.array_equal(oracle.encode_e4m3(v), torch_encode(v))


def test_breakpoints_vs_torch():
    bp = oracle.nonneg_breakpoints()
    assert len(bp) == 126 and np.all(np.diff(bp.astype(np.int64)) > 0)
    below = (bp - 1).view(np.float32)
    at = bp.view(np.float32)
    t_below = torch_encode(below).astype(int)
    t_at = torch_encode(at).astype(int)
    assert np.array_equal(t_at, t_below + 1)
    assert np.array_equal(t_at, np.arange(1, 127))
    # the first step is just above 2^-10 (the tie at 2^-10 goes to 0); the last at 432 (tie -> 448)
    assert bp[0] == np.float32(2.0 ** -10).view(np.uint32) + 1
    assert bp[-1] == np.float32(432.0).view(np.uint32)


@pytest.mark.parametrize("seed", [0, 1])
def test_encode_random_patterns_vs_torch(seed):
    rng = np.random.default_rng(seed)
    pats = rng.integers(0, 0x43E80000, 2_000_000, dtype=np.uint32)
    v = pats.view(np.float32)
    v = np.where(rng.random(v.shape) < 0.5, -v, v).astype(np.float32)
    assert np.array_equal(oracle.encode_e4m3(v), torch_encode(v))


def test_encode_nearest_by_brute_force():
    """Pure-Python nearest-code search over all 254 finite values on random inputs."""
    rng = np.random.default_rng(7)
    vals = (rng.standard_normal(3000) * np.exp2(rng.integers(-12, 9, 3000))).astype(np.float32)
    table = [(float(oracle.decode_e4m3(np.uint8(c))), c) for c in range(256) if c not in (0x7F, 0xFF)]
    for v, got in zip(vals, oracle.encode_e4m3(vals)):
        v = float(v)
        if abs(v) >= 448:
            want = 0xFE if v < 0 else 0x7E
        else:
            best = None
            for val, c in table:
                if (c & 0x80) != (0x80 if math.copysign(1.0, v) < 0 else 0):
                    continue
                d = abs(val - v)
                if best is None or d < best[0] or (d == best[0] and (c & 1) == 0):
                    best = (d, c)
            want = best[1]
        assert got == want, (v, got, want)
