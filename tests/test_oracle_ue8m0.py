"""Pins for the oracle's UE8M0 (power-of-two) block scales (CPU only).

References used: torch's float8_e8m0fnu dtype (library decode of all 256 codes; its
float -> e8m0 cast rounds to the nearest power of two, a different reading, so it is
not used), numpy.frexp, exact rational arithmetic with fractions.Fraction, brute force
over the 255 finite codes, the
float32-scale quantizer on blocks whose amax / 448 is a power of two, and a
pure-Python triple loop for the product.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle.ue8m0 import (e8m0_decode, e8m0_from_amax, quantize_groups_ue8m0,
                          gemm_blockwise_ue8m0_ref, bound_blockwise_ue8m0)

ALL16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def positive_finite(dtype):
    x = oracle.input_to_f32(ALL16, dtype)
    return np.unique(x[np.isfinite(x) & (x > 0)])


def test_decode_matches_torch_e8m0fnu():
    codes = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(codes).view(torch.float8_e8m0fnu).double().numpy()
    ours = e8m0_decode(codes)
    assert np.isnan(ours[255]) and np.isnan(lib[255])
    np.testing.assert_array_equal(ours[:255], lib[:255])
    # each code is twice the one before
    np.testing.assert_array_equal(ours[1:255], 2 * ours[:254])


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_scale_code_matches_frexp(dtype):
    """For every positive finite bf16 / fp16 amax whose amax / 448 lies in the byte's
    range: with amax / 448 = m * 2^p (numpy.frexp, 0.5 <= m < 1), the smallest power
    of two not below it is 2^(p - 1) when m = 0.5 and 2^p otherwise.  The float64
    quotient decides as the exact one would: away from a power of two it differs from
    one by at least the input's relative spacing (2^-11 or more)."""
    a = positive_finite(dtype)
    q = a.astype(np.float64) / 448.0
    inside = (q >= 2.0 ** -127) & (q <= 2.0 ** 127)
    a, q = a[inside], q[inside]
    m, p = np.frexp(q)
    want = (np.where(m == 0.5, p - 1, p) + 127).astype(np.uint8)
    np.testing.assert_array_equal(e8m0_from_amax(a), want)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_scale_code_is_smallest_power_not_below(dtype):
    """Exact rationals over every positive finite input value: 448 * s >= amax and,
    unless the code is the smallest one, 448 * s / 2 < amax."""
    for v in positive_finite(dtype):
        c = int(e8m0_from_amax(np.float32(v)))
        s = Fraction(2) ** (c - 127)
        assert 448 * s >= Fraction(float(v)), (v, c)
        assert c == 0 or 448 * s / 2 < Fraction(float(v)), (v, c)


def test_scale_code_brute_force_over_codes():
    """The smallest of the 255 finite codes whose value times 448 reaches amax, found
    by trying them all, on random and edge amax values."""
    rng = np.random.default_rng(7)
    vals = np.concatenate([
        np.float32(448.0) * np.float32(2.0) ** rng.integers(-120, 120, 64).astype(np.float32),
        (rng.standard_normal(200) * 10.0 ** rng.integers(-30, 30, 200)).astype(np.float32),
        np.array([448, 449, 447, 224, 225, 1, 1e-38, 3e38, 2 ** -133], np.float32)])
    vals = np.abs(vals[vals != 0]).astype(np.float32)
    for v in vals:
        want = next((c for c in range(255) if 448 * Fraction(2) ** (c - 127) >= Fraction(float(v))), 254)
        assert int(e8m0_from_amax(v)) == want, v


def test_scale_code_special_values():
    assert int(e8m0_from_amax(np.float32(448.0))) == 127
    assert int(e8m0_from_amax(np.float32(896.0))) == 128
    assert int(e8m0_from_amax(np.nextafter(np.float32(448.0), np.float32(np.inf)))) == 128
    assert int(e8m0_from_amax(np.float32(0.0))) == 127                  # all-zero block: 2^0
    assert int(e8m0_from_amax(np.float32(np.nan))) == 255
    assert int(e8m0_from_amax(np.float32(np.inf))) == 255
    assert int(e8m0_from_amax(np.float32(1e-45))) == 0                   # clamped to 2^-127


def test_quantize_power_of_two_amax_matches_float32_scales():
    """When every block's amax is 448 * 2^k, amax / 448 is exactly 2^k, so the
    float32-scale quantizer uses the same scale and must give the same codes."""
    rng = np.random.default_rng(3)
    R, C = 5, 384
    x = rng.standard_normal((R, C)) * 0.3
    ks = rng.integers(-20, 20, (R, C // 128))
    for r in range(R):
        for g in range(C // 128):
            blk = x[r, g * 128:(g + 1) * 128]
            blk *= 2.0 ** ks[r, g]
            blk[rng.integers(0, 128)] = 448.0 * 2.0 ** ks[r, g] * rng.choice([-1, 1])
    bits = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)   # exact: 448*2^k has 3 bits
    x32 = oracle.input_to_f32(bits, "bf16")
    assert np.all(oracle.amax_groups(x32, 1, 128) == (448.0 * 2.0 ** ks).astype(np.float32))
    q, codes = quantize_groups_ue8m0(bits, "bf16", 1, 128)
    q32, s32 = oracle.quantize_groups(bits, "bf16", 1, 128)
    np.testing.assert_array_equal(codes, (ks + 127).astype(np.uint8))
    np.testing.assert_array_equal(s32, (2.0 ** ks).astype(np.float32))
    np.testing.assert_array_equal(q, q32)


def test_quantize_brute_force_small():
    """Each code is the nearest e4m3 value (ties to the even code) to x / 2^e, found by
    a search over all 127 magnitudes in exact rationals."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((3, 200)) * 10.0 ** rng.integers(-3, 4, (3, 200))).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    q, codes = quantize_groups_ue8m0(bits, "bf16", 1, 128)
    x32 = oracle.input_to_f32(bits, "bf16")
    mags = [Fraction(float(v)) for v in oracle.positive_values()]
    for r in range(3):
        for c in range(200):
            s = Fraction(2) ** (int(codes[r, c // 128]) - 127)
            t = Fraction(float(x32[r, c])) / s
            best = min(range(127), key=lambda i: (abs(mags[i] - abs(t)), i & 1))
            want = best | (0x80 if x32[r, c] < 0 else 0)
            assert int(q[r, c]) == want, (r, c)


def test_quantize_never_saturates_and_uses_the_top_binade():
    """With the smallest power of two not below amax / 448, every |code| <= 448 and each
    block's largest element lands above 224 (unless its block is all zero)."""
    rng = np.random.default_rng(9)
    x = (rng.standard_t(4, (300, 640)) * np.exp(rng.standard_normal((1, 640)))).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    for gr in (1, 128):
        q, codes = quantize_groups_ue8m0(bits, "bf16", gr, 128)
        d = np.abs(oracle.decode_e4m3(q))
        assert np.all(d <= 448)
        rows = -(-300 // gr)
        pad = np.zeros((rows * gr, 640))
        pad[:300] = d
        gm = pad.reshape(rows, gr, 5, 128).max(axis=(1, 3))
        assert np.all(gm >= 224)      # amax / s > 224, and e4m3 rounds it to 224 or above


def test_quantize_special_blocks():
    x = np.zeros((3, 256), np.uint16)
    x[1, 5] = 0x7FC0          # NaN in group (1, 0)
    x[2, 130] = 0x7F80        # +inf in group (2, 1)
    x[2, 0] = 0x3F80          # 1.0 in group (2, 0)
    q, codes = quantize_groups_ue8m0(x, "bf16", 1, 128)
    assert codes[0, 0] == 127 and np.all(q[0] == 0)                  # zero group
    assert codes[1, 0] == 255 and np.all((q[1, :128] & 0x7F) == 0x7F)  # NaN scale -> NaN codes
    assert codes[2, 1] == 255 and np.all((q[2, 128:] & 0x7F) == 0x7F)
    assert codes[2, 0] == 127 - 8    # amax 1.0: 448 * 2^-9 < 1 <= 448 * 2^-8


def test_gemm_exact_rationals():
    """Two slabs, one output: C = 2^(1+3) * (slab 0 sum) + 2^(-2+0) * (slab 1 sum)."""
    rng = np.random.default_rng(1)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    qa, qb = rng.choice(finite, (1, 256)), rng.choice(finite, (1, 256))
    ea = np.array([[128, 125]], np.uint8)
    eb = np.array([[130, 127]], np.uint8)
    da = [Fraction(float(v)) for v in oracle.decode_e4m3(qa[0])]
    db = [Fraction(float(v)) for v in oracle.decode_e4m3(qb[0])]
    s0 = sum(da[k] * db[k] for k in range(128))
    s1 = sum(da[k] * db[k] for k in range(128, 256))
    want = Fraction(2) ** 4 * s0 + Fraction(1, 4) * s1
    got = gemm_blockwise_ue8m0_ref(qa, ea, qb, eb)
    assert Fraction(float(got[0, 0])) == want
    bnd = bound_blockwise_ue8m0(qa, ea, qb, eb)
    want_b = Fraction(2) ** 4 * sum(abs(da[k] * db[k]) for k in range(128)) + \
        Fraction(1, 4) * sum(abs(da[k] * db[k]) for k in range(128, 256))
    assert Fraction(float(bnd[0, 0])) == want_b


def test_gemm_triple_loop_small():
    rng = np.random.default_rng(2)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    M, N, K = 3, 130, 256
    qa, qb = rng.choice(finite, (M, K)), rng.choice(finite, (N, K))
    ea = rng.integers(100, 150, (M, 2)).astype(np.uint8)
    eb = rng.integers(100, 150, (2, 2)).astype(np.uint8)
    got = gemm_blockwise_ue8m0_ref(qa, ea, qb, eb)
    da, db = oracle.decode_e4m3(qa), oracle.decode_e4m3(qb)
    for m in range(M):
        for n in (0, 1, 127, 128, 129):
            want, mag = Fraction(0), Fraction(0)
            for k in range(K):
                g = k // 128
                s = Fraction(2) ** (int(ea[m, g]) - 127) * Fraction(2) ** (int(eb[n // 128, g]) - 127)
                t = Fraction(float(da[m, k])) * Fraction(float(db[n, k])) * s
                want += t
                mag += abs(t)
            # each slab's float64 sum is exact; adding the two slabs rounds once
            assert abs(Fraction(float(got[m, n])) - want) <= mag * Fraction(1, 2 ** 52), (m, n)


def test_gemm_nan_scale_code_propagates():
    qa = np.full((1, 128), 0x38, np.uint8)
    qb = np.full((2, 128), 0x38, np.uint8)
    got = gemm_blockwise_ue8m0_ref(qa, np.array([[255]], np.uint8), qb, np.array([[127]], np.uint8))
    assert np.all(np.isnan(got))
