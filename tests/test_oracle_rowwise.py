"""Pins for the oracle's per-channel (rowwise) scaling (CPU only).

References used: the per-tensor quantizer applied to each row alone, brute-force nearest
e4m3 search in exact rationals, a triple loop in exact rationals for the product, the
tensorwise product (equal scales), and invariances that a wrong axis would break.
"""

from fractions import Fraction

import numpy as np

import oracle
from oracle.rowwise import amax_rows, quantize_rowwise, gemm_rowwise_ref, bound_rowwise


def bf16(a):
    return (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_each_row_is_a_per_tensor_quantize():
    rng = np.random.default_rng(1)
    x = rng.standard_t(3, (7, 300)) * np.exp(rng.normal(0, 2, (7, 1)))
    bits = bf16(x)
    q, s = quantize_rowwise(bits, "bf16")
    assert q.shape == (7, 300) and s.shape == (7,)
    for r in range(7):
        qr, sr = oracle.quantize_per_tensor(bits[r:r + 1], "bf16")
        np.testing.assert_array_equal(q[r:r + 1], qr)
        assert s[r] == sr


def test_rowwise_brute_force_small():
    """3 x 5 by hand: the scale of each row is float32(max|row| / 448); each code is the
    nearest e4m3 value of the float32 quotient (ties to the even code), saturating."""
    x = np.array([[1.0, -3.5, 0.25, 7.0, -0.0],
                  [100.0, 2.0, -300.0, 0.5, 1e-3],
                  [0.0, 0.0, 0.0, 0.0, 0.0]], np.float32)
    bits = bf16(x)
    x32 = oracle.input_to_f32(bits, "bf16")
    q, s = quantize_rowwise(bits, "bf16")
    mags = [Fraction(float(v)) for v in oracle.positive_values()]
    for r in range(3):
        amax = max(abs(float(v)) for v in x32[r])
        want_s = np.float32(1.0) if amax == 0 else np.float32(np.float32(amax) / np.float32(448))
        assert s[r] == want_s
        for c in range(5):
            t = Fraction(float(np.float32(x32[r, c]) / want_s))
            code = 0x7E if abs(t) >= 448 else min(range(127), key=lambda i: (abs(mags[i] - abs(t)), i & 1))
            code |= 0x80 if np.signbit(x32[r, c]) else 0
            assert int(q[r, c]) == code, (r, c)


def test_rowwise_scale_invariance_and_special_rows():
    """Scaling one row by 2^k leaves every code alone and multiplies only that row's
    scale by 2^k (a column-wise or whole-tensor amax would change other rows); a zero row
    gets scale 1 and zero codes; a NaN makes only its own row NaN."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 256)).astype(np.float32)
    q0, s0 = quantize_rowwise(bf16(x), "bf16")
    y = x.copy()
    y[2] *= np.float32(2.0 ** 9)
    q1, s1 = quantize_rowwise(bf16(y), "bf16")
    np.testing.assert_array_equal(q0, q1)
    assert s1[2] == s0[2] * np.float32(2.0 ** 9)
    np.testing.assert_array_equal(np.delete(s1, 2), np.delete(s0, 2))
    z = x.copy()
    z[1] = 0.0
    z[3, 17] = np.nan
    q2, s2 = quantize_rowwise(bf16(z), "bf16")
    assert s2[1] == 1.0 and not q2[1].any()
    assert np.isnan(s2[3]) and (q2[3] == 0x7F).all()
    np.testing.assert_array_equal(q2[[0, 2]], q0[[0, 2]])
    np.testing.assert_array_equal(amax_rows(np.zeros((3, 0), np.float32)), np.zeros(3, np.float32))


def test_gemm_rowwise_exact_triple_loop():
    """sum_k (dec(qa) sa[m]) (dec(qb) sb[n]) in exact rationals; distinct scales per row
    and per column catch a transposed or swapped scale vector."""
    rng = np.random.default_rng(3)
    M, N, K = 3, 5, 48
    qa = rng.integers(0, 256, (M, K)).astype(np.uint8)
    qb = rng.integers(0, 256, (N, K)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x11
    qb[(qb & 0x7F) == 0x7F] = 0x22
    sa = (2.0 ** rng.uniform(-8, 8, M)).astype(np.float32)
    sb = (2.0 ** rng.uniform(-8, 8, N)).astype(np.float32)
    da, db = oracle.decode_e4m3(qa), oracle.decode_e4m3(qb)
    got = gemm_rowwise_ref(qa, sa, qb, sb)
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(float(da[m, k])) * Fraction(float(sa[m])) *
                        Fraction(float(db[n, k])) * Fraction(float(sb[n])) for k in range(K))
            assert abs(Fraction(float(got[m, n])) - exact) <= abs(exact) * Fraction(1, 2 ** 52), (m, n)
    bnd = bound_rowwise(qa, sa, qb, sb)
    assert (bnd >= np.abs(got) * (1 - 2.0 ** -50)).all()


def test_gemm_rowwise_equal_scales_is_tensorwise():
    rng = np.random.default_rng(4)
    qa = rng.integers(0, 0x7E, (6, 64)).astype(np.uint8)
    qb = rng.integers(0, 0x7E, (9, 64)).astype(np.uint8)
    sa, sb = np.float32(0.013), np.float32(3.75)
    r = gemm_rowwise_ref(qa, np.full(6, sa), qb, np.full(9, sb))
    t = oracle.gemm_tensorwise_ref(qa, sa, qb, sb)
    np.testing.assert_array_equal(r, t)
    np.testing.assert_array_equal(bound_rowwise(qa, np.full(6, sa), qb, np.full(9, sb)),
                                  oracle.bound_tensorwise(qa, sa, qb, sb))
