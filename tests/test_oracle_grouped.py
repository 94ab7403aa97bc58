"""Pins for the oracle's grouped (MoE) blockwise GEMM (CPU only).

References used: the dense blockwise product (one expert), an exact rational triple loop
that looks up each row's expert by searching the offsets, the invariance of the result
under relabelling the experts, and empty groups.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.grouped import (offsets_from_sizes, gemm_grouped_blockwise_ref, bound_grouped_blockwise,
                            gemm_grouped_blockwise_ue8m0_ref)

FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def case(sizes, N, K, seed):
    rng = np.random.default_rng(seed)
    E, T = len(sizes), int(np.sum(sizes))
    qa = rng.choice(FINITE, (T, K))
    qb = rng.choice(FINITE, (E, N, K))
    sa = (2.0 ** rng.uniform(-6, 6, (T, K // 128))).astype(np.float32)
    sb = (2.0 ** rng.uniform(-6, 6, (E, -(-N // 128), K // 128))).astype(np.float32)
    return qa, sa, qb, sb, offsets_from_sizes(sizes)


def test_offsets():
    np.testing.assert_array_equal(offsets_from_sizes([3, 0, 2]), [0, 3, 3, 5])
    np.testing.assert_array_equal(offsets_from_sizes([]), [0])


def test_one_expert_is_the_dense_product():
    qa, sa, qb, sb, off = case([37], 200, 256, 1)
    np.testing.assert_array_equal(gemm_grouped_blockwise_ref(qa, sa, qb, sb, off),
                                  oracle.gemm_blockwise_ref(qa, sa, qb[0], sb[0]))
    np.testing.assert_array_equal(bound_grouped_blockwise(qa, sa, qb, sb, off),
                                  oracle.bound_blockwise(qa, sa, qb[0], sb[0]))


def test_exact_triple_loop_with_empty_groups():
    """Sizes [2, 0, 3, 1] (an empty expert between two others), N = 130 (two weight-block
    rows), K = 256 (two slabs): every output against an exact rational sum over k with the
    row's expert found by searching the offsets and the block indices written out."""
    sizes = [2, 0, 3, 1]
    qa, sa, qb, sb, off = case(sizes, 130, 256, 2)
    got = gemm_grouped_blockwise_ref(qa, sa, qb, sb, off)
    da, db = oracle.decode_e4m3(qa), oracle.decode_e4m3(qb)
    for t in range(qa.shape[0]):
        e = int(np.searchsorted(off, t, side="right") - 1)
        for n in (0, 1, 127, 128, 129):
            terms = [Fraction(float(da[t, k])) * Fraction(float(db[e, n, k])) *
                     Fraction(float(sa[t, k // 128])) * Fraction(float(sb[e, n // 128, k // 128]))
                     for k in range(256)]
            exact, mag = sum(terms), sum(abs(x) for x in terms)
            assert abs(Fraction(float(got[t, n])) - exact) <= mag * Fraction(1, 2 ** 50), (t, n)


def test_relabelling_experts_moves_their_rows():
    """Swap experts 0 and 2 (weights and segments): the output rows move with them, so the
    result depends on the pairing of segment and weight, not on the order of the experts."""
    sizes = [3, 4, 5]
    qa, sa, qb, sb, off = case(sizes, 64, 128, 3)
    c = gemm_grouped_blockwise_ref(qa, sa, qb, sb, off)
    seg = [np.arange(off[e], off[e + 1]) for e in range(3)]
    perm = np.concatenate([seg[2], seg[1], seg[0]])
    c2 = gemm_grouped_blockwise_ref(qa[perm], sa[perm], qb[[2, 1, 0]], sb[[2, 1, 0]],
                                    offsets_from_sizes([5, 4, 3]))
    np.testing.assert_array_equal(c2, c[perm])
    # pairing a segment with the wrong expert changes it
    c3 = gemm_grouped_blockwise_ref(qa, sa, qb[[1, 0, 2]], sb[[1, 0, 2]], off)
    assert not np.array_equal(c3[:3], c[:3])


def test_ue8m0_grouped_is_the_decoded_float_product():
    rng = np.random.default_rng(4)
    sizes = [5, 0, 7]
    T, N, K = 12, 140, 256
    qa, qb = rng.choice(FINITE, (T, K)), rng.choice(FINITE, (3, N, K))
    ea = rng.integers(110, 140, (T, 2)).astype(np.uint8)
    eb = rng.integers(110, 140, (3, 2, 2)).astype(np.uint8)
    off = offsets_from_sizes(sizes)
    got = gemm_grouped_blockwise_ue8m0_ref(qa, ea, qb, eb, off)
    want = gemm_grouped_blockwise_ref(qa, np.exp2(ea.astype(np.float64) - 127).astype(np.float32), qb,
                                      np.exp2(eb.astype(np.float64) - 127).astype(np.float32), off)
    np.testing.assert_array_equal(got, want)


def test_offsets_must_cover_the_rows():
    qa, sa, qb, sb, off = case([2, 2], 16, 128, 5)
    with pytest.raises(AssertionError):
        gemm_grouped_blockwise_ref(qa, sa, qb, sb, np.array([0, 2, 3]))
    with pytest.raises(AssertionError):
        gemm_grouped_blockwise_ref(qa, sa, qb, sb, np.array([0, 3, 2]))


def test_ue8m0_grouped_bound_exact_and_decoded():
    """bound_grouped_blockwise_ue8m0 is the magnitude term of the grouped UE8M0 tolerance.
    Pinned three ways: it equals the float-scale grouped bound with the bytes decoded to
    2^(c - 127); a few entries equal an exact rational sum over k of
    |dec(qa)·2^(ea-127)|·|dec(qb)·2^(eb-127)| with the row's expert found by searching the
    offsets (taking the scale bytes as plain numbers instead would miss by a factor of about
    127^2 and fail here); and it is at least |C| everywhere, with equality where every
    product of a row and column has one sign."""
    from oracle.grouped import bound_grouped_blockwise_ue8m0
    rng = np.random.default_rng(7)
    sizes = [3, 0, 4]
    T, N, K = 7, 140, 256
    qa, qb = rng.choice(FINITE, (T, K)), rng.choice(FINITE, (3, N, K))
    ea = rng.integers(112, 142, (T, 2)).astype(np.uint8)
    eb = rng.integers(112, 142, (3, 2, 2)).astype(np.uint8)
    off = offsets_from_sizes(sizes)
    got = bound_grouped_blockwise_ue8m0(qa, ea, qb, eb, off)
    dec = lambda e: np.exp2(e.astype(np.float64) - 127).astype(np.float32)
    np.testing.assert_array_equal(got, bound_grouped_blockwise(qa, dec(ea), qb, dec(eb), off))
    da, db = oracle.decode_e4m3(qa), oracle.decode_e4m3(qb)
    for t in (0, 2, 3, 6):
        e = int(np.searchsorted(off, t, side="right") - 1)
        for n in (0, 127, 128, 139):
            mag = sum(abs(Fraction(float(da[t, k])) * Fraction(2) ** (int(ea[t, k // 128]) - 127) *
                          Fraction(float(db[e, n, k])) * Fraction(2) ** (int(eb[e, n // 128, k // 128]) - 127))
                      for k in range(K))
            assert abs(Fraction(float(got[t, n])) - mag) <= mag * Fraction(1, 2 ** 50), (t, n)
    c = gemm_grouped_blockwise_ue8m0_ref(qa, ea, qb, eb, off)
    assert np.all(got >= np.abs(c))
    # one sign everywhere: the bound equals |C|
    qa1, qb1 = qa & 0x7F, qb & 0x7F
    np.testing.assert_allclose(bound_grouped_blockwise_ue8m0(qa1, ea, qb1, eb, off),
                               np.abs(gemm_grouped_blockwise_ue8m0_ref(qa1, ea, qb1, eb, off)), rtol=1e-14)
