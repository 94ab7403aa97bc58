"""Pins for the oracle's scaled GEMM references and tolerance check (CPU only).

References: exact rational arithmetic (fractions.Fraction) on tiny products,
one-hot selections, algebraic identities between the tensorwise and blockwise
forms, and the Transformer Engine page's mechanism written with torch's own
float8_e4m3fn dtype and matmul.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from fp8_quantized_gemm_amax_amd import workloads as wl

FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def rand_codes(rng, shape):
    return rng.choice(FINITE, size=shape)


def frac_dec(c):
    return Fraction(float(oracle.decode_e4m3(np.uint8(c))))


@pytest.mark.parametrize("M,N,K", [(3, 5, 16), (8, 8, 128), (2, 7, 256)])
def test_tensorwise_vs_exact_rationals(M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    qa, qb = rand_codes(rng, (M, K)), rand_codes(rng, (N, K))
    sa, sb = np.float32(rng.random() * 3), np.float32(rng.random() * 1e-3)
    c = oracle.gemm_tensorwise_ref(qa, sa, qb, sb)
    for m in range(M):
        for n in range(N):
            exact = sum(frac_dec(qa[m, k]) * frac_dec(qb[n, k]) for k in range(K))
            exact *= Fraction(float(sa)) * Fraction(float(sb))
            assert c[m, n] == float(exact)          # one rounding: float() rounds to nearest


@pytest.mark.parametrize("M,N,K", [(3, 130, 256), (5, 4, 384)])
def test_blockwise_vs_exact_rationals(M, N, K):
    rng = np.random.default_rng(K + N)
    qa, qb = rand_codes(rng, (M, K)), rand_codes(rng, (N, K))
    G = K // 128
    sa = (rng.random((M, G)) * 2).astype(np.float32)
    sb = (rng.random((-(-N // 128), G)) * 0.01).astype(np.float32)
    c = oracle.gemm_blockwise_ref(qa, sa, qb, sb)
    for m in range(M):
        for n in list(range(min(N, 4))) + [N - 1]:
            exact = Fraction(0)
            mag = Fraction(0)
            for g in range(G):
                part = sum(frac_dec(qa[m, k]) * frac_dec(qb[n, k]) for k in range(g * 128, (g + 1) * 128))
                term = part * Fraction(float(sa[m, g])) * Fraction(float(sb[n // 128, g]))
                exact += term
                mag += abs(term)
            # slab sums are exact; each slab adds one product and one sum rounding (2^-53 each)
            assert abs(Fraction(c[m, n]) - exact) <= 2 * G * mag * Fraction(1, 2 ** 53)


def test_one_hot_selects_columns():
    rng = np.random.default_rng(1)
    M, N, K = 6, 9, 144
    qa = rand_codes(rng, (M, K))
    sel = rng.integers(0, K, N)
    qb = np.zeros((N, K), np.uint8)
    qb[np.arange(N), sel] = 0x38                     # 1.0
    sa, sb = np.float32(0.75), np.float32(2.0)
    c = oracle.gemm_tensorwise_ref(qa, sa, qb, sb)
    want = oracle.decode_e4m3(qa)[:, sel] * 1.5
    assert np.array_equal(c, want)


def test_blockwise_constant_scales_equals_tensorwise():
    rng = np.random.default_rng(2)
    M, N, K = 7, 300, 512
    qa, qb = rand_codes(rng, (M, K)), rand_codes(rng, (N, K))
    sa, sb = np.float32(0.125), np.float32(3.0)      # powers-of-two-friendly: no rounding
    ct = oracle.gemm_tensorwise_ref(qa, sa, qb, sb)
    cb = oracle.gemm_blockwise_ref(qa, np.full((M, K // 128), sa), qb, np.full((3, K // 128), sb))
    assert np.allclose(cb, ct, rtol=1e-14, atol=0)
    # a single slab is the tensorwise product with that slab's scales
    sa1 = (rng.random((M, 1)) + 0.5).astype(np.float32)
    sb1 = (rng.random((3, 1)) + 0.5).astype(np.float32)
    cb1 = oracle.gemm_blockwise_ref(qa[:, :128], sa1, qb[:, :128], sb1)
    for m in range(M):
        for nb in range(3):
            cols = slice(nb * 128, min(N, nb * 128 + 128))
            ct1 = oracle.gemm_tensorwise_ref(qa[m:m + 1, :128], sa1[m, 0], qb[cols, :128], sb1[nb, 0])
            assert np.array_equal(cb1[m:m + 1, cols], ct1)


def test_swap_operands_transposes():
    rng = np.random.default_rng(3)
    qa, qb = rand_codes(rng, (5, 256)), rand_codes(rng, (11, 256))
    c1 = oracle.gemm_tensorwise_ref(qa, 0.5, qb, 0.25)
    c2 = oracle.gemm_tensorwise_ref(qb, 0.25, qa, 0.5)
    assert np.array_equal(c1, c2.T)


def test_bound_dominates_and_is_exact_for_same_signs():
    rng = np.random.default_rng(4)
    qa = rand_codes(rng, (4, 256)) & 0x7F            # all non-negative codes
    qb = rand_codes(rng, (6, 256)) & 0x7F
    qa[qa == 0x7F] = 0x7E
    qb[qb == 0x7F] = 0x7E
    c = oracle.gemm_tensorwise_ref(qa, 0.5, qb, 2.0)
    assert np.array_equal(oracle.bound_tensorwise(qa, 0.5, qb, 2.0), c)
    qs = qa.copy()
    qs[:, ::2] |= 0x80
    assert np.all(oracle.bound_tensorwise(qs, 0.5, qb, 2.0) >= np.abs(oracle.gemm_tensorwise_ref(qs, 0.5, qb, 2.0)))


def test_output_ulp_values():
    assert oracle.output_ulp(1.0, "bf16") == 2.0 ** -7
    assert oracle.output_ulp(1.5, "f16") == 2.0 ** -10
    assert oracle.output_ulp(-1000.0, "bf16") == 2.0 ** (9 - 7)
    assert oracle.output_ulp(0.0, "f16") == 2.0 ** -24
    assert oracle.output_ulp(1e-40, "bf16") == 2.0 ** -133
    # compare with torch's spacing: next representable after 3.0 in bf16
    t = torch.tensor([3.0], dtype=torch.bfloat16)
    nxt = torch.nextafter(t.float(), torch.tensor([4.0])).to(torch.bfloat16)
    assert float(oracle.output_ulp(3.0, "bf16")) == 2.0 ** -6 and float(nxt) == 3.0


def test_check_gemm_inside_and_outside_bound():
    rng = np.random.default_rng(5)
    c = rng.standard_normal((8, 8)) * 10
    bnd = np.abs(c) * 3 + 1
    tol = 2e-3 * np.abs(c) + 1e-4 * bnd + oracle.output_ulp(c, "bf16")
    assert oracle.check_gemm(c + 0.999 * tol, c, bnd, "bf16")["ok"]
    assert oracle.check_gemm(c - 0.999 * tol, c, bnd, "bf16")["ok"]
    bad = c.copy()
    bad[3, 4] += 1.001 * tol[3, 4]
    r = oracle.check_gemm(bad, c, bnd, "bf16")
    assert not r["ok"] and r["n_bad"] == 1 and r["worst_index"] == (3, 4)
    nan = c.copy()
    nan[0, 0] = np.nan
    assert not oracle.check_gemm(nan, c, bnd, "bf16")["ok"]


@pytest.mark.parametrize("name", ["pertensor_16x64x128", "tinyllama_upproj_prefill"])
def test_oracle_against_torch_e4m3_cast_and_matmul(name):
    """An independent cross-check of the per-tensor path: the oracle's amax and scale (its
    own API) fed to torch's float8_e4m3fn conversion give the oracle's codes byte for byte,
    and torch's float64 matmul of the decoded codes, times both scales, is the oracle's
    exact product (so a dropped scale or a transposed operand in either would show)."""
    w = wl.WORKLOADS[name]
    a_bits, b_bits = wl.make_inputs(name)
    qa, sa = oracle.quantize_per_tensor(a_bits, "bf16")
    qb, sb = oracle.quantize_per_tensor(b_bits, "bf16")
    for bits, q, s in ((a_bits, qa, sa), (b_bits, qb, sb)):
        x32 = oracle.input_to_f32(bits, "bf16")
        scale = oracle.scale_from_amax(oracle.amax_per_tensor(x32))
        assert np.float32(scale) == s
        # float32 quotient (IEEE division in torch), then torch's round-to-nearest-even cast;
        # nothing here saturates, since |x| / scale <= 448
        t = (torch.from_numpy(x32) / torch.tensor(np.float32(scale))).to(torch.float8_e4m3fn)
        assert np.array_equal(t.view(torch.uint8).numpy(), q)
    da = torch.from_numpy(oracle.decode_e4m3(qa).astype(np.float64))
    db = torch.from_numpy(oracle.decode_e4m3(qb).astype(np.float64))
    c_torch = (da @ db.T).numpy() * (np.float64(sa) * np.float64(sb))
    c64 = oracle.gemm_tensorwise_ref(qa, sa, qb, sb)
    # exact products of 3-bit mantissas summed in float64: equal up to summation order
    bnd = oracle.bound_tensorwise(qa, sa, qb, sb)
    assert np.all(np.abs(c_torch - c64) <= 1e-12 * bnd + 1e-300)
    tdt = torch.float16 if w.out_dtype == "f16" else torch.bfloat16
    r = oracle.check_gemm(torch.from_numpy(c_torch).to(tdt).double().numpy(), c64, bnd, w.out_dtype)
    assert r["ok"], r


def test_blockwise_row_subset_with_nblock():
    rng = np.random.default_rng(6)
    qa, qb = rand_codes(rng, (3, 256)), rand_codes(rng, (300, 256))
    sa = (rng.random((3, 2)) + 0.5).astype(np.float32)
    sb = (rng.random((3, 2)) + 0.5).astype(np.float32)
    full = oracle.gemm_blockwise_ref(qa, sa, qb, sb)
    cols = np.array([0, 127, 128, 200, 299])
    sub = oracle.gemm_blockwise_ref(qa, sa, qb[cols], sb, nblock=cols // 128)
    assert np.array_equal(sub, full[:, cols])

