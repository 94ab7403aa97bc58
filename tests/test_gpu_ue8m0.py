"""GPU parity for the UE8M0 (power-of-two, e8m0fnu byte) scale mode: the quantizer's codes
and scale bytes bit for bit against the oracle, and the blockwise product through every
kernel path within the product tolerance, all through the C ABI (Python binding)."""

import numpy as np
import pytest
import torch

import oracle
import fp8_quantized_gemm_amax_amd as fp8
from fp8_quantized_gemm_amax_amd import workloads as wl
from parity_util import (DEV, to_dev, u8_to_dev, guarded_u8, guarded_out, guard_intact, host_u8,
                         out_to_f64, assert_bytes_equal)

pytestmark = pytest.mark.gpu

TDT = {"bf16": torch.bfloat16, "f16": torch.float16}
FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
ALL16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def packed(codes):
    """The oracle's [rows, groups] codes in the library's layout: rows padded with 127 to a
    multiple of four bytes."""
    codes = np.asarray(codes, np.uint8)
    g4 = fp8.e8m0_row_bytes(codes.shape[1])
    out = np.full((codes.shape[0], g4), 127, np.uint8)
    out[:, :codes.shape[1]] = codes
    return out


# ----------------------------------------------------------------------------- quantizer

def check_groups(bits, dtype, gr, label):
    R, C = bits.shape
    q_want, e_want = oracle.quantize_groups_ue8m0(bits, dtype, gr, 128)
    want = packed(e_want)
    x = to_dev(bits, dtype)
    q, qfull = guarded_u8((R, C))
    s, sfull = guarded_u8(want.shape)
    fp8.fp8_quantize_per_token_group_ue8m0(x, gr, 128, q=q, scales=s)
    assert_bytes_equal(host_u8(s), want, f"{label} scale bytes (padding included)")
    assert_bytes_equal(host_u8(q), q_want, f"{label} codes")
    assert guard_intact(qfull, R * C, "u8") and guard_intact(sfull, want.size, "u8"), label


@pytest.mark.parametrize("name,which,gr", [("llama3_8b_mlp_blockwise", "a", 1), ("deepseek_v3_blockwise", "a", 1),
                                           ("deepseek_v3_blockwise", "b", 128), ("llama3_8b_mlp_blockwise", "b", 128)])
def test_workload_operands(name, which, gr):
    a_bits, b_bits = wl.make_inputs(name)
    check_groups(a_bits if which == "a" else b_bits, "bf16", gr, f"{name} {which}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("gr", [1, 128])
def test_all_bit_patterns(dtype, gr):
    """Every 16-bit pattern once (NaN, inf, subnormal and zero groups included)."""
    check_groups(ALL16.reshape(-1, 512), dtype, gr, f"all patterns {dtype} {gr}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_every_finite_amax(dtype):
    """One 1x128 group per finite positive input value a: x[0] = +-a and 127 smaller
    random elements, so every branch of the scale exponent (fraction above or below 1.75,
    clamping at 2^-127, subnormal amax) is taken."""
    x32 = oracle.input_to_f32(ALL16, dtype)
    vals = ALL16[np.isfinite(x32) & (x32 > 0)]
    rng = np.random.default_rng(3)
    rows = np.zeros((len(vals), 128), np.uint16)
    rows[:, 0] = vals | (rng.integers(0, 2, len(vals)) << 15).astype(np.uint16)
    small = (vals.astype(np.int64)[:, None] - rng.integers(1, 64, (len(vals), 127))).clip(0, None)
    rows[:, 1:] = small.astype(np.uint16) | (rng.integers(0, 2, small.shape) << 15).astype(np.uint16)
    check_groups(rows, dtype, 1, f"every amax {dtype}")


@pytest.mark.parametrize("shape,gr", [((3, 200), 1), ((5, 136), 1), ((1, 7), 1), ((129, 129), 1),
                                      ((130, 260), 128), ((257, 1000), 128), ((64, 384), 1),
                                      ((200, 640), 128), ((7, 1544), 1)])
def test_ragged(shape, gr):
    """Ragged rows and columns, rows whose length is not a multiple of 8 (scalar path),
    and 1, 2, 3 or 4+ groups per row (1, 2 or 3 padding bytes, or none)."""
    rng = np.random.default_rng(shape[0] * 7 + shape[1])
    a = rng.standard_t(4, shape) * np.exp(rng.normal(0, 2, (1, shape[1])))
    check_groups(wl.to_bf16_bits(a), "bf16", gr, f"ragged {shape} gr={gr}")


# ----------------------------------------------------------------------------- product

def random_case(M, N, K, seed):
    """UE8M0-quantized operands from heavy-tailed activations and lognormal weights."""
    rng = np.random.default_rng(seed)
    a = rng.standard_t(5, (M, K)) * np.exp(rng.normal(0, 1, (M, 1)))
    b = 0.02 * rng.standard_normal((N, K)) * np.exp(rng.normal(0, 0.5, (N, 1)))
    qa, ea = oracle.quantize_groups_ue8m0(wl.to_bf16_bits(a), "bf16", 1, 128)
    qb, eb = oracle.quantize_groups_ue8m0(wl.to_bf16_bits(b), "bf16", 128, 128)
    return qa, ea, qb, eb


def run_gemm(qa, ea, qb, eb, out_dtype):
    M, N = qa.shape[0], qb.shape[0]
    c, full = guarded_out((M, N), TDT[out_dtype])
    fp8.fp8_gemm_scaled_blockwise_ue8m0(u8_to_dev(qa), u8_to_dev(packed(ea)), u8_to_dev(qb),
                                       u8_to_dev(packed(eb)), out=c)
    got = out_to_f64(c)
    assert guard_intact(full, M * N, "out"), "write past the end of C"
    return got


def check(got, qa, ea, qb, eb, out_dtype, label):
    c64 = oracle.gemm_blockwise_ue8m0_ref(qa, ea, qb, eb)
    bnd = oracle.bound_blockwise_ue8m0(qa, ea, qb, eb)
    r = oracle.check_gemm(got, c64, bnd, out_dtype)
    assert r["ok"], f"{label}: {r}"


@pytest.mark.parametrize("M,N,K", [(1, 300, 640), (1, 1000, 2048), (3, 130, 256), (5, 70, 1152), (16, 256, 128),
                                   (17, 300, 384), (33, 1000, 640), (64, 4100, 256), (100, 290, 2176),
                                   (128, 12300, 384), (300, 520, 640), (130, 257, 512)])
@pytest.mark.parametrize("out_dtype", ["bf16", "f16"])
def test_shapes(M, N, K, out_dtype):
    """Every kernel path: the one-token vector-ALU kernel (M = 1), the MFMA decode kernel
    (2-16), the few-token kernel (17-128) and the 128x128 tiles, with ragged N and K/128
    of 1 to 17 slabs (padded scale rows included)."""
    qa, ea, qb, eb = random_case(M, N, K, M * 31 + N * 7 + K)
    check(run_gemm(qa, ea, qb, eb, out_dtype), qa, ea, qb, eb, out_dtype, f"{M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(128, 130, 8192), (128, 130, 65536), (100, 130, 65664), (64, 40, 131072),
                                   (64, 40, 131200)])
def test_few_token_scale_block_staging(M, N, K):
    """The few-token kernel stages a workgroup's UE8M0 activation-scale rows into LDS from 64
    tokens on while 16 MB rows of padded scale bytes fit in 64 KB, and takes them slab by
    slab past that: both sides of the limit for 128- and 64-row tiles."""
    qa, ea, qb, eb = random_case(M, N, K, M + K)
    check(run_gemm(qa, ea, qb, eb, "bf16"), qa, ea, qb, eb, "bf16", f"staging {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(2050, 8200, 256), (1030, 4100, 384), (520, 33000, 128), (520, 18000, 256)])
def test_large_tile_paths(M, N, K):
    """The 256x256 tile (at least one tile per CU) with its 128x128 tail, the four-wave
    128x128 tile, and whole rounds of it with a tail launch of eight-wave 128x128 tiles."""
    qa, ea, qb, eb = random_case(M, N, K, M + N + K)
    check(run_gemm(qa, ea, qb, eb, "bf16"), qa, ea, qb, eb, "bf16", f"{M}x{N}x{K}")


@pytest.mark.parametrize("M", [1, 5, 40, 300])
def test_scale_exponents_reach_every_slab_and_row(M):
    """Scale bytes drawn at random per (row, slab) and per (block, slab), over a wide
    exponent range, with uniform codes: a scale byte applied to the wrong slab, row or
    block shows up as an error far beyond the tolerance."""
    rng = np.random.default_rng(M)
    N, K = 260, 1152
    qa = rng.choice(FINITE[(FINITE & 0x78) >= 0x30], (M, K))     # moderate magnitudes
    qb = rng.choice(FINITE[(FINITE & 0x78) >= 0x30], (N, K))
    ea = rng.integers(110, 145, (M, K // 128)).astype(np.uint8)
    eb = rng.integers(110, 145, (-(-N // 128), K // 128)).astype(np.uint8)
    check(run_gemm(qa, ea, qb, eb, "bf16"), qa, ea, qb, eb, "bf16", f"exponents M={M}")


@pytest.mark.parametrize("M", [1, 3, 40, 300])
def test_nan_scale_byte(M):
    """Scale byte 255 (NaN) for one activation group makes that row's outputs NaN and
    leaves the other rows finite."""
    qa, ea, qb, eb = random_case(M, 200, 384, 11)
    ea = ea.copy()
    ea[M - 1, 1] = 255
    got = run_gemm(qa, ea, qb, eb, "bf16")
    assert np.all(np.isnan(got[M - 1]))
    assert np.all(np.isfinite(got[:M - 1]))


@pytest.mark.parametrize("name", ["llama3_8b_mlp_blockwise", "deepseek_v3_blockwise"])
def test_workload_end_to_end(name):
    """bf16 activations and weights of the workload (M = 128 rows of A) quantized on the GPU
    with UE8M0 scales, then multiplied: bytes equal to the oracle's, product within the
    tolerance."""
    a_bits, b_bits = wl.make_inputs(name)
    a_bits = a_bits[:128]
    qa_w, ea_w = oracle.quantize_groups_ue8m0(a_bits, "bf16", 1, 128)
    qb_w, eb_w = oracle.quantize_groups_ue8m0(b_bits, "bf16", 128, 128)
    qa, sa = fp8.fp8_quantize_per_token_group_ue8m0(to_dev(a_bits), 1, 128)
    qb, sb = fp8.fp8_quantize_per_token_group_ue8m0(to_dev(b_bits), 128, 128)
    assert_bytes_equal(host_u8(qa), qa_w, f"{name} qA")
    assert_bytes_equal(host_u8(sa), packed(ea_w), f"{name} sA")
    assert_bytes_equal(host_u8(qb), qb_w, f"{name} qB")
    assert_bytes_equal(host_u8(sb), packed(eb_w), f"{name} sB")
    c = fp8.fp8_gemm_scaled_blockwise_ue8m0(qa, sa, qb, sb)
    check(out_to_f64(c), qa_w, ea_w, qb_w, eb_w, "bf16", name)


@pytest.mark.parametrize("scale_mode", ["float32", "ue8m0"])
def test_register_staged_path_huge_k(scale_mode):
    """K = 2^23: 256 rows of K bytes overflow the 32-bit buffer offsets of the LDS-DMA
    tiles, so 17 tokens take the register-staged kernel (65536 slabs in one workgroup),
    for both blockwise scale formats."""
    rng = np.random.default_rng(23)
    M, N, K = 17, 16, 1 << 23
    mid = FINITE[((FINITE & 0x78) >= 0x28) & ((FINITE & 0x78) <= 0x48)]
    qa, qb = rng.choice(mid, (M, K)), rng.choice(mid, (N, K))
    c, full = guarded_out((M, N), torch.bfloat16)
    if scale_mode == "ue8m0":
        ea = rng.integers(120, 135, (M, K // 128)).astype(np.uint8)
        eb = rng.integers(120, 135, (1, K // 128)).astype(np.uint8)
        fp8.fp8_gemm_scaled_blockwise_ue8m0(u8_to_dev(qa), u8_to_dev(packed(ea)), u8_to_dev(qb),
                                           u8_to_dev(packed(eb)), out=c)
        c64 = oracle.gemm_blockwise_ue8m0_ref(qa, ea, qb, eb)
        bnd = oracle.bound_blockwise_ue8m0(qa, ea, qb, eb)
    else:
        sa = (rng.random((M, K // 128)) + 0.5).astype(np.float32)
        sb = (rng.random((1, K // 128)) + 0.5).astype(np.float32) * np.float32(1e-3)
        fp8.fp8_gemm_scaled_blockwise(u8_to_dev(qa), torch.from_numpy(sa).to(DEV), u8_to_dev(qb),
                                      torch.from_numpy(sb).to(DEV), out=c)
        c64 = oracle.gemm_blockwise_ref(qa, sa, qb, sb)
        bnd = oracle.bound_blockwise(qa, sa, qb, sb)
    got = out_to_f64(c)
    assert guard_intact(full, M * N, "out")
    r = oracle.check_gemm(got, c64, bnd, "bf16")
    assert r["ok"], r
