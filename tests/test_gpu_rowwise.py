"""GPU parity for per-channel ("rowwise") scaling: fp8_quantize_rowwise bit for bit against
the oracle on every kernel path of the row quantizer, and fp8_gemm_scaled_rowwise element by
element within the product tolerance on every GEMM kernel path, separately and end to end on
the workload shapes."""

import functools

import numpy as np
import pytest
import torch

import oracle
import fp8_quantized_gemm_amax_amd as fp8
from fp8_quantized_gemm_amax_amd import workloads as wl
from parity_util import (DEV, to_dev, u8_to_dev, f32_to_dev, guarded_u8, guarded_f32, guarded_out,
                         guard_intact, host_u8, host_f32, out_to_f64, assert_bytes_equal)

pytestmark = pytest.mark.gpu

TDT = {"bf16": torch.bfloat16, "f16": torch.float16}
FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def rows_input(rows, cols, dtype, seed):
    """Heavy-tailed rows whose magnitudes differ by up to 2^+-12 from row to row."""
    rng = np.random.default_rng(seed)
    a = rng.standard_t(4, (rows, cols)) * np.exp2(rng.uniform(-12, 12, (rows, 1)))
    if dtype == "bf16":
        return wl.to_bf16_bits(a)
    with np.errstate(over="ignore"):
        return np.clip(a, -6e4, 6e4).astype(np.float16).view(np.uint16)


def run_rows(bits, dtype):
    R, C = bits.shape
    q, qfull = guarded_u8((R, C))
    s, sfull = guarded_f32((R,))
    fp8.fp8_quantize_rowwise(to_dev(bits, dtype), q=q, scales=s)
    got_q, got_s = host_u8(q), host_f32(s)
    assert guard_intact(qfull, R * C, "u8"), "write past the end of q"
    assert guard_intact(sfull, R, "f32"), "write past the end of scales"
    return got_q, got_s


# cols picks the path: <= 4096 a row per wave (1, 2, 4 or 8 pieces per lane), <= 16384 a
# row per workgroup (4 or 8 pieces per thread), above that two passes; cols % 8 != 0 the
# scalar two-pass path
@pytest.mark.parametrize("cols", [1, 7, 8, 120, 300, 512, 520, 1024, 1032, 2048, 2056, 4096, 4104,
                                  8192, 8200, 16384, 16392, 20000, 20001])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_rowwise_quantize_paths(cols, dtype):
    rows = 37 if cols <= 4104 else 5
    bits = rows_input(rows, cols, dtype, cols)
    q_want, s_want = oracle.quantize_rowwise(bits, dtype)
    q, s = run_rows(bits, dtype)
    assert_bytes_equal(s, s_want, f"{cols} {dtype} scales")
    assert_bytes_equal(q, q_want, f"{cols} {dtype} codes")


@pytest.mark.parametrize("cols", [256, 6000, 19000, 301])
def test_rowwise_special_rows(cols):
    """A zero row (scale 1), a row holding a NaN (NaN scale, all codes 0x7F), a row with an
    infinity (infinite scale), a row of subnormals only, and ordinary rows between them."""
    bits = rows_input(7, cols, "bf16", 99)
    bits[1] = 0
    bits[3, cols // 2] = 0x7FC0
    bits[4, cols - 1] = 0xFF80
    bits[5] = (np.arange(cols) % 127 + 1).astype(np.uint16)          # bf16 subnormals
    q_want, s_want = oracle.quantize_rowwise(bits, "bf16")
    q, s = run_rows(bits, "bf16")
    assert s[1] == 1.0 and np.isnan(s[3]) and np.isinf(s[4])
    assert_bytes_equal(s, s_want, f"{cols} scales")
    assert_bytes_equal(q, q_want, f"{cols} codes")


@pytest.mark.parametrize("rows,cols", [(70000, 8), (65537, 512), (16390, 8192)])
def test_rowwise_quantize_many_rows_sampled(rows, cols):
    """More rows than one grid covers (the kernels loop over rows): every scale and the codes
    of sampled rows, including both ends of every pass of the grid."""
    rng = np.random.default_rng(rows)
    bits = wl.to_bf16_bits(rng.standard_normal((rows, cols)) * np.exp2(rng.uniform(-6, 6, (rows, 1))))
    q, s = run_rows(bits, "bf16")
    x32 = oracle.input_to_f32(bits, "bf16")
    s_want = oracle.scale_from_amax(oracle.amax_rows(x32))
    assert_bytes_equal(s, s_want, "all scales")
    pick = np.unique(np.concatenate([np.arange(5), rows - 5 + np.arange(5), [16383, 16384, 65535, 65536],
                                     rng.choice(rows, 40, replace=False)]))
    pick = pick[pick < rows]
    q_want, _ = oracle.quantize_rowwise(bits[pick], "bf16")
    assert_bytes_equal(q[pick], q_want, "sampled rows")


def test_rowwise_quantize_empty():
    q, s = fp8.fp8_quantize_rowwise(torch.empty((0, 64), dtype=torch.bfloat16, device=DEV))
    assert q.shape == (0, 64) and s.shape == (0,)
    q, s = fp8.fp8_quantize_rowwise(torch.empty((3, 0), dtype=torch.bfloat16, device=DEV))
    assert q.shape == (3, 0) and host_f32(s).tolist() == [1.0, 1.0, 1.0]   # empty rows: amax 0


# ----------------------------------------------------------------------------- GEMM

def random_rowwise_case(M, N, K, seed):
    """Operands as the row quantizer produces them: per-token magnitudes over 2^+-6, per
    output channel weight magnitudes lognormal."""
    rng = np.random.default_rng(seed)
    a = rng.standard_t(5, (M, K)) * np.exp2(rng.uniform(-6, 6, (M, 1)))
    b = 0.02 * rng.standard_normal((N, K)) * np.exp(rng.normal(0, 1, (N, 1)))
    qa, sa = oracle.quantize_rowwise(wl.to_bf16_bits(a), "bf16")
    qb, sb = oracle.quantize_rowwise(wl.to_bf16_bits(b), "bf16")
    return qa, sa, qb, sb


def run_gemm(qa, sa, qb, sb, out_dtype="bf16"):
    M, N = qa.shape[0], qb.shape[0]
    c, full = guarded_out((M, N), TDT[out_dtype])
    fp8.fp8_gemm_scaled_rowwise(u8_to_dev(qa), f32_to_dev(sa), u8_to_dev(qb), f32_to_dev(sb), out=c)
    got = out_to_f64(c)
    assert guard_intact(full, M * N, "out"), "write past the end of C"
    return got


def check(got, qa, sa, qb, sb, out_dtype, label):
    r = oracle.check_gemm(got, oracle.gemm_rowwise_ref(qa, sa, qb, sb), oracle.bound_rowwise(qa, sa, qb, sb),
                          out_dtype)
    assert r["ok"], f"{label}: {r}"
    return r


# M picks the kernel: 1 the vector-ALU GEMV, 2-16 the MFMA GEMV, 17-128 the few-token
# kernel, above that the LDS-DMA tile kernels (three tile configurations by size); K % 128
# != 0 or huge K the register-staged kernel
@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (1, 300, 4096), (1, 37, 2192), (3, 17, 48), (5, 290, 656),
                                   (16, 64, 128), (17, 130, 272), (33, 1000, 2048), (65, 4100, 256),
                                   (128, 12300, 384), (130, 257, 528), (300, 520, 256), (600, 600, 384),
                                   (1030, 4100, 384), (2050, 8200, 256), (520, 18000, 256)])
@pytest.mark.parametrize("out_dtype", ["bf16", "f16"])
def test_rowwise_gemm_shapes(M, N, K, out_dtype):
    qa, sa, qb, sb = random_rowwise_case(M, N, K, M * 31 + N * 7 + K)
    got = run_gemm(qa, sa, qb, sb, out_dtype)
    check(got, qa, sa, qb, sb, out_dtype, f"rowwise {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(1, 70, 1040), (5, 70, 256), (20, 70, 384), (128, 300, 256), (300, 260, 256),
                                   (64, 64, 272)])
def test_rowwise_scales_land_on_their_row_and_column(M, N, K):
    """B one-hot at column k_n with code 1.0, distinct power-of-two scales per row and per
    column: C[m, n] = dec(qa[m, k_n]) * sa[m] * sb[n] exactly, so a scale applied to the
    wrong row or column shows up as a wrong element."""
    rng = np.random.default_rng(M + N + K)
    qa = rng.choice(FINITE, (M, K))
    sel = rng.integers(0, K, N)
    qb = np.zeros((N, K), np.uint8)
    qb[np.arange(N), sel] = 0x38
    sa = np.exp2(rng.integers(-6, 7, M)).astype(np.float32)
    sb = np.exp2(rng.integers(-6, 7, N)).astype(np.float32)
    got = run_gemm(qa, sa, qb, sb)
    want = oracle.decode_e4m3(qa)[:, sel] * sa[:, None].astype(np.float64) * sb[None, :].astype(np.float64)
    bad = np.argwhere(got != want)
    assert len(bad) == 0, f"{len(bad)} wrong; first {bad[:3].tolist()}"


def test_rowwise_equal_scales_match_tensorwise():
    rng = np.random.default_rng(5)
    M, N, K = 130, 300, 512
    qa, qb = rng.choice(FINITE, (M, K)), rng.choice(FINITE, (N, K))
    r = run_gemm(qa, np.full(M, 0.5, np.float32), qb, np.full(N, 0.25, np.float32))
    t = fp8.fp8_gemm_scaled_tensorwise(u8_to_dev(qa), f32_to_dev(np.float32(0.5)), u8_to_dev(qb),
                                       f32_to_dev(np.float32(0.25)))
    np.testing.assert_array_equal(r, out_to_f64(t))     # same sums, same single scale product


@pytest.mark.parametrize("M", [1, 3, 40, 300])
def test_rowwise_nan_scale_stays_in_its_row_and_column(M):
    rng = np.random.default_rng(M)
    qa, qb = rng.choice(FINITE, (M, 256)), rng.choice(FINITE, (50, 256))
    sa = np.ones(M, np.float32)
    sb = np.ones(50, np.float32)
    sa[M // 2] = np.nan
    sb[7] = np.nan
    got = run_gemm(qa, sa, qb, sb)
    assert np.all(np.isnan(got[M // 2])) and np.all(np.isnan(got[:, 7]))
    assert np.sum(np.isnan(got)) == 50 + M - 1


# ----------------------------------------------------------------------------- workloads

@functools.lru_cache(maxsize=None)
def _inputs(name):
    return wl.make_inputs(name)


@functools.lru_cache(maxsize=None)
def _quantized_w(name):
    return oracle.quantize_rowwise(_inputs(name)[1], "bf16")


@pytest.mark.parametrize("name,m", [("tinyllama_upproj_prefill", 512), ("llama7b_decode", 1),
                                    ("llama7b_decode", 128), ("deepseek_v3_blockwise", 1),
                                    ("deepseek_v3_blockwise", 128)])
def test_rowwise_workload_end_to_end(name, m):
    """The workload's activations per token and weights per output channel, quantized on the
    GPU, multiplied on the GPU: codes and scales bit for bit, every output within tolerance."""
    w = wl.WORKLOADS[name]
    a_bits, b_bits = _inputs(name)
    a_bits = a_bits[:m]
    qa, sa = oracle.quantize_rowwise(a_bits, "bf16")
    qb, sb = _quantized_w(name)
    gqa, gsa = fp8.fp8_quantize_rowwise(to_dev(a_bits))
    gqb, gsb = fp8.fp8_quantize_rowwise(to_dev(b_bits))
    c = fp8.fp8_gemm_scaled_rowwise(gqa, gsa, gqb, gsb, out_dtype=TDT[w.out_dtype])
    assert_bytes_equal(host_u8(gqa), qa, f"{name} qA")
    assert_bytes_equal(host_f32(gsa), sa, f"{name} sA")
    assert_bytes_equal(host_u8(gqb), qb, f"{name} qB")
    assert_bytes_equal(host_f32(gsb), sb, f"{name} sB")
    r = check(out_to_f64(c), qa, sa, qb, sb, w.out_dtype, f"{name} M={m}")
    print(f"{name} M={m} rowwise: max rel dev {r['max_rel_dev']:.3e}, worst err/tol {r['worst_ratio']:.3f}")


def test_rowwise_prefill_sampled():
    """Llama-3-8B MLP shape at M = 4096 (per-channel weight magnitudes lognormal): the GPU
    computes the whole product, the oracle checks 48 rows and 48 columns."""
    name = "llama3_8b_mlp_blockwise"
    w = wl.WORKLOADS[name]
    a_bits, b_bits = _inputs(name)
    qa, sa = oracle.quantize_rowwise(a_bits, "bf16")
    qb, sb = _quantized_w(name)
    gqa, gsa = fp8.fp8_quantize_rowwise(to_dev(a_bits))
    gqb, gsb = fp8.fp8_quantize_rowwise(to_dev(b_bits))
    c = fp8.fp8_gemm_scaled_rowwise(gqa, gsa, gqb, gsb)
    assert_bytes_equal(host_u8(gqa), qa, "qA")
    assert_bytes_equal(host_f32(gsb), sb, "sB")
    got = out_to_f64(c)
    rng = np.random.default_rng(0)
    M, N = got.shape
    rows = np.sort(rng.choice(M, 48, replace=False))
    rows[-1] = M - 1
    check(got[rows], qa[rows], sa[rows], qb, sb, w.out_dtype, "sampled rows")
    cols = np.sort(rng.choice(N, 48, replace=False))
    cols[-1] = N - 1
    check(got[:, cols], qa, sa, qb[cols], sb[cols], w.out_dtype, "sampled cols")
