"""GPU parity for the fused one-token step fp8_gemv_dynamic (the activation row quantized
and multiplied in one launch): its codes and scales bit for bit against the oracle's
quantizer of the matching scheme, its output element by element against the oracle's
product within the product tolerance, and every output bit for bit against the two-call
path (the quantizer entry point, then the GEMM entry point; NaN outputs as NaN), in every scale mode, for both
input and output dtypes, ragged K, the shapes that take the two-launch fallback (K > 8192),
special inputs, graph replays and the decode workloads' full shapes."""

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
MODES = ["tensorwise", "rowwise", "blockwise", "blockwise_ue8m0"]
BLOCK = ("blockwise", "blockwise_ue8m0")


def pad_e8m0(codes):
    """[rows, groups] UE8M0 codes in the library's layout: rows padded with 127 to whole words."""
    g4 = fp8.e8m0_row_bytes(codes.shape[1])
    return np.concatenate([codes, np.full((codes.shape[0], g4 - codes.shape[1]), 127, np.uint8)], axis=1)


def to_bits(a, dtype):
    if dtype == "bf16":
        return wl.to_bf16_bits(a)
    with np.errstate(over="ignore"):
        return np.clip(a, -6e4, 6e4).astype(np.float16).view(np.uint16)


def activation(K, dtype, seed):
    """One token: heavy-tailed values, a few outlier channels 40x larger (the case dynamic
    per-group scaling exists for)."""
    rng = np.random.default_rng(seed)
    a = rng.standard_t(4, K) * 1.5
    a[rng.choice(K, max(1, K // 500), replace=False)] *= 40.0
    return to_bits(a, dtype)


def quantize_weights(mode, bits):
    """Weight codes and the scales the GEMM of `mode` takes (stored layout), from the oracle's
    weight quantizer of that scheme (per tensor, per output channel, 128 x 128 blocks), and
    the unpadded UE8M0 codes (None for the other modes)."""
    if mode == "tensorwise":
        qb, sb = oracle.quantize_per_tensor(bits, "bf16")
        return qb, np.array([sb], np.float32), None
    if mode == "rowwise":
        qb, sb = oracle.quantize_rowwise(bits, "bf16")
        return qb, sb, None
    if mode == "blockwise":
        qb, sb = oracle.quantize_groups(bits, "bf16", 128, 128)
        return qb, sb, None
    qb, eb = oracle.quantize_groups_ue8m0(bits, "bf16", 128, 128)
    return qb, pad_e8m0(eb), eb


def weights(mode, N, K, seed):
    rng = np.random.default_rng(seed)
    w = 0.02 * rng.standard_normal((N, K)) * np.exp(rng.normal(0, 0.5, (N, 1)))
    return quantize_weights(mode, wl.to_bf16_bits(w))


def oracle_quant(mode, xbits, dtype):
    """The oracle's quantize of x as [1, K] with the scheme of `mode`: codes, the scales in the
    library's stored layout, and the scales the oracle's product takes."""
    x2 = xbits.reshape(1, -1)
    if mode == "tensorwise":
        qa, s = oracle.quantize_per_tensor(x2, dtype)
        return qa, np.array([s], np.float32), s
    if mode == "rowwise":
        qa, sa = oracle.quantize_rowwise(x2, dtype)
        return qa, sa, sa
    if mode == "blockwise":
        qa, sa = oracle.quantize_groups(x2, dtype, 1, 128)
        return qa, sa, sa
    qa, ea = oracle.quantize_groups_ue8m0(x2, dtype, 1, 128)
    return qa, pad_e8m0(ea), ea


def oracle_product(mode, qa, sa, qb, sb, eb, nblock=None):
    """Float64 product of the mode and its magnitude term (sa, sb as oracle_quant and
    quantize_weights hand them over; nblock: weight block of each row of qb)."""
    if mode == "tensorwise":
        return oracle.gemm_tensorwise_ref(qa, sa, qb, sb[0]), oracle.bound_tensorwise(qa, sa, qb, sb[0])
    if mode == "rowwise":
        return oracle.gemm_rowwise_ref(qa, sa, qb, sb), oracle.bound_rowwise(qa, sa, qb, sb)
    if mode == "blockwise":
        return (oracle.gemm_blockwise_ref(qa, sa, qb, sb, nblock=nblock),
                oracle.bound_blockwise(qa, sa, qb, sb, nblock=nblock))
    return (oracle.gemm_blockwise_ue8m0_ref(qa, sa, qb, eb, nblock=nblock),
            oracle.bound_blockwise_ue8m0(qa, sa, qb, eb, nblock=nblock))


def oracle_step(mode, xbits, dtype, qb, sb, eb):
    qa, stored, s = oracle_quant(mode, xbits, dtype)
    c64, bnd = oracle_product(mode, qa, s, qb, sb, eb)
    return qa, stored, c64, bnd


def sa_buffer(mode, K):
    if mode in ("tensorwise", "rowwise"):
        return guarded_f32((1,)), 1, "f32"
    if mode == "blockwise":
        return guarded_f32((1, K // 128)), K // 128, "f32"
    g4 = fp8.e8m0_row_bytes(K // 128)
    return guarded_u8((1, g4)), g4, "u8"


def sb_dev(mode, sb):
    return u8_to_dev(sb) if mode == "blockwise_ue8m0" else f32_to_dev(sb)


def run_dynamic(mode, xbits, dtype, qb, sb, out_dtype):
    """fp8_gemv_dynamic with guard-banded outputs; returns host (qa, sa, c as float64, c bits)."""
    K, N = xbits.size, qb.shape[0]
    qa, qfull = guarded_u8((1, K))
    (sa, sfull), ns, skind = sa_buffer(mode, K)
    c, cfull = guarded_out((1, N), TDT[out_dtype])
    fp8.fp8_gemv_dynamic(mode, to_dev(xbits.reshape(1, K), dtype), u8_to_dev(qb), sb_dev(mode, sb),
                         out=c, qa=qa, sa=sa)
    torch.cuda.synchronize()
    assert guard_intact(qfull, K, "u8"), "write past the end of qa"
    assert guard_intact(sfull, ns, skind), "write past the end of sa"
    assert guard_intact(cfull, N, "out"), "write past the end of c"
    got_sa = host_u8(sa) if skind == "u8" else host_f32(sa)
    return host_u8(qa), got_sa, out_to_f64(c), c.view(torch.int16).cpu().numpy().view(np.uint16)


def run_two_calls(mode, xbits, dtype, qb, sb, out_dtype):
    """The quantizer entry point of the mode, then its GEMM entry point (M = 1)."""
    x = to_dev(xbits.reshape(1, -1), dtype)
    if mode == "tensorwise":
        qa, sa = fp8.fp8_quantize_per_tensor(x)
        c = fp8.fp8_gemm_scaled_tensorwise(qa, sa, u8_to_dev(qb), sb_dev(mode, sb), out_dtype=TDT[out_dtype])
    elif mode == "rowwise":
        qa, sa = fp8.fp8_quantize_rowwise(x)
        c = fp8.fp8_gemm_scaled_rowwise(qa, sa, u8_to_dev(qb), sb_dev(mode, sb), out_dtype=TDT[out_dtype])
    elif mode == "blockwise":
        qa, sa = fp8.fp8_quantize_per_token_group(x, 1, 128)
        c = fp8.fp8_gemm_scaled_blockwise(qa, sa, u8_to_dev(qb), sb_dev(mode, sb), out_dtype=TDT[out_dtype])
    else:
        qa, sa = fp8.fp8_quantize_per_token_group_ue8m0(x, 1, 128)
        c = fp8.fp8_gemm_scaled_blockwise_ue8m0(qa, sa, u8_to_dev(qb), sb_dev(mode, sb), out_dtype=TDT[out_dtype])
    torch.cuda.synchronize()
    got_sa = host_u8(sa) if mode == "blockwise_ue8m0" else host_f32(sa)
    return host_u8(qa), got_sa.reshape(1, -1) if mode in BLOCK else got_sa, \
        c.view(torch.int16).cpu().numpy().view(np.uint16)


def same_outputs(a, b, out_dtype):
    """Output bit patterns equal, except that a NaN may differ from another NaN in sign and
    payload (which operand's NaN a multiply passes on is the compiler's operand order)."""
    top = 0x7F80 if out_dtype == "bf16" else 0x7C00
    na, nb = (a & 0x7FFF) > top, (b & 0x7FFF) > top
    return bool(np.array_equal(na, nb) and np.array_equal(a[~na], b[~nb]))


def check_all(mode, xbits, dtype, qb, sb, eb, out_dtype, label):
    qa_w, sa_w, c64, bnd = oracle_step(mode, xbits, dtype, qb, sb, eb)
    qa, sa, c, cbits = run_dynamic(mode, xbits, dtype, qb, sb, out_dtype)
    assert_bytes_equal(qa, qa_w, f"{label} codes")
    assert_bytes_equal(sa.reshape(sa_w.shape), sa_w, f"{label} scales")
    r = oracle.check_gemm(c, c64, bnd, out_dtype)
    assert r["ok"], (label, r)
    qa2, sa2, cbits2 = run_two_calls(mode, xbits, dtype, qb, sb, out_dtype)
    assert_bytes_equal(qa, qa2, f"{label} codes against the quantizer entry point")
    assert_bytes_equal(sa.reshape(sa2.shape), sa2, f"{label} scales against the quantizer entry point")
    assert same_outputs(cbits, cbits2, out_dtype), f"{label}: output differs from the two-call path " \
        f"({int((cbits != cbits2).sum())} of {cbits.size})"


# K: one chunk and less, ragged chunks (1152, 2944), whole chunks (4096, 8192), the largest
# one-launch K and the two-launch fallback beyond it (8320, 12288); N: one row, ragged
# workgroups (7, 130, 257: eight weight rows per workgroup), a weight block straddled, and
# more rows than the persistent form has waves (3072), so that waves take one, two or five
# rows and the last refill runs past N (3100, 12289)
SHAPES = [(1, 128), (7, 1152), (130, 4096), (257, 7168), (33, 8192), (64, 2944), (5, 8320), (3, 12288),
          (3100, 1024), (12289, 256)]
SHAPES_K16 = [(40, 16), (9, 1040), (17, 8208)]          # K % 128 != 0: per tensor and per row only


@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("dtype,out_dtype", [("bf16", "bf16"), ("f16", "f16")])
def test_dynamic_against_oracle_and_two_calls(N, K, mode, dtype, out_dtype):
    qb, sb, eb = weights(mode, N, K, N * 7 + K)
    xbits = activation(K, dtype, K + N)
    check_all(mode, xbits, dtype, qb, sb, eb, out_dtype, f"{mode} {dtype}->{out_dtype} N={N} K={K}")


@pytest.mark.parametrize("N,K", SHAPES_K16)
@pytest.mark.parametrize("mode", ["tensorwise", "rowwise"])
def test_dynamic_k_not_whole_slabs(N, K, mode):
    qb, sb, eb = weights(mode, N, K, N + K)
    xbits = activation(K, "bf16", K)
    check_all(mode, xbits, "bf16", qb, sb, eb, "f16", f"{mode} N={N} K={K}")


@pytest.mark.parametrize("mode", MODES)
def test_dynamic_special_rows(mode):
    """A zero row (scale 1, or UE8M0 code 127), a row whose amax is a lone outlier group, a
    row of subnormals, and rows holding a NaN or an infinity (NaN or infinite scales, NaN
    outputs): codes and scales against the oracle, every output bit against the two-call path,
    and the product against the oracle's for the first two.  The subnormal row's scale is
    itself a float32 subnormal near 2^-135, and the epilogue factor sa * sb formed from it in
    float32 keeps only a few significant bits, so its product is checked against the two-call
    path alone (the GEMM entry points form the same factor)."""
    N, K = 130, 1152
    qb, sb, eb = weights(mode, N, K, 5)
    rows = []
    rows.append(np.zeros(K, np.uint16))
    a = np.full(K, 1e-3)
    a[300] = 3e4
    rows.append(wl.to_bf16_bits(a))
    rows.append((np.arange(K) % 127 + 1).astype(np.uint16))             # bf16 subnormals
    nan_row = activation(K, "bf16", 9)
    nan_row[700] = 0x7FC0
    rows.append(nan_row)
    inf_row = activation(K, "bf16", 10)
    inf_row[5] = 0xFF80
    rows.append(inf_row)
    for i, xbits in enumerate(rows):
        qa_w, sa_w, c64, bnd = oracle_step(mode, xbits, "bf16", qb, sb, eb)
        qa, sa, c, cbits = run_dynamic(mode, xbits, "bf16", qb, sb, "bf16")
        assert_bytes_equal(qa, qa_w, f"row {i} codes")
        assert_bytes_equal(sa.reshape(sa_w.shape), sa_w, f"row {i} scales")
        qa2, sa2, cbits2 = run_two_calls(mode, xbits, "bf16", qb, sb, "bf16")
        assert same_outputs(cbits, cbits2, "bf16"), f"row {i}: output differs from the two-call path"
        if i < 2:
            r = oracle.check_gemm(c, c64, bnd, "bf16")
            assert r["ok"], (i, r)
        elif i > 2:
            assert np.isnan(c).any(), f"row {i}: a NaN or infinite input must give NaN outputs"


@pytest.mark.parametrize("mode", MODES)
def test_dynamic_no_weight_rows(mode):
    """N == 0: the activation is still quantized (the quantizer's launch alone); out is empty."""
    K = 1024
    xbits = activation(K, "bf16", 3)
    sb = {"tensorwise": np.ones((1,), np.float32), "rowwise": np.zeros((0,), np.float32),
          "blockwise": np.zeros((0, K // 128), np.float32),
          "blockwise_ue8m0": np.zeros((0, fp8.e8m0_row_bytes(K // 128)), np.uint8)}[mode]
    qa_w, sa_w, _ = oracle_quant(mode, xbits, "bf16")
    out, qa, sa = fp8.fp8_gemv_dynamic(mode, to_dev(xbits, "bf16"), u8_to_dev(np.zeros((0, K), np.uint8)),
                                       sb_dev(mode, sb))
    assert out.shape == (1, 0)
    assert_bytes_equal(host_u8(qa), qa_w, "codes")
    got = host_u8(sa) if mode == "blockwise_ue8m0" else host_f32(sa)
    assert_bytes_equal(got.reshape(sa_w.shape), sa_w, "scales")


@pytest.mark.parametrize("mode", MODES)
def test_dynamic_graph_replays(mode):
    """Captured in a HIP graph and replayed with new activations copied in between (eager
    work and synchronisations between replays): every replay equals the eager call."""
    N, K = 300, 2048
    qb, sb, eb = weights(mode, N, K, 11)
    qbd, sbd = u8_to_dev(qb), sb_dev(mode, sb)
    x = torch.empty((1, K), dtype=torch.bfloat16, device=DEV)
    x.copy_(to_dev(activation(K, "bf16", 0).reshape(1, K), "bf16"))
    out, qa, sa = fp8.fp8_gemv_dynamic(mode, x, qbd, sbd)          # outputs allocated once
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fp8.fp8_gemv_dynamic(mode, x, qbd, sbd, out=out, qa=qa, sa=sa)
    for r in range(4):
        xbits = activation(K, "bf16", 100 + r)
        x.copy_(to_dev(xbits.reshape(1, K), "bf16"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (out.clone(), qa.clone(), sa.clone())
        want = fp8.fp8_gemv_dynamic(mode, x, qbd, sbd)
        torch.cuda.synchronize()
        for a, b, what in zip(got, want, ("out", "qa", "sa")):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {r}: {what}"


@functools.lru_cache(maxsize=None)
def _workload_operands(workload, mode):
    """The workload's own one-token activation and weights (its seeded generators), the
    weights quantized by the oracle with the scheme of `mode`."""
    a_bits, b_bits = wl.make_inputs(workload, 1)
    return (a_bits[0],) + quantize_weights(mode, b_bits)


@pytest.mark.parametrize("workload,mode", [("llama7b_decode", "tensorwise"), ("llama7b_decode", "rowwise"),
                                           ("deepseek_v3_blockwise", "blockwise"),
                                           ("deepseek_v3_blockwise", "blockwise_ue8m0")])
def test_dynamic_workload_shapes(workload, mode):
    """The decode workloads at full size (Llama-7B W[11008, 4096], DeepSeek-V3 W[18432, 7168])
    in the launch configuration the bench times: every output bit for bit against the two-call
    path, codes and scales against the oracle, 96 sampled output rows against the oracle's
    product."""
    xbits, qb, sb, eb = _workload_operands(workload, mode)
    N = qb.shape[0]
    qa, sa, c, cbits = run_dynamic(mode, xbits, "bf16", qb, sb, "bf16")
    qa2, sa2, cbits2 = run_two_calls(mode, xbits, "bf16", qb, sb, "bf16")
    assert same_outputs(cbits, cbits2, "bf16"), f"{int((cbits != cbits2).sum())} outputs differ from the two-call path"
    qa_w, sa_w, s = oracle_quant(mode, xbits, "bf16")
    assert_bytes_equal(qa, qa_w, "codes")
    assert_bytes_equal(sa.reshape(sa_w.shape), sa_w, "scales")
    rng = np.random.default_rng(N)
    pick = np.unique(np.concatenate([np.arange(8), N - 8 + np.arange(8), rng.choice(N, 80, replace=False)]))
    if mode == "rowwise":
        c64, bnd = oracle_product(mode, qa_w, s, qb[pick], sb[pick], None)
    elif mode == "tensorwise":
        c64, bnd = oracle_product(mode, qa_w, s, qb[pick], sb, None)
    else:
        c64, bnd = oracle_product(mode, qa_w, s, qb[pick], sb if mode == "blockwise" else None, eb,
                                  nblock=pick // 128)
    r = oracle.check_gemm(c[:, pick], c64, bnd, "bf16")
    assert r["ok"], r
