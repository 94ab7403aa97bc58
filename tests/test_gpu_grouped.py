"""GPU parity for the grouped (mixture-of-experts) blockwise GEMM: every output row against the
oracle's grouped product within the product tolerance, for ragged and empty groups, groups
spanning several 128-token chunks, many experts, both scale formats, offsets that need
clamping, and HIP-graph replays whose routing changes on the device between replays."""

import numpy as np
import pytest
import torch

import oracle
import fp8_quantized_gemm_amax_amd as fp8
from fp8_quantized_gemm_amax_amd import workloads as wl
from parity_util import DEV, to_dev, u8_to_dev, f32_to_dev, guarded_out, guard_intact, out_to_f64, host_u8, \
    host_f32, assert_bytes_equal

pytestmark = pytest.mark.gpu

TDT = {"bf16": torch.bfloat16, "f16": torch.float16}


def grouped_case(sizes, N, K, seed, ue8m0=False):
    """Operands as the quantizers produce them: heavy-tailed routed tokens (1 x 128 groups) and
    per-expert weights of different magnitudes (128 x 128 blocks)."""
    rng = np.random.default_rng(seed)
    E, T = len(sizes), int(np.sum(sizes))
    a = rng.standard_t(5, (T, K)) * np.exp(rng.normal(0, 1, (T, 1)))
    b = 0.02 * rng.standard_normal((E, N, K)) * np.exp(rng.normal(0, 1, (E, 1, 1)))
    a_bits = wl.to_bf16_bits(a)
    if ue8m0:
        qa, sa = oracle.quantize_groups_ue8m0(a_bits, "bf16", 1, 128)
        qs = [oracle.quantize_groups_ue8m0(wl.to_bf16_bits(b[e]), "bf16", 128, 128) for e in range(E)]
    else:
        qa, sa = oracle.quantize_groups(a_bits, "bf16", 1, 128)
        qs = [oracle.quantize_groups(wl.to_bf16_bits(b[e]), "bf16", 128, 128) for e in range(E)]
    qb = np.stack([q for q, _ in qs])
    sb = np.stack([s for _, s in qs])
    return qa, sa, qb, sb, oracle.offsets_from_sizes(sizes)


def pad4(codes):
    """UE8M0 codes [..., G] -> the device layout [..., G4] (padding bytes 127)."""
    g = codes.shape[-1]
    g4 = fp8.e8m0_row_bytes(g)
    out = np.full(codes.shape[:-1] + (g4,), 127, np.uint8)
    out[..., :g] = codes
    return out


def run_grouped(qa, sa, qb, sb, offsets, out_dtype="bf16", ue8m0=False, T=None):
    T = qa.shape[0] if T is None else T
    N = qb.shape[1]
    c, full = guarded_out((T, N), TDT[out_dtype])
    off = torch.from_numpy(np.asarray(offsets, np.int32)).to(DEV)
    if ue8m0:
        fp8.fp8_gemm_grouped_blockwise_ue8m0(u8_to_dev(qa), u8_to_dev(pad4(sa)), u8_to_dev(qb),
                                             u8_to_dev(pad4(sb)), off, out=c)
    else:
        fp8.fp8_gemm_grouped_blockwise(u8_to_dev(qa), f32_to_dev(sa), u8_to_dev(qb), f32_to_dev(sb), off, out=c)
    got = out_to_f64(c)
    assert guard_intact(full, T * N, "out"), "write past the end of C"
    return got


def check(got, qa, sa, qb, sb, offsets, out_dtype, label, ue8m0=False):
    if ue8m0:
        c64 = oracle.gemm_grouped_blockwise_ue8m0_ref(qa, sa, qb, sb, offsets)
        bnd = oracle.bound_grouped_blockwise_ue8m0(qa, sa, qb, sb, offsets)
    else:
        c64 = oracle.gemm_grouped_blockwise_ref(qa, sa, qb, sb, offsets)
        bnd = oracle.bound_grouped_blockwise(qa, sa, qb, sb, offsets)
    r = oracle.check_gemm(got, c64, bnd, out_dtype)
    assert r["ok"], f"{label}: {r}"
    return r


# sizes: one expert; empty experts first, in the middle and last; groups of exactly one and
# two 128-token chunks and just past them; a group of three chunks; N with a partial weight
# block and partial workgroup tiles; K of one slab and of many
@pytest.mark.parametrize("sizes,N,K", [
    ([37], 256, 128),
    ([0, 5, 0, 128, 129, 0], 130, 256),
    ([1, 256, 257, 2], 300, 384),
    ([300, 0, 7], 448, 1152),
    ([64] * 9 + [3, 200], 520, 256),
])
@pytest.mark.parametrize("out_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("ue8m0", [False, True])
def test_grouped_matches_oracle(sizes, N, K, out_dtype, ue8m0):
    qa, sa, qb, sb, off = grouped_case(sizes, N, K, len(sizes) * 7 + N + K, ue8m0)
    got = run_grouped(qa, sa, qb, sb, off, out_dtype, ue8m0)
    check(got, qa, sa, qb, sb, off, out_dtype, f"{sizes} N={N} K={K}", ue8m0)


@pytest.mark.parametrize("K", [16384, 16512])
def test_grouped_scale_block_staging(K):
    """The grouped launch stages a chunk's float32 activation scales into LDS when it has at
    least 64 tokens and 128 rows x K/128 scales fit in 64 KB: at K = 16384 the chunks of 128
    and 72 tokens stage them and the 56-token chunk takes them slab by slab; at K = 16512
    every chunk does."""
    qa, sa, qb, sb, off = grouped_case([200, 0, 56], 130, K, K)
    got = run_grouped(qa, sa, qb, sb, off, "bf16")
    check(got, qa, sa, qb, sb, off, "bf16", f"staging K={K}")


def test_grouped_many_experts():
    """96 experts with sizes 0..40 (a third of them empty): the tile search crosses two
    64-expert batches."""
    rng = np.random.default_rng(11)
    sizes = rng.integers(0, 41, 96) * (rng.random(96) > 0.33)
    qa, sa, qb, sb, off = grouped_case(sizes, 144, 256, 12)
    got = run_grouped(qa, sa, qb, sb, off)
    check(got, qa, sa, qb, sb, off, "bf16", "96 experts")


@pytest.mark.parametrize("off,good", [([-5, 6, 6, 99], [0, 6, 6, 12]),    # clamped to [0, T]
                                      ([0, 4, 12, 8], [0, 4, 12, 12])])   # an end before its start
def test_grouped_offsets_are_clamped(off, good):
    """Offsets outside [0, T] are clamped and an expert that ends before it starts is empty:
    the rows are those of the clamped grouping and nothing is written outside C."""
    qa, sa, qb, sb, _ = grouped_case([4, 4, 4], 128, 128, 13)
    got = run_grouped(qa, sa, qb, sb, np.array(off, np.int64))
    want = oracle.gemm_grouped_blockwise_ref(qa, sa, qb, sb, np.array(good))
    bnd = oracle.bound_grouped_blockwise(qa, sa, qb, sb, np.array(good))
    r = oracle.check_gemm(got, want, bnd, "bf16")
    assert r["ok"], r


def test_grouped_rows_outside_segments_are_untouched():
    qa, sa, qb, sb, _ = grouped_case([3, 5], 128, 128, 14)
    off = np.array([0, 3, 6], np.int64)            # rows 6, 7 belong to no expert
    c = torch.full((8, 128), -3.0, dtype=torch.bfloat16, device=DEV)
    fp8.fp8_gemm_grouped_blockwise(u8_to_dev(qa), f32_to_dev(sa), u8_to_dev(qb), f32_to_dev(sb),
                                   torch.from_numpy(off.astype(np.int32)).to(DEV), out=c)
    got = out_to_f64(c)
    assert (got[6:] == -3.0).all()
    want = oracle.gemm_grouped_blockwise_ref(qa[:6], sa[:6], qb, sb, off)
    r = oracle.check_gemm(got[:6], want, oracle.bound_grouped_blockwise(qa[:6], sa[:6], qb, sb, off), "bf16")
    assert r["ok"], r


def test_grouped_graph_follows_routing_on_the_device():
    """The offsets are read by the kernel, not by the host: a graph captured once and replayed
    after new offsets are written into the same device tensor computes the new grouping."""
    qa, sa, qb, sb, off0 = grouped_case([100, 0, 60, 96], 256, 512, 15)
    T, N = qa.shape[0], qb.shape[1]
    routings = [np.array(off0), oracle.offsets_from_sizes([0, 256, 0, 0]),
                oracle.offsets_from_sizes([10, 20, 30, 196]), np.array(off0)]
    d_qa, d_sa, d_qb, d_sb = u8_to_dev(qa), f32_to_dev(sa), u8_to_dev(qb), f32_to_dev(sb)
    d_off = torch.from_numpy(routings[0].astype(np.int32)).to(DEV)
    c = torch.empty((T, N), dtype=torch.bfloat16, device=DEV)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            fp8.fp8_gemm_grouped_blockwise(d_qa, d_sa, d_qb, d_sb, d_off, out=c)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    for i, off in enumerate(routings):
        d_off.copy_(torch.from_numpy(off.astype(np.int32)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check(out_to_f64(c), qa, sa, qb, sb, off, "bf16", f"replay {i}")


def test_grouped_empty_and_validation():
    qa = torch.empty((0, 128), dtype=torch.uint8, device=DEV)
    qb = torch.zeros((2, 64, 128), dtype=torch.uint8, device=DEV)
    off = torch.zeros(3, dtype=torch.int32, device=DEV)
    c = fp8.fp8_gemm_grouped_blockwise(qa, torch.ones((0, 1), device=DEV), qb, torch.ones((2, 1, 1), device=DEV), off)
    assert c.shape == (0, 64)
    with pytest.raises(TypeError):
        fp8.fp8_gemm_grouped_blockwise(qa, torch.ones((0, 1), device=DEV), qb, torch.ones((2, 1, 1), device=DEV),
                                       off.to(torch.int64))


# ----------------------------------------------------------------------------- workload

MOE = "deepseek_v3_moe_grouped"
_cache = {}


def _expert_weights_on_gpu():
    """Every expert's weight drawn on the host and quantized by the GPU (as the bench does)."""
    if "gpu_w" not in _cache:
        w = wl.WORKLOADS[MOE]
        qb = torch.empty((w.experts, w.n, w.k), dtype=torch.uint8, device=DEV)
        sb = torch.empty((w.experts, w.n // 128, w.k // 128), dtype=torch.float32, device=DEV)
        for e in range(w.experts):
            fp8.fp8_quantize_per_token_group(to_dev(wl.expert_weight_bits(MOE, e)), 128, 128, q=qb[e], scales=sb[e])
        _cache["gpu_w"] = (qb, sb)
    return _cache["gpu_w"]


def _oracle_expert(e):
    key = ("w", e)
    if key not in _cache:
        _cache[key] = oracle.quantize_groups(wl.expert_weight_bits(MOE, e), "bf16", 128, 128)
    return _cache[key]


@pytest.mark.parametrize("m", [256, 4096])
def test_moe_workload_sampled_experts(m):
    """The MoE workload at full size in the bench's launch: all 32 experts' weights, the routed
    rows quantized per token on the GPU, one grouped launch.  Three experts (the first, the
    one with the most rows, the last) are checked in full: their weight codes and scales bit
    for bit, and every output row routed to them within the product tolerance."""
    w = wl.WORKLOADS[MOE]
    a_bits, _ = wl.make_inputs(MOE, m)
    sizes = wl.group_sizes(MOE, m)
    off = oracle.offsets_from_sizes(sizes)
    qb, sb = _expert_weights_on_gpu()
    qa, sa = fp8.fp8_quantize_per_token_group(to_dev(a_bits), 1, 128)
    d_off = torch.from_numpy(off.astype(np.int32)).to(DEV)
    c = fp8.fp8_gemm_grouped_blockwise(qa, sa, qb, sb, d_off)
    got = out_to_f64(c)
    qa_h, sa_h = host_u8(qa), host_f32(sa)
    for e in sorted({0, int(np.argmax(sizes)), w.experts - 1}):
        qb_e, sb_e = _oracle_expert(e)
        assert_bytes_equal(host_u8(qb[e]), qb_e, f"expert {e} weight codes")
        assert_bytes_equal(host_f32(sb[e]), sb_e, f"expert {e} weight scales")
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        qa_e, sa_e = oracle.quantize_groups(a_bits[lo:hi], "bf16", 1, 128)
        assert_bytes_equal(qa_h[lo:hi], qa_e, f"expert {e} routed rows codes")
        assert_bytes_equal(sa_h[lo:hi], sa_e, f"expert {e} routed rows scales")
        one = np.array([0, hi - lo])
        r = oracle.check_gemm(got[lo:hi], oracle.gemm_grouped_blockwise_ref(qa_e, sa_e, qb_e[None], sb_e[None], one),
                              oracle.bound_grouped_blockwise(qa_e, sa_e, qb_e[None], sb_e[None], one), "bf16")
        assert r["ok"], f"M={m} expert {e} ({hi - lo} rows): {r}"
