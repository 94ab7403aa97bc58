"""The C-ABI library loads, exports every function include/fp8amax.h declares, and
rejects bad arguments with the documented status codes before any HIP call (so these
run on a machine without a GPU: no call here reaches a kernel launch)."""

import ctypes
import os
import re

import pytest

from fp8_quantized_gemm_amax_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, NULLP, SHAPE, DTYPE, ALIGN, LAUNCH, LARGE = range(7)
A16 = 0x10000          # fake, 16-byte aligned addresses (never dereferenced: validation fails first)
MIS = 0x10001


def header_functions():
    text = open(os.path.join(ROOT, "include", "fp8amax.h")).read()
    return re.findall(r"^(?:fp8_status_t|const char\*)\s+(fp8_\w+)\s*\(", text, flags=re.M)


@pytest.fixture(scope="module")
def L():
    return binding.lib()


def test_exports_every_declared_symbol(L):
    names = header_functions()
    assert set(names) == {"fp8_status_string", "fp8_amax", "fp8_quantize_per_tensor",
                          "fp8_quantize_per_token_group", "fp8_gemm_scaled_tensorwise",
                          "fp8_gemm_scaled_blockwise", "fp8_debug_cast_f32",
                          "fp8_quantize_per_token_group_ue8m0", "fp8_gemm_scaled_blockwise_ue8m0",
                          "fp8_quantize_static", "fp8_delayed_scaling_update", "fp8_quantize_delayed",
                          "fp8_quantize_rowwise", "fp8_gemm_scaled_rowwise",
                          "fp8_gemm_grouped_blockwise", "fp8_gemm_grouped_blockwise_ue8m0",
                          "fp8_debug_byte_mix", "fp8_debug_gemm_plan", "fp8_gemv_dynamic"}
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(binding._SIGNATURES)


def test_status_strings(L):
    for code, name in binding.STATUS_NAMES.items():
        assert L.fp8_status_string(code).decode().startswith(name)
    assert L.fp8_status_string(99) == b"unknown fp8_status_t"


@pytest.mark.parametrize("fn", ["fp8_gemm_scaled_tensorwise", "fp8_gemm_scaled_blockwise",
                                "fp8_gemm_scaled_blockwise_ue8m0", "fp8_gemm_scaled_rowwise"])
def test_gemm_validation(L, fn):
    f = getattr(L, fn)
    good = (A16, A16, A16, A16)
    assert f(*good, 4, 4, 0, A16, 0, None) == SHAPE          # K == 0
    assert f(*good, -1, 4, 128, A16, 0, None) == SHAPE
    assert f(*good, 4, -2, 128, A16, 0, None) == SHAPE
    assert f(*good, 4, 4, 120 if "blockwise" in fn else 24, A16, 0, None) == SHAPE   # K rule
    assert f(*good, 4, 4, 128, A16, 7, None) == DTYPE
    assert f(*good, 0, 4, 128, A16, 0, None) == OK            # empty: nothing launched
    assert f(*good, 4, 0, 128, A16, 0, None) == OK
    assert f(None, A16, A16, A16, 4, 4, 128, A16, 0, None) == NULLP
    assert f(A16, A16, A16, A16, 4, 4, 128, None, 0, None) == NULLP
    assert f(MIS, A16, A16, A16, 4, 4, 128, A16, 0, None) == ALIGN
    assert f(A16, A16, A16, A16, 4, 4, 128, MIS, 0, None) == ALIGN
    assert f(A16, A16 + 2, A16, A16, 4, 4, 128, A16, 0, None) == ALIGN   # float pointer needs 4 B
    assert f(*good, 2 ** 31, 4, 128, A16, 0, None) == LARGE


@pytest.mark.parametrize("fn", ["fp8_quantize_per_token_group", "fp8_quantize_per_token_group_ue8m0"])
def test_group_quantize_validation(L, fn):
    q = getattr(L, fn)
    assert q(A16, 0, 4, 256, 2, 128, A16, A16, None) == SHAPE      # unsupported group
    assert q(A16, 0, 4, 256, 1, 64, A16, A16, None) == SHAPE
    assert q(A16, 0, -4, 256, 1, 128, A16, A16, None) == SHAPE
    assert q(A16, 2, 4, 256, 1, 128, A16, A16, None) == DTYPE
    assert q(A16, 0, 0, 256, 1, 128, None, None, None) == OK        # empty
    assert q(None, 0, 4, 256, 1, 128, A16, A16, None) == NULLP
    assert q(MIS, 0, 4, 256, 128, 128, A16, A16, None) == ALIGN
    assert q(A16, 0, 4, 256, 128, 128, MIS, A16, None) == ALIGN
    assert q(A16, 0, 4, 256, 128, 128, A16, A16 + 2, None) == ALIGN   # scale rows are 4-byte words


def test_quantize_validation(L):
    q = L.fp8_quantize_per_token_group
    assert q(A16, 0, 4, 256, 2, 128, A16, A16, None) == SHAPE      # unsupported group
    assert q(A16, 0, 4, 256, 1, 64, A16, A16, None) == SHAPE
    assert q(A16, 0, -4, 256, 1, 128, A16, A16, None) == SHAPE
    assert q(A16, 2, 4, 256, 1, 128, A16, A16, None) == DTYPE
    assert q(A16, 0, 0, 256, 1, 128, None, None, None) == OK        # empty
    assert q(None, 0, 4, 256, 1, 128, A16, A16, None) == NULLP
    assert q(MIS, 0, 4, 256, 128, 128, A16, A16, None) == ALIGN
    assert q(A16, 0, 4, 256, 128, 128, MIS, A16, None) == ALIGN
    p = L.fp8_quantize_per_tensor
    assert p(A16, 0, 4, 256, A16, None, None) == NULLP               # scale is always written
    assert p(A16, 5, 4, 256, A16, A16, None) == DTYPE
    assert p(A16, 0, 4, -1, A16, A16, None) == SHAPE
    assert p(A16, 0, 2 ** 31, 2, A16, A16, None) == LARGE
    assert p(A16, 0, 2 ** 30, 2 ** 30, A16, A16, None) == LARGE      # 2^60 elements
    a = L.fp8_amax
    assert a(A16, 0, 4, 256, 1, 64, A16, None) == SHAPE
    assert a(A16, 0, 4, 256, 0, 128, A16, None) == SHAPE
    assert a(A16, 0, 0, 256, 1, 128, None, None) == OK               # empty grid
    assert a(A16, 0, 4, 256, 0, 0, None, None) == NULLP
    assert a(A16, 0, 4, 256, 0, 0, A16 + 1, None) == ALIGN
    d = L.fp8_debug_cast_f32
    assert d(A16, A16, -1, None) == SHAPE
    assert d(A16, A16, 0, None) == OK
    assert d(None, A16, 8, None) == NULLP
    bm = L.fp8_debug_byte_mix
    assert bm(A16, A16, -1, None) == SHAPE
    assert bm(A16, A16, 0, None) == OK
    assert bm(None, A16, 8, None) == NULLP
    assert bm(A16, A16 + 8, 8, None) == ALIGN
    assert bm(A16, A16, 2 ** 62, None) == LARGE


def test_static_and_delayed_validation(L):
    st = L.fp8_quantize_static
    assert st(A16, 3, 4, 256, A16, A16, None, None) == DTYPE
    assert st(A16, 0, -1, 256, A16, A16, None, None) == SHAPE
    assert st(A16, 0, 0, 256, None, None, None, None) == OK             # empty: nothing launched
    assert st(None, 0, 4, 256, A16, A16, None, None) == NULLP
    assert st(A16, 0, 4, 256, None, A16, None, None) == NULLP           # scale is required
    assert st(A16, 0, 4, 256, A16 + 2, A16, None, None) == ALIGN
    assert st(A16, 0, 4, 256, A16, A16, A16 + 1, None) == ALIGN
    up = L.fp8_delayed_scaling_update
    assert up(A16, 0, A16, A16, 4, 0, A16, None) == SHAPE                # empty history
    assert up(A16, 8, A16, A16, 0, 0, A16, None) == SHAPE                # interval 0
    assert up(A16, 8, A16, A16, 4, 127, A16, None) == SHAPE              # margin out of range
    assert up(None, 8, A16, A16, 4, 0, A16, None) == NULLP
    assert up(A16, 8, A16, A16 + 2, 4, 0, A16, None) == ALIGN


@pytest.mark.parametrize("fn", ["fp8_gemm_grouped_blockwise", "fp8_gemm_grouped_blockwise_ue8m0"])
def test_grouped_validation(L, fn):
    """(qa, sa, qb, sb, offsets, E, T, N, K, c, out_dt, stream)"""
    f = getattr(L, fn)

    def call(qa=A16, sa=A16, qb=A16, sb=A16, off=A16, E=4, T=64, N=256, K=256, c=A16, dt=0):
        return f(qa, sa, qb, sb, off, E, T, N, K, c, dt, None)

    assert call(E=0) == SHAPE
    assert call(T=-1) == SHAPE
    assert call(K=200) == SHAPE
    assert call(K=0) == SHAPE
    assert call(E=1 << 17) == LARGE
    assert call(K=1 << 24) == LARGE
    assert call(dt=9) == DTYPE
    assert call(T=0, qa=None, off=None) == OK                       # nothing to compute
    assert call(N=0) == OK
    assert call(off=None) == NULLP
    assert call(sb=None) == NULLP
    assert call(qa=MIS) == ALIGN
    assert call(off=A16 + 2) == ALIGN
    assert call(c=A16 + 8) == ALIGN


def test_rowwise_quantize_validation(L):
    f = L.fp8_quantize_rowwise
    assert f(A16, 2, 4, 256, A16, A16, None) == DTYPE
    assert f(A16, 0, -1, 256, A16, A16, None) == SHAPE
    assert f(A16, 0, 4, -256, A16, A16, None) == SHAPE
    assert f(None, 0, 0, 256, None, None, None) == OK                # no rows: nothing launched
    assert f(A16, 0, 4, 256, A16, None, None) == NULLP               # scales are required
    assert f(None, 0, 4, 256, A16, A16, None) == NULLP
    assert f(A16, 0, 4, 256, None, A16, None) == NULLP
    assert f(MIS, 0, 4, 256, A16, A16, None) == ALIGN
    assert f(A16, 0, 4, 256, A16 + 8, A16, None) == ALIGN
    assert f(A16, 0, 4, 256, A16, A16 + 2, None) == ALIGN
    assert f(A16, 0, 1 << 31, 256, A16, A16, None) == LARGE


def test_fused_delayed_validation(L):
    """fp8_quantize_delayed(x, dt, rows, cols, history, len, acc, step, interval, margin,
    scale, scale_used, q, stream): only failing cases (an empty tensor still launches the
    update)."""
    fq = L.fp8_quantize_delayed

    def call(x=A16, dt=0, rows=4, cols=256, hist=A16, n=8, acc=A16, step=A16, interval=4, margin=0,
             scale=A16, used=A16, q=A16):
        return fq(x, dt, rows, cols, hist, n, acc, step, interval, margin, scale, used, q, None)

    assert call(dt=5) == DTYPE
    assert call(rows=-1) == SHAPE
    assert call(n=0) == SHAPE
    assert call(interval=0) == SHAPE
    assert call(margin=-127) == SHAPE
    assert call(x=None) == NULLP
    assert call(q=None) == NULLP
    assert call(rows=0, hist=None) == NULLP                             # state is needed even when empty
    assert call(step=None) == NULLP
    assert call(used=None) == NULLP
    assert call(x=A16 + 4) == ALIGN
    assert call(step=A16 + 2) == ALIGN
    assert call(rows=0, x=MIS, q=MIS, used=A16 + 1) == ALIGN             # x, q unused when empty


def test_gemv_dynamic_validation(L):
    """fp8_gemv_dynamic(mode, x, in_dt, qb, sb, N, K, qa, sa, c, out_dt, stream): only failing
    cases, and the argument order of their checks (mode, shape, dtype, pointers, alignment)."""
    f = L.fp8_gemv_dynamic

    def call(mode=0, x=A16, dt=0, qb=A16, sb=A16, N=64, K=256, qa=A16, sa=A16, c=A16, odt=0):
        return f(mode, x, dt, qb, sb, N, K, qa, sa, c, odt, None)

    assert call(mode=-1) == SHAPE
    assert call(mode=4) == SHAPE
    assert call(K=0) == SHAPE
    assert call(K=24) == SHAPE                                        # K % 16
    assert call(mode=1, K=1040) == SHAPE                              # blockwise: K % 128
    assert call(mode=2, K=1040) == SHAPE
    assert call(N=-1) == SHAPE
    assert call(N=2 ** 31) == LARGE
    assert call(dt=2) == DTYPE
    assert call(odt=9) == DTYPE
    assert call(x=None) == NULLP
    assert call(qa=None) == NULLP
    assert call(sa=None) == NULLP
    assert call(qb=None) == NULLP
    assert call(c=None) == NULLP
    assert call(N=0, qb=None, sb=None, c=None, x=MIS) == ALIGN        # N == 0: x is still quantized
    assert call(x=A16 + 8) == ALIGN
    assert call(qa=MIS) == ALIGN
    assert call(sa=A16 + 2) == ALIGN
    assert call(c=MIS) == ALIGN
    assert call(qb=MIS) == ALIGN
    assert call(sb=A16 + 1) == ALIGN


def test_binding_refuses_cpu_tensors():
    import torch
    import fp8_quantized_gemm_amax_amd as f
    with pytest.raises(ValueError):
        f.fp8_quantize_per_token_group(torch.zeros(4, 128, dtype=torch.bfloat16))
    with pytest.raises(TypeError):
        f.fp8_gemm_scaled_tensorwise(torch.zeros(4, 128, dtype=torch.float32), torch.ones(1),
                                     torch.zeros(4, 128, dtype=torch.uint8), torch.ones(1))
