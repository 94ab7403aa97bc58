"""The Python binding rejects caller-supplied output buffers that the kernels would write
past (wrong shape, dtype, strides) or that share memory with an input, before any library
call.  CPU only: the device checks are replaced by no-ops and the library by a stub that
fails the test if it is ever reached."""

import pytest
import torch

import fp8_quantized_gemm_amax_amd.binding as b


class _NoLib:
    def __getattr__(self, name):
        raise AssertionError(f"library call {name} reached with an invalid output")


@pytest.fixture
def cpu_binding(monkeypatch):
    monkeypatch.setattr(b, "_need_cuda", lambda *ts: None)
    monkeypatch.setattr(b, "lib", lambda: _NoLib())
    return b


def x16(r, c):
    return torch.zeros((r, c), dtype=torch.bfloat16)


def test_check_out_rules():
    x = x16(4, 8)
    ok = torch.empty((4, 8), dtype=torch.uint8)
    with pytest.raises(TypeError):
        b._check_out(torch.empty((4, 8), dtype=torch.int8), (4, 8), b._CODES, "q", x)
    with pytest.raises(ValueError, match="shape"):
        b._check_out(torch.empty((4, 7), dtype=torch.uint8), (4, 8), b._CODES, "q", x)
    with pytest.raises(ValueError, match="shape"):
        b._check_out(torch.empty((32,), dtype=torch.uint8), (4, 8), b._CODES, "q", x)
    with pytest.raises(ValueError, match="contiguous"):
        b._check_out(torch.empty((8, 4), dtype=torch.uint8).t(), (4, 8), b._CODES, "q", x)
    with pytest.raises(ValueError, match="overlaps"):
        b._check_out(x.view(torch.uint8).reshape(-1)[:32].view(4, 8), (4, 8), b._CODES, "q", x, (x,))
    assert not b._overlaps(ok, x)
    big = torch.empty(100, dtype=torch.uint8)
    assert b._overlaps(big[10:20], big[15:30]) and not b._overlaps(big[10:20], big[20:30])


@pytest.mark.parametrize("call", [
    lambda b: b.fp8_quantize_per_tensor(x16(4, 256), q=torch.empty((4, 255), dtype=torch.uint8)),
    lambda b: b.fp8_quantize_per_tensor(x16(4, 256), q=torch.empty((4, 256), dtype=torch.int32)),
    lambda b: b.fp8_quantize_per_tensor(x16(4, 256), scale=torch.empty((2,), dtype=torch.float32)),
    lambda b: b.fp8_quantize_per_token_group(x16(4, 256), 1, 128, scales=torch.empty((4, 1), dtype=torch.float32)),
    lambda b: b.fp8_quantize_per_token_group(x16(4, 256), 1, 128, q=torch.empty((256, 4), dtype=torch.uint8).t()),
    lambda b: b.fp8_quantize_per_token_group(x16(256, 256), 128, 128, scales=torch.empty((2, 2), dtype=torch.float16)),
    lambda b: b.fp8_quantize_per_token_group_ue8m0(x16(4, 256), 1, 128, scales=torch.empty((4, 2), dtype=torch.uint8)),
    lambda b: b.fp8_quantize_rowwise(x16(4, 256), scales=torch.empty((4, 1), dtype=torch.float32)),
    lambda b: b.fp8_amax(x16(4, 256), 1, 128, out=torch.empty((4,), dtype=torch.float32)),
    lambda b: b.fp8_gemm_scaled_tensorwise(torch.zeros((4, 32), dtype=torch.uint8), torch.ones(1),
                                           torch.zeros((8, 32), dtype=torch.uint8), torch.ones(1),
                                           out=torch.empty((4, 7), dtype=torch.bfloat16)),
    lambda b: b.fp8_gemm_scaled_tensorwise(torch.zeros((4, 32), dtype=torch.uint8), torch.ones(1),
                                           torch.zeros((8, 32), dtype=torch.uint8), torch.ones(1),
                                           out=torch.empty((4, 8), dtype=torch.float32)),
    lambda b: b.fp8_gemm_scaled_blockwise(torch.zeros((4, 128), dtype=torch.uint8), torch.ones((4, 1)),
                                          torch.zeros((8, 128), dtype=torch.uint8), torch.ones((1, 1)),
                                          out=torch.empty((8, 4), dtype=torch.bfloat16).t()),
    lambda b: b.fp8_gemm_scaled_rowwise(torch.zeros((4, 32), dtype=torch.uint8), torch.ones(4),
                                        torch.zeros((8, 32), dtype=torch.uint8), torch.ones(8),
                                        out=torch.empty((32,), dtype=torch.bfloat16)),
    lambda b: b.fp8_gemm_grouped_blockwise(torch.zeros((6, 128), dtype=torch.uint8), torch.ones((6, 1)),
                                           torch.zeros((2, 8, 128), dtype=torch.uint8), torch.ones((2, 1, 1)),
                                           torch.tensor([0, 3, 6], dtype=torch.int32),
                                           out=torch.empty((6, 9), dtype=torch.bfloat16)),
    lambda b: b.fp8_quantize_static(x16(4, 32), torch.ones(1), q=torch.empty((4, 31), dtype=torch.uint8)),
    lambda b: b.fp8_debug_cast_f32(torch.zeros(16), q=torch.empty(15, dtype=torch.uint8)),
    lambda b: b.fp8_gemv_dynamic("tensorwise", x16(1, 256), torch.zeros((8, 256), dtype=torch.uint8), torch.ones(1),
                                 out=torch.empty((8,), dtype=torch.bfloat16)),
    lambda b: b.fp8_gemv_dynamic("blockwise", x16(1, 256), torch.zeros((8, 256), dtype=torch.uint8),
                                 torch.ones((1, 2)), sa=torch.empty((1,), dtype=torch.float32)),
    lambda b: b.fp8_gemv_dynamic("blockwise_ue8m0", x16(1, 256), torch.zeros((8, 256), dtype=torch.uint8),
                                 torch.ones((1, 4), dtype=torch.uint8), sa=torch.empty((1, 2), dtype=torch.uint8)),
    lambda b: b.fp8_gemv_dynamic("rowwise", x16(1, 256), torch.zeros((8, 256), dtype=torch.uint8), torch.ones(8),
                                 qa=torch.empty((256,), dtype=torch.uint8)),
    lambda b: b.fp8_gemv_dynamic("rowwise", x16(1, 256), torch.zeros((8, 256), dtype=torch.uint8),
                                 torch.ones(1)),                                  # weight scales: [N]
    lambda b: b.fp8_gemv_dynamic("blockwise", x16(2, 256), torch.zeros((8, 256), dtype=torch.uint8),
                                 torch.ones((1, 2))),                             # one token only
    lambda b: b.fp8_gemv_dynamic("per_tensor", x16(1, 256), torch.zeros((8, 256), dtype=torch.uint8),
                                 torch.ones(1)),                                  # unknown mode
])
def test_bad_outputs_rejected_before_the_library(cpu_binding, call):
    with pytest.raises((TypeError, ValueError)):
        call(cpu_binding)


def test_per_tensor_q_must_not_overlap_x(cpu_binding):
    """The per-tensor quantizer keeps partial maxima in q between its two launches and
    reads x again in the second; q inside x's memory is refused."""
    x = x16(8, 256)
    with pytest.raises(ValueError, match="overlaps"):
        cpu_binding.fp8_quantize_per_tensor(x, q=x.view(torch.uint8).reshape(-1)[:2048].view(8, 256))


def test_gemm_out_must_not_overlap_operands(cpu_binding):
    qa = torch.zeros((4, 64), dtype=torch.uint8)
    with pytest.raises(ValueError, match="overlaps"):
        cpu_binding.fp8_gemm_scaled_tensorwise(qa, torch.ones(1), torch.zeros((8, 64), dtype=torch.uint8),
                                               torch.ones(1), out=qa.reshape(-1)[:64].view(torch.bfloat16).view(4, 8))


def test_gemv_dynamic_outputs_must_not_overlap_x(cpu_binding):
    """Every workgroup of the fused step reads x while the first one writes qa and sa."""
    x = x16(1, 512)
    qb = torch.zeros((8, 512), dtype=torch.uint8)
    with pytest.raises(ValueError, match="overlaps"):
        cpu_binding.fp8_gemv_dynamic("tensorwise", x, qb, torch.ones(1), qa=x.view(torch.uint8)[:, :512])
    with pytest.raises(ValueError, match="overlaps"):
        cpu_binding.fp8_gemv_dynamic("tensorwise", x, qb, torch.ones(1), out=x[:, :8])
