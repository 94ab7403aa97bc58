"""The hot path captured in a HIP graph (as bench.py runs it) reproduces the eager
results on every replay, with eager work and synchronisations between replays.  The
per-tensor path clears nothing between calls: its partial maxima live in q, which is
filled with junk before every replay here."""

import numpy as np
import pytest
import torch

import oracle
import fp8_quantized_gemm_amax_amd as fp8
from fp8_quantized_gemm_amax_amd import workloads as wl
from parity_util import DEV, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tinyllama_upproj_prefill", "deepseek_v3_blockwise"])
def test_graph_replays_match_eager(name):
    w = wl.WORKLOADS[name]
    m = 512 if name == "tinyllama_upproj_prefill" else 128
    a_bits, b_bits = wl.make_inputs(name, m)
    a, b = to_dev(a_bits), to_dev(b_bits)
    blockwise = w.mode == "blockwise"
    if blockwise:
        qb, sb = fp8.fp8_quantize_per_token_group(b, 128, 128)
        qa = torch.empty((m, w.k), dtype=torch.uint8, device=DEV)
        sa = torch.empty((m, w.k // 128), dtype=torch.float32, device=DEV)
    else:
        qb, sb = fp8.fp8_quantize_per_tensor(b)
        qa = torch.empty((m, w.k), dtype=torch.uint8, device=DEV)
        sa = torch.empty((1,), dtype=torch.float32, device=DEV)
    c = torch.empty((m, w.n), dtype=torch.float16 if w.out_dtype == "f16" else torch.bfloat16, device=DEV)

    def step():
        if blockwise:
            fp8.fp8_quantize_per_token_group(a, 1, 128, q=qa, scales=sa)
            fp8.fp8_gemm_scaled_blockwise(qa, sa, qb, sb, out=c)
        else:
            fp8.fp8_quantize_per_tensor(a, q=qa, scale=sa)
            fp8.fp8_gemm_scaled_tensorwise(qa, sa, qb, sb, out=c)

    step()
    torch.cuda.synchronize()
    ref = (qa.clone(), sa.clone(), c.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        qa.fill_(0x55)
        sa.fill_(-3.0)
        c.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(qa, ref[0]), f"replay {rep}: codes differ"
        assert torch.equal(sa.view(torch.int32), ref[1].view(torch.int32)), f"replay {rep}: scales differ"
        assert torch.equal(c.view(torch.int16), ref[2].view(torch.int16)), f"replay {rep}: output differs"
        _ = (a.float() * 2).sum()           # unrelated eager work between replays
    # and the eager result itself is the oracle's
    if not blockwise:
        q_want, s_want = oracle.quantize_per_tensor(a_bits, "bf16")
        assert np.array_equal(ref[0].cpu().numpy(), q_want)
        assert ref[1].cpu().numpy()[0] == s_want
