"""Seeded synthetic inputs for the FP8 scaled-GEMM workloads.

Shared by the tests, the bench and the smoke check; used by both the HIP path and
the CPU oracle.  It holds no step of the method (no amax, scale, cast or
product): it only draws numbers with NumPy's PCG64 generator and rounds them to
bf16 with torch's round-to-nearest-even conversion.

The five workloads are the shapes and distributions of the model layers the
pages name (TinyLlama-1.1B on the task page, Llama-2-7B on the Transformer Engine
page, Llama-3-8B and DeepSeek-V3 on the Transformers fine-grained FP8 page); the
pages print no layer sizes, so the sizes are those of the public model
configurations.  Real activations and weights are not available; normal,
lognormal and Student-t draws stand in for them.
"""

from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    m_values: tuple          # M (tokens) variants; inputs for smaller M are row prefixes
    n: int                   # output channels (rows of W / B)
    k: int                   # input channels
    mode: str                # "tensorwise" or "blockwise"
    out_dtype: str           # "bf16" or "f16"
    quantize_b_per_call: bool
    description: str
    experts: int = 0         # grouped workloads: experts on this GPU (B is [experts * n, k])


WORKLOADS = {
    "pertensor_16x64x128": Workload(
        "pertensor_16x64x128", 0, (16,), 64, 128, "tensorwise", "bf16", True,
        "A[16,128] ~ N(0,1), B[64,128] ~ N(0,0.02^2); both quantized per tensor on every call"),
    "tinyllama_upproj_prefill": Workload(
        "tinyllama_upproj_prefill", 1, (512,), 5632, 2048, "tensorwise", "f16", False,
        "TinyLlama-1.1B MLP up-projection prefill: A[512,2048] ~ N(0,1) with 20 (1%) "
        "outlier channels scaled x20, W[5632,2048] ~ N(0,0.02^2); per-tensor scales; fp16 out"),
    "llama7b_decode": Workload(
        "llama7b_decode", 2, (1, 128), 11008, 4096, "tensorwise", "bf16", False,
        "Llama-7B MLP decode: A[M,4096] ~ N(0,1) for M in {1,128}, W[11008,4096] ~ N(0,0.02^2); "
        "per-tensor scales"),
    "llama3_8b_mlp_blockwise": Workload(
        "llama3_8b_mlp_blockwise", 3, (4096,), 14336, 4096, "blockwise", "bf16", False,
        "Llama-3-8B MLP: A[4096,4096] = N(0,1) * lognormal(0,1) per input channel, "
        "W[14336,4096] = N(0,0.02^2) * lognormal(0,1) per output channel; "
        "1x128 activation groups, 128x128 weight blocks"),
    "deepseek_v3_blockwise": Workload(
        "deepseek_v3_blockwise", 4, (1, 128, 4096), 18432, 7168, "blockwise", "bf16", False,
        "DeepSeek-V3: A[M,7168] ~ Student-t(nu=4) for M in {1,128,4096}, "
        "W[18432,7168] ~ N(0,0.02^2); 1x128 activation groups, 128x128 weight blocks"),
    "deepseek_v3_moe_grouped": Workload(
        "deepseek_v3_moe_grouped", 5, (256, 4096), 4096, 7168, "grouped", "bf16", False,
        "DeepSeek-V3 routed experts, gate and up projections fused (N = 2 x 2048), on one GPU "
        "of eight-way expert parallelism (32 of 256 experts): M routed token rows in {256, "
        "4096} ~ Student-t(nu=4), split over the experts by a multinomial draw with "
        "Dirichlet(4) expert weights; each expert's W[4096,7168] ~ N(0,0.02^2) with its own "
        "seed; 1x128 activation groups, 128x128 weight blocks", experts=32),
}

ORDER = ["pertensor_16x64x128", "tinyllama_upproj_prefill", "llama7b_decode",
         "llama3_8b_mlp_blockwise", "deepseek_v3_blockwise", "deepseek_v3_moe_grouped"]


def to_bf16_bits(x):
    """float array -> uint16 bf16 bit patterns (round to nearest even, via torch)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def to_f16_bits(x):
    """float array -> uint16 fp16 bit patterns (round to nearest even)."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def make_inputs(name, m=None):
    """Return (a_bits [M,K] uint16, b_bits [N,K] uint16) bf16 patterns for a workload.

    ``m`` picks one of the workload's M variants (default: the largest).  Smaller
    M variants are the first rows of the largest draw, so all variants of a
    workload see the same weights and the same leading tokens.
    """
    w = WORKLOADS[name]
    mmax = max(w.m_values)
    m = mmax if m is None else m
    if m not in w.m_values:
        raise ValueError(f"{name}: M must be one of {w.m_values}")
    rng = np.random.default_rng(w.seed)
    K, N = w.k, w.n
    if name == "pertensor_16x64x128":
        a = rng.standard_normal((mmax, K))
        b = 0.02 * rng.standard_normal((N, K))
    elif name == "tinyllama_upproj_prefill":
        a = rng.standard_normal((mmax, K))
        idx = rng.choice(K, 20, replace=False)        # 1% of 2048 channels
        a[:, idx] *= 20.0
        b = 0.02 * rng.standard_normal((N, K), dtype=np.float32)
    elif name == "llama7b_decode":
        a = rng.standard_normal((mmax, K))
        b = 0.02 * rng.standard_normal((N, K), dtype=np.float32)
    elif name == "llama3_8b_mlp_blockwise":
        a = rng.standard_normal((mmax, K), dtype=np.float32)
        a *= rng.lognormal(0.0, 1.0, K).astype(np.float32)[None, :]
        b = rng.standard_normal((N, K), dtype=np.float32)
        b *= (0.02 * rng.lognormal(0.0, 1.0, N)).astype(np.float32)[:, None]
    elif name == "deepseek_v3_blockwise":
        a = rng.standard_t(4.0, (mmax, K))
        b = 0.02 * rng.standard_normal((N, K), dtype=np.float32)
    elif w.mode == "grouped":
        # the routed rows; the expert weights come from expert_weight_bits, one expert at a time
        return to_bf16_bits(rng.standard_t(4.0, (m, K)).astype(np.float32)), None
    else:
        raise KeyError(name)
    return to_bf16_bits(a[:m]), to_bf16_bits(b)


def group_sizes(name, m):
    """Rows per expert for a grouped workload with m routed rows: a multinomial draw of m over
    the experts with Dirichlet(4) expert probabilities (imbalanced routing), seeded."""
    w = WORKLOADS[name]
    rng = np.random.default_rng([w.seed, m])
    p = rng.dirichlet(np.full(w.experts, 4.0))
    return rng.multinomial(m, p).astype(np.int64)


def expert_weight_bits(name, e):
    """Expert e's weight W_e [n, k] of a grouped workload, bf16 bit patterns, with its own
    seed (so any subset of experts can be drawn alone)."""
    w = WORKLOADS[name]
    rng = np.random.default_rng([w.seed, 1000 + e])
    return to_bf16_bits(0.02 * rng.standard_normal((w.n, w.k), dtype=np.float32))


def bits_to_tensor(bits, dtype="bf16", device="cpu"):
    """uint16 bit patterns -> torch bfloat16 / float16 tensor with the same bits."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy())
    t = t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)
    return t.to(device)
