"""Grouped (mixture-of-experts) blockwise FP8 GEMM on the CPU.  Test infrastructure only.

Source: "FP8 chi tiết" (the Transformers fine-grained FP8 page): its section on MoE experts
routes the expert matrix products through grouped_mm / batched_mm (float32 scales) or
DeepGEMM's expert kernels (UE8M0 scales on the newest parts), and its opening bullets define
the scaling of each product: 1x128 per-token activation groups, 128x128 weight blocks.

Readings where the page is silent (it names the backends, not their layout):
* E experts, each with its own weight W_e [N, K] in 128x128 blocks: qb [E, N, K] and
  sb [E, ceil(N/128), K/128] (float32) or [E, ceil(N/128), G4] (UE8M0 bytes);
* the tokens are already routed and permuted so that expert e's rows are the contiguous
  segment A[offsets[e] : offsets[e+1]] (offsets [E+1], non-decreasing, offsets[0] = 0,
  offsets[E] = T); a token sent to k experts appears k times;
* C[offsets[e] + i] = the blockwise product of that row with W_e, exactly as the dense
  blockwise GEMM defines it; an expert with no tokens contributes nothing;
* the routing itself (gating, top-k, the permutation, combining the expert outputs) is not
  part of the operation.
"""

import numpy as np

from .gemm import gemm_blockwise_ref, bound_blockwise
from .ue8m0 import gemm_blockwise_ue8m0_ref, bound_blockwise_ue8m0


def offsets_from_sizes(sizes):
    """Segment boundaries [E+1] (int64) of groups with the given sizes."""
    return np.concatenate([[0], np.cumsum(np.asarray(sizes, dtype=np.int64))])


def _grouped(fn, qa, sa, qb, sb, offsets):
    qa = np.asarray(qa, dtype=np.uint8)
    offsets = np.asarray(offsets, dtype=np.int64)
    T = qa.shape[0]
    E, N = qb.shape[0], qb.shape[1]
    assert offsets.shape == (E + 1,) and offsets[0] == 0 and offsets[-1] == T
    assert np.all(np.diff(offsets) >= 0)
    out = np.zeros((T, N), dtype=np.float64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            out[lo:hi] = fn(qa[lo:hi], sa[lo:hi], qb[e], sb[e])
    return out


def gemm_grouped_blockwise_ref(qa, sa, qb, sb, offsets):
    """C64 [T, N]: each segment of A times its expert's weight, float32 block scales."""
    return _grouped(gemm_blockwise_ref, qa, sa, qb, sb, offsets)


def bound_grouped_blockwise(qa, sa, qb, sb, offsets):
    return _grouped(bound_blockwise, qa, sa, qb, sb, offsets)


def gemm_grouped_blockwise_ue8m0_ref(qa, ea, qb, eb, offsets):
    """The same with UE8M0 (e8m0fnu byte) scales."""
    return _grouped(gemm_blockwise_ue8m0_ref, qa, ea, qb, eb, offsets)


def bound_grouped_blockwise_ue8m0(qa, ea, qb, eb, offsets):
    return _grouped(bound_blockwise_ue8m0, qa, ea, qb, eb, offsets)
