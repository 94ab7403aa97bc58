"""Scaled FP8 GEMM reference and the tolerance check.  Test infrastructure only.

Transformer Engine page ("Что такое FP8 инференс на H100 (Transformer
Engine)?") §3 steps 5-6 and its pseudocode: the FP8 operands are multiplied with
a wide accumulator and the product is multiplied by scale_A * scale_B before the
16-bit output.  "FP8 chi tiết" (Transformers fine-grained FP8 page), opening
bullets: with 1x128 activation groups and 128x128 weight blocks the scales
change every 128 input channels, so each 128-wide K slab carries its own
scale_A[m, g] * scale_B[n // 128, g].

Readings:
* operands are A [M, K] and B [N, K], both K-contiguous, C = A @ B^T (the
  B[N,K] / W[N,K] shapes of the workloads);
* the reference accumulates in float64.  Every e4m3 value is an integer multiple
  of 2^-9 below 2^9, so each product is a multiple of 2^-18 below 2^18 and any
  sum of up to 2^13 of them (K <= 8192) is held exactly by float64 whatever the
  summation order: the unscaled product is exact, and the tensorwise result
  carries one rounding (blockwise: one per slab plus the slab sum);
* the output dtype rounding is not applied here; ``check_gemm`` allows one
  output ulp on top of the relative and magnitude terms.
"""

import numpy as np

from .e4m3 import decode_e4m3

SLAB = 128


def _dec(q):
    return decode_e4m3(np.asarray(q, dtype=np.uint8))


def gemm_tensorwise_ref(qa, sa, qb, sb):
    """C64[m, n] = (sum_k dec(qa[m,k]) * dec(qb[n,k])) * (sa * sb), float64."""
    da, db = _dec(qa), _dec(qb)
    s = np.float64(np.float32(sa)) * np.float64(np.float32(sb))
    return (da @ db.T) * s


def bound_tensorwise(qa, sa, qb, sb):
    """Bnd[m, n] = sum_k |dec(qa) * sa| * |dec(qb) * sb| (the magnitude term)."""
    da, db = np.abs(_dec(qa)), np.abs(_dec(qb))
    s = abs(np.float64(np.float32(sa)) * np.float64(np.float32(sb)))
    return (da @ db.T) * s


def _slab_loop(qa, sa, qb, sb, absval, nblock):
    qa = np.asarray(qa, dtype=np.uint8)
    qb = np.asarray(qb, dtype=np.uint8)
    M, K = qa.shape
    N = qb.shape[0]
    assert K % SLAB == 0, "blockwise operands need K to be a multiple of 128"
    sa = np.asarray(sa, dtype=np.float32).astype(np.float64)
    sb = np.asarray(sb, dtype=np.float32).astype(np.float64)
    nblk = np.arange(N) // SLAB if nblock is None else np.asarray(nblock)
    out = np.zeros((M, N), dtype=np.float64)
    for g in range(K // SLAB):
        da = _dec(qa[:, g * SLAB:(g + 1) * SLAB])
        db = _dec(qb[:, g * SLAB:(g + 1) * SLAB])
        if absval:
            da, db = np.abs(da), np.abs(db)
        part = da @ db.T                                      # exact
        scale = sa[:, g][:, None] * sb[nblk, g][None, :]      # exact (24b x 24b)
        if absval:
            scale = np.abs(scale)
        out += part * scale
    return out


def gemm_blockwise_ref(qa, sa, qb, sb, nblock=None):
    """C64[m, n] = sum_g (sum_{k in slab g} dec(qa)dec(qb)) * sa[m, g] * sb[n // 128, g].

    sa is float32 [M, K/128] (one scale per token per 128 input channels), sb is
    float32 [ceil(N/128), K/128] (one scale per 128x128 weight block).  ``nblock``
    optionally gives the weight-block row of each row of qb (default n // 128), so a
    subset of B's rows can be checked against the full sb.
    """
    return _slab_loop(qa, sa, qb, sb, False, nblock)


def bound_blockwise(qa, sa, qb, sb, nblock=None):
    """Magnitude term for the blockwise product: same sum with |.| everywhere."""
    return _slab_loop(qa, sa, qb, sb, True, nblock)


def output_ulp(c, out_dtype):
    """Spacing of the output format ("bf16" or "f16") at |c|."""
    a = np.abs(np.asarray(c, dtype=np.float64))
    if out_dtype == "bf16":
        mant, emin = 7, -126
    elif out_dtype == "f16":
        mant, emin = 10, -14
    else:
        raise ValueError(out_dtype)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(np.where(a > 0, e, emin), emin)
    return np.exp2(e - mant)


def check_gemm(gpu, c64, bnd, out_dtype, rel=2e-3, mag=1e-4):
    """Element-wise test |gpu - C64| <= rel*|C64| + mag*Bnd + ulp_out(C64).

    Returns a dict: ok, n_bad, worst ratio err/tol, the index of the worst
    element, and the largest relative deviation |gpu - C64| / |C64| over
    elements with C64 != 0.
    """
    g = np.asarray(gpu, dtype=np.float64)
    c = np.asarray(c64, dtype=np.float64)
    b = np.asarray(bnd, dtype=np.float64)
    err = np.abs(g - c)
    tol = rel * np.abs(c) + mag * b + output_ulp(c, out_dtype)
    both_nan = np.isnan(g) & np.isnan(c)
    bad = ~((err <= tol) | both_nan)
    ratio = np.where(both_nan, 0.0, err / tol)
    ratio = np.where(np.isnan(ratio), np.inf, ratio)
    nz = c != 0
    max_rel = float(np.max(err[nz] / np.abs(c[nz]))) if nz.any() else 0.0
    worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape) if ratio.size else None
    return {
        "ok": not bool(bad.any()),
        "n_bad": int(bad.sum()),
        "worst_ratio": float(ratio.max()) if ratio.size else 0.0,
        "worst_index": tuple(int(i) for i in worst) if worst is not None else None,
        "max_rel_dev": max_rel,
    }
