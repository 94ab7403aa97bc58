"""Helpers shared by the GPU parity tests: moving bit patterns between NumPy and the
device, and guard-banded output buffers that catch writes past an output's end."""

import numpy as np
import torch

from fp8_quantized_gemm_amax_amd import workloads as wl

DEV = "cuda:0"
GUARD = 256            # bytes / elements of sentinel after each output
SENTINEL_U8 = 0xA5


def to_dev(bits, dtype="bf16"):
    return wl.bits_to_tensor(bits, dtype, DEV)


def u8_to_dev(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).to(DEV)


def f32_to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32).reshape(-1) if np.ndim(a) == 0
                            else np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def guarded_u8(shape):
    """(view of `shape`, full buffer) with GUARD sentinel bytes after the view."""
    n = int(np.prod(shape))
    full = torch.full((n + GUARD,), SENTINEL_U8, dtype=torch.uint8, device=DEV)
    return full[:n].view(*shape), full


def guarded_f32(shape):
    n = int(np.prod(shape))
    full = torch.full((n + GUARD,), -12345.0, dtype=torch.float32, device=DEV)
    return full[:n].view(*shape), full


def guarded_out(shape, dtype):
    n = int(np.prod(shape))
    full = torch.full((n + GUARD,), -7.0, dtype=dtype, device=DEV)
    return full[:n].view(*shape), full


def guard_intact(full, n, kind):
    tail = full[n:]
    if kind == "u8":
        return bool((tail == SENTINEL_U8).all())
    if kind == "f32":
        return bool((tail == -12345.0).all())
    return bool((tail == -7.0).all())


def host_u8(t):
    torch.cuda.synchronize()
    return t.cpu().numpy().view(np.uint8)


def host_f32(t):
    torch.cuda.synchronize()
    return t.cpu().numpy().astype(np.float32)


def out_to_f64(t):
    torch.cuda.synchronize()
    return t.float().cpu().numpy().astype(np.float64)


def assert_bytes_equal(got, want, what):
    got = np.atleast_1d(np.asarray(got))
    want = np.atleast_1d(np.asarray(want))
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.nonzero(got.view(np.uint8) != want.view(np.uint8)) if got.dtype == np.uint8 else \
        np.nonzero(got.view(np.uint32) != want.view(np.uint32))
    n_bad = len(bad[0])
    if n_bad:
        idx = tuple(int(b[0]) for b in bad)
        raise AssertionError(f"{what}: {n_bad} mismatches; first at {idx}: got {got[idx]!r} "
                             f"want {want[idx]!r}")
