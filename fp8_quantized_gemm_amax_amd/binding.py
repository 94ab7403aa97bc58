"""ctypes binding of libfp8amax.so: the C ABI of include/fp8amax.h with the same names.

Argument marshalling only.  torch supplies device memory (outputs are allocated with
``torch.empty``) and the current HIP stream; every step of the path runs in the
library's HIP kernels.  There is no fallback: if the library is missing or fails to
load, every call raises.
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# FP8AMAX_LIBRARY selects another build of the same library (the tests load a host-sanitized
# build of the argument checks this way); by default the in-tree build.
LIB_PATH = os.environ.get("FP8AMAX_LIBRARY") or os.path.join(_PKG, "libfp8amax.so")

FP8_BF16, FP8_F16 = 0, 1
STATUS_NAMES = {0: "FP8_OK", 1: "FP8_ERR_NULL_POINTER", 2: "FP8_ERR_BAD_SHAPE", 3: "FP8_ERR_BAD_DTYPE",
                4: "FP8_ERR_MISALIGNED", 5: "FP8_ERR_LAUNCH", 6: "FP8_ERR_TOO_LARGE"}

_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SIGNATURES = {
    "fp8_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "fp8_amax": ([_P, ctypes.c_int, _I64, _I64, _I32, _I32, _P, _P], ctypes.c_int),
    "fp8_quantize_per_tensor": ([_P, ctypes.c_int, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "fp8_quantize_per_token_group": ([_P, ctypes.c_int, _I64, _I64, _I32, _I32, _P, _P, _P], ctypes.c_int),
    "fp8_gemm_scaled_tensorwise": ([_P, _P, _P, _P, _I64, _I64, _I64, _P, ctypes.c_int, _P], ctypes.c_int),
    "fp8_gemm_scaled_blockwise": ([_P, _P, _P, _P, _I64, _I64, _I64, _P, ctypes.c_int, _P], ctypes.c_int),
    "fp8_quantize_per_token_group_ue8m0": ([_P, ctypes.c_int, _I64, _I64, _I32, _I32, _P, _P, _P], ctypes.c_int),
    "fp8_gemm_scaled_blockwise_ue8m0": ([_P, _P, _P, _P, _I64, _I64, _I64, _P, ctypes.c_int, _P], ctypes.c_int),
    "fp8_quantize_rowwise": ([_P, ctypes.c_int, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "fp8_gemm_scaled_rowwise": ([_P, _P, _P, _P, _I64, _I64, _I64, _P, ctypes.c_int, _P], ctypes.c_int),
    "fp8_gemm_grouped_blockwise": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, ctypes.c_int, _P],
                                   ctypes.c_int),
    "fp8_gemm_grouped_blockwise_ue8m0": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, ctypes.c_int, _P],
                                         ctypes.c_int),
    "fp8_quantize_static": ([_P, ctypes.c_int, _I64, _I64, _P, _P, _P, _P], ctypes.c_int),
    "fp8_delayed_scaling_update": ([_P, _I32, _P, _P, _I32, _I32, _P, _P], ctypes.c_int),
    "fp8_quantize_delayed": ([_P, ctypes.c_int, _I64, _I64, _P, _I32, _P, _P, _I32, _I32, _P, _P, _P, _P],
                             ctypes.c_int),
    "fp8_debug_cast_f32": ([_P, _P, _I64, _P], ctypes.c_int),
    "fp8_debug_byte_mix": ([_P, _P, _I64, _P], ctypes.c_int),
    "fp8_debug_gemm_plan": ([_I32, _I64, _I64, _I64, _P], ctypes.c_int),
    "fp8_gemv_dynamic": ([_I32, _P, ctypes.c_int, _P, _P, _I64, _I64, _P, _P, _P, ctypes.c_int, _P], ctypes.c_int),
}


class Fp8Error(RuntimeError):
    """A non-zero fp8_status_t from the library."""

    def __init__(self, fn, code, text):
        super().__init__(f"{fn}: {text}")
        self.code = code
        self.status = STATUS_NAMES.get(code, str(code))


def lib():
    """Load libfp8amax.so once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m fp8_quantized_gemm_amax_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


def _check(fn, code):
    if code != 0:
        text = lib().fp8_status_string(code).decode()
        raise Fp8Error(fn, code, text)


def _dt(t):
    if t.dtype == torch.bfloat16:
        return FP8_BF16
    if t.dtype == torch.float16:
        return FP8_F16
    raise TypeError(f"expected a bfloat16 or float16 tensor, got {t.dtype}")


def _out_dt(dtype):
    if dtype == torch.bfloat16:
        return FP8_BF16
    if dtype == torch.float16:
        return FP8_F16
    raise TypeError(f"output dtype must be bfloat16 or float16, got {dtype}")


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else ctypes.c_void_p(0)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")


def _same_device(like, *ts):
    """Every tensor on like's GPU (the library launches on like's stream)."""
    _need_cuda(like, *ts)
    for t in ts:
        if t is not None and t.device != like.device:
            raise ValueError(f"all tensors must be on {like.device}, got one on {t.device}")


def _span(t):
    """[first, last) byte addresses a contiguous tensor covers."""
    lo = t.data_ptr()
    return lo, lo + t.numel() * t.element_size()


def _overlaps(a, b):
    if a is None or b is None or a.numel() == 0 or b.numel() == 0:
        return False
    (a0, a1), (b0, b1) = _span(a), _span(b)
    return a0 < b1 and b0 < a1


def _check_out(t, shape, dtypes, what, like, inputs=()):
    """A caller-supplied output buffer: on like's device, contiguous, one of `dtypes`, exactly
    `shape`, and sharing no memory with any of `inputs`.  Checked before any library call:
    the kernels write the full extent of an output, so a smaller or strided buffer would be
    written past its end."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{what} must be {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    for x in inputs:
        if _overlaps(t, x):
            raise ValueError(f"{what} overlaps an input")
    _same_device(like, t)
    return t


_CODES = (torch.uint8, torch.float8_e4m3fn)
_F32 = (torch.float32,)
_U8 = (torch.uint8,)
_OUT = (torch.bfloat16, torch.float16)


def _as_2d(x):
    if x.dim() != 2:
        raise ValueError(f"expected a 2-D tensor, got shape {tuple(x.shape)}")
    return x.contiguous()


def _codes(t):
    """Accept uint8 or float8_e4m3fn code tensors; return a uint8 view."""
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8)
    if t.dtype != torch.uint8:
        raise TypeError(f"FP8 operands must be uint8 or float8_e4m3fn, got {t.dtype}")
    return t


def fp8_amax(x, block_rows=0, block_cols=0, out=None):
    """amax per tensor ((0,0) -> shape [1]) or per (1,128) / (128,128) block."""
    x = _as_2d(x)
    _need_cuda(x)
    R, C = x.shape
    shape = (1,) if (block_rows, block_cols) == (0, 0) else (
        -(-R // max(block_rows, 1)), -(-C // max(block_cols, 1)))
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=x.device)
    _check_out(out, shape, _F32, "out", x, (x,))
    _check("fp8_amax", lib().fp8_amax(_ptr(x), _dt(x), R, C, block_rows, block_cols,
                                      ctypes.c_void_p(out.data_ptr()), _stream(x)))
    return out


def fp8_quantize_per_tensor(x, q=None, scale=None):
    """Returns (q uint8 [R, C], scale float32 [1])."""
    x = _as_2d(x)
    _need_cuda(x)
    R, C = x.shape
    if q is None:
        q = torch.empty((R, C), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty((1,), dtype=torch.float32, device=x.device)
    # q also holds the partial maxima between the call's two launches: it must not share
    # memory with x, which the second launch reads again
    _check_out(q, (R, C), _CODES, "q", x, (x,))
    _check_out(scale, (1,), _F32, "scale", x, (x, q))
    _check("fp8_quantize_per_tensor",
           lib().fp8_quantize_per_tensor(_ptr(x), _dt(x), R, C, _ptr(q),
                                         ctypes.c_void_p(scale.data_ptr()), _stream(x)))
    return q, scale


def fp8_quantize_per_token_group(x, group_rows=1, group_cols=128, q=None, scales=None):
    """Returns (q uint8 [R, C], scales float32 [ceil(R/group_rows), ceil(C/group_cols)])."""
    x = _as_2d(x)
    _need_cuda(x)
    R, C = x.shape
    if q is None:
        q = torch.empty((R, C), dtype=torch.uint8, device=x.device)
    grid = (-(-R // max(group_rows, 1)), -(-C // max(group_cols, 1)))
    if scales is None:
        scales = torch.empty(grid, dtype=torch.float32, device=x.device)
    _check_out(q, (R, C), _CODES, "q", x, (x,))
    _check_out(scales, grid, _F32, "scales", x, (x, q))
    _check("fp8_quantize_per_token_group",
           lib().fp8_quantize_per_token_group(_ptr(x), _dt(x), R, C, group_rows, group_cols,
                                              _ptr(q), _ptr(scales), _stream(x)))
    return q, scales


def fp8_quantize_rowwise(x, q=None, scales=None):
    """One scale per row (a token of the activations, an output channel of the weights).
    Returns (q uint8 [R, C], scales float32 [R])."""
    x = _as_2d(x)
    _need_cuda(x)
    R, C = x.shape
    if q is None:
        q = torch.empty((R, C), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((R,), dtype=torch.float32, device=x.device)
    _check_out(q, (R, C), _CODES, "q", x, (x,))
    _check_out(scales, (R,), _F32, "scales", x, (x, q))
    _check("fp8_quantize_rowwise",
           lib().fp8_quantize_rowwise(_ptr(x), _dt(x), R, C, _ptr(q), _ptr(scales), _stream(x)))
    return q, scales


def e8m0_row_bytes(groups):
    """Bytes per row of a UE8M0 scale tensor with `groups` scales (four per 32-bit word)."""
    return (groups + 3) // 4 * 4


def fp8_quantize_per_token_group_ue8m0(x, group_rows=1, group_cols=128, q=None, scales=None):
    """Like fp8_quantize_per_token_group with power-of-two (UE8M0) scales.  Returns
    (q uint8 [R, C], scales uint8 e8m0fnu [ceil(R/group_rows), G4]) where G4 is
    ceil(C/group_cols) rounded up to a multiple of 4; the padding bytes are 127."""
    x = _as_2d(x)
    _need_cuda(x)
    R, C = x.shape
    if q is None:
        q = torch.empty((R, C), dtype=torch.uint8, device=x.device)
    grid = (-(-R // max(group_rows, 1)), e8m0_row_bytes(-(-C // max(group_cols, 1))))
    if scales is None:
        scales = torch.empty(grid, dtype=torch.uint8, device=x.device)
    _check_out(q, (R, C), _CODES, "q", x, (x,))
    _check_out(scales, grid, _U8, "scales", x, (x, q))
    _check("fp8_quantize_per_token_group_ue8m0",
           lib().fp8_quantize_per_token_group_ue8m0(_ptr(x), _dt(x), R, C, group_rows, group_cols,
                                                    _ptr(q), _ptr(scales), _stream(x)))
    return q, scales


def _gemm(name, qa, sa, qb, sb, out_dtype, out, scale_dtype=torch.float32):
    qa, qb = _codes(_as_2d(qa)), _codes(_as_2d(qb))
    _same_device(qa, qb, sa, sb)
    M, K = qa.shape
    N, K2 = qb.shape
    if K != K2:
        raise ValueError(f"K mismatch: qa has {K}, qb has {K2}")
    sa = sa.contiguous()
    sb = sb.contiguous()
    if sa.dtype != scale_dtype or sb.dtype != scale_dtype:
        raise TypeError(f"scales must be {scale_dtype}")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=qa.device)
    _check_out(out, (M, N), _OUT, "out", qa, (qa, qb, sa, sb))
    fn = getattr(lib(), name)
    _check(name, fn(_ptr(qa), _ptr(sa), _ptr(qb), _ptr(sb), M, N, K, _ptr(out), _out_dt(out.dtype),
                    _stream(qa)))
    return out


def fp8_gemm_scaled_tensorwise(qa, sa, qb, sb, out_dtype=torch.bfloat16, out=None):
    """C [M, N] = (qa @ qb^T) * sa * sb; qa [M, K], qb [N, K] e4m3 codes, sa/sb float32 [1]."""
    if sa.numel() != 1 or sb.numel() != 1:
        raise ValueError("tensorwise scales are single float32 values")
    return _gemm("fp8_gemm_scaled_tensorwise", qa, sa, qb, sb, out_dtype, out)


def fp8_gemm_scaled_rowwise(qa, sa, qb, sb, out_dtype=torch.bfloat16, out=None):
    """C [M, N] = (qa @ qb^T) * sa[m] * sb[n]; sa float32 [M] (per token), sb float32 [N]
    (per output channel)."""
    M, N = qa.shape[0], qb.shape[0]
    if sa.numel() != M or sb.numel() != N:
        raise ValueError(f"rowwise scales must have {M} and {N} entries, got {sa.numel()} and {sb.numel()}")
    return _gemm("fp8_gemm_scaled_rowwise", qa, sa, qb, sb, out_dtype, out)


def _grouped(name, qa, sa, qb, sb, offsets, out_dtype, out, scale_dtype):
    qa = _codes(_as_2d(qa))
    qb = _codes(qb)
    if qb.dim() != 3:
        raise ValueError(f"expert weights must be [E, N, K], got {tuple(qb.shape)}")
    qb = qb.contiguous()
    _same_device(qa, qb, sa, sb, offsets)
    T, K = qa.shape
    E, N, K2 = qb.shape
    if K != K2:
        raise ValueError(f"K mismatch: qa has {K}, qb has {K2}")
    if offsets.dtype != torch.int32 or offsets.numel() != E + 1:
        raise TypeError(f"offsets must be int32 [{E + 1}]")
    sa, sb, offsets = sa.contiguous(), sb.contiguous(), offsets.contiguous()
    if sa.dtype != scale_dtype or sb.dtype != scale_dtype:
        raise TypeError(f"scales must be {scale_dtype}")
    if K % 128 == 0 and K > 0:
        g = K // 128 if scale_dtype == torch.float32 else e8m0_row_bytes(K // 128)
        if tuple(sa.shape) != (T, g) or tuple(sb.shape) != (E, -(-N // 128), g):
            raise ValueError(f"grouped scales must be [{T}, {g}] and [{E}, {-(-N // 128)}, {g}], "
                             f"got {tuple(sa.shape)} and {tuple(sb.shape)}")
    if out is None:
        out = torch.empty((T, N), dtype=out_dtype, device=qa.device)
    _check_out(out, (T, N), _OUT, "out", qa, (qa, qb, sa, sb, offsets))
    fn = getattr(lib(), name)
    _check(name, fn(_ptr(qa), _ptr(sa), _ptr(qb), _ptr(sb), _ptr(offsets), E, T, N, K, _ptr(out),
                    _out_dt(out.dtype), _stream(qa)))
    return out


def fp8_gemm_grouped_blockwise(qa, sa, qb, sb, offsets, out_dtype=torch.bfloat16, out=None):
    """Mixture-of-experts product: rows offsets[e]:offsets[e+1] of qa [T, K] times expert
    weight qb[e] ([E, N, K]); sa float32 [T, K/128], sb float32 [E, ceil(N/128), K/128],
    offsets int32 [E + 1] on the device.  Returns C [T, N]."""
    return _grouped("fp8_gemm_grouped_blockwise", qa, sa, qb, sb, offsets, out_dtype, out, torch.float32)


def fp8_gemm_grouped_blockwise_ue8m0(qa, sa, qb, sb, offsets, out_dtype=torch.bfloat16, out=None):
    """The grouped product with UE8M0 scales: sa uint8 [T, G4], sb uint8 [E, ceil(N/128), G4]."""
    return _grouped("fp8_gemm_grouped_blockwise_ue8m0", qa, sa, qb, sb, offsets, out_dtype, out, torch.uint8)


def fp8_gemm_scaled_blockwise(qa, sa, qb, sb, out_dtype=torch.bfloat16, out=None):
    """Per 128-wide K slab scales: sa [M, K/128], sb [ceil(N/128), K/128]."""
    M, K = qa.shape
    N = qb.shape[0]
    if K % 128 == 0 and K > 0:
        if tuple(sa.shape) != (M, K // 128) or tuple(sb.shape) != (-(-N // 128), K // 128):
            raise ValueError(f"blockwise scales must be [{M}, {K // 128}] and [{-(-N // 128)}, {K // 128}], "
                             f"got {tuple(sa.shape)} and {tuple(sb.shape)}")
    return _gemm("fp8_gemm_scaled_blockwise", qa, sa, qb, sb, out_dtype, out)


def fp8_gemm_scaled_blockwise_ue8m0(qa, sa, qb, sb, out_dtype=torch.bfloat16, out=None):
    """Blockwise product with UE8M0 scales: sa uint8 [M, G4], sb uint8 [ceil(N/128), G4],
    G4 = K/128 rounded up to a multiple of 4 (the layout the UE8M0 quantizer writes)."""
    M, K = qa.shape
    N = qb.shape[0]
    if K % 128 == 0 and K > 0:
        g4 = e8m0_row_bytes(K // 128)
        if tuple(sa.shape) != (M, g4) or tuple(sb.shape) != (-(-N // 128), g4):
            raise ValueError(f"UE8M0 scales must be [{M}, {g4}] and [{-(-N // 128)}, {g4}], "
                             f"got {tuple(sa.shape)} and {tuple(sb.shape)}")
    return _gemm("fp8_gemm_scaled_blockwise_ue8m0", qa, sa, qb, sb, out_dtype, out, torch.uint8)


def fp8_quantize_static(x, scale, q=None, amax_acc=None):
    """q = e4m3(x / scale) with a given float32 [1] device scale (static or delayed scaling),
    saturating; if amax_acc (uint32 [1], or int32 viewed as such) is given, the tensor's amax
    is folded into it for fp8_delayed_scaling_update.  Returns q."""
    x = _as_2d(x)
    _need_cuda(x, scale)
    if scale.dtype != torch.float32 or scale.numel() != 1:
        raise TypeError("scale must be one float32 value on the device")
    R, C = x.shape
    if q is None:
        q = torch.empty((R, C), dtype=torch.uint8, device=x.device)
    _same_device(x, scale)
    _check_out(q, (R, C), _CODES, "q", x, (x, scale))
    acc = None
    if amax_acc is not None:
        _same_device(x, amax_acc)
        if amax_acc.element_size() != 4 or amax_acc.numel() != 1:
            raise TypeError("amax_acc must be one 32-bit word on the device")
        acc = ctypes.c_void_p(amax_acc.data_ptr())
    _check("fp8_quantize_static",
           lib().fp8_quantize_static(_ptr(x), _dt(x), R, C, ctypes.c_void_p(scale.data_ptr()), _ptr(q),
                                     acc, _stream(x)))
    return q


class DelayedScaling:
    """Device-resident delayed-scaling state: history float32 [len] (a ring), the amax
    accumulator (int32 storage of the uint32 word), the step count (int32), the scale
    (float32 [1], initially `init_scale`) and the scale the last quantize_step cast with
    (scale_used)."""

    def __init__(self, history_len, interval, margin=0, init_scale=1.0, device="cuda"):
        self.history = torch.zeros(history_len, dtype=torch.float32, device=device)
        self.amax_acc = torch.zeros(1, dtype=torch.int32, device=device)
        self.step = torch.zeros(1, dtype=torch.int32, device=device)
        self.scale = torch.full((1,), float(init_scale), dtype=torch.float32, device=device)
        self.scale_used = torch.full((1,), float(init_scale), dtype=torch.float32, device=device)
        self.interval, self.margin = int(interval), int(margin)

    def quantize_step(self, x, q=None):
        """One whole step in one call: cast x with the current scale (copied to
        scale_used, the scale to hand to the GEMM), push its amax, refresh the scale every
        interval steps.  Returns q."""
        return fp8_quantize_delayed(x, self.history, self.amax_acc, self.step, self.interval, self.margin,
                                    self.scale, self.scale_used, q=q)

    def quantize(self, x, q=None):
        """Cast x with the current scale and record its amax."""
        return fp8_quantize_static(x, self.scale, q=q, amax_acc=self.amax_acc)

    def update(self):
        """Push the recorded amax into the history; refresh the scale every interval steps."""
        fp8_delayed_scaling_update(self.history, self.amax_acc, self.step, self.interval, self.margin,
                                   self.scale)


def fp8_delayed_scaling_update(history, amax_acc, step, interval, margin, scale):
    _need_cuda(history, amax_acc, step, scale)
    _check("fp8_delayed_scaling_update",
           lib().fp8_delayed_scaling_update(ctypes.c_void_p(history.data_ptr()), history.numel(),
                                            ctypes.c_void_p(amax_acc.data_ptr()),
                                            ctypes.c_void_p(step.data_ptr()), interval, margin,
                                            ctypes.c_void_p(scale.data_ptr()), _stream(history)))


def fp8_quantize_delayed(x, history, amax_acc, step, interval, margin, scale, scale_used, q=None):
    """fp8_quantize_static followed by fp8_delayed_scaling_update in one call; the scale
    the codes were made with is written to scale_used.  Returns q."""
    x = _as_2d(x)
    _need_cuda(x, history, amax_acc, step, scale, scale_used)
    for t, what in ((scale, "scale"), (scale_used, "scale_used")):
        if t.dtype != torch.float32 or t.numel() != 1:
            raise TypeError(f"{what} must be one float32 value on the device")
    for t, what in ((amax_acc, "amax_acc"), (step, "step")):
        if t.element_size() != 4 or t.numel() != 1:
            raise TypeError(f"{what} must be one 32-bit word on the device")
    if history.dtype != torch.float32 or not history.is_contiguous():
        raise TypeError("history must be a contiguous float32 tensor")
    R, C = x.shape
    if q is None:
        q = torch.empty((R, C), dtype=torch.uint8, device=x.device)
    _same_device(x, history, amax_acc, step, scale, scale_used)
    _check_out(q, (R, C), _CODES, "q", x, (x, history, amax_acc, step, scale, scale_used))
    vp = lambda t: ctypes.c_void_p(t.data_ptr())
    _check("fp8_quantize_delayed",
           lib().fp8_quantize_delayed(_ptr(x), _dt(x), R, C, vp(history), history.numel(), vp(amax_acc),
                                      vp(step), int(interval), int(margin), vp(scale), vp(scale_used),
                                      _ptr(q), _stream(x)))
    return q


def fp8_debug_cast_f32(v, q=None):
    """q = e4m3(v) elementwise with the library's device encoder (test hook)."""
    v = v.contiguous()
    _need_cuda(v)
    if v.dtype != torch.float32:
        raise TypeError("fp8_debug_cast_f32 takes float32")
    if q is None:
        q = torch.empty(v.shape, dtype=torch.uint8, device=v.device)
    _check_out(q, v.shape, _CODES, "q", v, (v,))
    _check("fp8_debug_cast_f32", lib().fp8_debug_cast_f32(_ptr(v), _ptr(q), v.numel(), _stream(v)))
    return q


def fp8_debug_byte_mix(x, q=None):
    """q = the high byte of every 16-bit element of x (measurement reference: a quantizer's
    byte mix without its arithmetic)."""
    x = x.contiguous()
    _need_cuda(x)
    if x.element_size() != 2:
        raise TypeError("fp8_debug_byte_mix takes a 16-bit tensor")
    if q is None:
        q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _check_out(q, x.shape, _U8, "q", x, (x,))
    _check("fp8_debug_byte_mix", lib().fp8_debug_byte_mix(_ptr(x), _ptr(q), x.numel(), _stream(x)))
    return q


class _GemmLaunch(ctypes.Structure):
    _fields_ = [("kernel", _I32), ("tile_m", _I32), ("tile_n", _I32), ("variant", _I32), ("waves", _I32),
                ("paired", _I32), ("grid", _I64), ("threads", _I64), ("n_begin", _I64), ("n_end", _I64),
                ("max_range", _I64), ("max_offset", _I64)]


class _GemmPlan(ctypes.Structure):
    _fields_ = [("launches", _I32), ("reserved", _I32), ("launch", _GemmLaunch * 2)]


GEMM_MODES = {"tensorwise": 0, "blockwise": 1, "blockwise_ue8m0": 2, "rowwise": 3}
GEMM_KERNELS = {1: "gemv_stream", 2: "gemv_valu", 3: "gemv_mfma", 4: "skinny", 5: "tile", 6: "staged"}


def fp8_debug_gemm_plan(mode, M, N, K):
    """The launches a scaled GEMM of this shape makes (host arithmetic only, no GPU): a list
    of dicts with the kernel's name and the fields of fp8_gemm_launch_t."""
    plan = _GemmPlan()
    _check("fp8_debug_gemm_plan", lib().fp8_debug_gemm_plan(GEMM_MODES[mode], M, N, K, ctypes.byref(plan)))
    out = []
    for i in range(plan.launches):
        l = plan.launch[i]
        d = {name: getattr(l, name) for name, _ in _GemmLaunch._fields_}
        d["kernel"] = GEMM_KERNELS[l.kernel]
        out.append(d)
    return out


def _act_scale_spec(mode, K):
    """Shape and dtype of the activation scales fp8_gemv_dynamic writes for x as [1, K]: those
    of the quantizer that pairs with `mode`."""
    if mode in ("tensorwise", "rowwise"):
        return (1,), torch.float32
    if mode == "blockwise":
        return (1, K // 128), torch.float32
    return (1, e8m0_row_bytes(K // 128)), torch.uint8


def _weight_scale_spec(mode, N, K):
    """Shape and dtype of the weight scales the GEMM of `mode` takes for qb [N, K]."""
    if mode == "tensorwise":
        return (1,), torch.float32
    if mode == "rowwise":
        return (N,), torch.float32
    if mode == "blockwise":
        return (-(-N // 128), K // 128), torch.float32
    return (-(-N // 128), e8m0_row_bytes(K // 128)), torch.uint8


def fp8_gemv_dynamic(mode, x, qb, sb, out_dtype=torch.bfloat16, out=None, qa=None, sa=None):
    """The whole one-token step in one call: x ([K] or [1, K], bf16/fp16) quantized with the
    scheme that pairs with `mode` ("tensorwise": one scale; "rowwise": the row's scale;
    "blockwise": 1x128 groups with float32 scales; "blockwise_ue8m0": 1x128 groups with UE8M0
    scales), then multiplied with qb [N, K] and its scales sb as the GEMM of that mode takes
    them.  Returns (out [1, N], qa uint8 [1, K], sa), qa and sa as the matching quantizer
    writes them for x as [1, K]."""
    if mode not in GEMM_MODES:
        raise ValueError(f"mode must be one of {sorted(GEMM_MODES)}, got {mode!r}")
    if x.dim() == 1:
        x = x.reshape(1, -1)
    x = _as_2d(x)
    if x.shape[0] != 1:
        raise ValueError(f"one token: x must be [K] or [1, K], got {tuple(x.shape)}")
    qb = _codes(_as_2d(qb))
    _same_device(x, qb, sb)
    K = x.shape[1]
    N, K2 = qb.shape
    if K != K2:
        raise ValueError(f"K mismatch: x has {K}, qb has {K2}")
    sb = sb.contiguous()
    if K > 0 and (K % 128 == 0 or mode in ("tensorwise", "rowwise")):
        shape, dtype = _weight_scale_spec(mode, N, K)
        if tuple(sb.shape) != shape or sb.dtype != dtype:
            raise ValueError(f"{mode} weight scales must be {dtype} {shape}, got {sb.dtype} {tuple(sb.shape)}")
    a_shape, a_dtype = _act_scale_spec(mode, K)
    if qa is None:
        qa = torch.empty((1, K), dtype=torch.uint8, device=x.device)
    if sa is None:
        sa = torch.empty(a_shape, dtype=a_dtype, device=x.device)
    if out is None:
        out = torch.empty((1, N), dtype=out_dtype, device=x.device)
    _check_out(qa, (1, K), _CODES, "qa", x, (x, qb, sb))
    _check_out(sa, a_shape, (a_dtype,), "sa", x, (x, qb, sb, qa))
    _check_out(out, (1, N), _OUT, "out", x, (x, qb, sb, qa, sa))
    _check("fp8_gemv_dynamic",
           lib().fp8_gemv_dynamic(GEMM_MODES[mode], _ptr(x), _dt(x), _ptr(qb), _ptr(sb), N, K, _ptr(qa), _ptr(sa),
                                  _ptr(out), _out_dt(out.dtype), _stream(x)))
    return out, qa, sa
