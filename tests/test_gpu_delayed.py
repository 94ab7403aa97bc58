"""GPU parity for static scaling (fp8_quantize_static) and the delayed-scaling update
(fp8_delayed_scaling_update): codes, recorded amax, history ring, step count and scale bit
for bit against the oracle, eagerly and as replays of a captured HIP graph."""

import numpy as np
import pytest
import torch

import oracle
import fp8_quantized_gemm_amax_amd as fp8
from fp8_quantized_gemm_amax_amd import workloads as wl
from parity_util import (DEV, to_dev, u8_to_dev, f32_to_dev, guarded_u8, guard_intact, host_u8,
                         out_to_f64, assert_bytes_equal)

pytestmark = pytest.mark.gpu


def scale_dev(v):
    return torch.tensor([float(np.float32(v))], dtype=torch.float32, device=DEV)


def acc_bits(acc):
    torch.cuda.synchronize()
    return int(acc.cpu().numpy().view(np.uint32)[0])


def f32_bits(v):
    return int(np.array([v], np.float32).view(np.uint32)[0])


def canonical_bits(v):
    return 0x7FC00000 if np.isnan(v) else f32_bits(v)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", [(1, 1), (3, 5), (37, 300), (257, 509), (1000, 1001), (2, 4096)])
@pytest.mark.parametrize("which", ["own", "small", "tiny"])
def test_static_matches_oracle(dtype, shape, which):
    """The tensor's own scale (must equal the dynamic quantizer), a scale four times too
    small (a quarter of the elements saturate), and a scale below 2^-100 (the exact
    division path); ragged tails; the recorded amax bits."""
    rng = np.random.default_rng(shape[0] * 13 + shape[1])
    a = rng.standard_t(4, shape) * (3.0 if dtype == "bf16" else 0.5)
    bits = wl.to_bf16_bits(a) if dtype == "bf16" else a.astype(np.float16).view(np.uint16)
    x32 = oracle.input_to_f32(bits, dtype)
    amax = oracle.amax_per_tensor(x32)
    own = oracle.scale_from_amax(amax)
    scale = {"own": own, "small": own / np.float32(4), "tiny": np.float32(2.0 ** -110)}[which]
    q_want, amax_want = oracle.quantize_static(bits, dtype, scale)
    q, qfull = guarded_u8(shape)
    acc = torch.zeros(1, dtype=torch.int32, device=DEV)
    fp8.fp8_quantize_static(to_dev(bits, dtype), scale_dev(scale), q=q, amax_acc=acc)
    assert_bytes_equal(host_u8(q), q_want, f"{which} {shape} {dtype} codes")
    assert guard_intact(qfull, int(np.prod(shape)), "u8")
    assert acc_bits(acc) == canonical_bits(amax_want)
    if which == "own":
        q_dyn, _ = oracle.quantize_per_tensor(bits, dtype)
        assert_bytes_equal(host_u8(q), q_dyn, "equals the dynamic quantizer")


def test_static_without_record_and_specials():
    bits = np.array([[0x3F80, 0xFF80, 0x7FC0, 0x0000, 0x8001, 0x4480, 0xC480, 0x7F7F]], np.uint16)
    for scale in (np.float32(1.0), np.float32(0.01)):
        q_want, amax_want = oracle.quantize_static(bits, "bf16", scale)
        q = fp8.fp8_quantize_static(to_dev(bits), scale_dev(scale))
        assert_bytes_equal(host_u8(q), q_want, f"specials at scale {scale}")
        acc = torch.zeros(1, dtype=torch.int32, device=DEV)
        fp8.fp8_quantize_static(to_dev(bits), scale_dev(scale), amax_acc=acc)
        assert acc_bits(acc) == 0x7FC00000                      # NaN amax is recorded as NaN


def sweep_scales():
    rng = np.random.default_rng(17)
    edges = [2.0 ** -80, 2.0 ** 119, 2.0 ** -100, 2.0 ** 126, 2.0 ** 127, 1.0, 1 / 448]
    out = [np.float32(e) for e in edges]
    out += [np.nextafter(np.float32(e), np.float32(np.inf)) for e in edges[:2]]
    out += [np.nextafter(np.float32(e), np.float32(0)) for e in edges[:2]]
    out += [np.float32(2.0 ** rng.uniform(-100, 127)) for _ in range(24)]
    return out


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_static_scale_sweep(dtype):
    """Scales over the float32 range, on both sides of the bounds of the fast quotient
    (2^-80, 2^119), with inputs proportional to the scale: quotients at e4m3 midpoints (exact
    ties when the scale is a power of two), near the smallest code 2^-10, above 448 and
    infinite, plus signed zeros and NaNs."""
    rng = np.random.default_rng(5 if dtype == "bf16" else 6)
    mids = np.array(oracle.positive_values(), np.float64)
    mids = (mids[1:] + mids[:-1]) / 2
    base = np.concatenate([mids, -mids, 2.0 ** -10 * np.array([0.5, 1, 1.5, 2, 3]),
                           rng.standard_t(3, 700) * 60, [1e6, -1e6, 0.0, -0.0]])
    for scale in sweep_scales():
        x = base * float(scale)
        with np.errstate(over="ignore"):                # inputs beyond the format become inf
            if dtype == "bf16":
                bits = wl.to_bf16_bits(x)
                bits[:3] = [0x7F80, 0xFF80, 0x7FC1]
            else:
                bits = x.astype(np.float16).view(np.uint16).copy()
                bits[:3] = [0x7C00, 0xFC00, 0x7E01]
        bits = bits.reshape(1, -1)
        q_want, amax_want = oracle.quantize_static(bits, dtype, scale)
        acc = torch.zeros(1, dtype=torch.int32, device=DEV)
        q = fp8.fp8_quantize_static(to_dev(bits, dtype), scale_dev(scale), amax_acc=acc)
        assert_bytes_equal(host_u8(q), q_want, f"{dtype} scale {float(scale)!r}")
        assert acc_bits(acc) == 0x7FC00000


def test_recorded_amax_accumulates_over_calls():
    rng = np.random.default_rng(4)
    acc = torch.zeros(1, dtype=torch.int32, device=DEV)
    want = np.float32(0)
    for k in range(3):
        bits = wl.to_bf16_bits(rng.standard_normal((64, 384)) * (10.0 if k == 1 else 1.0))
        fp8.fp8_quantize_static(to_dev(bits), scale_dev(1.0), amax_acc=acc)
        want = max(want, oracle.amax_per_tensor(oracle.input_to_f32(bits, "bf16")))
    assert acc_bits(acc) == f32_bits(want)


def ring_to_recent_first(ring, step):
    L = len(ring)
    return np.array([ring[(step - 1 - i) % L] for i in range(L)], np.float32)


def check_state(ds, h_want, step_want, scale_want, label):
    torch.cuda.synchronize()
    step = int(ds.step.cpu()[0])
    assert step == step_want, label
    ring = ds.history.cpu().numpy()
    np.testing.assert_array_equal(ring_to_recent_first(ring, step)[:min(step, len(ring))],
                                  h_want[:min(step, len(ring))], err_msg=label)
    assert canonical_bits(float(ds.scale.cpu()[0])) == canonical_bits(scale_want), label
    assert acc_bits(ds.amax_acc) == 0, f"{label}: the update clears the recorded amax"


@pytest.mark.parametrize("length,interval,margin", [(3, 4, 0), (5, 2, 1), (1, 1, -2), (70, 3, 0)])
def test_delayed_sequence_matches_oracle(length, interval, margin):
    """Twelve steps on tensors whose magnitude changes from step to step (so the scale
    rises and falls and saturation happens when it lags), each step's codes against the
    oracle quantizing with the oracle's scale, then the state after the update."""
    rng = np.random.default_rng(length * 100 + interval * 10 + margin)
    ds = fp8.DelayedScaling(length, interval, margin, init_scale=0.5, device=DEV)
    h, step, scale = np.zeros(length, np.float32), 0, np.float32(0.5)
    for k in range(12):
        mag = 2.0 ** rng.integers(-6, 8)
        bits = wl.to_bf16_bits(rng.standard_t(4, (33, 640)) * mag)
        q = ds.quantize(to_dev(bits))
        q_want, amax = oracle.quantize_static(bits, "bf16", scale)
        assert_bytes_equal(host_u8(q), q_want, f"step {k} codes")
        ds.update()
        h, step, scale = oracle.delayed_step(h, step, scale, amax, interval, margin)
        check_state(ds, h, step, scale, f"step {k}")


def test_delayed_step_captured_in_a_graph():
    """quantize + update captured once and replayed: every replay advances the
    device-resident state exactly as the eager steps would (no memset nodes; the amax word
    is cleared by the update kernel)."""
    rng = np.random.default_rng(9)
    xs = [wl.to_bf16_bits(rng.standard_normal((64, 512)) * 2.0 ** e) for e in (0, 3, -2)]
    xdev = [to_dev(b) for b in xs]
    ds = fp8.DelayedScaling(4, 2, 0, init_scale=1.0, device=DEV)
    q = torch.empty((64, 512), dtype=torch.uint8, device=DEV)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for x in xdev:
                ds.quantize(x, q=q)
                ds.update()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    # capture ran nothing: the state is still the initial one
    check_state(ds, np.zeros(4, np.float32), 0, np.float32(1.0), "after capture")
    h, step, scale = np.zeros(4, np.float32), 0, np.float32(1.0)
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        for b in xs:
            q_want, amax = oracle.quantize_static(b, "bf16", scale)
            h, step, scale = oracle.delayed_step(h, step, scale, amax, 2, 0)
        assert_bytes_equal(host_u8(q), q_want, f"replay {rep} last codes")
        check_state(ds, h, step, scale, f"replay {rep}")


# ---- the whole step in one call (fp8_quantize_delayed) ----

def check_fused_state(ds, h_want, step_want, scale_want, used_want, label):
    check_state(ds, h_want, step_want, scale_want, label)
    assert canonical_bits(float(ds.scale_used.cpu()[0])) == canonical_bits(used_want), label


@pytest.mark.parametrize("shape", [(33, 640), (64, 512), (257, 509), (1000, 1001), (3, 8191)])
@pytest.mark.parametrize("length,interval,margin", [(3, 4, 0), (5, 1, 1), (70, 3, -1)])
def test_fused_sequence_matches_oracle(shape, length, interval, margin):
    """Up to 32768 elements: one launch, one workgroup; above: the static cast and the
    update.  Every step's codes and scale_used against the oracle's static cast with the
    scale before the step, then the state after it."""
    rng = np.random.default_rng(shape[0] + 7 * length)
    ds = fp8.DelayedScaling(length, interval, margin, init_scale=0.25, device=DEV)
    h, step, scale = np.zeros(length, np.float32), 0, np.float32(0.25)
    for k in range(10):
        bits = wl.to_bf16_bits(rng.standard_t(4, shape) * 2.0 ** rng.integers(-5, 9))
        q = ds.quantize_step(to_dev(bits))
        q_want, amax = oracle.quantize_static(bits, "bf16", scale)
        assert_bytes_equal(host_u8(q), q_want, f"{shape} step {k} codes")
        used = scale
        h, step, scale = oracle.delayed_step(h, step, scale, amax, interval, margin)
        check_fused_state(ds, h, step, scale, used, f"{shape} step {k}")


@pytest.mark.parametrize("shape", [(16, 128), (512, 2048)])
def test_fused_folds_in_recorded_amax_and_empty_tensors(shape):
    """Amaxes recorded by fp8_quantize_static since the last update are folded into the
    fused call's push; an empty tensor pushes what was recorded (0 when nothing was)."""
    rng = np.random.default_rng(3)
    ds = fp8.DelayedScaling(4, 1, 0, init_scale=1.0, device=DEV)
    big = wl.to_bf16_bits(rng.standard_normal(shape) * 300.0)
    small = wl.to_bf16_bits(rng.standard_normal(shape))
    fp8.fp8_quantize_static(to_dev(big), ds.scale, amax_acc=ds.amax_acc)
    ds.quantize_step(to_dev(small))
    h, step, scale = np.zeros(4, np.float32), 0, np.float32(1.0)
    amax = max(oracle.quantize_static(big, "bf16", scale)[1], oracle.quantize_static(small, "bf16", scale)[1])
    h, step, scale = oracle.delayed_step(h, step, scale, amax, 1, 0)
    check_fused_state(ds, h, step, scale, np.float32(1.0), "folded")
    empty = torch.empty((0, shape[1]), dtype=torch.bfloat16, device=DEV)
    used = scale
    ds.quantize_step(empty)
    h, step, scale = oracle.delayed_step(h, step, scale, np.float32(0), 1, 0)
    check_fused_state(ds, h, step, scale, used, "empty tensor")


def test_fused_step_captured_in_a_graph():
    """One graph holding fused steps on a one-workgroup tensor and (twice) a many-workgroup
    tensor, and a tensorwise GEMM fed by scale_used, replayed several times with eager work
    between the replays; every replay against the oracle's sequence."""
    rng = np.random.default_rng(11)
    shapes = [(16, 1024), (512, 2048), (512, 2048)]
    xs = [wl.to_bf16_bits(rng.standard_normal(s) * 2.0 ** e) for s, e in zip(shapes, (0, 4, -3))]
    xdev = [to_dev(b) for b in xs]
    ds_small = fp8.DelayedScaling(3, 2, 0, init_scale=1.0, device=DEV)
    ds_big = fp8.DelayedScaling(3, 2, 0, init_scale=1.0, device=DEV)
    qs = [torch.empty(s, dtype=torch.uint8, device=DEV) for s in shapes]
    w_bits = wl.to_bf16_bits(rng.standard_normal((256, 2048)) * 0.02)
    qw_h, sw_h = oracle.quantize_per_tensor(w_bits, "bf16")
    qw, sw = u8_to_dev(qw_h), f32_to_dev(sw_h)
    c = torch.empty((512, 256), dtype=torch.bfloat16, device=DEV)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            ds_small.quantize_step(xdev[0], q=qs[0])
            ds_big.quantize_step(xdev[1], q=qs[1])
            ds_big.quantize_step(xdev[2], q=qs[2])
            fp8.fp8_gemm_scaled_tensorwise(qs[2], ds_big.scale_used, qw, sw, out=c)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    check_fused_state(ds_big, np.zeros(3, np.float32), 0, np.float32(1.0), np.float32(1.0), "after capture")
    st_s = (np.zeros(3, np.float32), 0, np.float32(1.0))
    st_b = (np.zeros(3, np.float32), 0, np.float32(1.0))
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert torch.ones(1024, device=DEV).sum().item() == 1024.0      # eager work between replays
        used_s = st_s[2]
        q0, a0 = oracle.quantize_static(xs[0], "bf16", used_s)
        st_s = oracle.delayed_step(*st_s, a0, 2, 0)
        assert_bytes_equal(host_u8(qs[0]), q0, f"replay {rep} small codes")
        check_fused_state(ds_small, *st_s, used_s, f"replay {rep} small")
        for i in (1, 2):
            used_b = st_b[2]
            qi, ai = oracle.quantize_static(xs[i], "bf16", used_b)
            st_b = oracle.delayed_step(*st_b, ai, 2, 0)
            assert_bytes_equal(host_u8(qs[i]), qi, f"replay {rep} big codes {i}")
        check_fused_state(ds_big, *st_b, used_b, f"replay {rep} big")
        r = oracle.check_gemm(out_to_f64(c), oracle.gemm_tensorwise_ref(qi, used_b, qw_h, sw_h),
                              oracle.bound_tensorwise(qi, used_b, qw_h, sw_h), "bf16")
        assert r["ok"], f"replay {rep} GEMM: {r}"
