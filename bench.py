"""Throughput of the FP8 E4M3 scaled-GEMM hot path on one MI355X.

One step = the whole hot path over one batch of synthetic input: amax + scale + cast of
the activations (per tensor, or per 1x128 token group), then the FP8 x FP8 GEMM with
float32 accumulation and the scale epilogue; for one token with dynamic scales both in one
launch (fp8_gemv_dynamic; --two-launch times the pair).  Weights are quantized once before
timing (as a serving stack does at load time), except in the small per-tensor workload,
where both operands are quantized on every call.

Inputs stay resident in HBM; each step reads a different copy of the input set from a
rotation whose footprint exceeds 1 GiB, so reads come from HBM rather than the 256 MB
Infinity Cache.

Prints one JSON line.  `value` is the whole step's throughput (TFLOP/s including the
activation quantize; GB/s for M <= 16 decode) from HIP events around the graph replays of
the timed region (mean, with the median and 10th/90th percentiles over replays);
`roofline` rates the dominant kernel (the GEMM) from HIP events around each of its
launches in a step-by-step pass where every GEMM follows its own quantize, as in the
timed steps; `cpu_baseline` times the CPU oracle on a bounded sample of the same workload;
`machine` records the GPU's compute units and clock, the ROCm version and the host CPU.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FP8 scaled-GEMM TFLOP/s incl. quantize (% MFMA FP8 peak); decode GB/s (% HBM)"
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA, 5.0 PFLOP/s
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, 8 TB/s
DEFAULT_WORKLOAD = "deepseek_v3_blockwise"   # the largest configuration: M=4096, N=18432, K=7168
ROTATION_BYTES = 1 << 30
DELAYED_HISTORY = 16          # amax history length of the delayed recipe (the pages give none)
DELAYED_INTERVAL = 4          # the recipe's interval and margin
DELAYED_MARGIN = 0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=500)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--m", type=int, default=None, help="M variant of the workload (default: largest)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--act-scaling", choices=["dynamic", "delayed"], default="dynamic",
                   help="per-tensor workloads: scale from this step's amax (dynamic), or the "
                        "delayed-scaling recipe (static cast with the scale left by the amax "
                        "history; margin 0, interval 4)")
    p.add_argument("--rowwise", action="store_true",
                   help="per-channel scaling on any workload shape: A per token every step, W per "
                        "output channel once, the rowwise GEMM")
    p.add_argument("--scale-fmt", choices=["float32", "ue8m0"], default="float32",
                   help="blockwise workloads: float32 scales (amax/448) or UE8M0 power-of-two "
                        "scale bytes on the scaled MFMA")
    p.add_argument("--quantize-only", choices=["activations", "weights"], default=None,
                   help="time only the workload's activation quantize (per token 1x128 groups or per "
                        "tensor) or its weight quantize (128x128 blocks), next to the byte-mix "
                        "reference (2 B read, 1 B written per element, no arithmetic) on the same tensors")
    p.add_argument("--vendor-gemm", action="store_true",
                   help="time the workload's GEMM (per tensor and per row/column scales) in this "
                        "library and in the vendor FP8 GEMM behind torch._scaled_mm on the same codes "
                        "and scales, cold inputs, HIP graphs; one JSON line")
    p.add_argument("--two-launch", action="store_true",
                   help="one token: time the quantize launch followed by the one-token GEMM instead "
                        "of the fused step (fp8_gemv_dynamic, one launch)")
    p.add_argument("--copy-mb", type=int, default=0,
                   help="instead of the hot path, run a plain device copy of this many MiB "
                        "(the known-size reference for rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    return p.parse_args()


_CSRC = "fp8_quantized_gemm_amax_amd/csrc/"
# the sources of each kernel family's code: the tiled and few-token GEMMs (M > 16), and the
# decode kernels with the fused one-token step (M <= 16)
KERNEL_SOURCES = {
    "gemm": [_CSRC + f for f in ("gemm.hip", "gemm_common.hpp", "dma.hpp", "fp8_device.hpp", "gemm_plan.hpp")],
    "decode": [_CSRC + f for f in ("gemv.hip", "fp8_device.hpp", "quant_device.hpp", "gemm_plan.hpp")],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_traffic.json")


def strip_comments(src):
    """C/C++ source without its comments and with runs of white space folded to one blank, so
    that an edit of a comment leaves the hash of the code unchanged.  String and character
    literals are kept as written."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash(M):
    """Hash of the code of the kernel family that runs M tokens (comments and layout
    excluded): the counter table's entries hold only while it is unchanged."""
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES["decode" if M <= 16 else "gemm"]:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(strip_comments(f.read()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def scheme_of(w, scale_fmt="float32", act_scaling="dynamic", rowwise=False):
    """How a step is scaled: tensorwise, tensorwise-delayed, blockwise, blockwise-ue8m0 or
    rowwise."""
    if rowwise:
        return "rowwise"
    if w.mode == "grouped":
        return "grouped-ue8m0" if scale_fmt == "ue8m0" else "grouped"
    if w.mode == "tensorwise":
        return "tensorwise-delayed" if act_scaling == "delayed" else "tensorwise"
    return "blockwise-ue8m0" if scale_fmt == "ue8m0" else "blockwise"


def traffic_key(workload, M, scheme="tensorwise", fused=False):
    """Counter-table key of a GEMM launch (delayed scaling runs the tensorwise GEMM; `fused`:
    the one-token step's single launch)."""
    suffix = {"blockwise-ue8m0": "/ue8m0", "grouped-ue8m0": "/ue8m0", "rowwise": "/rowwise"}.get(scheme, "")
    return f"{workload}/M={M}" + suffix + ("/fused" if fused else "")


def measured_traffic(workload, M, scheme="tensorwise", fused=False):
    """HBM bytes per GEMM launch from the committed rocprofv3 counter runs, or None when
    there is no entry for this workload or the kernel sources changed since it was taken."""
    import json as _json
    try:
        with open(TRAFFIC_FILE) as f:
            table = _json.load(f)
    except (OSError, ValueError):
        return None
    e = table.get(traffic_key(workload, M, scheme, fused))
    if not e or e.get("kernel_source_sha") != kernel_source_hash(M):
        return None
    return e.get("traffic_bytes_per_launch")


def shader_clock():
    """The current shader clock level of the first GPU that lists one in sysfs (MHz), or None.
    Read from a file: no child process is started (a process that has initialised the GPU
    must not exec another program on the box)."""
    import glob
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(path) as f:
                for ln in f:
                    if ln.rstrip().endswith("*"):
                        return ln.split(":", 1)[1].strip().rstrip("*").strip()
        except OSError:
            continue
    return None


def machine_facts():
    """Compute units and clocks of GPU 0, the ROCm and HIP versions, the host CPU model."""
    import torch
    props = torch.cuda.get_device_properties(0)
    facts = {"gpu": props.name, "gcn_arch": getattr(props, "gcnArchName", None),
             "compute_units": props.multi_processor_count, "hip": torch.version.hip}
    try:
        with open("/opt/rocm/.info/version") as f:
            facts["rocm"] = f.read().strip()
    except OSError:
        facts["rocm"] = None
    try:
        with open("/proc/cpuinfo") as f:
            facts["host_cpu"] = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        facts["host_cpu"] = None
    facts["host_threads"] = len(os.sched_getaffinity(0))
    facts["sclk"] = shader_clock()
    return facts


def percentiles(xs):
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {"median": round(float(np.median(a)), 6), "p10": round(float(np.percentile(a, 10)), 6),
            "p90": round(float(np.percentile(a, 90)), 6), "n": int(a.size)}


def quantize_reference(args):
    """The quantize pass alone (cold inputs, HIP graphs) and the byte-mix reference on the same
    tensors; one JSON line with both rates."""
    import numpy as np
    import torch
    import fp8_quantized_gemm_amax_amd as fp8
    from fp8_quantized_gemm_amax_amd import workloads as wl
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = wl.WORKLOADS[args.workload]
    M = args.m if args.m is not None else max(w.m_values)
    a_bits, b_bits = wl.make_inputs(args.workload, M)
    weights = args.quantize_only == "weights"
    bits = b_bits if weights else a_bits
    R_, C_ = bits.shape
    gr = 128 if weights else 1
    blockwise = w.mode == "blockwise" or weights
    x0 = wl.bits_to_tensor(bits, device=dev)
    per_set = 3 * R_ * C_
    R = max(2, min(256, -(-ROTATION_BYTES // per_set)))
    sets = []
    for _ in range(R):
        sx = {"x": x0.clone(), "q": torch.empty((R_, C_), dtype=torch.uint8, device=dev)}
        sx["s"] = (torch.empty((-(-R_ // gr), -(-C_ // 128)), dtype=torch.float32, device=dev) if blockwise
                   else torch.empty((1,), dtype=torch.float32, device=dev))
        sets.append(sx)
    del x0

    def quant(sx):
        if blockwise:
            fp8.fp8_quantize_per_token_group(sx["x"], gr, 128, q=sx["q"], scales=sx["s"])
        else:
            fp8.fp8_quantize_per_tensor(sx["x"], q=sx["q"], scale=sx["s"])

    def mix(sx):
        fp8.fp8_debug_byte_mix(sx["x"], q=sx["q"])

    def timed(fn):
        for i in range(R):
            fn(sets[i])
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(R):
                fn(sets[i])
        g.replay()
        torch.cuda.synchronize()
        reps = max(2, -(-args.steps // R))
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        per = [a.elapsed_time(b) / R for a, b in ev]
        return sum(per) / len(per), percentiles(per)

    q_ms, q_dist = timed(quant)
    m_ms, m_dist = timed(mix)
    nscale = sets[0]["s"].numel()
    q_bytes = 3 * R_ * C_ + 4 * nscale
    m_bytes = 3 * R_ * C_
    q_gbs = q_bytes / (q_ms * 1e-3) / 1e9
    m_gbs = m_bytes / (m_ms * 1e-3) / 1e9
    what = ("weights 128x128 blocks" if weights else
            "activations 1x128 groups" if blockwise else "activations per tensor")
    print(json.dumps({
        "metric": "quantize GB/s (% HBM)", "value": round(q_gbs, 1), "unit": "GB/s",
        "frac_of_hbm": round(q_gbs / PEAK_HBM_GBS, 4), "ms": round(q_ms, 6), "ms_dist": q_dist,
        "config": {"workload": args.workload, "tensor": what, "shape": [R_, C_], "rotation_sets": R,
                   "algorithmic_bytes": q_bytes},
        "byte_mix_reference": {"GBps": round(m_gbs, 1), "frac_of_hbm": round(m_gbs / PEAK_HBM_GBS, 4),
                               "ms": round(m_ms, 6), "ms_dist": m_dist, "bytes": m_bytes},
        "quantize_vs_reference": round(q_gbs / m_gbs, 4),
        "machine": machine_facts()}), flush=True)


def vendor_reference(args):
    """This library's per-tensor and per-row/column scaled GEMMs next to the vendor FP8 GEMM
    (torch._scaled_mm, hipBLASLt on ROCm) on the workload's shape: the same codes and scales,
    rotation sets of cold operands, each graph of R products replayed with events around it.
    The two outputs are compared on the first set (a reference, not a parity test)."""
    import torch
    import fp8_quantized_gemm_amax_amd as fp8
    from fp8_quantized_gemm_amax_amd import workloads as wl
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = wl.WORKLOADS[args.workload]
    M = args.m if args.m is not None else max(w.m_values)
    N, K = w.n, w.k
    a_bits, b_bits = wl.make_inputs(args.workload, M)
    out_dtype = torch.float16 if w.out_dtype == "f16" else torch.bfloat16
    a = wl.bits_to_tensor(a_bits, device=dev)
    b = wl.bits_to_tensor(b_bits, device=dev)
    qa, sa = fp8.fp8_quantize_per_tensor(a)
    qb, sb = fp8.fp8_quantize_per_tensor(b)
    ra, rsa = fp8.fp8_quantize_rowwise(a)
    rb, rsb = fp8.fp8_quantize_rowwise(b)
    del a, b
    per_set = 2 * (M * K + N * K) + 2 * M * N
    R = max(2, min(64, -(-ROTATION_BYTES // per_set)))
    sets = [{"qa": qa.clone(), "qb": qb.clone(), "ra": ra.clone(), "rb": rb.clone(),
             "c": torch.empty((M, N), dtype=out_dtype, device=dev)} for _ in range(R)]
    e4m3 = torch.float8_e4m3fn
    rsa2, rsb2 = rsa.reshape(M, 1), rsb.reshape(1, N)
    legs = {
        "ours_tensorwise": lambda x: fp8.fp8_gemm_scaled_tensorwise(x["qa"], sa, x["qb"], sb, out=x["c"]),
        "vendor_tensorwise": lambda x: torch._scaled_mm(x["qa"].view(e4m3), x["qb"].view(e4m3).t(), scale_a=sa[0],
                                                        scale_b=sb[0], out_dtype=out_dtype),
        "ours_rowwise": lambda x: fp8.fp8_gemm_scaled_rowwise(x["ra"], rsa, x["rb"], rsb, out=x["c"]),
        "vendor_rowwise": lambda x: torch._scaled_mm(x["ra"].view(e4m3), x["rb"].view(e4m3).t(), scale_a=rsa2,
                                                     scale_b=rsb2, out_dtype=out_dtype),
    }
    flops = 2.0 * M * N * K
    result = {}
    for name, fn in legs.items():
        try:
            out = fn(sets[0]).float()
            torch.cuda.synchronize()
            for x in sets:
                fn(x)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for x in sets:
                    fn(x)
            g.replay()
            torch.cuda.synchronize()
            reps = max(3, -(-args.steps // R))
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
            for s0, s1 in ev:
                s0.record()
                g.replay()
                s1.record()
            torch.cuda.synchronize()
            per = [s0.elapsed_time(s1) / R for s0, s1 in ev]
            ms = sum(per) / len(per)
            result[name] = {"us": round(ms * 1e3, 2), "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 1),
                            "frac_of_fp8_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
                            "us_dist": {k: round(v * 1e3, 2) for k, v in percentiles(per).items() if k != "n"},
                            "_out": out}
        except Exception as e:     # the vendor path may not exist for a dtype or shape
            result[name] = {"error": repr(e)[:200]}
    for kind in ("tensorwise", "rowwise"):
        o, v = result.get("ours_" + kind, {}), result.get("vendor_" + kind, {})
        if "_out" in o and "_out" in v:
            d = (o["_out"] - v["_out"]).abs()
            result[kind + "_max_rel_diff"] = round(float(d.max() / v["_out"].abs().max()), 6)
    for r in result.values():
        if isinstance(r, dict):
            r.pop("_out", None)
    print(json.dumps({"metric": "GEMM TFLOP/s, this library and the vendor FP8 GEMM",
                      "config": {"workload": args.workload, "M": M, "N": N, "K": K, "rotation_sets": R,
                                 "out": "f16" if out_dtype == torch.float16 else "bf16", "launch": "hip_graph"},
                      **result, "machine": machine_facts()}), flush=True)


def copy_reference(mib, steps):
    """A plain device copy of `mib` MiB, `steps` times (known bytes: mib MiB read + written)."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / steps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms_per_copy": round(ms, 4),
                      "GBps_read_plus_write": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)


def algorithmic_bytes(w, M, scheme="tensorwise", fused=False):
    """ABI-level bytes of one step: A read as bf16, qA written and read, scales, W read
    as FP8 with its scales, C written; plus B's quantize when it runs every call.  UE8M0
    scales are one byte each in rows padded to four bytes; rowwise scales one float per
    row of A and of W.  Delayed scaling adds, per delayed tensor, the recorded amax word
    and the update's history, step and scale.  The fused one-token step (`fused`) writes qA
    and its scales but does not read them back.  Returns (step bytes, bytes of the GEMM
    launch; for the fused step, its one launch's)."""
    N, K = w.n, w.k
    if w.mode == "grouped":                 # B is every expert's weight and block scales
        g = (K // 128 + 3) // 4 * 4 if scheme == "grouped-ue8m0" else 4 * (K // 128)
        sa_bytes, sb_bytes = M * g, w.experts * -(-N // 128) * g
        quant_a = 2 * M * K + M * K + sa_bytes
        gemm = M * K + sa_bytes + w.experts * N * K + sb_bytes + 2 * M * N + 4 * (w.experts + 1)
        return quant_a + gemm, gemm
    if scheme.startswith("tensorwise"):
        sa_bytes, sb_bytes = 4, 4
    elif scheme == "rowwise":
        sa_bytes, sb_bytes = 4 * M, 4 * N
    elif scheme == "blockwise-ue8m0":
        g4 = (K // 128 + 3) // 4 * 4
        sa_bytes, sb_bytes = M * g4, -(-N // 128) * g4
    else:
        sa_bytes, sb_bytes = M * (K // 128) * 4, -(-N // 128) * (K // 128) * 4
    quant_a = 2 * M * K + M * K + sa_bytes
    gemm = M * K + sa_bytes + N * K + sb_bytes + 2 * M * N
    if fused:
        step = quant_a + N * K + sb_bytes + 2 * M * N
        return step, step
    quant_b = (2 * N * K + N * K + sb_bytes) if w.quantize_b_per_call else 0
    if scheme == "tensorwise-delayed":
        # beyond the cast (whose scale_used write is sa_bytes): the scale read by the cast, the
        # amax word (recorded, read, cleared), the history read, one entry written, the step
        # read and written, the scale read and rewritten
        update = 4 + 12 + DELAYED_HISTORY * 4 + 4 + 8 + 8
        quant_a += update
        quant_b += update if w.quantize_b_per_call else 0
    return quant_a + gemm + quant_b, gemm


def cpu_baseline(w, a_bits, b_bits, budget_s=20.0, scheme="tensorwise", gpu_c=None):
    """The oracle's quantize(A) + scaled GEMM on the host, on a row sample of A sized to
    roughly `budget_s` seconds; returns TFLOP/s (float64 arithmetic).  With delayed
    scaling the step is the oracle's static cast with the history's scale, its history
    update, and the GEMM.  With `gpu_c` (the GPU step's output for the same inputs) the
    sampled rows of it are also checked against the oracle's, outside the timing, with the
    product tolerance."""
    import numpy as np
    import oracle
    cores = len(os.sched_getaffinity(0))
    M, N, K = a_bits.shape[0], w.n, w.k
    if w.mode == "grouped":
        return cpu_baseline_grouped(w, a_bits, scheme, cores)
    ue8m0 = scheme == "blockwise-ue8m0"
    delayed = scheme == "tensorwise-delayed"
    if delayed:
        hist, step_a, scale_a = np.zeros(DELAYED_HISTORY, np.float32), 0, np.float32(1)
        amax_a = oracle.amax_per_tensor(oracle.input_to_f32(a_bits, "bf16"))
        for _ in range(DELAYED_INTERVAL):                      # reach the recipe's steady state
            hist, step_a, scale_a = oracle.delayed_step(hist, step_a, scale_a, amax_a, DELAYED_INTERVAL,
                                                        DELAYED_MARGIN)
    if scheme == "rowwise":
        qb, sb = oracle.quantize_rowwise(b_bits, "bf16")
    elif w.mode == "tensorwise":
        qb, sb = oracle.quantize_per_tensor(b_bits, "bf16")
    elif ue8m0:
        qb, sb = oracle.quantize_groups_ue8m0(b_bits, "bf16", 128, 128)
    else:
        qb, sb = oracle.quantize_groups(b_bits, "bf16", 128, 128)
    rows = min(M, 64)          # a first timing on a few rows sizes the sample
    runs = []
    t_start = time.perf_counter()
    while True:
        a = a_bits[:rows]
        t0 = time.perf_counter()
        if scheme == "rowwise":
            qa, sa = oracle.quantize_rowwise(a, "bf16")
            if w.quantize_b_per_call:
                qb, sb = oracle.quantize_rowwise(b_bits, "bf16")
            c_or = oracle.gemm_rowwise_ref(qa, sa, qb, sb)
        elif delayed:
            qa, amax = oracle.quantize_static(a, "bf16", scale_a)
            oracle.delayed_step(hist, step_a, scale_a, amax, DELAYED_INTERVAL, DELAYED_MARGIN)
            if w.quantize_b_per_call:
                qb, _ = oracle.quantize_static(b_bits, "bf16", sb)
            c_or = oracle.gemm_tensorwise_ref(qa, scale_a, qb, sb)
        elif w.mode == "tensorwise":
            qa, sa = oracle.quantize_per_tensor(a, "bf16")
            if w.quantize_b_per_call:
                qb, sb = oracle.quantize_per_tensor(b_bits, "bf16")
            c_or = oracle.gemm_tensorwise_ref(qa, sa, qb, sb)
        elif ue8m0:
            qa, sa = oracle.quantize_groups_ue8m0(a, "bf16", 1, 128)
            c_or = oracle.gemm_blockwise_ue8m0_ref(qa, sa, qb, sb)
        else:
            qa, sa = oracle.quantize_groups(a, "bf16", 1, 128)
            c_or = oracle.gemm_blockwise_ref(qa, sa, qb, sb)
        dt = time.perf_counter() - t0
        runs.append(dt)
        if len(runs) == 1 and (dt * 3 > budget_s and rows > 1 or dt * 3 < 0.5 * budget_s and rows < M):
            rows = max(1, min(M, int(rows * budget_s / (3 * max(dt, 1e-6)))))
            runs = []
            continue
        if len(runs) >= 3 or time.perf_counter() - t_start > budget_s:
            break
    best = min(runs)
    flops = 2.0 * rows * N * K
    out = {"value": round(flops / best / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
           "sample": f"oracle {'delayed-scaling ' if delayed else ''}quantize(A[{rows},{K}]) + "
                     f"{scheme} GEMM with W[{N},{K}], best of "
                     f"{len(runs)} ({best:.2f} s); float64 NumPy, {cores} host threads"}
    if gpu_c is not None:
        if scheme == "rowwise":
            bnd = oracle.bound_rowwise(qa, sa, qb, sb)
        elif delayed:
            bnd = oracle.bound_tensorwise(qa, scale_a, qb, sb)
        elif w.mode == "tensorwise":
            # the GPU's activation scale comes from the whole A: quantize the sample with it
            sa = np.float32(oracle.scale_from_amax(oracle.amax_per_tensor(oracle.input_to_f32(a_bits, "bf16"))))
            qa = oracle.quantize_with_scale(oracle.input_to_f32(a_bits[:rows], "bf16"), sa)
            c_or = oracle.gemm_tensorwise_ref(qa, sa, qb, sb)
            bnd = oracle.bound_tensorwise(qa, sa, qb, sb)
        elif ue8m0:
            bnd = oracle.bound_blockwise_ue8m0(qa, sa, qb, sb)
        else:
            bnd = oracle.bound_blockwise(qa, sa, qb, sb)
        got = gpu_c[:rows].float().cpu().numpy().astype(np.float64)
        r = oracle.check_gemm(got, c_or, bnd, w.out_dtype)
        out["check"] = {"rows": rows, "ok": bool(r["ok"]), "n_bad": int(r["n_bad"]),
                        "worst_ratio": round(float(r["worst_ratio"]), 4),
                        "tolerance": "2e-3 |C| + 1e-4 sum|qa sa||qb sb| + one output ulp"}
    return out


def cpu_baseline_grouped(w, a_bits, scheme, cores):
    """The oracle's quantize + grouped product on a bounded sample: the rows routed to
    expert 0 (its weight quantized beforehand, as the GPU step does)."""
    import numpy as np
    import oracle
    from fp8_quantized_gemm_amax_amd import workloads as wl
    M, N, K = a_bits.shape[0], w.n, w.k
    sizes = wl.group_sizes(w.name, M)
    rows = int(sizes[0])
    ue8m0 = scheme == "grouped-ue8m0"
    quant = oracle.quantize_groups_ue8m0 if ue8m0 else oracle.quantize_groups
    gemm = oracle.gemm_grouped_blockwise_ue8m0_ref if ue8m0 else oracle.gemm_grouped_blockwise_ref
    qb, sb = quant(wl.expert_weight_bits(w.name, 0), "bf16", 128, 128)
    off = np.array([0, rows])
    runs = []
    for _ in range(3):
        t0 = time.perf_counter()
        qa, sa = quant(a_bits[:rows], "bf16", 1, 128)
        gemm(qa, sa, qb[None], sb[None], off)
        runs.append(time.perf_counter() - t0)
    best = min(runs)
    return {"value": round(2.0 * rows * N * K / best / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"oracle quantize + {scheme} product of the {rows} rows routed to expert 0 "
                      f"(W_0[{N},{K}]), best of 3 ({best:.2f} s); float64 NumPy, {cores} host threads"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.copy_mb:
        copy_reference(args.copy_mb, args.steps)
        return
    if args.quantize_only:
        quantize_reference(args)
        return
    if args.vendor_gemm:
        vendor_reference(args)
        return

    import numpy as np
    import torch
    import fp8_quantized_gemm_amax_amd as fp8
    from fp8_quantized_gemm_amax_amd import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = wl.WORKLOADS[args.workload]
    M = args.m if args.m is not None else max(w.m_values)
    N, K = w.n, w.k
    a_bits, b_bits = wl.make_inputs(args.workload, M)
    out_dtype = torch.float16 if w.out_dtype == "f16" else torch.bfloat16
    blockwise = w.mode == "blockwise"
    grouped = w.mode == "grouped"
    ue8m0 = args.scale_fmt == "ue8m0"
    if grouped and (args.rowwise or args.act_scaling == "delayed"):
        print(f"{args.workload} is a grouped (expert) workload with block scales only", file=sys.stderr)
        sys.exit(2)
    if ue8m0 and not (blockwise or grouped):
        print(f"--scale-fmt ue8m0 needs a blockwise workload; {args.workload} is {w.mode}", file=sys.stderr)
        sys.exit(2)
    delayed = args.act_scaling == "delayed"
    if delayed and blockwise:
        print(f"--act-scaling delayed is per-tensor scaling; {args.workload} is {w.mode}", file=sys.stderr)
        sys.exit(2)
    rowwise = args.rowwise
    if rowwise and (ue8m0 or delayed):
        print("--rowwise replaces the workload's scaling; it takes neither --scale-fmt ue8m0 nor "
              "--act-scaling delayed", file=sys.stderr)
        sys.exit(2)
    if rowwise:
        blockwise = False                   # the workload's shape with per-row scales
    scheme = scheme_of(w, args.scale_fmt, args.act_scaling, rowwise)
    # one token with dynamic activation scales: the whole step is one fused launch
    fused = (M == 1 and not grouped and not delayed and not w.quantize_b_per_call and not args.two_launch)
    fused_mode = ("rowwise" if rowwise else "blockwise_ue8m0" if (blockwise and ue8m0)
                  else "blockwise" if blockwise else "tensorwise")
    ds_a = ds_b = None
    if delayed:
        # one delayed-scaling state per quantized tensor, shared by the rotation sets: the
        # sets are successive inputs of the same layer
        ds_a = fp8.DelayedScaling(DELAYED_HISTORY, DELAYED_INTERVAL, DELAYED_MARGIN, device=dev)
        if w.quantize_b_per_call:
            ds_b = fp8.DelayedScaling(DELAYED_HISTORY, DELAYED_INTERVAL, DELAYED_MARGIN, device=dev)

    a0 = wl.bits_to_tensor(a_bits, device=dev)
    b0 = wl.bits_to_tensor(b_bits, device=dev) if b_bits is not None else None
    if grouped:
        pass
    elif rowwise:
        qb0, sb0 = fp8.fp8_quantize_rowwise(b0)
    elif blockwise:
        quant_groups = fp8.fp8_quantize_per_token_group_ue8m0 if ue8m0 else fp8.fp8_quantize_per_token_group
        qb0, sb0 = quant_groups(b0, 128, 128)
    else:
        qb0, sb0 = fp8.fp8_quantize_per_tensor(b0)

    if grouped:
        # every expert's weight drawn and quantized on the GPU once (128 x 128 blocks), shared
        # by all steps: at 0.94 GB it is read from HBM on every step; the routed rows rotate
        E = w.experts
        sizes = wl.group_sizes(args.workload, M)
        offsets = torch.from_numpy(np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)).to(dev)
        quant_groups = fp8.fp8_quantize_per_token_group_ue8m0 if ue8m0 else fp8.fp8_quantize_per_token_group
        g = fp8.e8m0_row_bytes(K // 128) if ue8m0 else K // 128
        qb0 = torch.empty((E, N, K), dtype=torch.uint8, device=dev)
        sb0 = torch.empty((E, -(-N // 128), g), dtype=torch.uint8 if ue8m0 else torch.float32, device=dev)
        for e in range(E):
            be = wl.bits_to_tensor(wl.expert_weight_bits(args.workload, e), device=dev)
            quant_groups(be, 128, 128, q=qb0[e], scales=sb0[e])
            del be
        gemm_grouped = fp8.fp8_gemm_grouped_blockwise_ue8m0 if ue8m0 else fp8.fp8_gemm_grouped_blockwise
        per_set = 2 * M * K + M * K + 2 * M * N
    else:
        per_set = 2 * M * K + M * K + 2 * M * N + N * K + (2 * N * K if w.quantize_b_per_call else 0)
    R = max(2, min(256, -(-ROTATION_BYTES // per_set)))
    sets = []
    for _ in range(R):
        if grouped:
            sets.append({"a": a0.clone(), "c": torch.empty((M, N), dtype=out_dtype, device=dev),
                         "qa": torch.empty((M, K), dtype=torch.uint8, device=dev),
                         "sa": torch.empty((M, g), dtype=torch.uint8 if ue8m0 else torch.float32, device=dev)})
            continue
        s = {"a": a0.clone(), "c": torch.empty((M, N), dtype=out_dtype, device=dev)}
        if w.quantize_b_per_call:
            s["b"] = b0.clone()
        else:
            s["qb"], s["sb"] = qb0.clone(), sb0.clone()
        if rowwise:
            s["qa"] = torch.empty((M, K), dtype=torch.uint8, device=dev)
            s["sa"] = torch.empty((M,), dtype=torch.float32, device=dev)
            if w.quantize_b_per_call:
                s["qb"] = torch.empty((N, K), dtype=torch.uint8, device=dev)
                s["sb"] = torch.empty((N,), dtype=torch.float32, device=dev)
        elif blockwise:
            s["qa"] = torch.empty((M, K), dtype=torch.uint8, device=dev)
            s["sa"] = (torch.empty((M, fp8.e8m0_row_bytes(K // 128)), dtype=torch.uint8, device=dev) if ue8m0
                       else torch.empty((M, K // 128), dtype=torch.float32, device=dev))
        else:
            s["qa"] = torch.empty((M, K), dtype=torch.uint8, device=dev)
            s["sa"] = torch.empty((1,), dtype=torch.float32, device=dev)
            if w.quantize_b_per_call:
                s["qb"] = torch.empty((N, K), dtype=torch.uint8, device=dev)
                s["sb"] = torch.empty((1,), dtype=torch.float32, device=dev)
        sets.append(s)
    del a0, b0

    def quantize(s):
        if grouped:
            quant_groups(s["a"], 1, 128, q=s["qa"], scales=s["sa"])
        elif rowwise:
            fp8.fp8_quantize_rowwise(s["a"], q=s["qa"], scales=s["sa"])
            if w.quantize_b_per_call:
                fp8.fp8_quantize_rowwise(s["b"], q=s["qb"], scales=s["sb"])
        elif blockwise:
            quant_groups(s["a"], 1, 128, q=s["qa"], scales=s["sa"])
        elif delayed:                       # cast, push the amax, refresh the scale: one launch
            ds_a.quantize_step(s["a"], q=s["qa"])
            if ds_b is not None:
                ds_b.quantize_step(s["b"], q=s["qb"])
        else:
            fp8.fp8_quantize_per_tensor(s["a"], q=s["qa"], scale=s["sa"])
            if w.quantize_b_per_call:
                fp8.fp8_quantize_per_tensor(s["b"], q=s["qb"], scale=s["sb"])

    def gemm(s):
        if grouped:
            gemm_grouped(s["qa"], s["sa"], qb0, sb0, offsets, out=s["c"])
        elif rowwise:
            fp8.fp8_gemm_scaled_rowwise(s["qa"], s["sa"], s["qb"], s["sb"], out=s["c"])
        elif blockwise:
            gemm_blockwise = fp8.fp8_gemm_scaled_blockwise_ue8m0 if ue8m0 else fp8.fp8_gemm_scaled_blockwise
            gemm_blockwise(s["qa"], s["sa"], s["qb"], s["sb"], out=s["c"])
        elif delayed:
            fp8.fp8_gemm_scaled_tensorwise(s["qa"], ds_a.scale_used, s["qb"],
                                           ds_b.scale_used if ds_b else s["sb"], out=s["c"])
        else:
            fp8.fp8_gemm_scaled_tensorwise(s["qa"], s["sa"], s["qb"], s["sb"], out=s["c"])

    def step(s):
        if fused:
            fp8.fp8_gemv_dynamic(fused_mode, s["a"], s["qb"], s["sb"], out=s["c"], qa=s["qa"], sa=s["sa"])
            return
        quantize(s)
        gemm(s)

    # eager warm-up: the first launches and lazy initialisation, at most one step per rotation
    # set (with delayed scaling at least two intervals, so the scale has reached its steady
    # state); then one eager reference output
    for i in range(max(1, min(args.warmup, R), 2 * DELAYED_INTERVAL if delayed else 1)):
        step(sets[i % R])
    step(sets[0])
    torch.cuda.synchronize()
    ref_c = sets[0]["c"].clone()

    # HIP graphs: one replay runs `R` steps (one per rotation set); a tail graph runs the
    # remaining K mod R, so exactly K steps are timed.
    K_steps = args.steps
    def capture(n, fn, first=0):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(first, first + n):
                fn(sets[i % R])
        return g
    n_full, tail = divmod(K_steps, R)
    g_full = capture(R, step) if n_full else None
    g_tail = capture(tail, step) if tail else None
    # graph warm-up: the W untimed steps as replays, back to back, so that the GPU runs them
    # under load as it runs the timed steps (eager launches leave it idle between steps);
    # every graph is replayed at least twice
    warm, per_warm = (g_full, R) if g_full is not None else (g_tail, tail)
    for _ in range(max(2, -(-args.warmup // per_warm))):
        warm.replay()
    if g_full is not None and g_tail is not None:
        g_tail.replay()
        g_tail.replay()
    torch.cuda.synchronize()

    # timed region: an event pair around every replay; the per-step time of a replay is its
    # duration over the steps it holds
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n_full + (1 if tail else 0))]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n_full):
        ev[i][0].record()
        g_full.replay()
        ev[i][1].record()
    if g_tail:
        ev[-1][0].record()
        g_tail.replay()
        ev[-1][1].record()
    torch.cuda.synchronize()
    host_s = time.perf_counter() - t0
    sizes_ = [R] * n_full + ([tail] if tail else [])
    durs = [a.elapsed_time(b) for a, b in ev]
    total_ms = ev[0][0].elapsed_time(ev[-1][1])
    ms_per_step = total_ms / K_steps
    step_dist = percentiles([d / n for d, n in zip(durs, sizes_)])

    # the same steps replayed must reproduce the eager output bit for bit
    if not torch.equal(sets[0]["c"].view(torch.int16), ref_c.view(torch.int16)):
        raise RuntimeError("graph replay output differs from the eager step")

    # the GEMM's time per launch: the same steps without their GEMMs (a graph of the R
    # quantizes, replayed as often as the step graph) are timed with events on the same
    # stream, and their time per step is taken off the step's.  Every GEMM thus runs right
    # after its own quantize, as in the timed steps, and no launch gap or event sits between
    # a GEMM and the next kernel.  The fused one-token step is one launch: its time is the
    # step's.
    if fused:
        quant_ms = None
        gemm_ms = ms_per_step
    else:
        g_q = capture(R, quantize)
        g_q.replay()
        torch.cuda.synchronize()
        reps = max(1, -(-K_steps // R))
        qev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in qev:
            a.record()
            g_q.replay()
            b.record()
        torch.cuda.synchronize()
        quant_ms = sum(a.elapsed_time(b) for a, b in qev) / (reps * R)
        gemm_ms = ms_per_step - quant_ms

    flops = 2.0 * M * N * K
    step_bytes, gemm_bytes = algorithmic_bytes(w, M, scheme, fused)
    decode = M <= 16
    if decode:
        value = step_bytes / (ms_per_step * 1e-3) / 1e9
        unit = "GB/s"
    else:
        value = flops / (ms_per_step * 1e-3) / 1e12
        unit = "TFLOP/s"
    # the GEMM kernel's roofline: whichever of MFMA time and HBM time at peak is longer
    t_mfma = flops / (PEAK_FP8_TFLOPS * 1e12)
    t_hbm = gemm_bytes / (PEAK_HBM_GBS * 1e9)
    if t_hbm >= t_mfma:
        roof = {"bound": "hbm", "achieved": round(gemm_bytes / (gemm_ms * 1e-3) / 1e9, 2),
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": round(flops / (gemm_ms * 1e-3) / 1e12, 2),
                "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = measured_traffic(args.workload, M, scheme, fused)

    result = {
        "metric": METRIC, "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": K_steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3", "data": "synthetic",
        "config": {"workload": args.workload, "M": M, "N": N, "K": K,
                   "scaling": "rowwise" if rowwise else w.mode,
                   "scale_fmt": args.scale_fmt if (blockwise or grouped) else "float32",
                   "act_scaling": args.act_scaling if not blockwise else "dynamic",
                   "in": "bf16", "out": w.out_dtype, "rotation_sets": R, "launch": "hip_graph",
                   "step": ("fused: quantize + GEMV in one launch (fp8_gemv_dynamic)" if fused
                            else "quantize launch(es), then the GEMM launch(es)"),
                   "gemm_ms": round(gemm_ms, 6),
                   "quantize_ms": round(quant_ms, 6) if quant_ms is not None else None,
                   "host_s": round(host_s, 4), "step_bytes": step_bytes},
        "step_ms": step_dist,
        "roofline": roof,
    }
    if delayed:
        result["config"].update({"history": DELAYED_HISTORY, "interval": DELAYED_INTERVAL,
                                 "margin": DELAYED_MARGIN})
    if grouped:
        result["config"].update({"experts": w.experts, "rows_per_expert_min": int(sizes.min()),
                                 "rows_per_expert_max": int(sizes.max())})
    result["machine"] = machine_facts()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, a_bits, b_bits, scheme=scheme, gpu_c=None if grouped else ref_c)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
