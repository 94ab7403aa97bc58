"""Throughput of the FP8 E4M3 scaled-GEMM hot path on one MI355X.

One step = the whole hot path over one batch of synthetic input: amax + scale + cast of
the activations (per tensor, or per 1x128 token group), then the FP8 x FP8 GEMM with
float32 accumulation and the scale epilogue.  Weights are quantized once before timing
(as a serving stack does at load time), except in the small per-tensor workload, where
both operands are quantized on every call.

Inputs stay resident in HBM; each step reads a different copy of the input set from a
rotation whose footprint exceeds 1 GiB, so reads come from HBM rather than the 256 MB
Infinity Cache.

Prints one JSON line.  `value` is the whole step's throughput (TFLOP/s including the
activation quantize; GB/s for M <= 16 decode), `roofline` rates the dominant kernel
(the GEMM) from HIP events around each of its launches in the timed region, and
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.
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
DEFAULT_WORKLOAD = "tinyllama_upproj_prefill"
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
    p.add_argument("--copy-mb", type=int, default=0,
                   help="instead of the hot path, run a plain device copy of this many MiB "
                        "(the known-size reference for rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    return p.parse_args()


KERNEL_SOURCES = ["fp8_quantized_gemm_amax_amd/csrc/gemm.hip", "fp8_quantized_gemm_amax_amd/csrc/gemv.hip",
                  "fp8_quantized_gemm_amax_amd/csrc/dma.hpp", "fp8_quantized_gemm_amax_amd/csrc/fp8_device.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_traffic.json")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
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


def traffic_key(workload, M, scheme="tensorwise"):
    """Counter-table key of a GEMM launch (delayed scaling runs the tensorwise GEMM)."""
    suffix = {"blockwise-ue8m0": "/ue8m0", "grouped-ue8m0": "/ue8m0", "rowwise": "/rowwise"}.get(scheme, "")
    return f"{workload}/M={M}" + suffix


def measured_traffic(workload, M, scheme="tensorwise"):
    """HBM bytes per GEMM launch from the committed rocprofv3 counter runs, or None when
    there is no entry for this workload or the kernel sources changed since it was taken."""
    import json as _json
    try:
        with open(TRAFFIC_FILE) as f:
            table = _json.load(f)
    except (OSError, ValueError):
        return None
    e = table.get(traffic_key(workload, M, scheme))
    if not e or e.get("kernel_source_sha") != kernel_source_hash():
        return None
    return e.get("traffic_bytes_per_launch")


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


def algorithmic_bytes(w, M, scheme="tensorwise"):
    """ABI-level bytes of one step: A read as bf16, qA written and read, scales, W read
    as FP8 with its scales, C written; plus B's quantize when it runs every call.  UE8M0
    scales are one byte each in rows padded to four bytes; rowwise scales one float per
    row of A and of W.  Delayed scaling adds, per delayed tensor, the recorded amax word
    and the update's history, step and scale."""
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
    quant_b = (2 * N * K + N * K + sb_bytes) if w.quantize_b_per_call else 0
    if scheme == "tensorwise-delayed":
        # beyond the cast (whose scale_used write is sa_bytes): the scale read by the cast, the
        # amax word (recorded, read, cleared), the history read, one entry written, the step
        # read and written, the scale read and rewritten
        update = 4 + 12 + DELAYED_HISTORY * 4 + 4 + 8 + 8
        quant_a += update
        quant_b += update if w.quantize_b_per_call else 0
    return quant_a + gemm + quant_b, gemm


def cpu_baseline(w, a_bits, b_bits, budget_s=20.0, scheme="tensorwise"):
    """The oracle's quantize(A) + scaled GEMM on the host, on a row sample of A sized to
    roughly `budget_s` seconds; returns TFLOP/s (float64 arithmetic).  With delayed
    scaling the step is the oracle's static cast with the history's scale, its history
    update, and the GEMM."""
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
    rows = M
    runs = []
    t_start = time.perf_counter()
    while True:
        a = a_bits[:rows]
        t0 = time.perf_counter()
        if scheme == "rowwise":
            qa, sa = oracle.quantize_rowwise(a, "bf16")
            if w.quantize_b_per_call:
                qb, sb = oracle.quantize_rowwise(b_bits, "bf16")
            oracle.gemm_rowwise_ref(qa, sa, qb, sb)
        elif delayed:
            qa, amax = oracle.quantize_static(a, "bf16", scale_a)
            oracle.delayed_step(hist, step_a, scale_a, amax, DELAYED_INTERVAL, DELAYED_MARGIN)
            if w.quantize_b_per_call:
                qb, _ = oracle.quantize_static(b_bits, "bf16", sb)
            oracle.gemm_tensorwise_ref(qa, scale_a, qb, sb)
        elif w.mode == "tensorwise":
            qa, sa = oracle.quantize_per_tensor(a, "bf16")
            if w.quantize_b_per_call:
                qb, sb = oracle.quantize_per_tensor(b_bits, "bf16")
            oracle.gemm_tensorwise_ref(qa, sa, qb, sb)
        elif ue8m0:
            qa, sa = oracle.quantize_groups_ue8m0(a, "bf16", 1, 128)
            oracle.gemm_blockwise_ue8m0_ref(qa, sa, qb, sb)
        else:
            qa, sa = oracle.quantize_groups(a, "bf16", 1, 128)
            oracle.gemm_blockwise_ref(qa, sa, qb, sb)
        dt = time.perf_counter() - t0
        runs.append(dt)
        if dt * 3 > budget_s and rows > 1 and len(runs) == 1:
            rows = max(1, int(rows * budget_s / (3 * dt)))
            runs = []
            continue
        if len(runs) >= 3 or time.perf_counter() - t_start > budget_s:
            break
    best = min(runs)
    flops = 2.0 * rows * N * K
    return {"value": round(flops / best / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"oracle {'delayed-scaling ' if delayed else ''}quantize(A[{rows},{K}]) + "
                      f"{scheme} GEMM with W[{N},{K}], best of "
                      f"{len(runs)} ({best:.2f} s); float64 NumPy, {cores} host threads"}


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
        quantize(s)
        gemm(s)

    # eager warm-up (first launches, lazy initialisation; with delayed scaling at least two
    # intervals, so the scale has reached its steady state), then one eager reference output
    for i in range(max(1, args.warmup, 2 * DELAYED_INTERVAL if delayed else 1)):
        step(sets[i % R])
    step(sets[0])
    torch.cuda.synchronize()
    ref_c = sets[0]["c"].clone()

    # HIP graphs: one replay runs `R` steps (one per rotation set); a tail graph runs the
    # remaining K mod R, so exactly K steps are timed.  A second graph holds the R GEMMs
    # alone; its replays time the dominant kernel.
    K_steps = args.steps
    def capture(n, fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(sets[i % R])
        return g
    n_full, tail = divmod(K_steps, R)
    g_full = capture(R, step) if n_full else None
    g_tail = capture(tail, step) if tail else None
    g_gemm = capture(R, gemm)
    for _ in range(2):                      # graph warm-up replays
        if g_full:
            g_full.replay()
        g_gemm.replay()
    torch.cuda.synchronize()

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(n_full):
        g_full.replay()
    if g_tail:
        g_tail.replay()
    end.record()
    torch.cuda.synchronize()
    host_s = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / K_steps

    # the same steps replayed must reproduce the eager output bit for bit
    if not torch.equal(sets[0]["c"].view(torch.int16), ref_c.view(torch.int16)):
        raise RuntimeError("graph replay output differs from the eager step")

    gemm_reps = max(1, -(-K_steps // R))
    gs, ge = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gs.record()
    for _ in range(gemm_reps):
        g_gemm.replay()
    ge.record()
    torch.cuda.synchronize()
    gemm_ms = gs.elapsed_time(ge) / (gemm_reps * R)

    flops = 2.0 * M * N * K
    step_bytes, gemm_bytes = algorithmic_bytes(w, M, scheme)
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
    roof["traffic"] = measured_traffic(args.workload, M, scheme)

    result = {
        "metric": METRIC, "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": K_steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3", "data": "synthetic",
        "config": {"workload": args.workload, "M": M, "N": N, "K": K,
                   "scaling": "rowwise" if rowwise else w.mode,
                   "scale_fmt": args.scale_fmt if (blockwise or grouped) else "float32",
                   "act_scaling": args.act_scaling if not blockwise else "dynamic",
                   "in": "bf16", "out": w.out_dtype, "rotation_sets": R, "launch": "hip_graph",
                   "gemm_ms": round(gemm_ms, 6), "host_s": round(host_s, 4),
                   "step_bytes": step_bytes},
        "roofline": roof,
    }
    if delayed:
        result["config"].update({"history": DELAYED_HISTORY, "interval": DELAYED_INTERVAL,
                                 "margin": DELAYED_MARGIN})
    if grouped:
        result["config"].update({"experts": w.experts, "rows_per_expert_min": int(sizes.min()),
                                 "rows_per_expert_max": int(sizes.max())})
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, a_bits, b_bits, scheme=scheme)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
