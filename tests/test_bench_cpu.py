"""Host-side pieces of bench.py (no GPU): the one-GPU guard and the code hash that keys the
committed HBM-traffic counters."""

import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_strip_comments_keeps_code_and_literals():
    b = load_bench()
    src = 'int a = 1; // note\n/* block\n comment */ const char* s = "//x/*y*/"; char c = \'/\';\n'
    assert b.strip_comments(src) == 'int a = 1; const char* s = "//x/*y*/"; char c = \'/\';'
    # layout and comments do not change the result, code does
    assert b.strip_comments("int  a=1;\n\n// c\n") == b.strip_comments("int a=1; /* d */")
    assert b.strip_comments("int a=1;") != b.strip_comments("int a=2;")


def test_traffic_table_matches_the_kernel_code_or_is_ignored():
    """Every entry of the counter table names the code hash it was taken with; bench.py uses
    an entry only while the hash of its kernel family (decode for M <= 16) matches."""
    import json
    b = load_bench()
    with open(b.TRAFFIC_FILE) as f:
        table = json.load(f)
    for key, e in table.items():
        workload, m = key.split("/")[:2]
        M = int(m.split("=")[1])
        parts = key.split("/")[2:]
        fused = "fused" in parts
        scheme = "rowwise" if "rowwise" in parts else ("blockwise-ue8m0" if "ue8m0" in parts else "x")
        assert b.traffic_key(workload, M, scheme, fused) == key or scheme == "x"
        got = b.measured_traffic(workload, M, scheme, fused)
        assert (got == e["traffic_bytes_per_launch"]) == (e["kernel_source_sha"] == b.kernel_source_hash(M)), key


def test_kernel_families_hash_their_own_sources():
    """A change to the decode kernels leaves the tiled GEMM's counters valid, and back."""
    b = load_bench()
    assert set(b.KERNEL_SOURCES["gemm"]) & set(b.KERNEL_SOURCES["decode"]) == {
        b._CSRC + "fp8_device.hpp", b._CSRC + "gemm_plan.hpp"}
    assert b.kernel_source_hash(1) == b.kernel_source_hash(16) != b.kernel_source_hash(17)


def test_fused_step_bytes():
    """The fused one-token step writes the activation codes and scales but never reads them
    back: its bytes are the two-launch step's less qA and sA."""
    b = load_bench()
    from fp8_quantized_gemm_amax_amd import workloads as wl
    w = wl.WORKLOADS["deepseek_v3_blockwise"]
    K = w.k
    two, _ = b.algorithmic_bytes(w, 1, "blockwise")
    one, one_launch = b.algorithmic_bytes(w, 1, "blockwise", fused=True)
    assert one == one_launch == two - (K + 4 * (K // 128))
    w = wl.WORKLOADS["llama7b_decode"]
    assert b.algorithmic_bytes(w, 1, "tensorwise", fused=True)[0] == \
        2 * w.k + w.k + 4 + w.n * w.k + 4 + 2 * w.n
