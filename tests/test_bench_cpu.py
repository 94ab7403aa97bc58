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
    an entry only while the hash matches."""
    import json
    b = load_bench()
    with open(b.TRAFFIC_FILE) as f:
        table = json.load(f)
    h = b.kernel_source_hash()
    for key, e in table.items():
        workload, m = key.split("/")[:2]
        scheme = "rowwise" if key.endswith("/rowwise") else ("blockwise-ue8m0" if key.endswith("/ue8m0") else "x")
        got = b.measured_traffic(workload, int(m.split("=")[1]), scheme)
        assert (got == e["traffic_bytes_per_launch"]) == (e["kernel_source_sha"] == h), key
