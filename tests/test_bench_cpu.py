"""The bench's contract and reporting logic, on the host: one GPU only, the
dominant kernel's roofline (units and bound per kernel family), counter traffic
only for the schedule it was taken with, and the comment-insensitive source
hash that keys it."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def _stats(**kw):
    base = {"launches": 0, "total_ms": 0.0, "min_ms": 0.0, "max_ms": 0.0, "work": 0.0}
    return {name: dict(base, **kw.get(name, {})) for name in ("materialize", "gemm1", "gemm2_reduce", "reduce")}


def test_fused_kernel_is_priced_against_hbm():
    # one step: a 4.7 MB cut in 4 us, GEMM1 4.8 GFLOP in 12 us, the fused GEMM2 57.8 MB in 16.5 us
    st = _stats(materialize=dict(launches=1, total_ms=0.004, work=4.72e6),
                gemm1=dict(launches=1, total_ms=0.012, work=4.83e9),
                gemm2_reduce=dict(launches=1, total_ms=0.0165, work=57.8e6))
    k = bench.kernel_table(st, 1)
    assert k["gemm1"]["unit"] == "TFLOP/s" and abs(k["gemm1"]["achieved"] - 402.5) < 1
    assert k["gemm2_reduce"]["unit"] == "GB/s" and abs(k["gemm2_reduce"]["achieved"] - 3503.0) < 1
    r = bench.roofline(k, "bf16", "no-such-workload")
    assert r["kernel"] == "gemm2_reduce" and r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert abs(r["frac"] - 3503.0 / 8000.0) < 1e-3


def test_traffic_only_for_the_default_schedule(monkeypatch):
    monkeypatch.setattr(bench, "measured_traffic", lambda workload, kernel: 123.0)
    k = bench.kernel_table(_stats(gemm1=dict(launches=1, total_ms=0.01, work=1e9)), 1)
    assert bench.roofline(k, "bf16", "w")["traffic"] == 123.0
    assert bench.roofline(k, "bf16", "w", default_schedule=False)["traffic"] is None


def test_source_hash_ignores_comments_and_layout():
    a = "int f(int x) {\n  return x + 1;  // one more\n}\n/* block\n comment */\n"
    b = "int f(int x) { return x + 1; }"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only("int f(int x) { return x + 2; }")
