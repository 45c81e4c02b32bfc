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
    k = bench.kernel_table(st, 1, "bf16")
    assert k["gemm1"]["unit"] == "TFLOP/s" and abs(k["gemm1"]["achieved"] - 402.5) < 1
    assert k["gemm2_reduce"]["unit"] == "GB/s" and abs(k["gemm2_reduce"]["achieved"] - 3503.0) < 1
    r = bench.roofline(k, "bf16", "no-such-workload")
    assert r["kernel"] == "gemm2_reduce" and r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert abs(r["frac"] - 3503.0 / 8000.0) < 1e-3


def test_traffic_only_for_the_default_schedule(monkeypatch):
    monkeypatch.setattr(bench, "measured_traffic", lambda workload, kernel: 123.0)
    k = bench.kernel_table(_stats(gemm1=dict(launches=1, total_ms=0.01, work=1e9)), 1, "bf16")
    assert bench.roofline(k, "bf16", "w")["traffic"] == 123.0
    assert bench.roofline(k, "bf16", "w", default_schedule=False)["traffic"] is None


def test_source_hash_ignores_comments_and_layout():
    a = "int f(int x) {\n  return x + 1;  // one more\n}\n/* block\n comment */\n"
    b = "int f(int x) { return x + 1; }"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only("int f(int x) { return x + 2; }")


def test_fractions_per_kernel_family():
    """Each kernel carries its own roofline: bf16 GEMMs against the MFMA peak,
    fp32 GEMMs (the tiny workload) against the fp32 vector peak, layout and
    reduce kernels against HBM."""
    st = _stats(materialize=dict(launches=2, total_ms=0.2, work=1.6e9),
                gemm1=dict(launches=2, total_ms=0.5, work=6.2e11),
                reduce=dict(launches=4, total_ms=0.4, work=1.8e9))
    k = bench.kernel_table(st, 2, "bf16")
    assert k["gemm1"]["bound"] == "mfma" and k["gemm1"]["peak"] == bench.PEAK_BF16_TFLOPS
    assert abs(k["gemm1"]["frac"] - (6.2e11 / 0.5e-3 / 1e12) / 2500.0) < 1e-9
    assert k["reduce"]["bound"] == "hbm" and abs(k["reduce"]["achieved"] - 4500.0) < 1e-6
    assert k["materialize"]["launches_per_step"] == 1.0 and k["reduce"]["work_per_launch"] == 4.5e8
    f = bench.kernel_table(_stats(gemm1=dict(launches=1, total_ms=0.01, work=1e8)), 1, "f32")
    assert f["gemm1"]["bound"] == "alu" and f["gemm1"]["peak"] == bench.PEAK_F32_TFLOPS
    r = bench.roofline(k, "bf16", "w")
    assert r["kernel"] == "gemm1" and r["avg_ms"] == 0.25 and r["timing"] == "cold"


def test_tail_reduce_is_its_own_hbm_kernel():
    """The last block's reduction (alone on a one-shot grid) is reported apart
    from the reductions beside the GEMMs, each priced against HBM, and neither
    is taken as the dominant kernel while GEMMs are present."""
    st = {name: {"launches": 0, "total_ms": 0.0, "min_ms": 0.0, "max_ms": 0.0, "work": 0.0}
          for name in ("gemm1", "gemm2", "reduce", "reduce_tail")}
    st["gemm2"].update(launches=4, total_ms=0.58, work=4 * 154.6e9)
    st["reduce"].update(launches=3, total_ms=0.45, work=3 * 453e6)
    st["reduce_tail"].update(launches=1, total_ms=0.075, work=453e6)
    k = bench.kernel_table(st, 1, "bf16")
    assert k["reduce_tail"]["unit"] == "GB/s" and k["reduce_tail"]["bound"] == "hbm"
    assert abs(k["reduce_tail"]["achieved"] - 6040.0) < 1 and abs(k["reduce"]["achieved"] - 3020.0) < 1
    assert bench.roofline(k, "bf16", "w")["kernel"] == "gemm2"


def test_spread_reports_median_and_percentiles():
    s = bench.spread([1.0, 2.0, 3.0, 4.0, 100.0])
    assert s["median"] == 3.0 and s["n"] == 5
    assert 1.0 <= s["p10"] <= 2.0 and 4.0 <= s["p90"] <= 100.0


def test_default_workload_is_the_largest_single_gpu_configuration():
    assert bench.HEADLINE == "gpt3-175b-tp8-2d-r2c2"
    assert set(bench.EXTRAS) == {"tiny-fp32-p2", "gpt2-small-tp4", "gpt3-6.7b-tp8-rowsplit2", "reshard-2x4-mesh",
                                 "shortrun-split-gather"}
    assert bench.FLUSH_BYTES >= 512 << 20


def test_schedule_label_from_launch_counts():
    """The record names the schedule the library chose, from its launch counts."""
    k = lambda **n: {name: {"launches_per_step": c} for name, c in n.items()}
    # a GEMM1 per chunk: the schedule as configured, no label
    assert bench.schedule_label(k(gemm1=2, gemm2=4, reduce=3, gemm2_reduce=1), 2, False) is None
    two = bench.schedule_label(k(gemm1=1, gemm2=3, reduce=3, gemm2_reduce=1), 2, False)
    assert two.startswith("two streams") and "epilogue" in two
    fold = bench.schedule_label(k(gemm1=1, gemm2_reduce=2), 2, False)
    assert fold.startswith("one stream (the second offered, unused)") and "folds" in fold
    assert bench.schedule_label(k(gemm1=1, gemm2_reduce=2), 2, True).startswith("one stream:")
    assert bench.schedule_label(k(gemm1=1, gemm2=1, reduce=1), 2, True).endswith("as one block")
