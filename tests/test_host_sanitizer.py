"""The library's host code (layout planning, the sharding checker, argument
validation and the two-stream scheduler) built with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer and driven through
brute-force layouts, every error status and several hundred valid MLP
configurations ([ONNX] sharding formalism, "validity check": a layout is
checked and refused with a reason).  The kernel launchers are replaced by
host stand-ins (tests/sanitizer/stub_kernels.cpp) that check every byte
range a kernel would touch against the buffers the driver registered; no GPU
is used."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sharded_gemm_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitizer")
ROCM = "/opt/rocm"
FLAGS = ["-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{ROOT}/include"]


def test_host_code_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(f"{ROCM}/lib/libamdhip64.so"):
        pytest.skip("needs g++ and the HIP runtime library")
    srcs = [os.path.join(CSRC, f) for f in ("plan.cpp", "checker.cpp", "api.cpp", "timing.cpp")] + \
           [os.path.join(SAN, f) for f in ("stub_kernels.cpp", "driver.cpp")]
    procs, objs = [], []
    for s in srcs:
        o = str(tmp_path / (os.path.basename(s) + ".o"))
        objs.append(o)
        procs.append(subprocess.Popen([gxx, *FLAGS, "-c", s, "-o", o], stdout=subprocess.PIPE,
                                      stderr=subprocess.STDOUT, text=True))
    for s, p in zip(srcs, procs):
        out = p.communicate(timeout=600)[0]
        assert p.returncode == 0, f"compile of {s} failed:\n{out}"
    exe = str(tmp_path / "driver")
    r = subprocess.run([gxx, "-fsanitize=address,undefined", *objs, f"-L{ROCM}/lib", "-lamdhip64",
                        f"-Wl,-rpath,{ROCM}/lib", "-o", exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    counts = dict(zip(r.stdout.split()[0::2], map(int, r.stdout.split()[1::2])))
    assert counts["ok"] > 1000 and counts["launches"] > 1000
    for kind in ("arg", "spec", "indivisible", "unsupported"):
        assert counts[kind] > 0, kind
