"""The C ABI from a plain C caller: include/tpshard.h compiles as strict C99
and C++11, and a C program linked against libtpshard.so plans a layout and
reads an error through the host-only entry points (no GPU needed)."""
import os
import shutil
import subprocess

import pytest

from sharded_gemm_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")

needs_gcc = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                               reason="gcc/g++ not available")

PROGRAM = r"""
#include <stdio.h>
#include "tpshard.h"

int main(void) {
  /* [ONNX] "index rule for multi-axis sharding": a 2 x 2 tensor cut in two
   * along axis 0 and in two along axis 1 gives four shards, axis 0 outer. */
  int64_t shape[2] = {2, 2};
  tp_simple_sharding two = {0, 2};
  tp_sharded_dim dims[2] = {{0, &two, 1}, {1, &two, 1}};
  int64_t dev[4] = {0, 1, 2, 3};
  tp_layout lay = {0};
  lay.kind = TP_LAYOUT_SPEC;
  lay.spec.device = dev;
  lay.spec.num_device = 4;
  lay.spec.sharded_dim = dims;
  lay.spec.num_sharded_dim = 2;
  int64_t n = 0, boxes[4 * 4], sod[4];
  int rc = tp_layout_plan(shape, 2, &lay, &n, boxes, 4, sod, 4);
  printf("rc %d shards %lld\n", rc, (long long)n);
  for (int s = 0; s < (int)n && s < 4; ++s)
    printf("box %lld %lld %lld %lld; device %d gets shard %lld\n", (long long)boxes[s * 4],
           (long long)boxes[s * 4 + 1], (long long)boxes[s * 4 + 2], (long long)boxes[s * 4 + 3], s, (long long)sod[s]);
  /* A dim of 3 cut in two is rejected before anything is done. */
  int64_t three[2] = {3, 2};
  rc = tp_layout_plan(three, 2, &lay, &n, NULL, 0, NULL, 0);
  printf("indivisible %d %s\n", rc, tp_last_error());
  printf("version %s\n", tp_version());
  return 0;
}
"""


@needs_gcc
@pytest.mark.parametrize("compiler,std", [("gcc", "c99"), ("g++", "c++11")])
def test_header_is_strict_c_and_cxx(tmp_path, compiler, std):
    src = tmp_path / "h.c"
    src.write_text('#include "tpshard.h"\nint main(void) { return tp_version() ? 0 : 1; }\n')
    lang = ["-x", "c++"] if compiler == "g++" else []
    subprocess.run([compiler, f"-std={std}", "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only", *lang,
                    "-I", INCLUDE, str(src)], check=True, capture_output=True, text=True)


@needs_gcc
def test_c_program_plans_a_layout(tmp_path):
    if not os.path.exists(_abi.LIB_PATH):
        pytest.skip("libtpshard.so is not built")
    src = tmp_path / "prog.c"
    exe = tmp_path / "prog"
    src.write_text(PROGRAM)
    lib_dir = os.path.dirname(_abi.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", INCLUDE, str(src), "-L", lib_dir, "-ltpshard",
                    f"-Wl,-rpath,{lib_dir}", "-o", str(exe)], check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True, timeout=60).stdout.splitlines()
    assert out[0] == "rc 0 shards 4"
    # Shard k = (row block k // 2, column block k % 2), received by device k.
    assert out[1:5] == ["box 0 1 0 1; device 0 gets shard 0", "box 0 1 1 2; device 1 gets shard 1",
                        "box 1 2 0 1; device 2 gets shard 2", "box 1 2 1 2; device 3 gets shard 3"]
    rc, msg = out[5].split(" ", 2)[1:]
    assert int(rc) == -3 and "divisible" in msg   # TP_ERR_INDIVISIBLE, with the reason
    assert out[6].startswith("version tpshard")
