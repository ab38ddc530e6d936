"""The boundary from C: a C99 program that includes include/lc_moe.h, takes the address of
every entry point the header declares, links against liblc_moe.so and calls the host-side
parts (sizes, names, and argument checks that return before anything is enqueued).  No GPU
is touched, so it runs on the CPU."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "mixture_experts_layer_router_amd")
HEADER = os.path.join(ROOT, "include", "lc_moe.h")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "lc_moe.h"

/* every entry point, by address: the declarations are valid C and the symbols link */
static void* const entry_points[] = {
@ENTRY_POINTS@
};

int main(void) {
  int fails = 0;
  const lc_moe_shape prefill = {16384, 6144, 512, 256, 12, 2048, LC_MOE_BF16};
  const lc_moe_shape bad = {16, 100, 4, 2, 3, 64, LC_MOE_BF16}; /* d not a multiple of 8 */
  const lc_moe_shape f32 = {64, 132, 8, 4, 3, 60, LC_MOE_F32};
  size_t n = sizeof entry_points / sizeof entry_points[0], i;
  for (i = 0; i < n; ++i) fails += entry_points[i] == NULL;
  fails += lc_moe_workspace_size(&prefill) == 0;
  fails += lc_moe_workspace_size(&bad) != 0;
  fails += lc_moe_workspace_size(&f32) == 0;
  fails += lc_moe_fp8_weights_size(&prefill) == 0;
  fails += lc_moe_packed_weights_size(&prefill) == 0;
  fails += lc_moe_backward_workspace_size(&prefill) == 0;
  fails += lc_moe_fp8_weights_size(&f32) != 0; /* fp32 layers have no FP8 form */
  for (i = 0; i <= LC_MOE_E_DEVICE; ++i) {
    const char* s = lc_moe_status_str((lc_moe_status)i);
    fails += s == NULL || strlen(s) == 0;
  }
  for (i = 0; i < LC_MOE_NUM_STAGES; ++i) {
    const char* s = lc_moe_stage_name((int)i);
    fails += s == NULL || strlen(s) == 0;
  }
  {
    lc_moe_weights w;
    memset(&w, 0, sizeof w);
    fails += lc_moe_forward(&prefill, NULL, &w, NULL, NULL, NULL, NULL, NULL, 0, NULL) != LC_MOE_E_NULLPTR;
    fails += lc_moe_route(&bad, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) != LC_MOE_E_SHAPE;
  }
  printf("entry points %zu, failures %d\n", n, fails);
  return fails != 0;
}
"""


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:lc_moe_status|size_t|const char\*)\s+(lc_moe_\w+)\(", text, re.M)))


def test_header_compiles_as_c_and_links(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    lib = os.path.join(PKG, "liblc_moe.so")
    assert os.path.exists(lib), "build the library first"
    names = declared_functions()
    assert len(names) == 17, names
    src = tmp_path / "consumer.c"
    src.write_text(PROGRAM.replace("@ENTRY_POINTS@", ",\n".join(f"  (void*)&{n}" for n in names)))
    exe = tmp_path / "consumer"
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-isystem", "/opt/rocm/include", str(src), "-o", str(exe), "-L", PKG, "-llc_moe", f"-Wl,-rpath,{PKG}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, (r.stdout, r.stderr)
    assert f"entry points {len(names)}, failures 0" in r.stdout
