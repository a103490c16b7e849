"""The C ABI from plain C: a C99 program that includes only include/flce.h,
links libflce.so and calls the host-side entry points (sizing, planning,
argument checks, status and kernel names).  No GPU and no Python types are
involved, which is what the boundary promises a C caller."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "linear_cross_entropy_04_amd")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "flce.h"

int main(void) {
  /* the Llama-3-8B head at chunk 1024: the planned workspace is what a call needs */
  size_t ws = flce_workspace_bytes(8192, 4096, 128256, FLCE_BF16, 1024);
  int64_t c = 1024;
  size_t peak = 0;
  int st = flce_plan(8192, 4096, 128256, FLCE_BF16, &c, 0, &peak);
  printf("workspace %zu plan %d chunk %lld peak %zu\n", ws, st, (long long)c, peak);
  if (ws == 0 || st != FLCE_OK || c != 1024 || peak != ws) return 1;
  /* with no chunk asked for, the default budget keeps scratch below the N x V bf16 logits */
  c = 0;
  st = flce_plan(8192, 4096, 128256, FLCE_BF16, &c, 0, &peak);
  if (st != FLCE_OK || c <= 0 || c >= 8192 || peak >= (size_t)8192 * 128256 * 2) return 10;
  /* scratch follows the chunk, not N */
  if (flce_workspace_bytes(4 * 8192, 4096, 128256, FLCE_BF16, 1024) - ws != 3 * 8192 * 4) return 2;
  /* invalid sizes: 0 bytes; H % 8 != 0 is unsupported on the bf16 path */
  if (flce_workspace_bytes(8192, 4095, 128256, FLCE_BF16, 1024) != 0) return 3;
  if (flce_workspace_bytes(8192, 4096, 0, FLCE_BF16, 1024) != 0) return 4;
  /* argument errors come back before any device work; outputs untouched */
  {
    float loss = -1.0f;
    st = flce_fwd_bwd(NULL, NULL, NULL, 8, 8, 8, FLCE_BF16, -100, 0, &loss, NULL, NULL, NULL,
                      NULL, NULL, 0, NULL);
    if (st != FLCE_EINVAL || loss != -1.0f) return 5;
    st = flce_fwd(NULL, NULL, NULL, 8, 8, 8, 7, -100, 0, &loss, NULL, NULL, NULL, 0, NULL);
    if (st != FLCE_EINVAL || loss != -1.0f) return 6;
  }
  /* every status and kernel class has a name */
  {
    int k;
    for (k = FLCE_OK; k <= FLCE_EUNSUPPORTED; ++k)
      if (flce_status_string(k) == NULL || strlen(flce_status_string(k)) == 0) return 7;
    for (k = 0; k < FLCE_K_COUNT; ++k)
      if (strlen(flce_kernel_name(k)) == 0) return 8;
    if (strlen(flce_kernel_name(FLCE_K_COUNT)) != 0) return 9;
  }
  printf("ok\n");
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_program_uses_the_abi(tmp_path):
    lib = os.path.join(PKG, "libflce.so")
    if not os.path.exists(lib):
        pytest.skip("libflce.so is not built")
    src = tmp_path / "consumer.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "consumer"
    cc = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                         "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                         "-L", PKG, "-lflce", f"-Wl,-rpath,{PKG}"],
                        capture_output=True, text=True)
    assert cc.returncode == 0, cc.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, (run.returncode, run.stdout, run.stderr)
    assert run.stdout.strip().endswith("ok")
