"""The boundary from plain C: a C program includes include/arnorm.h, links libarnorm.so
and calls entry points that validate and return without touching a GPU (a C client
needs no PyTorch and no C++)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "tp_all_reduce_arnorm_amd")

C_CLIENT = r"""
#include <stdio.h>
#include <string.h>
#include "arnorm.h"

int main(void) {
  int fails = 0;
  /* return codes and their names */
  if (strcmp(arnorm_strerror(ARNORM_OK), "ok") != 0) fails++;
  /* a NULL mailbox is malformed; nothing is launched */
  if (lamport_arm(NULL, 16, ARNORM_SENTINEL, 0) != ARNORM_BAD_ARG) fails++;
  /* zero words: nothing to do */
  if (lamport_arm((int32_t *)0x1000, 0, ARNORM_SENTINEL, 0) != ARNORM_OK) fails++;
  /* TP = 1 and M > cap are not served, as the pages' front-end returns None */
  if (arnorm_push((const uint16_t *)0x1000, (int32_t *)0x2000, 2, 1, 64, 0, 0, 1, 4, 0) != ARNORM_NOT_SERVED) fails++;
  if (gather_poll((int32_t *)0x1000, (int32_t *)0x2000, 8, 64, 896, 65, 1, 0) != ARNORM_NOT_SERVED) fails++;
  /* the spin limit round-trips */
  uint64_t old = arnorm_get_spin_limit();
  if (arnorm_set_spin_limit(12345) != ARNORM_OK || arnorm_get_spin_limit() != 12345) fails++;
  if (arnorm_set_spin_limit(old) != ARNORM_OK) fails++;
  printf("c client: %d failures\n", fails);
  return fails;
}
"""


def test_c_client_compiles_links_and_runs(tmp_path):
    lib = os.path.join(LIB_DIR, "libarnorm.so")
    if not os.path.exists(lib):
        pytest.skip("libarnorm.so not built")
    if shutil.which("gcc") is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("needs gcc and the ROCm headers")
    src = tmp_path / "client.c"
    src.write_text(C_CLIENT)
    exe = tmp_path / "client"
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", f"-I{ROOT}/include",
                    "-I/opt/rocm/include", str(src), "-o", str(exe), f"-L{LIB_DIR}", "-larnorm",
                    f"-Wl,-rpath,{LIB_DIR}"], check=True, capture_output=True, text=True, timeout=120)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout
