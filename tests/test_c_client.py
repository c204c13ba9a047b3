"""The boundary from plain C: a C program includes include/arnorm.h and links
libarnorm.so, with no PyTorch and no C++.  On the CPU it calls the entry points that
validate and return without touching a GPU; on a GPU (marked `gpu`) it allocates with
hipMalloc, runs one-launch ArNorm calls and writes their outputs for the oracle to check."""

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


C_GPU_CLIENT = r"""
#include <stdio.h>
#include <stdlib.h>
#include <stdint.h>
#include "arnorm.h"

#define CHECK(x) do { if ((x) != hipSuccess) { fprintf(stderr, "HIP error at line %d\n", __LINE__); return 3; } } while (0)

/* One-launch ArNorm calls from plain C: device memory from hipMalloc, no PyTorch.
   in.bin: int32 tp, m, cap, calls; then per call bf16 partials [tp, m, 7168]; then
   gamma [7168].  out.bin: per call out [m, 7168] then residual_out [m, 7168]. */
int main(int argc, char **argv) {
  if (argc != 3) return 2;
  FILE *f = fopen(argv[1], "rb");
  if (!f) return 2;
  int32_t hdr[4];
  if (fread(hdr, 4, 4, f) != 4) return 2;
  const int tp = hdr[0], m = hdr[1], cap = hdr[2], calls = hdr[3];
  const size_t row = ARNORM_HIDDEN, part_n = (size_t)tp * m * row;
  uint16_t *parts = malloc(part_n * 2 * calls), *gamma = malloc(row * 2), *res = malloc(2 * m * row * 2 * calls);
  if (fread(parts, 2, part_n * calls, f) != part_n * calls || fread(gamma, 2, row, f) != row) return 2;
  fclose(f);
  const size_t box_words = (size_t)2 * tp * cap * ARNORM_ROW_WORDS, nbox_words = (size_t)2 * cap * 256;
  int32_t *box, *nbox;
  uint16_t *d_parts, *d_gamma, *d_out, *d_rout;
  CHECK(hipMalloc((void **)&box, box_words * 4));
  CHECK(hipMalloc((void **)&nbox, nbox_words * 4));
  CHECK(hipMalloc((void **)&d_parts, part_n * 2 * calls));
  CHECK(hipMalloc((void **)&d_gamma, row * 2));
  CHECK(hipMalloc((void **)&d_out, (size_t)m * row * 2 * calls));
  CHECK(hipMalloc((void **)&d_rout, (size_t)m * row * 2 * calls));
  CHECK(hipMemcpy(d_parts, parts, part_n * 2 * calls, hipMemcpyHostToDevice));
  CHECK(hipMemcpy(d_gamma, gamma, row * 2, hipMemcpyHostToDevice));
  hipStream_t s;
  CHECK(hipStreamCreate(&s));
  if (lamport_arm(box, box_words, ARNORM_SENTINEL, s) != ARNORM_OK) return 4;
  if (lamport_arm(nbox, nbox_words, ARNORM_SENTINEL, s) != ARNORM_OK) return 4;
  for (int c = 0; c < calls; ++c) {
    int rc = arnorm_push_reduce_norm(d_parts + part_n * c, NULL, d_gamma, d_out + (size_t)m * row * c,
                                     d_rout + (size_t)m * row * c, box, nbox, 2, tp, cap, c % 2, m, 1e-6f, s);
    if (rc != ARNORM_OK) { fprintf(stderr, "call %d: %s\n", c, arnorm_strerror(rc)); return 5; }
  }
  int status = -1;
  if (arnorm_status(&status, s) != ARNORM_OK || status != ARNORM_OK) return 6;
  int32_t *hbox = malloc(box_words * 4);
  CHECK(hipMemcpy(hbox, box, box_words * 4, hipMemcpyDeviceToHost));
  for (size_t i = 0; i < box_words; ++i)
    if ((uint32_t)hbox[i] != ARNORM_SENTINEL) { fprintf(stderr, "mailbox word %zu not re-armed\n", i); return 7; }
  FILE *o = fopen(argv[2], "wb");
  if (!o) return 2;
  for (int c = 0; c < calls; ++c) {
    CHECK(hipMemcpy(res, d_out + (size_t)m * row * c, (size_t)m * row * 2, hipMemcpyDeviceToHost));
    CHECK(hipMemcpy(res + (size_t)m * row, d_rout + (size_t)m * row * c, (size_t)m * row * 2, hipMemcpyDeviceToHost));
    fwrite(res, 2, 2 * (size_t)m * row, o);
  }
  fclose(o);
  printf("c gpu client: %d calls ok\n", calls);
  return 0;
}
"""


@pytest.mark.gpu
def test_c_client_on_gpu(tmp_path):
    """A plain C program (hipMalloc, no PyTorch) runs one-launch ArNorm calls at TP=8, M=4
    over two parities; its outputs match the oracle and it finds the mailbox re-armed."""
    import numpy as np

    import oracle
    from tests.gpu_util import assert_bits_equal, assert_out_close, say
    from tp_all_reduce_arnorm_amd import workloads as wl

    lib = os.path.join(LIB_DIR, "libarnorm.so")
    if not os.path.exists(lib):
        pytest.skip("libarnorm.so not built")
    say("[c client] one-launch ArNorm from C on the GPU")
    cfg = wl.CONFIGS["tp8_m4"]
    src = wl.ArNormInputs(cfg)
    calls = 4
    parts = [src.call()[0] for _ in range(calls)]
    with open(tmp_path / "in.bin", "wb") as f:
        f.write(np.array([cfg.tp, cfg.m, cfg.cap, calls], dtype=np.int32).tobytes())
        for p in parts:
            f.write(np.ascontiguousarray(p, dtype=np.uint16).tobytes())
        f.write(np.ascontiguousarray(src.gamma, dtype=np.uint16).tobytes())
    (tmp_path / "client.c").write_text(C_GPU_CLIENT)
    exe = tmp_path / "client"
    subprocess.run(["gcc", "-std=c11", "-O1", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", f"-I{ROOT}/include",
                    "-I/opt/rocm/include", str(tmp_path / "client.c"), "-o", str(exe), f"-L{LIB_DIR}", "-larnorm",
                    "-L/opt/rocm/lib", "-lamdhip64", f"-Wl,-rpath,{LIB_DIR}", "-Wl,-rpath,/opt/rocm/lib"],
                   check=True, capture_output=True, text=True, timeout=120)
    r = subprocess.run([str(exe), str(tmp_path / "in.bin"), str(tmp_path / "out.bin")], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    got = np.fromfile(tmp_path / "out.bin", dtype=np.uint16).reshape(calls, 2, cfg.m, 7168)
    box_h = oracle.arm(np.empty((2, cfg.tp, cfg.cap, 3584), dtype=np.uint32))
    for c, p in enumerate(parts):
        oracle.arnorm_push(box_h, p, c % 2, 0)
        want_out, want_res = oracle.arnorm_reduce_norm(box_h, c % 2, cfg.m, None, src.gamma, cfg.eps)
        assert_bits_equal(got[c, 1], want_res, f"call {c} residual_out")
        assert_out_close(got[c, 0], want_out, f"call {c} out")
