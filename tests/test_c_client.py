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


C_GPU_GATHER_TWOSHOT = r"""
#include <stdio.h>
#include <stdlib.h>
#include <stdint.h>
#include "arnorm.h"

#define CHECK(x) do { if ((x) != hipSuccess) { fprintf(stderr, "HIP error at line %d\n", __LINE__); return 3; } } while (0)

/* Gather and two-shot calls from plain C (hipMalloc, no PyTorch).
   in.bin: int32 tp, m, cap, s (words per rank), width, calls; then per call the shards
   uint32 [tp, m, s]; then per call the two-shot partials bf16 [tp, m, width].
   out.bin: per call the gathered rows uint32 [m, tp*s]; then per call the two-shot
   rows bf16 [m, width]. */
int main(int argc, char **argv) {
  if (argc != 3) return 2;
  FILE *f = fopen(argv[1], "rb");
  if (!f) return 2;
  int32_t h[6];
  if (fread(h, 4, 6, f) != 6) return 2;
  const int tp = h[0], m = h[1], cap = h[2], s = h[3], width = h[4], calls = h[5];
  const size_t sh_n = (size_t)tp * m * s, g_n = (size_t)m * tp * s, p_n = (size_t)tp * m * width, o_n = (size_t)m * width;
  uint32_t *sh = malloc(sh_n * 4 * calls), *gout = malloc(g_n * 4);
  uint16_t *parts = malloc(p_n * 2 * calls), *tout = malloc(o_n * 2);
  if (fread(sh, 4, sh_n * calls, f) != sh_n * calls || fread(parts, 2, p_n * calls, f) != p_n * calls) return 2;
  fclose(f);
  const size_t gbox_words = (size_t)cap * tp * s;
  const size_t recv_words = (size_t)2 * tp * cap * (width / 2), gath_words = (size_t)2 * cap * (width / 2);
  int32_t *d_sh, *gbox, *d_gout, *recv, *gath;
  uint16_t *d_parts, *d_tout;
  CHECK(hipMalloc((void **)&d_sh, sh_n * 4 * calls));
  CHECK(hipMalloc((void **)&gbox, gbox_words * 4));
  CHECK(hipMalloc((void **)&d_gout, g_n * 4 * calls));
  CHECK(hipMalloc((void **)&recv, recv_words * 4));
  CHECK(hipMalloc((void **)&gath, gath_words * 4));
  CHECK(hipMalloc((void **)&d_parts, p_n * 2 * calls));
  CHECK(hipMalloc((void **)&d_tout, o_n * 2 * calls));
  CHECK(hipMemcpy(d_sh, sh, sh_n * 4 * calls, hipMemcpyHostToDevice));
  CHECK(hipMemcpy(d_parts, parts, p_n * 2 * calls, hipMemcpyHostToDevice));
  hipStream_t st;
  CHECK(hipStreamCreate(&st));
  if (lamport_arm(gbox, gbox_words, ARNORM_SENTINEL, st) != ARNORM_OK) return 4;
  if (lamport_arm(recv, recv_words, ARNORM_SENTINEL, st) != ARNORM_OK) return 4;
  if (lamport_arm(gath, gath_words, ARNORM_SENTINEL, st) != ARNORM_OK) return 4;
  for (int c = 0; c < calls; ++c) {
    int rc = gather_push_poll(d_sh + sh_n * c, gbox, d_gout + g_n * c, tp, cap, s, m, 1, st);
    if (rc != ARNORM_OK) { fprintf(stderr, "gather call %d: %s\n", c, arnorm_strerror(rc)); return 5; }
    rc = twoshot_push_reduce_read(d_parts + p_n * c, recv, gath, d_tout + o_n * c, 2, tp, cap, width, c % 2, m, st);
    if (rc != ARNORM_OK) { fprintf(stderr, "two-shot call %d: %s\n", c, arnorm_strerror(rc)); return 5; }
  }
  int status = -1;
  if (arnorm_status(&status, st) != ARNORM_OK || status != ARNORM_OK) return 6;
  int32_t *chk[3] = {gbox, recv, gath};
  const size_t chk_n[3] = {gbox_words, recv_words, gath_words};
  for (int b = 0; b < 3; ++b) {
    int32_t *hb = malloc(chk_n[b] * 4);
    CHECK(hipMemcpy(hb, chk[b], chk_n[b] * 4, hipMemcpyDeviceToHost));
    for (size_t i = 0; i < chk_n[b]; ++i)
      if ((uint32_t)hb[i] != ARNORM_SENTINEL) { fprintf(stderr, "buffer %d word %zu not re-armed\n", b, i); return 7; }
    free(hb);
  }
  FILE *o = fopen(argv[2], "wb");
  if (!o) return 2;
  for (int c = 0; c < calls; ++c) {
    CHECK(hipMemcpy(gout, d_gout + g_n * c, g_n * 4, hipMemcpyDeviceToHost));
    fwrite(gout, 4, g_n, o);
  }
  for (int c = 0; c < calls; ++c) {
    CHECK(hipMemcpy(tout, d_tout + o_n * c, o_n * 2, hipMemcpyDeviceToHost));
    fwrite(tout, 2, o_n, o);
  }
  fclose(o);
  printf("c gpu client: %d gather and %d two-shot calls ok\n", calls, calls);
  return 0;
}
"""


@pytest.mark.gpu
def test_c_client_gather_and_twoshot_on_gpu(tmp_path):
    """A plain C program (hipMalloc, no PyTorch) runs one-launch Gather calls (TP=8, M=4,
    S=896 words) and one-launch two-shot calls (TP=8, M=4, width 7168) over two parities;
    its outputs match the oracle and it finds every mailbox re-armed."""
    import dataclasses

    import numpy as np

    import oracle
    from tests.gpu_util import assert_bits_equal, say
    from tp_all_reduce_arnorm_amd import workloads as wl

    lib = os.path.join(LIB_DIR, "libarnorm.so")
    if not os.path.exists(lib):
        pytest.skip("libarnorm.so not built")
    say("[c client] one-launch Gather and two-shot calls from C on the GPU")
    gcfg = dataclasses.replace(wl.CONFIGS["gather_tp8_m32"], m=4)
    tcfg = wl.CONFIGS["tp8_m4"]
    width, calls = 7168, 4
    shards = [wl.gather_shards(dataclasses.replace(gcfg, seed=gcfg.seed + c)) for c in range(calls)]
    src = wl.ArNormInputs(tcfg)
    parts = [src.partials() for _ in range(calls)]
    with open(tmp_path / "in.bin", "wb") as f:
        f.write(np.array([gcfg.tp, gcfg.m, gcfg.cap, gcfg.s, width, calls], dtype=np.int32).tobytes())
        for x in shards:
            f.write(np.ascontiguousarray(x, dtype=np.uint32).tobytes())
        for p in parts:
            f.write(np.ascontiguousarray(p, dtype=np.uint16).tobytes())
    (tmp_path / "client.c").write_text(C_GPU_GATHER_TWOSHOT)
    exe = tmp_path / "client"
    subprocess.run(["gcc", "-std=c11", "-O1", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", f"-I{ROOT}/include",
                    "-I/opt/rocm/include", str(tmp_path / "client.c"), "-o", str(exe), f"-L{LIB_DIR}", "-larnorm",
                    "-L/opt/rocm/lib", "-lamdhip64", f"-Wl,-rpath,{LIB_DIR}", "-Wl,-rpath,/opt/rocm/lib"],
                   check=True, capture_output=True, text=True, timeout=120)
    r = subprocess.run([str(exe), str(tmp_path / "in.bin"), str(tmp_path / "out.bin")], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    raw = np.fromfile(tmp_path / "out.bin", dtype=np.uint8)
    g_bytes = calls * gcfg.m * gcfg.tp * gcfg.s * 4
    assert raw.size == g_bytes + calls * tcfg.m * width * 2
    got_g = raw[:g_bytes].view(np.uint32).reshape(calls, gcfg.m, gcfg.tp * gcfg.s)
    got_t = raw[g_bytes:].view(np.uint16).reshape(calls, tcfg.m, width)
    gbox_h = oracle.arm(np.empty((gcfg.cap, gcfg.tp * gcfg.s), dtype=np.uint32))
    recv_h = oracle.arm(np.empty((2, tcfg.tp, tcfg.cap, width // 2), dtype=np.uint32))
    gath_h = oracle.arm(np.empty((2, 1, tcfg.cap, width // 2), dtype=np.uint32))
    for c in range(calls):
        oracle.gather_push(gbox_h, shards[c], 0)
        assert_bits_equal(got_g[c], oracle.gather_poll(gbox_h, gcfg.m, True), f"call {c} gathered words")
        oracle.twoshot_push(recv_h, parts[c], c % 2, 0)
        oracle.twoshot_reduce(recv_h, gath_h, c % 2, tcfg.m)
        assert_bits_equal(got_t[c], oracle.twoshot_read(gath_h, c % 2, tcfg.m), f"call {c} two-shot rows")
