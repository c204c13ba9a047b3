"""The C ABI on the CPU: the library loads, exports every entry point that
include/arnorm.h declares, and its host-side argument checks answer without any GPU
call (the pointers below are never dereferenced: every case returns before a launch)."""

import ctypes
import os
import re
import subprocess

import pytest

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "arnorm.h")
FAKE = 0x1000  # a 16-byte aligned address that no call below may touch
MIS = 0x1004  # misaligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[a-z_0-9 ]+?\*?\s*\b([a-z_0-9]+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    from tp_all_reduce_arnorm_amd import _lib

    return _lib.LIB


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("lamport_arm", "arnorm_push", "arnorm_reduce_norm", "gather_push", "gather_poll"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    lib_path = os.path.join(ROOT, "tp_all_reduce_arnorm_amd", "libarnorm.so")
    dyn = subprocess.run(["nm", "-D", "--defined-only", lib_path], capture_output=True, text=True,
                         check=True).stdout
    exported = {ln.split()[-1] for ln in dyn.splitlines() if " T " in ln}
    for n in declared_functions():
        assert n in exported, n
        assert hasattr(L, n)


def test_strerror(L):
    assert L.arnorm_strerror(0) == b"ok"
    assert b"not served" in L.arnorm_strerror(1)
    assert L.arnorm_strerror(99) == b"unknown code"


def test_arm_checks(L):
    assert L.lamport_arm(None, 16, 0x80000000, None) == 2
    assert L.lamport_arm(MIS, 16, 0x80000000, None) == 2
    assert L.lamport_arm(FAKE, 0, 0x80000000, None) == 0  # nothing to launch


@pytest.mark.parametrize("tp", [0, 1, 9, 16])
def test_push_tp_not_served(L, tp):
    assert L.arnorm_push(FAKE, FAKE, 1, tp, 64, 0, 0, 1, 4, None) == 1


@pytest.mark.parametrize("m,cap", [(0, 64), (65, 64), (-1, 64), (200000, 200000)])
def test_push_rows_not_served(L, m, cap):
    assert L.arnorm_push(FAKE, FAKE, 1, 8, cap, 0, 0, 8, m, None) == 1


@pytest.mark.parametrize("args", [
    dict(parities=0), dict(cap=0), dict(parity=2), dict(parity=-1), dict(rank=-1), dict(nslots=0),
    dict(rank=7, nslots=2), dict(partial=None), dict(partial=MIS), dict(mailbox=None), dict(mailbox=MIS),
])
def test_push_bad_args(L, args):
    a = dict(partial=FAKE, mailbox=FAKE, parities=2, tp=8, cap=64, parity=0, rank=0, nslots=8, M=4)
    a.update(args)
    m = a.get("M")
    if a["cap"] == 0:
        m = 0  # M <= cap is checked after cap; cap < 1 is malformed whatever M is
    rc = L.arnorm_push(a["partial"], a["mailbox"], a["parities"], a["tp"], a["cap"], a["parity"], a["rank"],
                       a["nslots"], m, None)
    assert rc == 2, (args, rc)


def reduce_rc(L, **kw):
    a = dict(partial=None, residual=FAKE + 0x100000, gamma=FAKE + 0x200000, out=FAKE + 0x300000,
             residual_out=FAKE + 0x400000, mailbox=FAKE + 0x500000, norm_box=None, parities=2, tp=8, cap=64,
             parity=0, rank=0, M=4, eps=1e-6)
    a.update(kw)
    return L.arnorm_reduce_norm(a["partial"], a["residual"], a["gamma"], a["out"], a["residual_out"],
                                a["mailbox"], a["norm_box"], a["parities"], a["tp"], a["cap"], a["parity"],
                                a["rank"], a["M"], a["eps"], None)


def test_reduce_checks(L):
    assert reduce_rc(L, tp=1) == 1
    assert reduce_rc(L, M=0) == 1
    assert reduce_rc(L, M=65) == 1
    assert reduce_rc(L, gamma=None) == 2
    assert reduce_rc(L, out=MIS) == 2
    assert reduce_rc(L, residual=MIS) == 2
    assert reduce_rc(L, parity=2) == 2
    assert reduce_rc(L, partial=FAKE, rank=8) == 2
    assert reduce_rc(L, partial=FAKE, rank=-1) == 2
    # outputs may not alias inputs or each other; residual_out may equal residual
    assert reduce_rc(L, out=FAKE + 0x100000) == 2
    assert reduce_rc(L, residual_out=FAKE + 0x300000) == 2
    assert reduce_rc(L, residual_out=FAKE + 0x500000) == 2
    assert reduce_rc(L, out=FAKE + 0x200000) == 2
    # the norm box: aligned, and no alias of the mailbox or an output
    assert reduce_rc(L, norm_box=MIS) == 2
    assert reduce_rc(L, norm_box=FAKE + 0x500000) == 2
    assert reduce_rc(L, norm_box=FAKE + 0x300000) == 2
    assert reduce_rc(L, norm_box=FAKE + 0x400000) == 2
    assert reduce_rc(L, norm_box=FAKE + 0x600000, tp=1) == 1


def test_push_reduce_norm_checks(L):
    a = (FAKE, FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000, FAKE + 0x400000, FAKE + 0x500000,
         FAKE + 0x600000)
    assert L.arnorm_push_reduce_norm(*a, 2, 1, 64, 0, 4, 1e-6, None) == 1      # tp 1
    assert L.arnorm_push_reduce_norm(*a, 2, 8, 64, 0, 65, 1e-6, None) == 1     # M > cap
    assert L.arnorm_push_reduce_norm(*a, 2, 8, 64, 0, 0, 1e-6, None) == 1      # M = 0
    assert L.arnorm_push_reduce_norm(*a, 2, 8, 64, 2, 4, 1e-6, None) == 2      # parity
    assert L.arnorm_push_reduce_norm(MIS, *a[1:], 2, 8, 64, 0, 4, 1e-6, None) == 2
    b = list(a)
    b[6] = FAKE + 0x300000  # norm box aliases out
    assert L.arnorm_push_reduce_norm(*b, 2, 8, 64, 0, 4, 1e-6, None) == 2
    # the two-launch form (M=64, or no norm box) rejects a bad consumer argument before it
    # launches the push (which would fail here, with no GPU, as HIP_ERROR = 3)
    for m, box in ((64, FAKE + 0x600000), (4, None)):
        c = list(a)
        c[6] = box
        c[4] = c[3]  # residual_out aliases out
        assert L.arnorm_push_reduce_norm(*c, 2, 8, 64, 0, m, 1e-6, None) == 2
        c = list(a)
        c[6] = box
        c[2] = MIS  # misaligned gamma
        assert L.arnorm_push_reduce_norm(*c, 2, 8, 64, 0, m, 1e-6, None) == 2
        c = list(a)
        c[6] = box
        c[3] = c[5]  # out aliases the mailbox
        assert L.arnorm_push_reduce_norm(*c, 2, 8, 64, 0, m, 1e-6, None) == 2


def test_gather_checks(L):
    assert L.gather_push(FAKE, FAKE, 1, 64, 896, 0, 1, 32, None) == 1
    assert L.gather_push(FAKE, FAKE, 8, 64, 894, 0, 1, 32, None) == 1  # S % 4
    assert L.gather_push(FAKE, FAKE, 8, 64, 0, 0, 1, 32, None) == 1
    assert L.gather_push(FAKE, FAKE, 8, 64, 896, 0, 1, 65, None) == 1
    assert L.gather_push(FAKE, FAKE, 8, 64, 896, 7, 2, 32, None) == 2
    assert L.gather_push(MIS, FAKE, 8, 64, 896, 0, 1, 32, None) == 2
    # one slot's shard rows above 2^32 - 256 fragments (2^24 + 1 rows of 256): refused before any launch
    assert L.gather_push(FAKE, FAKE, 2, (1 << 24) + 1, 1024, 0, 1, (1 << 24) + 1, None) == 1
    assert L.gather_poll(FAKE, None, 8, 64, 896, 32, 1, None) == 2  # copy needs out
    assert L.gather_poll(FAKE, FAKE, 8, 64, 896, 32, 1, None) == 2  # out aliases mailbox
    assert L.gather_poll(FAKE, None, 8, 64, 896, 0, 0, None) == 1


def test_gather_push_poll_checks(L):
    assert L.gather_push_poll(FAKE, FAKE + 0x100000, FAKE + 0x200000, 1, 64, 896, 32, 1, None) == 1
    assert L.gather_push_poll(FAKE, FAKE + 0x100000, FAKE + 0x200000, 8, 64, 6, 32, 1, None) == 1
    assert L.gather_push_poll(FAKE, FAKE + 0x100000, FAKE + 0x200000, 8, 64, 896, 65, 1, None) == 1
    assert L.gather_push_poll(FAKE, FAKE + 0x100000, FAKE + 0x200000, 8, 64, 896, 0, 1, None) == 1
    for m in (4, 32):  # one launch, and the pair
        assert L.gather_push_poll(MIS, FAKE + 0x100000, FAKE + 0x200000, 8, 64, 896, m, 1, None) == 2
        assert L.gather_push_poll(FAKE, FAKE + 0x100000, FAKE + 0x100000, 8, 64, 896, m, 1, None) == 2
        assert L.gather_push_poll(FAKE, FAKE + 0x100000, FAKE, 8, 64, 896, m, 1, None) == 2
        assert L.gather_push_poll(FAKE, FAKE + 0x100000, None, 8, 64, 896, m, 1, None) == 2


def test_twoshot_checks(L):
    assert L.twoshot_push(FAKE, FAKE, 2, 1, 64, 7168, 0, 0, 1, 4, None) == 1   # tp 1
    assert L.twoshot_push(FAKE, FAKE, 2, 8, 64, 7164, 0, 0, 8, 4, None) == 1   # width % 8
    assert L.twoshot_push(FAKE, FAKE, 2, 8, 64, 7168, 0, 0, 8, 65, None) == 1  # M > cap
    assert L.twoshot_push(FAKE, FAKE, 2, 8, 64, 7168, 2, 0, 8, 4, None) == 2   # parity
    assert L.twoshot_push(FAKE, FAKE, 2, 8, 64, 7168, 0, 1, 8, 4, None) == 2   # rank + nslots
    assert L.twoshot_push(MIS, FAKE, 2, 8, 64, 7168, 0, 0, 8, 4, None) == 2
    assert L.twoshot_reduce(FAKE, FAKE + 0x100000, 2, 9, 64, 7168, 0, 4, None) == 1
    assert L.twoshot_reduce(FAKE, FAKE, 2, 8, 64, 7168, 0, 4, None) == 2      # recv == gather
    assert L.twoshot_reduce(FAKE, FAKE + 0x100000, 2, 8, 64, 0, 0, 4, None) == 1
    assert L.twoshot_read(FAKE, FAKE, 2, 64, 7168, 0, 4, None) == 2           # out == gather
    assert L.twoshot_read(FAKE, MIS, 2, 64, 7168, 0, 4, None) == 2
    assert L.twoshot_read(FAKE, FAKE + 0x100000, 2, 64, 7168, 0, 0, None) == 1


def test_twoshot_push_reduce_read_checks(L):
    P, R, G, O = FAKE, FAKE + 0x1000000, FAKE + 0x2000000, FAKE + 0x3000000
    f = L.twoshot_push_reduce_read
    assert f(P, R, G, O, 2, 1, 64, 7168, 0, 4, None) == 1    # tp 1
    assert f(P, R, G, O, 2, 9, 64, 7168, 0, 4, None) == 1    # tp 9
    assert f(P, R, G, O, 2, 8, 64, 7164, 0, 4, None) == 1    # width % 8
    assert f(P, R, G, O, 2, 8, 64, 7168, 0, 65, None) == 1   # M > cap
    assert f(P, R, G, O, 2, 8, 64, 7168, 0, 0, None) == 1    # M = 0
    assert f(P, R, G, O, 2, 8, 64, 7168, 2, 4, None) == 2    # parity
    for m in (4, 64):  # one launch, and the three launches
        assert f(MIS, R, G, O, 2, 8, 64, 7168, 0, m, None) == 2
        assert f(P, R, G, MIS, 2, 8, 64, 7168, 0, m, None) == 2
        assert f(P, R, R, O, 2, 8, 64, 7168, 0, m, None) == 2   # recv == gather
        assert f(P, R, G, G, 2, 8, 64, 7168, 0, m, None) == 2   # out == gather
        assert f(P, R, G, R, 2, 8, 64, 7168, 0, m, None) == 2   # out == recv
        assert f(P, R, G, P, 2, 8, 64, 7168, 0, m, None) == 2   # out == partial
        assert f(P, R, G, None, 2, 8, 64, 7168, 0, m, None) == 2


def test_poll_knob(L):
    for u, mode in ((3, 0), (2, 0), (0, 3), (0, -1), (8, 1)):
        assert L.arnorm_set_poll(u, mode) == 2
    for u in (0, 1, 4):
        for mode in (0, 1, 2):
            assert L.arnorm_set_poll(u, mode) == 0
    assert L.arnorm_set_poll(0, 0) == 0


def test_spin_limit_and_threads(L):
    old = L.arnorm_get_spin_limit()
    assert L.arnorm_set_spin_limit(0) == 2
    assert L.arnorm_set_spin_limit(12345) == 0
    assert L.arnorm_get_spin_limit() == 12345
    assert L.arnorm_set_spin_limit(old) == 0
    for k in (2, 3, 5, 16):
        assert L.arnorm_set_reduce_split(k) == 2
    for k in (4, 7, 8, 14, 1, 0):
        assert L.arnorm_set_reduce_split(k) == 0
    assert L.arnorm_set_reduce_threads(300) == 2
    for t in (896, 448, 256, 0):
        assert L.arnorm_set_reduce_threads(t) == 0
    assert L.arnorm_status(None, None) == 2


def test_binding_mirrors_the_abi():
    from tp_all_reduce_arnorm_amd import _lib

    for n in ("lamport_arm", "arnorm_push", "arnorm_reduce_norm", "arnorm_push_reduce_norm", "gather_push",
              "gather_poll", "gather_push_poll", "twoshot_push", "twoshot_reduce", "twoshot_read",
              "twoshot_push_reduce_read"):
        assert callable(getattr(_lib, n))


def test_binding_fails_loudly_without_the_library(tmp_path):
    """The binding has no fallback: imported from a package directory where libarnorm.so
    was never built, it raises ImportError naming the build command."""
    import shutil
    import sys

    pkg = tmp_path / "unbuilt_pkg"
    pkg.mkdir()
    (pkg / "__init__.py").write_text("")
    shutil.copy(os.path.join(ROOT, "tp_all_reduce_arnorm_amd", "_lib.py"), pkg / "_lib.py")
    r = subprocess.run([sys.executable, "-c", "import unbuilt_pkg._lib"], cwd=str(tmp_path), capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "is not built" in r.stderr
