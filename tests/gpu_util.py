"""Helpers for the GPU parity tests: host <-> device copies of bit patterns and the
comparison contract (bit-exact words; `out` within one BF16 ulp of the oracle)."""

import sys

import numpy as np

import oracle

S0 = 0x80000000
W = 7168


def say(*a):
    """Name the case before a GPU step (flushed, so a fault still leaves the name)."""
    print(*a, flush=True)
    sys.stdout.flush()


def dev16(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).to("cuda")


def dev32(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32)).to("cuda")


def host16(t):
    return t.cpu().numpy().view(np.uint16)


def host32(t):
    return t.cpu().numpy().view(np.uint32)


def empty16(shape):
    import torch

    return torch.empty(shape, dtype=torch.int16, device="cuda")


def armed_box(shape):
    """A device mailbox filled with the sentinel by the library's own lamport_arm."""
    import torch
    from tp_all_reduce_arnorm_amd import _lib

    box = torch.empty(shape, dtype=torch.int32, device="cuda")
    assert _lib.lamport_arm(box) is True
    return box


def assert_bits_equal(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.argwhere(got != want)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {i}: got {int(got[i]):#x}, "
                             f"want {int(want[i]):#x}")


# At most this fraction of the finite, nonzero oracle values of an `out` comparison may
# differ from the oracle's BF16 bits at all (each still within one ulp).
MAX_DIFFER = 0.01


def assert_out_close(got, want, what="out", exact_zero=None, max_differ=MAX_DIFFER):
    """Within one BF16 ulp of the oracle's value: |gpu - oracle| <= 2^-7 |oracle| for
    normal values, <= 2^-133 (the BF16 subnormal step) below the normal range.
    Elements whose exact value is zero (``exact_zero``; default: where the oracle is
    zero) must be exactly zero (+0 and -0 compare equal); infinities must be equal;
    NaN where the oracle has NaN (any NaN pattern).

    The one-ulp bound is the contract; on its own it would let a systematic error of the
    norm through (a sum of squares off by 0.1 %, say).  So, over comparisons of at least
    1024 finite nonzero oracle values, at most ``max_differ`` of them may differ from the
    oracle's bits at all.  A different FP32 order of the sum of squares moves rstd by a
    few FP32 ulps, which flips an element's BF16 rounding with a probability near 1e-4
    (the GPU tests differ from the oracle in 1e-5 of such elements overall, 7e-4 at
    most in one comparison); an error of 1e-4 in the sum of squares flips about 1 %."""
    g = oracle.widen(got).astype(np.float64)
    w = oracle.widen(want).astype(np.float64)
    if exact_zero is None:
        exact_zero = w == 0
    ulp = np.where(exact_zero, 0.0, np.maximum(2.0**-7 * np.abs(w), 2.0**-133))
    with np.errstate(invalid="ignore"):
        ok = (np.abs(g - w) <= ulp) | (g == w) | (np.isnan(g) & np.isnan(w))
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{what}: {(~ok).sum()} outside 1 ulp, first at {i}: got {g[i]!r} "
                             f"({int(np.asarray(got)[i]):#06x}), want {w[i]!r} ({int(np.asarray(want)[i]):#06x})")
    comparable = np.isfinite(w) & (w != 0)
    n = int(comparable.sum())
    if max_differ is not None and n >= 1024:
        differ = int((comparable & (np.asarray(got, dtype=np.uint16) != np.asarray(want, dtype=np.uint16))).sum())
        if differ > max_differ * n:
            raise AssertionError(f"{what}: {differ} of {n} finite nonzero values differ from the oracle's bits "
                                 f"(each within 1 ulp; at most {max_differ:.0%} may)")
