"""The comparison contract of `out` (tests/gpu_util.assert_out_close), checked on the CPU.

The pages fix the normed output only to one BF16 ulp, because the order of the sum of
squares is the implementation's.  One ulp alone is a loose test: a sum of squares off by
0.4 % still passes it.  The helper therefore also bounds how many values may differ from
the oracle's bits at all.  Here an FP32 model of the norm pins both sides of that bound:
correct FP32 sums in other orders pass, and a sum of squares off by 1e-3 or 4e-3 (inside
one ulp everywhere) fails."""

import numpy as np
import pytest

import oracle
from oracle.bf16 import round_to_bf16, widen
from tests.gpu_util import MAX_DIFFER, assert_out_close

M, W, EPS = 16, 7168, 1e-6


@pytest.fixture(scope="module")
def rows():
    rng = np.random.default_rng(5)
    n = round_to_bf16(rng.standard_normal((M, W), dtype=np.float32))
    gamma = round_to_bf16((1 + 0.1 * rng.standard_normal(W)).astype(np.float32))
    return n, gamma, oracle.rms_norm(n, gamma, EPS)


def fp32_norm(n, gamma, order, scale=1.0):
    """The norm as an FP32 kernel computes it: squares and their sum in FP32 (in the
    given order), rstd = 1 / sqrt(total / 7168 + eps) with FP32 roundings, then
    (x * rstd) * w rounded once to BF16.  ``scale`` multiplies the total: a planted error."""
    v, g = widen(n), widen(gamma)
    sq = (v * v).astype(np.float32)
    if order == "sequential":  # one running FP32 sum over the row: the largest rounding error
        total = np.zeros(M, dtype=np.float32)
        for c in range(W):
            total = (total + sq[:, c]).astype(np.float32)
    else:  # 64-lane partial sums, then their sum
        total = sq.reshape(M, W // 64, 64).sum(axis=2, dtype=np.float32).sum(axis=1, dtype=np.float32)
    total = (total * np.float32(scale)).astype(np.float32)
    rstd = (np.float32(1) / np.sqrt((total / np.float32(W) + np.float32(EPS)).astype(np.float32))).astype(np.float32)
    return round_to_bf16(((v * rstd[:, None]).astype(np.float32) * g).astype(np.float32))


@pytest.mark.parametrize("order", ["lanes", "sequential"])
def test_other_fp32_orders_pass(rows, order):
    n, gamma, want = rows
    got = fp32_norm(n, gamma, order)
    assert (got != want).mean() < MAX_DIFFER / 10  # far inside the bound
    assert_out_close(got, want)


@pytest.mark.parametrize("scale", [1 + 1e-3, 1 + 4e-3])
def test_a_norm_error_inside_one_ulp_fails(rows, scale):
    n, gamma, want = rows
    got = fp32_norm(n, gamma, "lanes", scale)
    assert_out_close(got, want, max_differ=None)  # the one-ulp bound alone lets it through
    with pytest.raises(AssertionError, match="differ from the oracle"):
        assert_out_close(got, want)
