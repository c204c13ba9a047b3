"""The Python binding refuses mismatched tensor shapes before anything reaches the
library: the kernels index the caller's buffers by the sizes passed, so a short buffer
would be read or written past its end.  These checks run before any device call, so
host tensors are enough to exercise them."""

import pytest
import torch

from tp_all_reduce_arnorm_amd import _lib as lib

W = 7168


def t16(*shape):
    return torch.zeros(shape, dtype=torch.int16)


def t32(*shape):
    return torch.zeros(shape, dtype=torch.int32)


@pytest.mark.parametrize("bad", ["residual", "residual_out", "gamma", "partial", "norm_box"])
def test_reduce_norm_shapes(bad):
    m = 4
    args = dict(residual=t16(m, W), gamma=t16(W), mailbox=t32(2, 8, 64, W // 2), parity=0, eps=1e-6,
                out=t16(m, W), residual_out=t16(m, W), partial=t16(m, W), norm_box=t32(2, 64, 256))
    args[bad] = {"residual": t16(m - 1, W), "residual_out": t16(m, W - 8), "gamma": t16(W // 2),
                 "partial": t16(m + 1, W), "norm_box": t32(2, 32, 256)}[bad]
    with pytest.raises(ValueError, match=bad):
        lib.arnorm_reduce_norm(**args)


@pytest.mark.parametrize("bad", ["out", "residual_out", "gamma", "residual", "partials", "norm_box"])
def test_push_reduce_norm_shapes(bad):
    m = 4
    args = dict(partials=t16(8, m, W), residual=t16(m, W), gamma=t16(W), mailbox=t32(2, 8, 64, W // 2), parity=0,
                eps=1e-6, out=t16(m, W), residual_out=t16(m, W), norm_box=t32(2, 64, 256))
    args[bad] = {"out": t16(m - 1, W), "residual_out": t16(m + 1, W), "gamma": t16(W + 8),
                 "residual": t16(2 * m, W), "partials": t16(7, m, W), "norm_box": t32(1, 64, 256)}[bad]
    with pytest.raises(ValueError):
        lib.arnorm_push_reduce_norm(**args)


def test_gather_shapes():
    box = t32(64, 8 * 896)
    with pytest.raises(ValueError):
        lib.gather_push(t32(8, 32, 895), box, 8, 0)          # S does not match the rows
    with pytest.raises(ValueError):
        lib.gather_poll(box, 8, 32, out=t32(31, 8 * 896))    # out one row short
    with pytest.raises(ValueError):
        lib.gather_poll(box, 8, 32, out=None, copy=True)     # copy needs out
    with pytest.raises(ValueError):
        lib.gather_poll(t32(64, 100), 8, 32, copy=False)     # rows do not split over tp
    with pytest.raises(ValueError):
        lib.gather_push_poll(t32(8, 32, 896), box, out=t32(32, 8 * 895))


def test_twoshot_shapes():
    recv, gath = t32(2, 8, 64, W // 2), t32(2, 1, 64, W // 2)
    with pytest.raises(ValueError):
        lib.twoshot_push(t16(8, 4, W - 8), recv, 0, 0)
    with pytest.raises(ValueError):
        lib.twoshot_reduce(recv, t32(2, 1, 32, W // 2), 0, 4)
    with pytest.raises(ValueError):
        lib.twoshot_read(t32(2, 2, 64, W // 2), 0, t16(4, W))
    with pytest.raises(ValueError):
        lib.twoshot_push_reduce_read(t16(8, 4, W), recv, gath, 0, t16(3, W))
    with pytest.raises(ValueError):
        lib.twoshot_push_reduce_read(t16(4, 4, W), recv, gath, 0, t16(4, W))
