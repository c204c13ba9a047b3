"""The pages' front-end gates, on the host: a BF16 argument of another dtype is not
served (None, as drafter.comm's DrafterComm.ar_norm returns), 32-bit word arguments of
another dtype are refused, and the DrafterComm-shaped front-end serves exactly the
shapes the pages' gather_context / gather_logits / ar_norm serve.  Every check runs
before any device call, so host tensors are enough."""

import pytest
import torch

from tp_all_reduce_arnorm_amd import _lib as lib
from tp_all_reduce_arnorm_amd import comm

W = 7168


def t(dtype, *shape):
    return torch.zeros(shape, dtype=dtype)


NOT_BF16 = [torch.float16, torch.float32, torch.int32, torch.uint8]


@pytest.mark.parametrize("dtype", NOT_BF16)
def test_arnorm_entry_points_do_not_serve_other_dtypes(dtype):
    m = 4
    box, nbox = t(torch.int32, 2, 8, 64, W // 2), t(torch.int32, 2, 64, 256)
    bf = torch.bfloat16
    assert lib.arnorm_push(t(dtype, 8, m, W), box, 0, 0) is None
    for bad in ("residual", "gamma", "out", "residual_out", "partial"):
        args = dict(residual=t(bf, m, W), gamma=t(bf, W), mailbox=box, parity=0, eps=1e-6, out=t(bf, m, W),
                    residual_out=t(bf, m, W), partial=t(bf, m, W), norm_box=nbox)
        args[bad] = t(dtype, *args[bad].shape)
        assert lib.arnorm_reduce_norm(**args) is None, bad
    for bad in ("partials", "residual", "gamma", "out", "residual_out"):
        args = dict(partials=t(bf, 8, m, W), residual=t(bf, m, W), gamma=t(bf, W), mailbox=box, parity=0,
                    eps=1e-6, out=t(bf, m, W), residual_out=t(bf, m, W), norm_box=nbox)
        args[bad] = t(dtype, *args[bad].shape)
        assert lib.arnorm_push_reduce_norm(**args) is None, bad


@pytest.mark.parametrize("dtype", NOT_BF16)
def test_twoshot_entry_points_do_not_serve_other_dtypes(dtype):
    recv, gath = t(torch.int32, 2, 8, 64, W // 2), t(torch.int32, 2, 1, 64, W // 2)
    assert lib.twoshot_push(t(dtype, 8, 4, W), recv, 0, 0) is None
    assert lib.twoshot_read(gath, 0, t(dtype, 4, W)) is None
    assert lib.twoshot_push_reduce_read(t(dtype, 8, 4, W), recv, gath, 0, t(torch.bfloat16, 4, W)) is None
    assert lib.twoshot_push_reduce_read(t(torch.int16, 8, 4, W), recv, gath, 0, t(dtype, 4, W)) is None


@pytest.mark.parametrize("dtype", [torch.float32, torch.int16, torch.int64, torch.float16])
def test_word_arguments_must_be_int32(dtype):
    bf = torch.bfloat16
    with pytest.raises(ValueError, match="32-bit words"):
        lib.arnorm_push(t(bf, 8, 4, W), t(dtype, 2, 8, 64, W // 2), 0, 0)
    with pytest.raises(ValueError, match="32-bit words"):
        lib.arnorm_reduce_norm(None, t(bf, W), t(torch.int32, 2, 8, 64, W // 2), 0, 1e-6, t(bf, 4, W),
                               t(bf, 4, W), norm_box=t(dtype, 2, 64, 256))
    with pytest.raises(ValueError, match="32-bit words"):
        lib.gather_push(t(dtype, 8, 32, 896), t(torch.int32, 64, 8 * 896), 8, 0)
    with pytest.raises(ValueError, match="32-bit words"):
        lib.gather_poll(t(torch.int32, 64, 8 * 896), 8, 32, out=t(dtype, 32, 8 * 896))
    with pytest.raises(ValueError, match="32-bit words"):
        lib.gather_push_poll(t(torch.int32, 8, 32, 896), t(dtype, 64, 8 * 896), out=t(torch.int32, 32, 8 * 896))
    with pytest.raises(ValueError, match="32-bit words"):
        lib.twoshot_reduce(t(dtype, 2, 8, 64, W // 2), t(torch.int32, 2, 1, 64, W // 2), 0, 4)
    with pytest.raises(ValueError, match="32-bit words"):
        lib.lamport_arm(t(dtype, 16))


def test_bit_views_of_bf16_are_served():
    assert lib.bf16_served(t(torch.bfloat16, 2), t(torch.int16, 2), t(torch.uint16, 2), None)
    assert not lib.bf16_served(t(torch.int16, 2), t(torch.float16, 2))


def test_ar_norm_gate():
    bf, tp, cap = torch.bfloat16, 8, 64
    x, w, r = t(bf, tp, 4, W), t(bf, W), t(bf, 4, W)
    assert comm.ar_norm_served(x, r, w, tp, cap)
    assert comm.ar_norm_served(x, None, w, tp, cap)
    assert comm.ar_norm_served(t(bf, tp, cap, W), None, w, tp, cap)
    assert not comm.ar_norm_served(t(bf, tp, cap + 1, W), None, w, tp, cap)       # rows above ROWS_CAP
    assert not comm.ar_norm_served(t(bf, tp, 0, W), None, w, tp, cap)             # no rows
    assert not comm.ar_norm_served(t(bf, tp, 4, W - 8), None, w, tp, cap)         # not the hidden width
    assert not comm.ar_norm_served(t(bf, tp - 1, 4, W), None, w, tp, cap)         # not every rank
    assert not comm.ar_norm_served(t(bf, 4, W), None, w, tp, cap)                 # one rank's rows only
    for dtype in (torch.float16, torch.float32):
        assert not comm.ar_norm_served(t(dtype, tp, 4, W), r, w, tp, cap)         # x
        assert not comm.ar_norm_served(x, r, t(dtype, W), tp, cap)                # the norm weight
        assert not comm.ar_norm_served(x, t(dtype, 4, W), w, tp, cap)             # the residual


def test_gather_gates():
    bf = torch.bfloat16
    for tp in (2, 4, 7, 8):
        assert comm.context_served(t(bf, tp, 3, W // tp), tp)
    assert not comm.context_served(t(bf, 8, 3, 1024), 8)             # shard width * TP != 7168
    assert not comm.context_served(t(torch.float16, 8, 3, 896), 8)   # not BF16
    assert not comm.context_served(t(bf, 7, 3, 896), 8)              # not every rank
    assert comm.logits_served(t(bf, 8, 4, 20480), 8, 20480)
    assert not comm.logits_served(t(bf, 8, 4, 20480), 8, None)       # no logits row built
    assert not comm.logits_served(t(bf, 8, 4, 20484), 8, 20484)      # vocab shard % 8 != 0: no row
    assert not comm.logits_served(t(bf, 8, 4, 20472), 8, 20480)      # not the vocab shard width
    assert not comm.logits_served(t(torch.float32, 8, 4, 20480), 8, 20480)
    assert comm.rows_served(t(bf, 8, 64, 896), 64)
    assert not comm.rows_served(t(bf, 8, 65, 896), 64)
    assert not comm.rows_served(t(bf, 8, 0, 896), 64)
    assert not comm.rows_served(t(bf, 8, 4, 1792)[:, :, ::2], 64)    # not contiguous
