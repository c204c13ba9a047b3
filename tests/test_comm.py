"""The DrafterComm-shaped front-end (tp_all_reduce_arnorm_amd.comm.StandInComm) on the
GPU: ar_norm, gather_context and gather_logits against the oracle on seeded inputs, and
None for every shape and dtype the pages' gates refuse (no launch, the mailboxes stay
armed)."""

import numpy as np
import pytest

import oracle
from tests.gpu_util import assert_bits_equal, assert_out_close, host16, host32, say
from tp_all_reduce_arnorm_amd import workloads as wl

pytestmark = pytest.mark.gpu
W = 7168
EPS = 1e-6


def bf16(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).cuda().view(torch.bfloat16)


def test_ar_norm_front_end(lib):
    import torch

    from tp_all_reduce_arnorm_amd.comm import StandInComm

    say("[comm] ar_norm front-end, TP=8, M=4 and 64")
    comm = StandInComm(8)
    box_h = oracle.arm(np.empty((2, 8, 64, W // 2), dtype=np.uint32))
    for call, (name, residual) in enumerate((("tp8_m4", False), ("tp8_m64", True), ("tp8_m4", True),
                                             ("tp8_m64", False))):
        import dataclasses

        cfg = dataclasses.replace(wl.CONFIGS[name], residual=residual, sigma_residual=1.0, seed=70 + call)
        src = wl.ArNormInputs(cfg)
        p, r = src.call()
        parity = call % 2
        got = comm.ar_norm(bf16(p), bf16(r) if residual else None, bf16(src.gamma), EPS, parity)
        assert got is not None
        out, res_out = got
        assert out.dtype == torch.bfloat16 and tuple(out.shape) == (cfg.m, W)
        oracle.arnorm_push(box_h, p, parity, 0)
        want_out, want_res = oracle.arnorm_reduce_norm(box_h, parity, cfg.m, r, src.gamma, EPS)
        assert_bits_equal(host16(res_out.view(torch.int16)), want_res, f"call {call} residual_out")
        assert_out_close(host16(out.view(torch.int16)), want_out, f"call {call} out")
    assert_bits_equal(host32(comm.ar), box_h, "mailbox")
    assert lib.status() == lib.OK


def test_ar_norm_front_end_not_served(lib):
    import torch

    from tp_all_reduce_arnorm_amd.comm import StandInComm

    say("[comm] ar_norm gates")
    comm = StandInComm(8, rows_cap=16)
    x = torch.zeros((8, 4, W), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(W, dtype=torch.bfloat16, device="cuda")
    assert comm.ar_norm(x.half(), None, w, EPS, 0) is None
    assert comm.ar_norm(x, None, w.float(), EPS, 0) is None
    assert comm.ar_norm(x, torch.zeros((4, W), dtype=torch.float16, device="cuda"), w, EPS, 0) is None
    assert comm.ar_norm(torch.zeros((8, 17, W), dtype=torch.bfloat16, device="cuda"), None, w, EPS, 0) is None
    assert comm.ar_norm(x[:7], None, w, EPS, 0) is None
    torch.cuda.synchronize()
    assert bool((comm.ar == -(1 << 31)).all()), "nothing was launched"
    assert comm.ar_norm(x, None, w, EPS, 0) is not None


@pytest.mark.parametrize("tp", [2, 4, 8])
def test_gather_context_front_end(lib, tp):
    import dataclasses

    from tp_all_reduce_arnorm_amd.comm import StandInComm

    say(f"[comm] gather_context TP={tp}")
    comm = StandInComm(tp)
    for m in (1, 64):
        cfg = dataclasses.replace(wl.CONFIGS["ctx"], tp=tp, m=m, s=W // 2 // tp, seed=80 + m)
        words = wl.bf16_shards(cfg)  # uint32 [tp, m, S] words of BF16 pairs
        halves = oracle.unpack_pairs(words)  # uint16 [tp, m, 7168 / tp]
        got = comm.gather_context(bf16(halves))
        assert got is not None and tuple(got.shape) == (m, W)
        gh = oracle.arm(np.empty((64, tp * cfg.s), dtype=np.uint32))
        oracle.gather_push(gh, words, 0)
        want = oracle.unpack_pairs(oracle.gather_poll(gh, m, True))
        import torch

        assert_bits_equal(host16(got.view(torch.int16)), want, f"context rows M={m}")
    assert comm.gather_context(bf16(np.zeros((tp, 65, W // tp), dtype=np.uint16))) is None  # above the cap
    assert comm.gather_context(bf16(np.zeros((tp, 4, W // tp + 8), dtype=np.uint16))) is None
    assert lib.status() == lib.OK


def test_gather_logits_front_end(lib):
    import dataclasses

    import torch

    from tp_all_reduce_arnorm_amd.comm import StandInComm

    say("[comm] gather_logits TP=8, V/TP = 20480")
    cfg = wl.CONFIGS["logits"]
    comm = StandInComm(8, vocab_shard=2 * cfg.s)
    for m in (1, 4):
        c = dataclasses.replace(cfg, m=m, seed=90 + m)
        words = wl.bf16_shards(c)
        got = comm.gather_logits(bf16(oracle.unpack_pairs(words)))
        assert got is not None and tuple(got.shape) == (m, 8 * 2 * cfg.s)
        gh = oracle.arm(np.empty((64, 8 * cfg.s), dtype=np.uint32))
        oracle.gather_push(gh, words, 0)
        assert_bits_equal(host16(got.view(torch.int16)), oracle.unpack_pairs(oracle.gather_poll(gh, m, True)),
                          f"logits M={m}")
    x = torch.zeros((8, 2, 2 * cfg.s), dtype=torch.bfloat16, device="cuda")
    assert comm.gather_logits(x.float()) is None
    assert comm.gather_logits(x[:, :, :-8].contiguous()) is None
    assert StandInComm(8).gather_logits(x) is None  # no logits row without a vocab shard
    assert StandInComm(8, vocab_shard=2 * cfg.s + 4).gather_logits(x) is None  # not a multiple of 8
    assert lib.status() == lib.OK
