"""Seeded random sweep of shapes, layouts and call forms on the GPU against the oracle.

Every case is drawn once, at import, from a fixed seed, so the collected cases are the
same on every run: TP, cap, M, parities, residual or not, the call form (push + consumer,
one call, the fused own push), the consumer layout (split rows, workgroup size), the
Gather poll layout, and the two-shot row width.  Each case makes a few calls over
alternating parities and compares every output and every mailbox with the oracle:
bit-exact, except the normed output within one BF16 ulp.
"""

import numpy as np
import pytest

import oracle
from tests.gpu_util import (S0, W, armed_box, assert_bits_equal, assert_out_close, dev16, dev32, empty16,
                            host16, host32, say)
from tests.test_parity import torture_partials

pytestmark = pytest.mark.gpu
EPS = 1e-6


def _draw_arnorm(rng, n):
    cases = []
    for i in range(n):
        tp = int(rng.integers(2, 9))
        cap = int(rng.integers(1, 49))
        c = dict(tp=tp, cap=cap, m=int(rng.integers(1, cap + 1)), parities=int(rng.integers(1, 4)),
                 residual=bool(rng.integers(0, 2)), torture=bool(rng.integers(0, 2)),
                 form=str(rng.choice(["pair", "one_call", "one_call_nobox", "fused"])),
                 split=int(rng.choice([0, 1, 7, 14])), threads=int(rng.choice([0, 448, 256])),
                 rank=int(rng.integers(0, tp)), seed=1000 + i)
        cases.append(c)
    return cases


def _draw_gather(rng, n):
    cases = []
    for i in range(n):
        cap = int(rng.integers(1, 80))
        cases.append(dict(tp=int(rng.integers(2, 9)), s=4 * int(rng.integers(1, 600)), cap=cap,
                          m=int(rng.integers(1, cap + 1)), form=str(rng.choice(["pair", "one_call"])),
                          copy=bool(rng.integers(0, 2)),
                          poll=[(0, 0), (1, 2), (4, 1), (4, 2), (1, 1)][int(rng.integers(0, 5))], seed=2000 + i))
    return cases


def _draw_twoshot(rng, n):
    cases = []
    for i in range(n):
        cap = int(rng.integers(1, 40))
        cases.append(dict(tp=int(rng.integers(2, 9)), width=8 * int(rng.integers(1, 1800)), cap=cap,
                          m=int(rng.integers(1, cap + 1)), parities=int(rng.integers(1, 4)),
                          form=str(rng.choice(["three", "one_call"])), seed=3000 + i))
    return cases


def _draw_arnorm_wide(rng, n):
    """Larger caps (up to 300 rows: the pair's 4-way split up to M=128 and its whole-row grid
    that loops over rows above 128; the one launch's 4-way rows up to M=256 and 2-way rows
    above), the splits of 4 and 8 ways, and the call with the library's own norm box
    (M <= 64)."""
    cases = []
    for i in range(n):
        tp = int(rng.integers(2, 9))
        cap = int(rng.integers(1, 301))
        m = int(rng.integers(1, cap + 1))
        form = str(rng.choice(["pair", "one_call", "fused", "static"]))
        if form == "static" and m > 64:
            form = "one_call"
        cases.append(dict(tp=tp, cap=cap, m=m, parities=int(rng.integers(1, 4)), residual=bool(rng.integers(0, 2)),
                          torture=bool(rng.integers(0, 2)), form=form, split=int(rng.choice([0, 1, 4, 8])),
                          threads=int(rng.choice([0, 448, 256])), rank=int(rng.integers(0, tp)), seed=4000 + i))
    return cases


_RNG = np.random.default_rng(20251202)
ARNORM_CASES = _draw_arnorm(_RNG, 64)
GATHER_CASES = _draw_gather(_RNG, 40)
TWOSHOT_CASES = _draw_twoshot(_RNG, 40)
ARNORM_WIDE_CASES = _draw_arnorm_wide(np.random.default_rng(20251203), 32)


def _case_id(c):
    return ",".join(f"{k}={v}" for k, v in c.items() if k != "seed")


@pytest.fixture(autouse=True)
def _defaults(lib):
    lib.set_reduce_threads(0)
    lib.set_reduce_split(0)
    lib.set_poll(0, 0)
    yield
    lib.set_reduce_threads(0)
    lib.set_reduce_split(0)
    lib.set_poll(0, 0)


def _bf16_rows(rng, shape):
    return (rng.standard_normal(shape, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("c", ARNORM_CASES, ids=_case_id)
def test_random_arnorm(lib, c):
    say(f"[random] arnorm {_case_id(c)}")
    _run_arnorm_case(lib, c)


@pytest.mark.parametrize("c", ARNORM_WIDE_CASES, ids=_case_id)
def test_random_arnorm_wide(lib, c):
    say(f"[random] arnorm wide {_case_id(c)}")
    _run_arnorm_case(lib, c)


def _run_arnorm_case(lib, c):
    rng = np.random.default_rng(c["seed"])
    tp, cap, m, parities = c["tp"], c["cap"], c["m"], c["parities"]
    lib.set_reduce_split(c["split"])
    lib.set_reduce_threads(c["threads"])
    shape = (parities, tp, cap, W // 2)
    box_d, box_h = armed_box(shape), oracle.arm(np.empty(shape, dtype=np.uint32))
    nbox = armed_box((parities, cap, 256))
    gamma = (np.float32(1) + np.float32(0.1) * rng.standard_normal(W, dtype=np.float32)).view(np.uint32)
    gamma = (gamma >> 16).astype(np.uint16)
    g_d = dev16(gamma)
    for call in range(3):
        parity = call % parities
        p = torture_partials(rng, tp, m) if c["torture"] else _bf16_rows(rng, (tp, m, W))
        res = _bf16_rows(rng, (m, W)) if c["residual"] else None
        res_d = dev16(res) if res is not None else None
        out_d, rout_d = empty16((m, W)), empty16((m, W))
        partial = None
        if c["form"] == "fused":
            k = c["rank"]
            others = [(0, k), (k + 1, tp - k - 1)]
            for rank, n in others:
                if n:
                    assert lib.arnorm_push(dev16(p[rank:rank + n]), box_d, parity, rank) is True
                    oracle.arnorm_push(box_h, p[rank:rank + n], parity, rank)
            partial = p[k]
            assert lib.arnorm_reduce_norm(res_d, g_d, box_d, parity, EPS, out_d, rout_d, partial=dev16(partial),
                                          rank=k, norm_box=nbox) is True
        elif c["form"] == "pair":
            assert lib.arnorm_push(dev16(p), box_d, parity, 0) is True
            oracle.arnorm_push(box_h, p, parity, 0)
            assert lib.arnorm_reduce_norm(res_d, g_d, box_d, parity, EPS, out_d, rout_d, norm_box=nbox) is True
        elif c["form"] == "static":
            assert lib.arnorm_push_reduce_norm_static(dev16(p), res_d, g_d, box_d, parity, EPS, out_d, rout_d) is True
            oracle.arnorm_push(box_h, p, parity, 0)
        else:
            box_arg = nbox if c["form"] == "one_call" else None
            assert lib.arnorm_push_reduce_norm(dev16(p), res_d, g_d, box_d, parity, EPS, out_d, rout_d,
                                               norm_box=box_arg) is True
            oracle.arnorm_push(box_h, p, parity, 0)
        want_out, want_res = oracle.arnorm_reduce_norm(box_h, parity, m, res, gamma, EPS, partial=partial,
                                                       rank=c["rank"] if partial is not None else 0)
        assert lib.status() == lib.OK
        assert_bits_equal(host16(rout_d), want_res, f"call {call} residual_out")
        exact_zero = (oracle.widen(want_res) == 0) | (oracle.widen(gamma) == 0)[None, :]
        assert_out_close(host16(out_d), want_out, f"call {call} out", exact_zero=exact_zero)
        assert_bits_equal(host32(box_d), box_h, f"call {call} mailbox")
        assert np.all(host32(nbox) == S0), "norm box left re-armed"


@pytest.mark.parametrize("c", GATHER_CASES, ids=_case_id)
def test_random_gather(lib, c):
    import torch

    say(f"[random] gather {_case_id(c)}")
    rng = np.random.default_rng(c["seed"])
    tp, s, cap, m = c["tp"], c["s"], c["cap"], c["m"]
    lib.set_poll(*c["poll"])
    gshape = (cap, tp * s)
    gbox_d, gbox_h = armed_box(gshape), oracle.arm(np.empty(gshape, dtype=np.uint32))
    for call in range(2):
        shards = rng.integers(0, 1 << 32, size=(tp, m, s), dtype=np.uint64).astype(np.uint32)
        shards[rng.random(size=shards.shape) < 0.03] = S0
        sh_d = dev32(shards)
        out_d = torch.empty((m, tp * s), dtype=torch.int32, device="cuda")
        copy = c["copy"]
        if c["form"] == "one_call":
            assert lib.gather_push_poll(sh_d, gbox_d, out=out_d if copy else None, copy=copy) is True
        else:
            assert lib.gather_push(sh_d, gbox_d, tp, 0) is True
            assert lib.gather_poll(gbox_d, tp, m, out=out_d if copy else None, copy=copy) is True
        oracle.gather_push(gbox_h, shards, 0)
        want = oracle.gather_poll(gbox_h, m, copy)
        if not copy:  # a later reader copies and re-arms
            assert lib.gather_poll(gbox_d, tp, m, out=out_d, copy=True) is True
            want = oracle.gather_poll(gbox_h, m, True)
        assert lib.status() == lib.OK
        assert_bits_equal(host32(out_d), want, f"call {call} gathered words")
        assert_bits_equal(host32(gbox_d), gbox_h, f"call {call} mailbox")


@pytest.mark.parametrize("c", TWOSHOT_CASES, ids=_case_id)
def test_random_twoshot(lib, c):
    say(f"[random] twoshot {_case_id(c)}")
    rng = np.random.default_rng(c["seed"])
    tp, width, cap, m, parities = c["tp"], c["width"], c["cap"], c["m"], c["parities"]
    rshape, gshape = (parities, tp, cap, width // 2), (parities, 1, cap, width // 2)
    recv_d, gath_d = armed_box(rshape), armed_box(gshape)
    recv_h, gath_h = oracle.arm(np.empty(rshape, dtype=np.uint32)), oracle.arm(np.empty(gshape, dtype=np.uint32))
    for call in range(3):
        parity = call % parities
        p = _bf16_rows(rng, (tp, m, width))
        p[:, :, 1::5] = 0x8000
        out_d = empty16((m, width))
        if c["form"] == "one_call":
            assert lib.twoshot_push_reduce_read(dev16(p), recv_d, gath_d, parity, out_d) is True
        else:
            assert lib.twoshot_push(dev16(p), recv_d, parity, 0) is True
            assert lib.twoshot_reduce(recv_d, gath_d, parity, m) is True
            assert lib.twoshot_read(gath_d, parity, out_d) is True
        oracle.twoshot_push(recv_h, p, parity, 0)
        want = oracle.twoshot_reduce(recv_h, gath_h, parity, m)
        assert_bits_equal(oracle.twoshot_read(gath_h, parity, m), want, "oracle read")
        assert lib.status() == lib.OK
        assert_bits_equal(host16(out_d), want, f"call {call} out")
        assert_bits_equal(host32(recv_d), recv_h, f"call {call} recv")
        assert_bits_equal(host32(gath_d), gath_h, f"call {call} gather row")
