"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle on the
same seeded inputs.  Bit-exact: residual_out (the all-reduced row when there is no
residual), every gathered word, and the mailbox after every call.  out: within one
BF16 ulp, with at most 1 % of its values off the oracle's bits.  Sizes: the five
workloads (tp2_m1..tp8_m4096, tp8_m4096 on sampled rows), plus edge cases."""

import numpy as np
import pytest

import oracle
from tests.gpu_util import (S0, W, armed_box, assert_bits_equal, assert_out_close, dev16, dev32, empty16,
                            host16, host32, say)
from tp_all_reduce_arnorm_amd import workloads as wl

pytestmark = pytest.mark.gpu
EPS = 1e-6


@pytest.fixture(autouse=True)
def _defaults(lib):
    lib.set_reduce_threads(0)
    lib.set_reduce_split(0)
    lib.set_poll(0, 0)
    yield
    lib.set_reduce_threads(0)
    lib.set_reduce_split(0)
    lib.set_poll(0, 0)


def norm_box_for(box_shape):
    """A sentinel-armed norm box [parities, cap, 256] for a mailbox of this shape."""
    return armed_box((box_shape[0], box_shape[2], 256))


def run_call(lib, box_d, box_h, partials, residual, gamma_d, gamma, parity, eps=EPS, pushes=None,
             fused_rank=None, norm_box=None):
    """One ArNorm call on both sides: pushes (list of (rank, nslots)), then the
    consumer; returns after comparing outputs and the whole mailbox."""
    tp = partials.shape[0]
    m = partials.shape[1]
    pushes = pushes or [(0, tp)]
    for rank, n in pushes:
        assert lib.arnorm_push(dev16(partials[rank:rank + n]), box_d, parity, rank) is True
        oracle.arnorm_push(box_h, partials[rank:rank + n], parity, rank)
    out_d, rout_d = empty16((m, W)), empty16((m, W))
    res_d = dev16(residual) if residual is not None else None
    part_d = dev16(partials[fused_rank]) if fused_rank is not None else None
    assert lib.arnorm_reduce_norm(res_d, gamma_d, box_d, parity, eps, out_d, rout_d, partial=part_d,
                                  rank=fused_rank or 0, norm_box=norm_box) is True
    want_out, want_res = oracle.arnorm_reduce_norm(
        box_h, parity, m, residual, gamma, eps,
        partial=partials[fused_rank] if fused_rank is not None else None, rank=fused_rank or 0)
    got_res = host16(rout_d)
    assert_bits_equal(got_res, want_res, "residual_out")
    exact_zero = (oracle.widen(want_res) == 0) | (oracle.widen(gamma) == 0)[None, :]
    assert_out_close(host16(out_d), want_out, exact_zero=exact_zero)
    assert_bits_equal(host32(box_d), box_h, "mailbox")
    if norm_box is not None:
        assert np.all(host32(norm_box) == S0), "the norm box is left re-armed"
    assert lib.status() == lib.OK
    return got_res


def run_config(lib, name, calls=None, threads=0, split=None):
    """split None: no norm box (one workgroup per row); else a norm box with
    arnorm_set_reduce_split(split)."""
    cfg = wl.CONFIGS[name]
    say(f"[parity] {name} threads={threads} split={split}")
    lib.set_reduce_threads(threads)
    src = wl.ArNormInputs(cfg)
    shape = (cfg.parities, cfg.tp, cfg.cap, W // 2)
    box_d = armed_box(shape)
    box_h = oracle.arm(np.empty(shape, dtype=np.uint32))
    nbox = None
    if split is not None:
        lib.set_reduce_split(split)
        nbox = norm_box_for(shape)
    gamma_d = dev16(src.gamma)
    for call in range(calls or cfg.calls):
        p, r = src.call()
        run_call(lib, box_d, box_h, p, r, gamma_d, src.gamma, call % cfg.parities, norm_box=nbox)


def test_tp2_m1(lib):
    run_config(lib, "tp2_m1")


def test_tp8_m4(lib):
    run_config(lib, "tp8_m4")


def test_tp8_m64(lib):
    run_config(lib, "tp8_m64")


@pytest.mark.parametrize("threads", [448, 256])
def test_tp8_m64_other_workgroup_sizes(lib, threads):
    run_config(lib, "tp8_m64", calls=4, threads=threads)


@pytest.mark.parametrize("split", [0, 4, 7, 8, 14])
@pytest.mark.parametrize("name", ["tp2_m1", "tp8_m4", "tp8_m64"])
def test_split_rows(lib, name, split):
    """Rows split over 4, 7, 8 or 14 workgroups (and the automatic choice; 4 and 8 leave
    lanes of each workgroup idle), the row's sum of squares exchanged through the norm
    box, which every call leaves re-armed."""
    run_config(lib, name, calls=min(wl.CONFIGS[name].calls, 12), split=split)


@pytest.mark.parametrize("name,with_box,split", [("tp2_m1", True, 0), ("tp8_m4", True, 0), ("tp8_m64", True, 0), ("tp8_m4", False, 0),
                                                ("tp2_m1", True, 14), ("tp8_m4", True, 14), ("tp8_m4", True, 4),
                                                ("tp8_m4", True, 8), ("tp8_m64", True, 4), ("tp8_m64", True, 8)])
def test_push_reduce_norm_one_call(lib, name, with_box, split):
    """arnorm_push_reduce_norm (with a norm box one launch, rows split the automatic 7 or 4
    ways or the forced 4, 8 or 14; without one the pair of launches) against the oracle's
    push of every slot followed by its consumer."""
    cfg = wl.CONFIGS[name]
    say(f"[parity] push_reduce_norm {name} norm_box={with_box} split={split}")
    lib.set_reduce_split(split)
    src = wl.ArNormInputs(cfg)
    shape = (cfg.parities, cfg.tp, cfg.cap, W // 2)
    box_d, box_h = armed_box(shape), oracle.arm(np.empty(shape, dtype=np.uint32))
    nbox = norm_box_for(shape) if with_box else None
    g_d = dev16(src.gamma)
    for call in range(min(cfg.calls, 12)):
        parity = call % cfg.parities
        p, r = src.call()
        out_d, rout_d = empty16((cfg.m, W)), empty16((cfg.m, W))
        assert lib.arnorm_push_reduce_norm(dev16(p), dev16(r) if r is not None else None, g_d, box_d, parity, EPS,
                                           out_d, rout_d, norm_box=nbox) is True
        oracle.arnorm_push(box_h, p, parity, 0)
        want_out, want_res = oracle.arnorm_reduce_norm(box_h, parity, cfg.m, r, src.gamma, EPS)
        assert_bits_equal(host16(rout_d), want_res, f"call {call} residual_out")
        exact_zero = (oracle.widen(want_res) == 0) | (oracle.widen(src.gamma) == 0)[None, :]
        assert_out_close(host16(out_d), want_out, f"call {call} out", exact_zero=exact_zero)
        assert_bits_equal(host32(box_d), box_h, f"call {call} mailbox")
        if nbox is not None:
            assert np.all(host32(nbox) == S0)
        assert lib.status() == lib.OK


@pytest.mark.parametrize("tp,split,m", [(2, 0, 13), (3, 0, 13), (8, 0, 13), (3, 14, 13), (8, 14, 13), (5, 4, 13),
                                        (8, 8, 13), (8, 0, 3), (8, 0, 4), (8, 0, 5), (8, 0, 9), (4, 0, 7),
                                        (8, 0, 14), (8, 0, 31), (8, 0, 32), (8, 0, 33), (8, 0, 34), (8, 0, 64),
                                        (8, 0, 65), (8, 0, 128), (8, 0, 129), (8, 0, 256), (8, 0, 257),
                                        (8, 0, 512), (8, 0, 513), (8, 0, 562), (8, 0, 563), (5, 0, 129),
                                        (4, 0, 200), (4, 0, 257), (4, 0, 936), (4, 0, 937), (6, 0, 704),
                                        (6, 0, 705), (2, 0, 300), (2, 0, 1024), (2, 0, 1025)])
def test_push_reduce_norm_torture(lib, tp, split, m):
    """Torture rows through arnorm_push_reduce_norm.  With the automatic split at TP=8 the
    one launch (a row's workgroups on one XCD, in blocks of 8 rows) takes 7 parts at M=3
    (one short block), 4, 5, 9 (a full block and one row), 13, 14 and 31 (an odd producer
    count per slot, rounded up to even: the extra producer has no fragments) and 32, and 4
    parts at M=33, 34, 64, 65, 128, 129 and 256 (from about M=100 the grid is larger than
    what the GPU holds at once), and 2 parts at M=257, 512, 513 (past the split grid's cap
    of 1024 workgroups) and 562 (the last row count whose grid, 10 M workgroups, fits the
    one launch's 5632); forced splits of 4, 8 and 14 ways run at M=13; at M=563 the pair of
    launches runs, one workgroup per row.  Below TP=8: 4 parts at TP=5 M=129 and TP=4 M=200,
    2 parts at TP=4 M=257 and 936, TP=6 M=704 and TP=2 M=300 and 1024, all one launch, and
    the pair at TP=4 M=937, TP=6 M=705 (one row past the grid limit) and TP=2
    M=1025 (past the one launch's 1024 rows)."""
    say(f"[parity] push_reduce_norm torture tp={tp} split={split} m={m}")
    lib.set_reduce_split(split)
    rng = np.random.default_rng(170 + tp + 32 * m)
    cap = max(17, m)
    shape = (2, tp, cap, W // 2)
    box_d, box_h, nbox = armed_box(shape), oracle.arm(np.empty(shape, dtype=np.uint32)), norm_box_for(shape)
    gamma = (rng.integers(0, 2, W) << 15 | (rng.integers(120, 132, W) << 7) | rng.integers(0, 128, W)).astype(np.uint16)
    for call in range(3):
        parity = call % 2
        p = torture_partials(rng, tp, m)
        res = torture_partials(rng, 1, m)[0] if call % 2 else None
        out_d, rout_d = empty16((m, W)), empty16((m, W))
        assert lib.arnorm_push_reduce_norm(dev16(p), dev16(res) if res is not None else None, dev16(gamma), box_d,
                                           parity, EPS, out_d, rout_d, norm_box=nbox) is True
        oracle.arnorm_push(box_h, p, parity, 0)
        want_out, want_res = oracle.arnorm_reduce_norm(box_h, parity, m, res, gamma, EPS)
        assert_bits_equal(host16(rout_d), want_res, "residual_out")
        exact_zero = (oracle.widen(want_res) == 0) | (oracle.widen(gamma) == 0)[None, :]
        assert_out_close(host16(out_d), want_out, exact_zero=exact_zero)
        assert_bits_equal(host32(box_d), box_h, "mailbox")
        assert lib.status() == lib.OK


def test_tp8_m64_per_rank_pushes_and_chained_residual(lib):
    """Ranks push one by one (and in groups), and each call's residual is the previous
    call's residual_out, as consecutive layers use it."""
    cfg = wl.CONFIGS["tp8_m64"]
    say("[parity] tp8_m64 per-rank pushes, chained residual")
    src = wl.ArNormInputs(cfg)
    shape = (2, 8, 64, W // 2)
    box_d, box_h = armed_box(shape), oracle.arm(np.empty(shape, dtype=np.uint32))
    gamma_d = dev16(src.gamma)
    residual = src.residual()
    groupings = [[(k, 1) for k in range(8)], [(0, 3), (3, 5)], [(7, 1), (0, 7)], [(4, 4), (0, 4)]]
    for call in range(8):
        p = src.partials()
        residual = run_call(lib, box_d, box_h, p, residual, gamma_d, src.gamma, call % 2,
                            pushes=groupings[call % len(groupings)])


def test_gather_tp8_m32(lib):
    cfg = wl.CONFIGS["gather_tp8_m32"]
    say("[parity] gather_tp8_m32 copy / no-copy")
    shards = wl.gather_shards(cfg)
    gshape = (cfg.cap, cfg.tp * cfg.s)
    gbox_d = armed_box(gshape)
    gbox_h = oracle.arm(np.empty(gshape, dtype=np.uint32))
    import torch

    for round_ in range(3):
        # ranks push one by one (round 0), all at once (1), in two groups (2)
        groups = [[(k, 1) for k in range(8)], [(0, 8)], [(0, 5), (5, 3)]][round_]
        for rank, n in groups:
            assert lib.gather_push(dev32(shards[rank:rank + n]), gbox_d, cfg.tp, rank) is True
            oracle.gather_push(gbox_h, shards[rank:rank + n], rank)
        assert_bits_equal(host32(gbox_d), gbox_h, "gather mailbox after push")
        if round_ == 1:
            # no copy: rows stay published for a later reader, which copies and re-arms
            assert lib.gather_poll(gbox_d, cfg.tp, cfg.m, copy=False) is True
            assert oracle.gather_poll(gbox_h, cfg.m, False) is None
            assert_bits_equal(host32(gbox_d), gbox_h, "gather mailbox after no-copy poll")
        out_d = torch.empty((cfg.m, cfg.tp * cfg.s), dtype=torch.int32, device="cuda")
        assert lib.gather_poll(gbox_d, cfg.tp, cfg.m, out=out_d, copy=True) is True
        want = oracle.gather_poll(gbox_h, cfg.m, True)
        assert_bits_equal(host32(out_d), want, "gathered words")
        assert_bits_equal(host32(gbox_d), gbox_h, "gather mailbox after copy")
        assert lib.status() == lib.OK
        # the words moved are the shards with only the sentinel pair changed
        for r in range(cfg.tp):
            blk = want[:, r * cfg.s:(r + 1) * cfg.s]
            src = shards[r]
            assert np.array_equal(blk[src != S0], src[src != S0]) and np.all(blk[src == S0] == 0)


@pytest.mark.parametrize("name,m,tp", [("ctx", 64, 8), ("ctx", 1, 8), ("ctx", 7, 4), ("ctx", 3, 2),
                                        ("logits", 4, 8), ("logits", 1, 8)])
def test_drafter_gather_shapes(lib, name, m, tp):
    """The drafter's own gathers: the context projection's [M, 7168/TP] BF16 rows and
    the lm_head's [M, V/TP] logits, moved as 32-bit words of BF16 pairs; bit-exact."""
    import dataclasses

    import torch

    say(f"[parity] drafter gather {name} M={m} TP={tp}")
    base = wl.CONFIGS[name]
    s = base.s * base.tp // tp  # same row width at another TP
    cfg = dataclasses.replace(base, m=m, tp=tp, s=s)
    shards = wl.bf16_shards(cfg)
    gshape = (cfg.cap, cfg.tp * cfg.s)
    gbox_d, gbox_h = armed_box(gshape), oracle.arm(np.empty(gshape, dtype=np.uint32))
    for rank in range(tp):
        assert lib.gather_push(dev32(shards[rank:rank + 1]), gbox_d, tp, rank) is True
        oracle.gather_push(gbox_h, shards[rank:rank + 1], rank)
    out_d = torch.empty((m, tp * s), dtype=torch.int32, device="cuda")
    assert lib.gather_poll(gbox_d, tp, m, out=out_d, copy=True) is True
    want = oracle.gather_poll(gbox_h, m, True)
    assert lib.status() == lib.OK
    assert_bits_equal(host32(out_d), want, "gathered words")
    assert_bits_equal(host32(gbox_d), gbox_h, "gather mailbox")
    # as BF16: the gathered row is the shards side by side, only (+0, -0) pairs made (+0, +0)
    row = oracle.unpack_pairs(want)
    for r in range(tp):
        src = oracle.unpack_pairs(shards[r])
        blk = row[:, r * 2 * s:(r + 1) * 2 * s]
        sent = (src[:, 0::2] == 0) & (src[:, 1::2] == 0x8000)
        assert np.array_equal(blk[:, 1::2][~sent], src[:, 1::2][~sent]) and np.all(blk[:, 1::2][sent] == 0)


@pytest.mark.parametrize("name,m", [("gather_tp8_m32", 32), ("gather_tp8_m32", 16), ("gather_tp8_m32", 1),
                                    ("gather_tp8_m32", 54), ("gather_tp8_m32", 64), ("ctx", 64), ("logits", 4),
                                    ("logits", 25), ("logits", 26), ("logits", 102), ("logits", 103),
                                    ("logits", 2), ("logits", 1)])
def test_gather_push_poll_one_call(lib, name, m):
    """gather_push_poll (one launch for calls within 32 MiB, else the pair; the logits rows,
    S=10240, fit 102 rows in it, not 103; its poll delay steps at 2, 4 and 8 MiB, which
    logits M=25 and 26 straddle) against the oracle's push of every rank followed by its
    poll: copy, then no-copy followed by a copying poll."""
    import dataclasses

    import torch

    say(f"[parity] gather_push_poll {name} M={m}")
    cfg = dataclasses.replace(wl.CONFIGS[name], m=m)
    cfg = dataclasses.replace(cfg, cap=max(cfg.cap, m))
    shards = wl.gather_shards(cfg) if name == "gather_tp8_m32" else wl.bf16_shards(cfg)
    gshape = (cfg.cap, cfg.tp * cfg.s)
    gbox_d, gbox_h = armed_box(gshape), oracle.arm(np.empty(gshape, dtype=np.uint32))
    sh_d = dev32(shards)
    for copy in (True, False):
        out_d = torch.empty((m, cfg.tp * cfg.s), dtype=torch.int32, device="cuda")
        assert lib.gather_push_poll(sh_d, gbox_d, out=out_d, copy=copy) is True
        oracle.gather_push(gbox_h, shards, 0)
        want = oracle.gather_poll(gbox_h, m, copy)
        if copy:
            assert_bits_equal(host32(out_d), want, "gathered words")
        assert_bits_equal(host32(gbox_d), gbox_h, f"gather mailbox (copy={copy})")
        assert lib.status() == lib.OK
    out_d = torch.empty((m, cfg.tp * cfg.s), dtype=torch.int32, device="cuda")
    assert lib.gather_poll(gbox_d, cfg.tp, m, out=out_d, copy=True) is True  # the later reader
    assert_bits_equal(host32(out_d), oracle.gather_poll(gbox_h, m, True), "later reader")
    assert_bits_equal(host32(gbox_d), gbox_h, "gather mailbox re-armed")


@pytest.mark.parametrize("u,mode", [(1, 2), (4, 1), (4, 2)])
@pytest.mark.parametrize("name,m", [("gather_tp8_m32", 54), ("gather_tp8_m32", 16), ("gather_tp8_m32", 1), ("ctx", 64),
                                    ("logits", 4), ("logits", 1)])
def test_gather_poll_layouts_one_launch(lib, name, m, u, mode):
    """gather_push_poll in one launch, its pollers forced to 1 or 4 fragments per thread and
    to re-read or witness waits: the producers in the same grid are still writing when
    the pollers start, so every wait path runs; out and mailbox bit-exact."""
    import dataclasses

    import torch

    say(f"[parity] gather one launch {name} M={m} frags/thread={u} mode={mode}")
    lib.set_poll(u, mode)
    cfg = dataclasses.replace(wl.CONFIGS[name], m=m)
    shards = wl.gather_shards(cfg) if name == "gather_tp8_m32" else wl.bf16_shards(cfg)
    gshape = (cfg.cap, cfg.tp * cfg.s)
    gbox_d, gbox_h = armed_box(gshape), oracle.arm(np.empty(gshape, dtype=np.uint32))
    sh_d = dev32(shards)
    for _ in range(3):
        out_d = torch.empty((m, cfg.tp * cfg.s), dtype=torch.int32, device="cuda")
        assert lib.gather_push_poll(sh_d, gbox_d, out=out_d, copy=True) is True
        oracle.gather_push(gbox_h, shards, 0)
        assert_bits_equal(host32(out_d), oracle.gather_poll(gbox_h, m, True), "gathered words")
        assert_bits_equal(host32(gbox_d), gbox_h, "gather mailbox")
        assert lib.status() == lib.OK


@pytest.mark.parametrize("tp,m,s", [(8, 4096, 896), (2, 4096, 4), (4, 1024, 10240), (2, 70000, 4)])
def test_gather_large(lib, tp, m, s):
    """Large gathers with M = cap: up to 168 MB of shards as the pair of launches, at S=4
    one launch over 4096 rows of 2 ranks, and M = 70000 rows (more than a grid's second
    dimension holds); through gather_push_poll with copy, then no copy followed by a
    copying gather_poll; every word and the whole mailbox compared with the oracle."""
    import dataclasses

    import torch

    say(f"[parity] gather large tp={tp} M={m} S={s}")
    cfg = dataclasses.replace(wl.CONFIGS["gather_tp8_m32"], tp=tp, m=m, s=s, cap=m, seed=40 + tp)
    shards = wl.gather_shards(cfg)
    gshape = (cfg.cap, tp * s)
    gbox_d, gbox_h = armed_box(gshape), oracle.arm(np.empty(gshape, dtype=np.uint32))
    sh_d = dev32(shards)
    out_d = torch.empty((m, tp * s), dtype=torch.int32, device="cuda")
    assert lib.gather_push_poll(sh_d, gbox_d, out=out_d, copy=True) is True
    oracle.gather_push(gbox_h, shards, 0)
    assert_bits_equal(host32(out_d), oracle.gather_poll(gbox_h, m, True), "gathered words")
    assert_bits_equal(host32(gbox_d), gbox_h, "mailbox re-armed")
    assert lib.gather_push_poll(sh_d, gbox_d, copy=False) is True
    oracle.gather_push(gbox_h, shards, 0)
    assert oracle.gather_poll(gbox_h, m, False) is None
    assert_bits_equal(host32(gbox_d), gbox_h, "mailbox left published")
    out_d.fill_(0x1234)
    assert lib.gather_poll(gbox_d, tp, m, out=out_d, copy=True) is True
    assert_bits_equal(host32(out_d), oracle.gather_poll(gbox_h, m, True), "later reader")
    assert_bits_equal(host32(gbox_d), gbox_h, "mailbox re-armed by the later reader")
    assert lib.status() == lib.OK


def test_tp8_m4096_full_size_every_row(lib):
    """M = 4096, TP = 8, in the launch configuration the benchmark times: every row of
    residual_out bit for bit and of out within the contract, against the oracle's push and
    reduce_norm run in blocks of 512 rows (rows are independent), and the whole mailbox
    re-armed."""
    import torch

    cfg = wl.CONFIGS["tp8_m4096"]
    say("[parity] tp8_m4096 full size, every row")
    src = wl.ArNormInputs(cfg)
    p, r = src.call()
    shape = (1, 8, cfg.cap, W // 2)
    box_d = armed_box(shape)
    p_d, r_d, g_d = dev16(p), dev16(r), dev16(src.gamma)
    out_d, rout_d = empty16((cfg.m, W)), empty16((cfg.m, W))
    assert lib.arnorm_push(p_d, box_d, 0, 0) is True
    assert lib.arnorm_reduce_norm(r_d, g_d, box_d, 0, EPS, out_d, rout_d) is True
    assert lib.status() == lib.OK
    assert bool((box_d == torch.tensor(-(1 << 31), dtype=torch.int32, device="cuda")).all())
    del box_d, p_d, r_d
    got_out, got_res = host16(out_d), host16(rout_d)
    blk = 512
    for r0 in range(0, cfg.m, blk):
        rows = slice(r0, r0 + blk)
        box_h = oracle.arm(np.empty((1, 8, blk, W // 2), dtype=np.uint32))
        oracle.arnorm_push(box_h, p[:, rows], 0, 0)
        want_out, want_res = oracle.arnorm_reduce_norm(box_h, 0, blk, r[rows], src.gamma, EPS)
        assert_bits_equal(got_res[rows], want_res, f"residual_out rows {r0}..{r0 + blk - 1}")
        assert_out_close(got_out[rows], want_out, f"out rows {r0}..{r0 + blk - 1}")


def test_max_rows_2gib_slot_block(lib):
    """The largest M served at TP=8: 149,796 rows, a slot block of 2,147,475,456 bytes, just
    under the 2 GiB a buffer resource spans (17 GB of mailbox).  Inputs are drawn on the
    device (seeded); the whole mailbox must be re-armed, and sampled rows, the first and
    last included, must match the oracle."""
    import torch

    tp, m = 8, (2**31 - 1) // (W * 2)
    assert m * W * 2 < 2**31 <= (m + 1) * W * 2
    free, _ = torch.cuda.mem_get_info()
    if free < 64 * 2**30:
        pytest.skip("needs about 45 GB of free device memory")
    say(f"[parity] max rows M={m}")
    gen = torch.Generator(device="cuda").manual_seed(2024)
    parts = torch.empty((tp, m, W), dtype=torch.bfloat16, device="cuda")
    for s in range(tp):
        parts[s] = torch.randn((m, W), generator=gen, device="cuda").to(torch.bfloat16)
    resid = torch.randn((m, W), generator=gen, device="cuda").to(torch.bfloat16)
    gamma = (1 + 0.1 * torch.randn(W, generator=gen, device="cuda")).to(torch.bfloat16)
    box_d = armed_box((1, tp, m, W // 2))
    out_d, rout_d = empty16((m, W)), empty16((m, W))
    assert lib.arnorm_push(parts, box_d, 0, 0) is True
    assert lib.arnorm_reduce_norm(resid, gamma, box_d, 0, EPS, out_d, rout_d) is True
    assert lib.status() == lib.OK
    assert bool((box_d == torch.tensor(-(1 << 31), dtype=torch.int32, device="cuda")).all())
    rng = np.random.default_rng(123)
    rows = np.unique(np.concatenate([[0, 1, m // 2, m - 2, m - 1], rng.choice(m, 59, replace=False)]))
    idx = torch.from_numpy(rows).cuda()
    p = host16(parts.view(torch.int16).index_select(1, idx))
    r = host16(resid.view(torch.int16).index_select(0, idx))
    g = host16(gamma.view(torch.int16))
    del parts, resid
    box_h = oracle.arm(np.empty((1, tp, len(rows), W // 2), dtype=np.uint32))
    oracle.arnorm_push(box_h, p, 0, 0)
    want_out, want_res = oracle.arnorm_reduce_norm(box_h, 0, len(rows), r, g, EPS)
    assert_bits_equal(host16(rout_d.index_select(0, idx)), want_res, "residual_out (sampled rows)")
    assert_out_close(host16(out_d.index_select(0, idx)), want_out, "out (sampled rows)")


def test_gather_max_row(lib):
    """The widest Gather row served at TP=8: S = 67,108,860 words per rank, a gathered row
    of 2,147,483,520 bytes, just under the 2 GiB a buffer resource spans.  Shards are
    drawn on the device (seeded, 3 % sentinel words); a no-copy poll, then a copying one.
    The mailbox must end re-armed, every gathered word must equal its shard word cleaned,
    and 4096 sampled columns of every rank (the first and last included) must match the
    oracle's gather."""
    import torch

    tp = 8
    s = ((2**31 - 1) // (tp * 4)) // 4 * 4
    assert tp * s * 4 < 2**31 <= tp * (s + 4) * 4
    free, _ = torch.cuda.mem_get_info()
    if free < 24 * 2**30:
        pytest.skip("needs about 12 GB of free device memory")
    say(f"[parity] gather max row S={s}")
    gen = torch.Generator(device="cuda").manual_seed(2025)
    sent = torch.tensor(-(1 << 31), dtype=torch.int32, device="cuda")
    shards = torch.randint(-(1 << 31), 1 << 31, (tp, 1, s), generator=gen, dtype=torch.int64, device="cuda")
    shards = shards.to(torch.int32)
    shards[torch.rand((tp, 1, s), generator=gen, device="cuda") < 0.03] = sent
    box = armed_box((1, tp * s))
    out = torch.empty((1, tp * s), dtype=torch.int32, device="cuda")
    assert lib.gather_push(shards, box, tp, 0) is True
    assert lib.gather_poll(box, tp, 1, copy=False) is True
    assert lib.gather_poll(box, tp, 1, out=out, copy=True) is True
    assert lib.status() == lib.OK
    assert bool((box == sent).all()), "mailbox not re-armed"
    zero = torch.zeros((), dtype=torch.int32, device="cuda")
    assert bool((out.view(tp, s) == torch.where(shards.view(tp, s) == sent, zero, shards.view(tp, s))).all())
    rng = np.random.default_rng(7)
    cols = np.sort(np.concatenate([[0, 1, s - 2, s - 1], 2 + rng.choice(s - 4, 4092, replace=False)]))
    idx = torch.from_numpy(cols).cuda()
    sh = host32(shards.index_select(2, idx))
    got = host32(out.view(tp, s).index_select(1, idx)).reshape(1, tp * len(cols))
    del shards, out, box
    gbox = oracle.arm(np.empty((1, tp * len(cols)), dtype=np.uint32))
    oracle.gather_push(gbox, sh, 0)
    assert_bits_equal(got, oracle.gather_poll(gbox, 1, True), "gathered words (sampled columns)")


def test_gather_range_beyond_4gib(lib):
    """A Gather whose rows < M span more than the 4 GiB a buffer resource can address: TP=2,
    the widest row (S = 268,435,452 words per rank, 2,147,483,616 bytes) and M=3, so the
    poll's flat range is 6.4 GB and every block of it gets a resource of its own.  Shards are
    drawn on the device (seeded, 3 % sentinel words); a no-copy poll, then a copying one.
    The mailbox must end re-armed, every gathered word must equal its shard word cleaned,
    and sampled columns of every row and rank must match the oracle's gather."""
    import torch

    tp, m = 2, 3
    s = ((2**31 - 1) // (tp * 4)) // 4 * 4
    assert tp * s * 4 < 2**31 and m * tp * s * 4 > 2**32
    free, _ = torch.cuda.mem_get_info()
    if free < 48 * 2**30:
        pytest.skip("needs about 32 GB of free device memory")
    say(f"[parity] gather range beyond 4 GiB: TP={tp}, M={m}, S={s}")
    gen = torch.Generator(device="cuda").manual_seed(2026)
    sent = torch.tensor(-(1 << 31), dtype=torch.int32, device="cuda")
    shards = torch.empty((tp, m, s), dtype=torch.int32, device="cuda")
    for r in range(tp):
        for row in range(m):
            x = torch.randint(-(1 << 31), (1 << 31) - 1, (s,), generator=gen, dtype=torch.int32, device="cuda")
            x[torch.rand(s, generator=gen, device="cuda") < 0.03] = sent
            shards[r, row] = x
            del x
    box = armed_box((m, tp * s))
    out = torch.empty((m, tp * s), dtype=torch.int32, device="cuda")
    assert lib.gather_push(shards, box, tp, 0) is True
    assert lib.gather_poll(box, tp, m, copy=False) is True
    assert lib.gather_poll(box, tp, m, out=out, copy=True) is True
    assert lib.status() == lib.OK
    for row in range(m):
        assert bool((box[row] == sent).all()), f"row {row} of the mailbox not re-armed"
        for r in range(tp):
            sh = shards[r, row]
            assert bool((out[row, r * s:(r + 1) * s] == torch.where(sh == sent, torch.zeros_like(sh), sh)).all()), \
                f"row {row}, rank {r}"
    rng = np.random.default_rng(8)
    cols = np.sort(np.concatenate([[0, 1, s - 2, s - 1], 2 + rng.choice(s - 4, 2044, replace=False)]))
    idx = torch.from_numpy(cols).cuda()
    sh = host32(shards.index_select(2, idx))
    got = host32(out.view(m, tp, s).index_select(2, idx)).reshape(m, tp * len(cols))
    del shards, out, box
    gbox = oracle.arm(np.empty((m, tp * len(cols)), dtype=np.uint32))
    oracle.gather_push(gbox, sh, 0)
    assert_bits_equal(got, oracle.gather_poll(gbox, m, True), "gathered words (sampled columns)")


# -- edge cases ------------------------------------------------------------------


def torture_partials(rng, tp, m):
    """Rows built to hit the rounding and sign corner cases: ties to even, carries into
    the next binade, cancellation to +-0, BF16 subnormals, overflow to inf, the
    sentinel pair and other -0 words."""
    p = np.zeros((tp, m, W), dtype=np.uint16)
    for r in range(m):
        kind = r % 6
        if kind == 0:  # random patterns over a wide exponent range
            e = rng.integers(-20, 20, size=(tp, W)) + 127
            p[:, r] = ((rng.integers(0, 2, (tp, W)) << 15) | (e << 7) | rng.integers(0, 128, (tp, W))).astype(np.uint16)
        elif kind == 1:  # subnormals and signed zeros
            p[:, r] = ((rng.integers(0, 2, (tp, W)) << 15) | rng.integers(0, 128, (tp, W))).astype(np.uint16)
        elif kind == 2:  # near-overflow values: sums overflow to +-inf
            p[:, r] = ((rng.integers(0, 2, (tp, W)) << 15) | (254 << 7) | rng.integers(100, 128, (tp, W))).astype(np.uint16)
        elif kind == 3:  # exact cancellation: slot 1 = -slot 0, the rest -0
            x = rng.integers(0, 1 << 15, W).astype(np.uint16) & np.uint16(0x7F7F)
            p[0, r] = x
            if tp > 1:
                p[1, r] = x ^ np.uint16(0x8000)
            p[2:, r] = 0x8000
        elif kind == 4:  # ties: 1.0 + k * 2^-8 style values per column
            p[0, r] = 0x3F80
            if tp > 1:
                p[1, r] = rng.choice([0x3B80, 0x3C40, 0x3BC0, 0x3C00], W)
            if tp > 2:
                p[2:, r] = rng.choice([0x0000, 0x8000, 0x3300], (tp - 2, W))
        else:  # the sentinel pair everywhere in some slots, -0 words in others
            p[:, r] = rng.integers(0, 1 << 16, (tp, W)).astype(np.uint16) & np.uint16(0xBF7F)
            p[: tp // 2, r, 0::2] = 0x0000
            p[: tp // 2, r, 1::2] = 0x8000
            p[tp // 2:, r, 0::4] = 0x8000
    return p


@pytest.mark.parametrize("tp", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("residual", [False, True])
def test_all_tp_torture_rows(lib, tp, residual):
    say(f"[parity] torture tp={tp} residual={residual}")
    rng = np.random.default_rng(100 + tp)
    m, cap = 13, 17  # ragged: rows 13..16 of the cap stay untouched
    shape = (2, tp, cap, W // 2)
    box_d, box_h = armed_box(shape), oracle.arm(np.empty(shape, dtype=np.uint32))
    gamma = (rng.integers(0, 2, W) << 15 | (rng.integers(120, 132, W) << 7) | rng.integers(0, 128, W)).astype(np.uint16)
    g_d = dev16(gamma)
    # leave the other parity published and unread: it must survive untouched
    other = torture_partials(rng, tp, m)
    assert lib.arnorm_push(dev16(other), box_d, 1, 0) is True
    oracle.arnorm_push(box_h, other, 1, 0)
    for call in range(2):
        p = torture_partials(rng, tp, m)
        res = torture_partials(rng, 1, m)[0] if residual else None
        run_call(lib, box_d, box_h, p, res, g_d, gamma, 0)


@pytest.mark.parametrize("tp", [2, 5, 8])
def test_torture_rows_split(lib, tp):
    say(f"[parity] torture tp={tp} split=14")
    lib.set_reduce_split(14)
    rng = np.random.default_rng(150 + tp)
    m, cap = 13, 17
    shape = (2, tp, cap, W // 2)
    box_d, box_h, nbox = armed_box(shape), oracle.arm(np.empty(shape, dtype=np.uint32)), norm_box_for(shape)
    gamma = (rng.integers(0, 2, W) << 15 | (rng.integers(120, 132, W) << 7) | rng.integers(0, 128, W)).astype(np.uint16)
    g_d = dev16(gamma)
    for call in range(3):
        p = torture_partials(rng, tp, m)
        res = torture_partials(rng, 1, m)[0] if call % 2 else None
        run_call(lib, box_d, box_h, p, res, g_d, gamma, call % 2, norm_box=nbox)


@pytest.mark.parametrize("threads", [896, 448, 256])
def test_norm_closed_form_rows(lib, threads):
    """All-zero row, one-hot row, constant row, an eps-dominated row and a row whose
    residual cancels the all-reduced value; tp=4, M=5."""
    say(f"[parity] closed-form rows threads={threads}")
    lib.set_reduce_threads(threads)
    tp, m = 4, 5
    p = np.zeros((tp, m, W), dtype=np.uint16)
    p[:, 0] = 0x0000                      # zero row
    p[0, 1, 123] = 0x3F80                 # one-hot 1.0
    p[:, 2] = 0x3E80                      # 4 x 0.25 = 1.0 everywhere
    p[0, 3] = 0x3A80                      # 2^-10 everywhere: mean ~ eps
    p[:, 4] = 0x3F80                      # 4.0, cancelled by residual -4.0
    res = np.zeros((m, W), dtype=np.uint16)
    res[4] = 0xC080
    gamma = np.full(W, 0x3F80, dtype=np.uint16)
    shape = (1, tp, m, W // 2)
    box_d, box_h = armed_box(shape), oracle.arm(np.empty(shape, dtype=np.uint32))
    got_res = run_call(lib, box_d, box_h, p, res, dev16(gamma), gamma, 0)
    assert np.all(got_res[4] == 0)


@pytest.mark.parametrize("rank,split", [(0, None), (3, None), (7, None), (3, 7), (5, 14)])
def test_fused_own_push(lib, rank, split):
    """The one-kernel form: the consumer brings rank `rank`'s row itself."""
    say(f"[parity] fused own push rank={rank} split={split}")
    cfg = wl.CONFIGS["tp8_m64"]
    src = wl.ArNormInputs(cfg)
    shape = (2, 8, 64, W // 2)
    box_d, box_h = armed_box(shape), oracle.arm(np.empty(shape, dtype=np.uint32))
    nbox = None
    if split is not None:
        lib.set_reduce_split(split)
        nbox = norm_box_for(shape)
    g_d = dev16(src.gamma)
    for call in range(3):
        p, r = src.call()
        pushes = [(k, 1) for k in range(8) if k != rank]
        run_call(lib, box_d, box_h, p, r, g_d, src.gamma, call % 2, pushes=pushes, fused_rank=rank,
                 norm_box=nbox)


def test_max_rows_and_single_row(lib):
    say("[parity] M = cap = 512 and M = 1")
    rng = np.random.default_rng(5)
    for m, cap in ((512, 512), (1, 512)):
        tp = 8
        p = (rng.standard_normal((tp, m, W), dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
        res = (rng.standard_normal((m, W), dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
        gamma = np.full(W, 0x3F80, dtype=np.uint16)
        shape = (1, tp, cap, W // 2)
        box_d, box_h = armed_box(shape), oracle.arm(np.empty(shape, dtype=np.uint32))
        run_call(lib, box_d, box_h, p, res, dev16(gamma), gamma, 0)


@pytest.mark.parametrize("m", [73, 74])
def test_push_layout_threshold(lib, m):
    """M=73 and M=74 at TP=8: a slot's rows just under and just over 1 MiB, where the
    producer switches from 2 fragments per thread to one (and the two-slot pushes of
    ranks 0-1 and the six of ranks 2-7 with it), with the one call beside the pair."""
    import dataclasses

    say(f"[parity] push layout threshold M={m}")
    cfg = dataclasses.replace(wl.CONFIGS["tp8_m64"], m=m, cap=80, sentinel_frac=0.05)
    src = wl.ArNormInputs(cfg)
    shape = (2, 8, cfg.cap, W // 2)
    box_d, box_h = armed_box(shape), oracle.arm(np.empty(shape, dtype=np.uint32))
    g_d = dev16(src.gamma)
    p, r = src.call()
    run_call(lib, box_d, box_h, p, r, g_d, src.gamma, 0, pushes=[(0, 2), (2, 6)])
    p, r = src.call()
    out_d, rout_d = empty16((m, W)), empty16((m, W))
    nbox = norm_box_for(shape)
    assert lib.arnorm_push_reduce_norm(dev16(p), dev16(r), g_d, box_d, 1, EPS, out_d, rout_d, norm_box=nbox) is True
    oracle.arnorm_push(box_h, p, 1, 0)
    want_out, want_res = oracle.arnorm_reduce_norm(box_h, 1, m, r, src.gamma, EPS)
    assert_bits_equal(host16(rout_d), want_res, "one-call residual_out")
    assert_out_close(host16(out_d), want_out)
    assert_bits_equal(host32(box_d), box_h, "mailbox")
    assert lib.status() == lib.OK


def test_in_place_residual(lib):
    say("[parity] residual_out == residual")
    cfg = wl.CONFIGS["tp8_m64"]
    src = wl.ArNormInputs(cfg)
    p, r = src.call()
    box_d = armed_box((2, 8, 64, W // 2))
    box_h = oracle.arm(np.empty((2, 8, 64, W // 2), dtype=np.uint32))
    assert lib.arnorm_push(dev16(p), box_d, 1, 0) is True
    oracle.arnorm_push(box_h, p, 1, 0)
    res_d = dev16(r)
    out_d = empty16((64, W))
    assert lib.arnorm_reduce_norm(res_d, dev16(src.gamma), box_d, 1, EPS, out_d, res_d) is True
    want_out, want_res = oracle.arnorm_reduce_norm(box_h, 1, 64, r, src.gamma, EPS)
    assert_bits_equal(host16(res_d), want_res, "in-place residual_out")
    assert_out_close(host16(out_d), want_out)


def test_not_served_shapes(lib):
    import torch

    box = armed_box((1, 8, 4, W // 2))
    p = torch.zeros((8, 5, W), dtype=torch.int16, device="cuda")
    assert lib.arnorm_push(p, box, 0, 0) is None  # M = 5 > cap = 4
    box1 = armed_box((1, 1, 4, W // 2))
    assert lib.arnorm_push(torch.zeros((1, 2, W), dtype=torch.int16, device="cuda"), box1, 0, 0) is None
    g = armed_box((4, 8 * 6))
    assert lib.gather_push(torch.zeros((1, 2, 6), dtype=torch.int32, device="cuda"), g, 8, 0) is None
    with pytest.raises(lib.ArnormError):
        lib.arnorm_push(torch.zeros((2, 2, W), dtype=torch.int16, device="cuda"), box, 0, 7)


def _golden_rows(fname, with_residual):
    """The hand cases of a golden file as (name, slot words, residual word or None,
    expected word)."""
    from tests.conftest import read_golden

    cases = []
    for ln in read_golden(fname):
        parts = [p.strip() for p in ln.split("|")]
        words = [int(x, 16) for x in parts[1].split(",")]
        res = int(parts[2], 16) if with_residual else None
        cases.append((parts[0], words, res, int(parts[-1], 16)))
    return cases


@pytest.mark.parametrize("one_launch", [False, True])
def test_golden_words_on_gpu(lib, one_launch):
    """The hand cases under tests/golden, whose expected words are derived from the pages
    and not from the oracle, through the HIP path: each slot word (and residual word) in
    the first two columns of an otherwise zero row; the new residual's first word, or the
    two-shot output's, must be the expected word, with every mailbox re-armed.  As the
    push + consumer pair, or as one launch per call."""
    say(f"[parity] golden words on the GPU one_launch={one_launch}")
    cases = [(n, w, None, e) for n, w, _, e in _golden_rows("allreduce_words.txt", False)]
    cases += _golden_rows("residual_words.txt", True)
    for name, words, res_word, want in cases:
        tp = len(words)
        partial = np.zeros((tp, 1, W), dtype=np.uint16)
        for k, w in enumerate(words):
            partial[k, 0, 0], partial[k, 0, 1] = w & 0xFFFF, w >> 16
        res_d = None
        if res_word is not None:
            residual = np.zeros((1, W), dtype=np.uint16)
            residual[0, 0], residual[0, 1] = res_word & 0xFFFF, res_word >> 16
            res_d = dev16(residual)
        box = armed_box((1, tp, 1, W // 2))
        nbox = armed_box((1, 1, 256))
        g_d = dev16(np.full(W, 0x3F80, dtype=np.uint16))
        out_d, rout_d = empty16((1, W)), empty16((1, W))
        if one_launch:
            assert lib.arnorm_push_reduce_norm(dev16(partial), res_d, g_d, box, 0, EPS, out_d, rout_d,
                                               norm_box=nbox) is True
        else:
            assert lib.arnorm_push(dev16(partial), box, 0, 0) is True
            assert lib.arnorm_reduce_norm(res_d, g_d, box, 0, EPS, out_d, rout_d) is True
        assert lib.status() == lib.OK
        got = host32(rout_d)[0, 0]
        assert got == want, f"{name}: new residual word {got:08X}, want {want:08X}"
        assert np.all(host32(box) == S0) and np.all(host32(nbox) == S0), f"{name}: not re-armed"
    for name, words, _, want in _golden_rows("twoshot_words.txt", False):
        tp, width = len(words), 8
        partial = np.zeros((tp, 1, width), dtype=np.uint16)
        for k, w in enumerate(words):
            partial[k, 0, 0], partial[k, 0, 1] = w & 0xFFFF, w >> 16
        recv, gath = armed_box((1, tp, 1, width // 2)), armed_box((1, 1, 1, width // 2))
        out_d = empty16((1, width))
        if one_launch:
            assert lib.twoshot_push_reduce_read(dev16(partial), recv, gath, 0, out_d) is True
        else:
            assert lib.twoshot_push(dev16(partial), recv, 0, 0) is True
            assert lib.twoshot_reduce(recv, gath, 0, 1) is True
            assert lib.twoshot_read(gath, 0, out_d) is True
        assert lib.status() == lib.OK
        got = host32(out_d)[0, 0]
        assert got == want, f"two-shot {name}: word {got:08X}, want {want:08X}"
        assert np.all(host32(recv) == S0) and np.all(host32(gath) == S0), f"two-shot {name}: not re-armed"
