"""Mailbox protocol on the GPU: bounded polls (a missing push is forced from the host
with a tiny spin limit, so every kernel still ends), recovery with lamport_arm, and
the stand-in call sequence captured in a HIP graph and replayed."""

import numpy as np
import pytest

import oracle
from tests.gpu_util import (W, armed_box, assert_bits_equal, assert_out_close, dev16, dev32, empty16, host16,
                            host32, say)
from tp_all_reduce_arnorm_amd import workloads as wl

pytestmark = pytest.mark.gpu
EPS = 1e-6


@pytest.fixture
def small_spin(lib):
    old = lib.get_spin_limit()
    lib.set_spin_limit(64)
    yield
    lib.set_spin_limit(old)


def test_missing_push_times_out_and_recovers(lib, small_spin):
    say("[protocol] arnorm missing push -> timeout -> lamport_arm -> exact")
    cfg = wl.CONFIGS["tp8_m4"]
    src = wl.ArNormInputs(cfg)
    shape = (2, 8, 64, W // 2)
    box_d = armed_box(shape)
    p, _ = src.call()
    assert lib.status() == lib.OK
    assert lib.arnorm_push(dev16(p[:7]), box_d, 0, 0) is True  # rank 7 never pushes
    out_d, rout_d = empty16((4, W)), empty16((4, W))
    g_d = dev16(src.gamma)
    assert lib.arnorm_reduce_norm(None, g_d, box_d, 0, EPS, out_d, rout_d) is True
    assert lib.status() == lib.TIMEOUT
    assert lib.status() == lib.OK  # read and cleared
    # timed-out fragments were not re-armed: slots 0..6 of rows < 4 still hold data
    assert not np.any(host32(box_d)[0, :7, :4] == 0x80000000)
    # recovery: re-arm the whole mailbox, then a normal call is exact
    assert lib.lamport_arm(box_d) is True
    box_h = oracle.arm(np.empty(shape, dtype=np.uint32))
    p, _ = src.call()
    assert lib.arnorm_push(dev16(p), box_d, 1, 0) is True
    oracle.arnorm_push(box_h, p, 1, 0)
    assert lib.arnorm_reduce_norm(None, g_d, box_d, 1, EPS, out_d, rout_d) is True
    want_out, want_res = oracle.arnorm_reduce_norm(box_h, 1, 4, None, src.gamma, EPS)
    assert lib.status() == lib.OK
    assert_bits_equal(host16(rout_d), want_res, "residual_out after recovery")
    assert_out_close(host16(out_d), want_out)
    assert_bits_equal(host32(box_d), box_h, "mailbox after recovery")


def test_gather_missing_push_times_out(lib, small_spin):
    import torch

    say("[protocol] gather missing push -> timeout -> lamport_arm -> exact")
    cfg = wl.CONFIGS["gather_tp8_m32"]
    shards = wl.gather_shards(cfg)
    gshape = (cfg.cap, cfg.tp * cfg.s)
    gbox_d = armed_box(gshape)
    assert lib.gather_push(dev32(shards[1:]), gbox_d, cfg.tp, 1) is True  # rank 0 missing
    out_d = torch.empty((cfg.m, cfg.tp * cfg.s), dtype=torch.int32, device="cuda")
    assert lib.gather_poll(gbox_d, cfg.tp, cfg.m, out=out_d, copy=True) is True
    assert lib.status() == lib.TIMEOUT
    assert lib.lamport_arm(gbox_d) is True
    gbox_h = oracle.arm(np.empty(gshape, dtype=np.uint32))
    assert lib.gather_push(dev32(shards), gbox_d, cfg.tp, 0) is True
    oracle.gather_push(gbox_h, shards, 0)
    assert lib.gather_poll(gbox_d, cfg.tp, cfg.m, out=out_d, copy=True) is True
    assert lib.status() == lib.OK
    assert_bits_equal(host32(out_d), oracle.gather_poll(gbox_h, cfg.m, True), "gathered words")
    assert_bits_equal(host32(gbox_d), gbox_h, "gather mailbox")


@pytest.mark.parametrize("form", ["pair", "one_call", "one_call_split14"])
def test_graph_replay_alternating_parities(lib, form):
    """push + reduce_norm (or the one-launch call, rows split 7 or 14 ways through a norm
    box) for parity 0, then parity 1, captured once and replayed; every replay (with eager
    work and synchronizations in between) matches the oracle."""
    import torch

    say(f"[protocol] HIP graph replay, tp8_m4 shape, {form}")
    lib.set_reduce_split(14 if form == "one_call_split14" else 0)
    cfg = wl.CONFIGS["tp8_m4"]
    src = wl.ArNormInputs(cfg)
    shape = (2, 8, 64, W // 2)
    box_d = armed_box(shape)
    p0, _ = src.call()
    p1, _ = src.call()
    p0_d, p1_d, g_d = dev16(p0), dev16(p1), dev16(src.gamma)
    outs = [(empty16((4, W)), empty16((4, W))) for _ in range(2)]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    nbox = armed_box((2, 64, 256))
    with torch.cuda.graph(graph):
        for parity, p_d in ((0, p0_d), (1, p1_d)):
            if form == "pair":
                assert lib.arnorm_push(p_d, box_d, parity, 0) is True
                assert lib.arnorm_reduce_norm(None, g_d, box_d, parity, EPS, outs[parity][0],
                                              outs[parity][1]) is True
            else:
                assert lib.arnorm_push_reduce_norm(p_d, None, g_d, box_d, parity, EPS, outs[parity][0],
                                                   outs[parity][1], norm_box=nbox) is True
    lib.set_reduce_split(0)
    box_h = oracle.arm(np.empty(shape, dtype=np.uint32))
    wants = []
    for parity, p in ((0, p0), (1, p1)):
        oracle.arnorm_push(box_h, p, parity, 0)
        wants.append(oracle.arnorm_reduce_norm(box_h, parity, 4, None, src.gamma, EPS))
    for replay in range(5):
        for o, r in outs:
            o.fill_(0)
            r.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for parity in (0, 1):
            assert_bits_equal(host16(outs[parity][1]), wants[parity][1], f"replay {replay} residual_out")
            assert_out_close(host16(outs[parity][0]), wants[parity][0], f"replay {replay} out")
        assert_bits_equal(host32(box_d), box_h, f"replay {replay} mailbox")
        assert np.all(host32(nbox) == 0x80000000), f"replay {replay} norm box"
        _ = torch.ones(1024, device="cuda").sum().item()  # eager work between replays
    assert lib.status() == lib.OK


@pytest.mark.parametrize("name,m", [("gather_tp8_m32", 4), ("gather_tp8_m32", 32), ("logits", 1)])
def test_graph_replay_gather(lib, name, m):
    """gather_push_poll with copy captured twice in one graph (two shard sets into one
    mailbox: each call leaves it re-armed for the next) and replayed; every replay, with
    eager work and synchronizations in between, matches the oracle.  M=4 and the logits
    row are one launch each, M=32 the pair gather_push + gather_poll."""
    import dataclasses

    import torch

    say(f"[protocol] HIP graph replay, gather_push_poll {name} M={m}")
    cfg = dataclasses.replace(wl.CONFIGS[name], m=m)
    gen = wl.gather_shards if name == "gather_tp8_m32" else wl.bf16_shards
    shards = [gen(cfg), gen(dataclasses.replace(cfg, seed=cfg.seed + 1))]
    assert not np.array_equal(shards[0], shards[1])
    gshape = (cfg.cap, cfg.tp * cfg.s)
    gbox_d = armed_box(gshape)
    sh_d = [dev32(x) for x in shards]
    outs = [torch.empty((m, cfg.tp * cfg.s), dtype=torch.int32, device="cuda") for _ in range(2)]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for x_d, o_d in zip(sh_d, outs):
            assert lib.gather_push_poll(x_d, gbox_d, out=o_d, copy=True) is True
    gbox_h = oracle.arm(np.empty(gshape, dtype=np.uint32))
    wants = []
    for x in shards:
        oracle.gather_push(gbox_h, x, 0)
        wants.append(oracle.gather_poll(gbox_h, m, True))
    for replay in range(5):
        for o_d in outs:
            o_d.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in range(2):
            assert_bits_equal(host32(outs[k]), wants[k], f"replay {replay} call {k} gathered words")
        assert_bits_equal(host32(gbox_d), gbox_h, f"replay {replay} gather mailbox")
        _ = torch.ones(1024, device="cuda").sum().item()  # eager work between replays
    assert lib.status() == lib.OK


@pytest.mark.parametrize("m,residual,split", [(4, False, None), (64, True, None), (1, True, None),
                                              (4, False, 14), (64, True, 7)])
def test_concurrent_consumer_polls_while_producer_pushes(lib, side_streams, m, residual, split):
    """The Lamport mode proper: the consumer is launched first on its own stream and
    spins on the mailbox while the producer, delayed on another stream, pushes; no
    kernel boundary orders them.  Every call must match the oracle."""
    import torch

    say(f"[protocol] concurrent consumer-first M={m} residual={residual} split={split}")
    old = lib.get_spin_limit()
    lib.set_spin_limit(1 << 16)
    lib.set_reduce_split(split or 0)
    try:
        rng = np.random.default_rng(40 + m)
        tp, cap = 8, 64
        shape = (2, tp, cap, W // 2)
        box_d = armed_box(shape)
        box_h = oracle.arm(np.empty(shape, dtype=np.uint32))
        nbox = armed_box((2, cap, 256)) if split else None
        gamma = (np.float32(1) + np.float32(0.1) * rng.standard_normal(W, dtype=np.float32)).view(np.uint32)
        gamma = (gamma >> 16).astype(np.uint16)
        g_d = dev16(gamma)
        cur = torch.cuda.current_stream()
        s_prod, s_cons = side_streams[0], side_streams[1]
        for call in range(6):
            parity = call % 2
            p = (rng.standard_normal((tp, m, W), dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
            res = (rng.standard_normal((m, W), dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16) \
                if residual else None
            p_d = dev16(p)
            res_d = dev16(res) if residual else None
            out_d, rout_d = empty16((m, W)), empty16((m, W))
            torch.cuda.synchronize()
            s_prod.wait_stream(cur)
            s_cons.wait_stream(cur)
            with torch.cuda.stream(s_cons):
                assert lib.arnorm_reduce_norm(res_d, g_d, box_d, parity, EPS, out_d, rout_d, norm_box=nbox) is True
            with torch.cuda.stream(s_prod):
                torch.cuda._sleep(200000)  # hold the producer back so that the consumer spins
                assert lib.arnorm_push(p_d, box_d, parity, 0) is True
            cur.wait_stream(s_prod)
            cur.wait_stream(s_cons)
            torch.cuda.synchronize()
            assert lib.status() == lib.OK, "a poll timed out: producer and consumer did not overlap"
            oracle.arnorm_push(box_h, p, parity, 0)
            want_out, want_res = oracle.arnorm_reduce_norm(box_h, parity, m, res, gamma, EPS)
            assert_bits_equal(host16(rout_d), want_res, f"call {call} residual_out")
            assert_out_close(host16(out_d), want_out, f"call {call} out")
            assert_bits_equal(host32(box_d), box_h, f"call {call} mailbox")
            if nbox is not None:
                assert np.all(host32(nbox) == 0x80000000), "the norm box is left re-armed"
    finally:
        lib.set_spin_limit(old)
        lib.set_reduce_split(0)


@pytest.mark.parametrize("frags_per_thread", [0, 4])
def test_concurrent_gather_consumer_first(lib, side_streams, frags_per_thread):
    """The poll launched first on its own stream, the push later and delayed, at gather_tp8_m32, with
    the witness wait forced: one fragment per thread (automatic) or 4 in flight per
    thread (forced)."""
    import torch

    say(f"[protocol] concurrent gather consumer-first frags/thread={frags_per_thread}")
    old = lib.get_spin_limit()
    lib.set_spin_limit(1 << 16)
    lib.set_poll(frags_per_thread, 2)
    try:
        cfg = wl.CONFIGS["gather_tp8_m32"]
        shards = wl.gather_shards(cfg)
        gshape = (cfg.cap, cfg.tp * cfg.s)
        gbox_d = armed_box(gshape)
        gbox_h = oracle.arm(np.empty(gshape, dtype=np.uint32))
        sh_d = dev32(shards)
        cur = torch.cuda.current_stream()
        s_prod, s_cons = side_streams[0], side_streams[1]
        for _ in range(3):
            out_d = torch.empty((cfg.m, cfg.tp * cfg.s), dtype=torch.int32, device="cuda")
            torch.cuda.synchronize()
            s_prod.wait_stream(cur)
            s_cons.wait_stream(cur)
            with torch.cuda.stream(s_cons):
                assert lib.gather_poll(gbox_d, cfg.tp, cfg.m, out=out_d, copy=True) is True
            with torch.cuda.stream(s_prod):
                torch.cuda._sleep(200000)
                assert lib.gather_push(sh_d, gbox_d, cfg.tp, 0) is True
            cur.wait_stream(s_prod)
            cur.wait_stream(s_cons)
            torch.cuda.synchronize()
            assert lib.status() == lib.OK
            oracle.gather_push(gbox_h, shards, 0)
            assert_bits_equal(host32(out_d), oracle.gather_poll(gbox_h, cfg.m, True), "gathered words")
            assert_bits_equal(host32(gbox_d), gbox_h, "gather mailbox")
    finally:
        lib.set_spin_limit(old)
        lib.set_poll(0, 0)


def test_three_host_threads_three_mailboxes(lib, side_streams):
    """Host threads calling the library at once, each on its own stream and mailbox: 24
    one-launch ArNorm calls (TP=8, M=4, rows split through a norm box), 24 one-launch
    Gathers (TP=8, M=4, S=896) and 24 one-launch two-shot calls (TP=8, M=4), all in flight
    together.  Every call's output and the final mailboxes must match the oracle."""
    import threading

    import torch

    say("[protocol] three host threads, three streams, three mailboxes")
    calls, tp, m, cap, s = 24, 8, 4, 64, 896
    rng = np.random.default_rng(404)

    def bf16(shape, scale):
        x = (np.float32(scale) * rng.standard_normal(shape, dtype=np.float32)).view(np.uint32)
        return (x >> 16).astype(np.uint16)

    ar_p = [bf16((tp, m, W), 0.02) for _ in range(calls)]
    gamma = ((np.float32(1) + np.float32(0.1) * rng.standard_normal(W, dtype=np.float32)).view(np.uint32) >> 16)
    gamma = gamma.astype(np.uint16)
    g_sh = []
    for _ in range(calls):
        w = rng.integers(0, 1 << 32, size=(tp, m, s), dtype=np.uint64).astype(np.uint32)
        w[rng.random(w.shape) < 0.03] = 0x80000000
        g_sh.append(w)
    ts_p = []
    for _ in range(calls):
        p = bf16((tp, m, W), 0.5)
        p[:, :, 3::7] = 0x8000
        ts_p.append(p)

    ar_box, nbox = armed_box((2, tp, cap, W // 2)), armed_box((2, cap, 256))
    g_box = armed_box((cap, tp * s))
    ts_recv, ts_gath = armed_box((2, tp, cap, W // 2)), armed_box((2, 1, cap, W // 2))
    ar_in, g_d = [dev16(p) for p in ar_p], dev16(gamma)
    g_in = [dev32(w) for w in g_sh]
    ts_in = [dev16(p) for p in ts_p]
    ar_out = [(empty16((m, W)), empty16((m, W))) for _ in range(calls)]
    g_out = [torch.empty((m, tp * s), dtype=torch.int32, device="cuda") for _ in range(calls)]
    ts_out = [empty16((m, W)) for _ in range(calls)]
    torch.cuda.synchronize()

    errors = []

    def run(stream, body):
        try:
            with torch.cuda.stream(stream):
                for i in range(calls):
                    assert body(i) is True
        except Exception as e:  # noqa: BLE001 -- reported after the join
            errors.append(e)

    jobs = [
        (side_streams[0], lambda i: lib.arnorm_push_reduce_norm(ar_in[i], None, g_d, ar_box, i % 2, EPS, ar_out[i][0],
                                                                ar_out[i][1], norm_box=nbox)),
        (side_streams[1], lambda i: lib.gather_push_poll(g_in[i], g_box, out=g_out[i], copy=True)),
        (side_streams[2], lambda i: lib.twoshot_push_reduce_read(ts_in[i], ts_recv, ts_gath, i % 2, ts_out[i])),
    ]
    threads = [threading.Thread(target=run, args=job) for job in jobs]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    assert lib.status() == lib.OK

    ar_h = oracle.arm(np.empty((2, tp, cap, W // 2), dtype=np.uint32))
    g_h = oracle.arm(np.empty((cap, tp * s), dtype=np.uint32))
    recv_h = oracle.arm(np.empty((2, tp, cap, W // 2), dtype=np.uint32))
    gath_h = oracle.arm(np.empty((2, 1, cap, W // 2), dtype=np.uint32))
    for i in range(calls):
        oracle.arnorm_push(ar_h, ar_p[i], i % 2, 0)
        want_out, want_res = oracle.arnorm_reduce_norm(ar_h, i % 2, m, None, gamma, EPS)
        assert_bits_equal(host16(ar_out[i][1]), want_res, f"ArNorm call {i} residual_out")
        exact_zero = (oracle.widen(want_res) == 0) | (oracle.widen(gamma) == 0)[None, :]
        assert_out_close(host16(ar_out[i][0]), want_out, f"ArNorm call {i} out", exact_zero=exact_zero)
        oracle.gather_push(g_h, g_sh[i], 0)
        assert_bits_equal(host32(g_out[i]), oracle.gather_poll(g_h, m, True), f"Gather call {i}")
        oracle.twoshot_push(recv_h, ts_p[i], i % 2, 0)
        want = oracle.twoshot_reduce(recv_h, gath_h, i % 2, m)
        assert_bits_equal(oracle.twoshot_read(gath_h, i % 2, m), want, "oracle two-shot read")
        assert_bits_equal(host16(ts_out[i]), want, f"two-shot call {i}")
    assert_bits_equal(host32(ar_box), ar_h, "ArNorm mailbox")
    assert np.all(host32(nbox) == 0x80000000), "norm box left re-armed"
    assert_bits_equal(host32(g_box), g_h, "Gather mailbox")
    assert_bits_equal(host32(ts_recv), recv_h, "two-shot slots")
    assert_bits_equal(host32(ts_gath), gath_h, "two-shot gather row")


def test_concurrent_consumer_first_m4096(lib, side_streams):
    """The whole-row consumer at M = 4096 (TP = 8, residual) launched first on its own
    stream, the push of all 8 slots later and delayed on another: the consumer's grid is
    capped at what the GPU holds at once with room left for the producer, so every poll
    ends within a bounded spin and every row matches the oracle."""
    import torch

    say("[protocol] concurrent consumer-first M=4096")
    old = lib.get_spin_limit()
    lib.set_spin_limit(1 << 18)
    try:
        cfg = wl.CONFIGS["tp8_m4096"]
        src = wl.ArNormInputs(cfg)
        p, r = src.call()
        box_d = armed_box((1, 8, cfg.cap, W // 2))
        p_d, r_d, g_d = dev16(p), dev16(r), dev16(src.gamma)
        out_d, rout_d = empty16((cfg.m, W)), empty16((cfg.m, W))
        cur = torch.cuda.current_stream()
        s_prod, s_cons = side_streams[0], side_streams[1]
        torch.cuda.synchronize()
        s_prod.wait_stream(cur)
        s_cons.wait_stream(cur)
        with torch.cuda.stream(s_cons):
            assert lib.arnorm_reduce_norm(r_d, g_d, box_d, 0, EPS, out_d, rout_d) is True
        with torch.cuda.stream(s_prod):
            torch.cuda._sleep(200000)
            assert lib.arnorm_push(p_d, box_d, 0, 0) is True
        cur.wait_stream(s_prod)
        cur.wait_stream(s_cons)
        torch.cuda.synchronize()
        assert lib.status() == lib.OK, "a poll timed out: the consumer's grid kept the producer out"
        assert bool((box_d == torch.tensor(-(1 << 31), dtype=torch.int32, device="cuda")).all())
        del box_d, p_d, r_d
        got_out, got_res = host16(out_d), host16(rout_d)
        blk = 1024
        for r0 in range(0, cfg.m, blk):
            box_h = oracle.arm(np.empty((1, 8, blk, W // 2), dtype=np.uint32))
            oracle.arnorm_push(box_h, p[:, r0:r0 + blk], 0, 0)
            want_out, want_res = oracle.arnorm_reduce_norm(box_h, 0, blk, r[r0:r0 + blk], src.gamma, EPS)
            assert_bits_equal(got_res[r0:r0 + blk], want_res, f"residual_out rows {r0}..")
            assert_out_close(got_out[r0:r0 + blk], want_out, f"out rows {r0}..")
    finally:
        lib.set_spin_limit(old)


def test_concurrent_gather_consumer_first_m4096(lib, side_streams):
    """gather_poll over 4096 rows of TP=8 x 896 words (7.3 M fragments, 4 per thread in
    flight over at most 1024 workgroups) launched before its push: every word and the
    mailbox must match the oracle and no poll may time out."""
    import dataclasses

    import torch

    say("[protocol] concurrent gather consumer-first M=4096")
    old = lib.get_spin_limit()
    lib.set_spin_limit(1 << 18)
    try:
        cfg = dataclasses.replace(wl.CONFIGS["gather_tp8_m32"], m=4096, cap=4096, seed=77)
        shards = wl.gather_shards(cfg)
        gshape = (cfg.cap, cfg.tp * cfg.s)
        gbox_d = armed_box(gshape)
        sh_d = dev32(shards)
        out_d = torch.empty((cfg.m, cfg.tp * cfg.s), dtype=torch.int32, device="cuda")
        cur = torch.cuda.current_stream()
        s_prod, s_cons = side_streams[0], side_streams[1]
        torch.cuda.synchronize()
        s_prod.wait_stream(cur)
        s_cons.wait_stream(cur)
        with torch.cuda.stream(s_cons):
            assert lib.gather_poll(gbox_d, cfg.tp, cfg.m, out=out_d, copy=True) is True
        with torch.cuda.stream(s_prod):
            torch.cuda._sleep(200000)
            assert lib.gather_push(sh_d, gbox_d, cfg.tp, 0) is True
        cur.wait_stream(s_prod)
        cur.wait_stream(s_cons)
        torch.cuda.synchronize()
        assert lib.status() == lib.OK
        gbox_h = oracle.arm(np.empty(gshape, dtype=np.uint32))
        oracle.gather_push(gbox_h, shards, 0)
        assert_bits_equal(host32(out_d), oracle.gather_poll(gbox_h, cfg.m, True), "gathered words")
        assert_bits_equal(host32(gbox_d), gbox_h, "gather mailbox")
    finally:
        lib.set_spin_limit(old)


def test_concurrent_twoshot_owner_first_m448(lib, side_streams):
    """The two-shot owner's reduce at M = 448 (1568 workgroups, at most 7 per CU: a grid
    that leaves a producer room) launched before the push, on its own stream, with the read
    of the gather row after it on that stream: no poll may time out, and every row, slot
    and the gather row must match the oracle."""
    import dataclasses

    import torch

    say("[protocol] concurrent two-shot owner-first M=448")
    old = lib.get_spin_limit()
    lib.set_spin_limit(1 << 18)
    try:
        cfg = dataclasses.replace(wl.CONFIGS["tp8_m4096"], m=448, cap=448, seed=44)
        p = wl.ArNormInputs(cfg).partials()
        recv_d = armed_box((1, 8, cfg.cap, W // 2))
        gath_d = armed_box((1, 1, cfg.cap, W // 2))
        p_d = dev16(p)
        out_d = empty16((cfg.m, W))
        cur = torch.cuda.current_stream()
        s_prod, s_own = side_streams[0], side_streams[1]
        torch.cuda.synchronize()
        for s in side_streams:
            s.wait_stream(cur)
        with torch.cuda.stream(s_own):
            assert lib.twoshot_reduce(recv_d, gath_d, 0, cfg.m) is True
            assert lib.twoshot_read(gath_d, 0, out_d) is True
        with torch.cuda.stream(s_prod):
            torch.cuda._sleep(200000)
            assert lib.twoshot_push(p_d, recv_d, 0, 0) is True
        for s in side_streams:
            cur.wait_stream(s)
        torch.cuda.synchronize()
        assert lib.status() == lib.OK
        s0 = torch.tensor(-(1 << 31), dtype=torch.int32, device="cuda")
        assert bool((recv_d == s0).all()) and bool((gath_d == s0).all())
        got = host16(out_d)
        assert_bits_equal(got, oracle.reduce_no_negative_zero(oracle.clean(oracle.pack_pairs(p))), "rows")
    finally:
        lib.set_spin_limit(old)


def test_status_taken_while_another_stream_times_out(lib, side_streams):
    """arnorm_status takes the status word with one device atomic: while a poll on one
    stream spins towards its limit (its push withheld), status reads on another stream
    report OK until the timeout lands, the timeout is reported exactly once, and the word
    is clear after."""
    import torch

    say("[protocol] status taken on one stream while another times out")
    old = lib.get_spin_limit()
    lib.set_spin_limit(1 << 14)
    try:
        box = armed_box((1, 8))  # TP=2 ranks of S=4 words, one row; never pushed
        cur = torch.cuda.current_stream()
        s_wait, s_read = side_streams[0], side_streams[1]
        assert lib.status() == lib.OK
        torch.cuda.synchronize()
        s_wait.wait_stream(cur)
        with torch.cuda.stream(s_wait):
            assert lib.gather_poll(box, 2, 1, copy=False) is True
        seen = []
        for _ in range(200):
            seen.append(lib.status(stream=s_read))
            if s_wait.query():
                break
        s_wait.synchronize()
        seen.append(lib.status(stream=s_read))
        seen.append(lib.status())
        assert seen.count(lib.TIMEOUT) == 1, seen
        assert seen[-1] == lib.OK and seen[-2] in (lib.OK, lib.TIMEOUT)
        assert lib.lamport_arm(box) is True
    finally:
        lib.set_spin_limit(old)
