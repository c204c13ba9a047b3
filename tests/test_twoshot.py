"""GPU parity of the two-shot all-reduce stand-in (owners = 1) against the oracle:
the gather row, the output and both mailboxes bit-exact after every step."""

import numpy as np
import pytest

import oracle
from tests.gpu_util import W, armed_box, assert_bits_equal, dev16, empty16, host16, host32, say
from tests.test_parity import torture_partials
from tp_all_reduce_arnorm_amd import workloads as wl

pytestmark = pytest.mark.gpu


def ts_call(lib, recv_d, gath_d, recv_h, gath_h, partials, parity, pushes=None):
    tp, m, width = partials.shape
    for rank, n in pushes or [(0, tp)]:
        assert lib.twoshot_push(dev16(partials[rank:rank + n]), recv_d, parity, rank) is True
        oracle.twoshot_push(recv_h, partials[rank:rank + n], parity, rank)
    assert lib.twoshot_reduce(recv_d, gath_d, parity, m) is True
    want = oracle.twoshot_reduce(recv_h, gath_h, parity, m)
    assert_bits_equal(host32(recv_d), recv_h, "recv after reduce")
    assert_bits_equal(host32(gath_d), gath_h, "gather row after reduce")
    out_d = empty16((m, width))
    assert lib.twoshot_read(gath_d, parity, out_d) is True
    got = host16(out_d)
    assert_bits_equal(got, oracle.twoshot_read(gath_h, parity, m), "read")
    assert_bits_equal(got, want, "read vs reduce")
    assert_bits_equal(host32(gath_d), gath_h, "gather row after read")
    assert lib.status() == lib.OK
    return got


def boxes(parities, tp, cap, width):
    rshape, gshape = (parities, tp, cap, width // 2), (parities, 1, cap, width // 2)
    return (armed_box(rshape), armed_box(gshape), oracle.arm(np.empty(rshape, dtype=np.uint32)),
            oracle.arm(np.empty(gshape, dtype=np.uint32)))


@pytest.mark.parametrize("name", ["tp8_m4", "tp8_m64"])
def test_workload_shapes(lib, name):
    cfg = wl.CONFIGS[name]
    say(f"[twoshot] {name}")
    src = wl.ArNormInputs(cfg)
    recv_d, gath_d, recv_h, gath_h = boxes(2, cfg.tp, cfg.cap, W)
    for call in range(min(cfg.calls, 12)):
        p = src.partials()
        pushes = [(0, 8)] if call % 3 else [(k, 1) for k in range(8)]
        ts_call(lib, recv_d, gath_d, recv_h, gath_h, p, call % 2, pushes)


@pytest.mark.parametrize("tp", [2, 3, 4, 5, 6, 7, 8])
def test_torture_rows(lib, tp):
    say(f"[twoshot] torture tp={tp}")
    rng = np.random.default_rng(200 + tp)
    m, cap = 13, 17
    recv_d, gath_d, recv_h, gath_h = boxes(2, tp, cap, W)
    # the other parity published and unread must survive untouched
    other = torture_partials(rng, tp, m)
    assert lib.twoshot_push(dev16(other), recv_d, 1, 0) is True
    oracle.twoshot_push(recv_h, other, 1, 0)
    for _ in range(2):
        got = ts_call(lib, recv_d, gath_d, recv_h, gath_h, torture_partials(rng, tp, m), 0)
        assert not np.any(got == 0x8000), "no negative zero in the reduced row"


@pytest.mark.parametrize("width", [8, 64, 7176, 2 * 7168])
def test_widths_and_three_parities(lib, width):
    say(f"[twoshot] width={width}, 3 parities")
    rng = np.random.default_rng(width)
    tp, m, cap = 8, 5, 9
    recv_d, gath_d, recv_h, gath_h = boxes(3, tp, cap, width)
    for call in range(6):
        p = (rng.standard_normal((tp, m, width), dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
        p[:, :, 1::7] = 0x8000
        ts_call(lib, recv_d, gath_d, recv_h, gath_h, p, call % 3)


def test_not_served(lib):
    import torch

    recv = armed_box((1, 8, 4, 6))
    gath = armed_box((1, 1, 4, 6))
    assert lib.twoshot_push(torch.zeros((8, 2, 12), dtype=torch.int16, device="cuda"), recv, 0, 0) is None
    assert lib.twoshot_reduce(recv, gath, 0, 2) is None  # width 12 % 8 != 0
    recv = armed_box((1, 8, 4, 8))
    gath = armed_box((1, 1, 4, 8))
    assert lib.twoshot_reduce(recv, gath, 0, 5) is None  # M > cap


def test_m4096_every_row(lib):
    """M = 4096 at TP = 8, width 7168, as the benchmark runs it (push, owner's reduce, read
    of the gather row): every row bit for bit against the oracle, in blocks of 512 rows,
    and every slot and the gather row re-armed."""
    import torch

    say("[twoshot] M=4096 every row")
    cfg = wl.CONFIGS["tp8_m4096"]
    src = wl.ArNormInputs(cfg)
    p = src.partials()
    recv_d = armed_box((1, 8, cfg.cap, W // 2))
    gath_d = armed_box((1, 1, cfg.cap, W // 2))
    assert lib.twoshot_push(dev16(p), recv_d, 0, 0) is True
    assert lib.twoshot_reduce(recv_d, gath_d, 0, cfg.m) is True
    out_d = empty16((cfg.m, W))
    assert lib.twoshot_read(gath_d, 0, out_d) is True
    assert lib.status() == lib.OK
    s0 = torch.tensor(-(1 << 31), dtype=torch.int32, device="cuda")
    assert bool((recv_d == s0).all()) and bool((gath_d == s0).all())
    del recv_d, gath_d
    got = host16(out_d)
    blk = 512
    for r0 in range(0, cfg.m, blk):
        recv_h = oracle.arm(np.empty((1, 8, blk, W // 2), dtype=np.uint32))
        gath_h = oracle.arm(np.empty((1, 1, blk, W // 2), dtype=np.uint32))
        oracle.twoshot_push(recv_h, p[:, r0:r0 + blk], 0, 0)
        oracle.twoshot_reduce(recv_h, gath_h, 0, blk)
        assert_bits_equal(got[r0:r0 + blk], oracle.twoshot_read(gath_h, 0, blk), f"rows {r0}..{r0 + blk - 1}")


@pytest.mark.parametrize("m", [4, 64])
def test_concurrent_owner_and_reader(lib, side_streams, m):
    """Reader first, owner second, producer last and delayed, each on its own stream:
    every wait is a Lamport poll; each call matches the oracle."""
    import torch

    say(f"[twoshot] concurrent M={m}")
    old = lib.get_spin_limit()
    lib.set_spin_limit(1 << 16)
    try:
        rng = np.random.default_rng(300 + m)
        tp, cap = 8, 64
        recv_d, gath_d, recv_h, gath_h = boxes(2, tp, cap, W)
        cur = torch.cuda.current_stream()
        s_prod, s_own, s_read = side_streams
        for call in range(4):
            parity = call % 2
            p = (rng.standard_normal((tp, m, W), dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
            p_d = dev16(p)
            out_d = empty16((m, W))
            torch.cuda.synchronize()
            for s in (s_prod, s_own, s_read):
                s.wait_stream(cur)
            with torch.cuda.stream(s_read):
                assert lib.twoshot_read(gath_d, parity, out_d) is True
            with torch.cuda.stream(s_own):
                assert lib.twoshot_reduce(recv_d, gath_d, parity, m) is True
            with torch.cuda.stream(s_prod):
                torch.cuda._sleep(200000)
                assert lib.twoshot_push(p_d, recv_d, parity, 0) is True
            for s in (s_prod, s_own, s_read):
                cur.wait_stream(s)
            torch.cuda.synchronize()
            assert lib.status() == lib.OK, "a poll timed out"
            oracle.twoshot_push(recv_h, p, parity, 0)
            want = oracle.twoshot_reduce(recv_h, gath_h, parity, m)
            oracle.twoshot_read(gath_h, parity, m)
            assert_bits_equal(host16(out_d), want, f"call {call} out")
            assert_bits_equal(host32(recv_d), recv_h, f"call {call} recv")
            assert_bits_equal(host32(gath_d), gath_h, f"call {call} gather row")
    finally:
        lib.set_spin_limit(old)


def tsr_call(lib, recv_d, gath_d, recv_h, gath_h, partials, parity):
    """twoshot_push_reduce_read of every rank against the oracle's push, reduce and read;
    both mailboxes bit-exact afterwards."""
    tp, m, width = partials.shape
    out_d = empty16((m, width))
    assert lib.twoshot_push_reduce_read(dev16(partials), recv_d, gath_d, parity, out_d) is True
    oracle.twoshot_push(recv_h, partials, parity, 0)
    want = oracle.twoshot_reduce(recv_h, gath_h, parity, m)
    assert_bits_equal(oracle.twoshot_read(gath_h, parity, m), want, "oracle read vs reduce")
    got = host16(out_d)
    assert_bits_equal(got, want, "one-call out")
    assert_bits_equal(host32(recv_d), recv_h, "recv after the call")
    assert_bits_equal(host32(gath_d), gath_h, "gather row after the call")
    assert lib.status() == lib.OK
    return got


@pytest.mark.parametrize("name,calls", [("tp8_m4", 8), ("tp8_m64", 4)])
def test_one_call_workloads(lib, name, calls):
    """tp8_m4 (TP=8, M=4: one launch) and tp8_m64 (M=64: the three launches)."""
    cfg = wl.CONFIGS[name]
    say(f"[twoshot] one call {name}")
    src = wl.ArNormInputs(cfg)
    recv_d, gath_d, recv_h, gath_h = boxes(2, cfg.tp, cfg.cap, W)
    for call in range(calls):
        tsr_call(lib, recv_d, gath_d, recv_h, gath_h, src.partials(), call % 2)


@pytest.mark.parametrize("tp,m", [(2, 13), (3, 13), (4, 13), (5, 13), (6, 9), (7, 9), (8, 9), (8, 13), (8, 1),
                                  (8, 6), (8, 7), (8, 8), (8, 73), (8, 74), (8, 292), (8, 293),
                                  (8, 585), (8, 586), (4, 1170), (4, 1171), (2, 2340), (2, 2341)])
def test_one_call_torture(lib, tp, m):
    """Torture rows through the one call, one launch where the TP slots of rows < M fit
    64 MiB (at TP=8 M=585 is the last row count within it, M=586 the first above, at TP=4
    1170 / 1171, at TP=2 2340 / 2341; M=292 and 293 straddle its former limit of 32 MiB, M=73
    and 74 the one of 8 MiB), with the
    other parity published and left untouched.  The one launch pads its producer groups to
    multiples of 8 workgroups from 24 per slot: TP=2..5 at M=13 and TP=8 at M=7, 8 and 13
    take the padded layout, TP=8 at M=6 the largest unpadded one, and M=9 and 73 (32 and 256
    per slot) need no padding."""
    say(f"[twoshot] one call torture tp={tp} m={m}")
    rng = np.random.default_rng(400 + 16 * tp + m)
    cap = max(17, m)
    recv_d, gath_d, recv_h, gath_h = boxes(2, tp, cap, W)
    other = torture_partials(rng, tp, m)
    assert lib.twoshot_push(dev16(other), recv_d, 1, 0) is True
    oracle.twoshot_push(recv_h, other, 1, 0)
    for _ in range(2):
        got = tsr_call(lib, recv_d, gath_d, recv_h, gath_h, torture_partials(rng, tp, m), 0)
        assert not np.any(got == 0x8000), "no negative zero in the reduced row"


@pytest.mark.parametrize("width,m", [(8, 1), (64, 7), (7176, 3), (2 * 7168, 4)])
def test_one_call_widths(lib, width, m):
    say(f"[twoshot] one call width={width} m={m}")
    rng = np.random.default_rng(500 + width + m)
    tp, cap = 8, 9
    recv_d, gath_d, recv_h, gath_h = boxes(3, tp, cap, width)
    for call in range(4):
        p = (rng.standard_normal((tp, m, width), dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
        p[:, :, 1::7] = 0x8000
        tsr_call(lib, recv_d, gath_d, recv_h, gath_h, p, call % 3)


def test_one_call_graph_replay(lib):
    """Captured one-call two-shot calls over two parities, replayed three times with
    eager work between the replays; every replay matches the oracle."""
    import torch

    say("[twoshot] one call graph replay")
    rng = np.random.default_rng(600)
    tp, m, cap = 8, 4, 64
    recv_d, gath_d, recv_h, gath_h = boxes(2, tp, cap, W)
    parts = [(rng.standard_normal((tp, m, W), dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
             for _ in range(2)]
    parts_d = [dev16(p) for p in parts]
    outs = [empty16((m, W)) for _ in range(2)]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for k in range(2):
            assert lib.twoshot_push_reduce_read(parts_d[k], recv_d, gath_d, k, outs[k]) is True
    for rep in range(3):
        for o in outs:
            o.fill_(0x1234)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert lib.status() == lib.OK
        for k in range(2):
            oracle.twoshot_push(recv_h, parts[k], k, 0)
            want = oracle.twoshot_reduce(recv_h, gath_h, k, m)
            oracle.twoshot_read(gath_h, k, m)
            assert_bits_equal(host16(outs[k]), want, f"replay {rep} parity {k}")
        assert_bits_equal(host32(recv_d), recv_h, f"replay {rep} recv")
        assert_bits_equal(host32(gath_d), gath_h, f"replay {rep} gather row")
