#!/usr/bin/env python3
"""Benchmark of the Lamport-mailbox ArNorm on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one ArNorm call of the one-GPU stand-in at TP=8, M=4 (the embedding
call: residual = AR(x)): one arnorm_push_reduce_norm, the 8 ranks' pushes of their
partial rows and the consumer (poll, re-arm, rank-order sum, RMSNorm; rows split over
7 workgroups through a norm box) in one launch, alternating the two layer parities.
The calls are captured in HIP graphs of 200 calls and replayed; the timed region holds
max(K, 2000) calls (about 9 ms), timed with HIP events recorded on the stream the graphs
run on, behind a short spin kernel so that the host has queued them before the GPU
reaches them (the span is GPU time only, less the measured cost of an empty pair of
events), with a device synchronization on both sides; inputs are already resident in
HBM.  The floor of 2000 calls is there because a span of a few calls mostly times the
start of a graph launch: at K = 20 the same calls read about 10 % above the figure of
20,000 (4.9 against 4.4 µs per call).

The same JSON line carries:
  roofline      the consumer kernel at TP=8, M=4096 with residual (the HBM-bound
                workload): algorithmic bytes per launch / its average duration, HIP
                events around each launch on the stream it runs on, against 8 TB/s;
                and (roofline.call) the whole call at that size, push + consumer, as
                it repeats back to back
  push          the producer kernel at the same size, same method
  gather        Gather calls (TP=8, M=32, S=896, and the drafter's shapes)
  twoshot       the two-shot stand-in call at M=4 and its kernels at M=4096
  drafter_step  a drafter decode step's collectives: 11 ArNorm calls and 2 Gathers
  workloads     GPU µs per call at the named ArNorm configurations as stated: tp2_m1
                (TP=2, M=1, residual), tp8_m4 and tp8_m64 (TP=8, M=64, residual)
  cpu_baseline  the CPU oracle on this host's cores, one thread: the same TP=8, M=4
                call (the headline), and per workload tp2_m1, tp8_m4, tp8_m64,
                gather_tp8_m32 and tp8_m4096
Prints exactly one JSON line (rank 0, one GPU).
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HIDDEN = 7168
ROW_BYTES = HIDDEN * 2
PEAK_HBM_GBPS = 8000.0
EPS = 1e-6
MIN_TIMED_CALLS = 2000
METRIC = "ArNorm µs/call at TP=8 M=4; HBM GB/s (fraction of peak) at M=4096"


def reduce_bytes(tp, m, residual):
    """Algorithmic bytes of one arnorm_reduce_norm launch: TP slot reads, residual,
    gamma, out + residual_out, TP slot re-arm writes."""
    return tp * m * ROW_BYTES + (m * ROW_BYTES if residual else 0) + ROW_BYTES + 2 * m * ROW_BYTES \
        + tp * m * ROW_BYTES


def push_bytes(nslots, m):
    return 2 * nslots * m * ROW_BYTES


def kernel_sources_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tp_all_reduce_arnorm_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def committed_traffic(kernel_key):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None when
    there is none or the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(kernel_key)
    if not entry or entry.get("sources_sha") != kernel_sources_hash():
        return None
    return entry.get("bytes_per_launch")


_SPIN_CYCLES_PER_US = []


def _spin_rate(torch):
    """Cycles per µs of torch's spin kernel (torch.cuda._sleep) on this GPU, measured once
    with HIP events."""
    if not _SPIN_CYCLES_PER_US:
        cycles = 1_000_000
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.cuda._sleep(cycles)
        e1.record()
        torch.cuda.synchronize()
        _SPIN_CYCLES_PER_US.append(cycles / max(e0.elapsed_time(e1) * 1e3, 1.0))
    return _SPIN_CYCLES_PER_US[0]


def _raw_span_us(torch, enqueue, lead_us):
    torch.cuda.synchronize()
    torch.cuda._sleep(int(lead_us * _spin_rate(torch)))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    enqueue()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3


_EVENT_PAIR_US = []


def event_pair_us(torch):
    """The span of two HIP events recorded back to back with nothing between them (the
    timestamp packets' own cost, about 4 µs on MI355X): median of 9, measured once."""
    if not _EVENT_PAIR_US:
        _EVENT_PAIR_US.append(float(np.median([_raw_span_us(torch, lambda: None, 200.0) for _ in range(9)])))
    return _EVENT_PAIR_US[0]


def gpu_span_us(torch, enqueue, lead_us=2000.0):
    """GPU time in µs of the work that ``enqueue()`` queues on torch's current stream: HIP
    events recorded on that stream right before and right after it, less the span of an
    empty pair of events (event_pair_us).  A spin kernel of about ``lead_us`` is queued
    ahead of the first event, so the host has queued the timed work before the GPU gets
    there and no host launch time falls inside the span.  The device is synchronized
    before and after."""
    return _raw_span_us(torch, enqueue, lead_us) - event_pair_us(torch)


def time_latency(lib, torch, steps, warmup, chunk=200, one_launch=True, m=None):
    """GPU seconds for exactly `steps` stand-in calls at TP=8, M=4 (or M=m), no
    residual, graph-replayed (graphs of `chunk` calls and one of the remainder), timed
    by gpu_span_us.  one_launch: arnorm_push_reduce_norm (every rank's push and the
    consumer in one launch within the library's one-launch limits, M <= 562 at TP=8, else
    the pair); else the pair arnorm_push + arnorm_reduce_norm."""
    import dataclasses

    from tp_all_reduce_arnorm_amd import workloads as wl

    cfg = wl.CONFIGS["tp8_m4"] if m is None else dataclasses.replace(wl.CONFIGS["tp8_m4"], m=m, cap=max(m, 64))
    src = wl.ArNormInputs(cfg)
    box = torch.empty((2, cfg.tp, cfg.cap, HIDDEN // 2), dtype=torch.int32, device="cuda")
    nbox = torch.empty((2, cfg.cap, 256), dtype=torch.int32, device="cuda")
    assert lib.lamport_arm(box) is True and lib.lamport_arm(nbox) is True
    parts = [torch.from_numpy(src.partials().view(np.int16)).cuda() for _ in range(2)]
    gamma = torch.from_numpy(src.gamma.view(np.int16)).cuda()
    outs = [(torch.empty((cfg.m, HIDDEN), dtype=torch.int16, device="cuda"),
             torch.empty((cfg.m, HIDDEN), dtype=torch.int16, device="cuda")) for _ in range(2)]

    def call(i):
        parity = i % 2
        if one_launch:
            assert lib.arnorm_push_reduce_norm(parts[parity], None, gamma, box, parity, EPS, outs[parity][0],
                                               outs[parity][1], norm_box=nbox) is True
            return
        assert lib.arnorm_push(parts[parity], box, parity, 0) is True
        assert lib.arnorm_reduce_norm(None, gamma, box, parity, EPS, outs[parity][0], outs[parity][1],
                                      norm_box=nbox) is True

    def capture(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                call(i)
        return g

    # eager warmup (also loads the kernels), then graphs of `chunk` calls (even: parities alternate)
    for i in range(4):
        call(i)
    torch.cuda.synchronize()
    chunk = max(2, min(chunk, steps) // 2 * 2)
    g_main = capture(chunk)
    rem = steps % chunk
    g_rem = capture(rem) if rem else None
    for _ in range(max(3, warmup // chunk)):  # a new graph's first replays run slower
        g_main.replay()
        if g_rem is not None:
            g_rem.replay()
    torch.cuda.synchronize()
    reps = steps // chunk

    def timed():
        for _ in range(reps):
            g_main.replay()
        if g_rem is not None:
            g_rem.replay()

    elapsed = gpu_span_us(torch, timed) * 1e-6
    assert lib.status() == lib.OK
    return elapsed


def time_config(lib, torch, name, calls=2000, chunk=200):
    """GPU µs per stand-in ArNorm call at one of the named workload configurations, as that
    configuration states it (TP, M, residual, capacity, parities): one arnorm_push_reduce_norm
    per call with a norm box, the residual an input of its own and residual_out another
    buffer, graph-replayed and timed as time_latency."""
    from tp_all_reduce_arnorm_amd import workloads as wl

    cfg = wl.CONFIGS[name]
    src = wl.ArNormInputs(cfg)
    box = torch.empty((cfg.parities, cfg.tp, cfg.cap, HIDDEN // 2), dtype=torch.int32, device="cuda")
    nbox = torch.empty((cfg.parities, cfg.cap, 256), dtype=torch.int32, device="cuda")
    assert lib.lamport_arm(box) is True and lib.lamport_arm(nbox) is True
    parts = [torch.from_numpy(src.partials().view(np.int16)).cuda() for _ in range(2)]
    res = torch.from_numpy(src.residual().view(np.int16)).cuda() if cfg.residual else None
    gamma = torch.from_numpy(src.gamma.view(np.int16)).cuda()
    out = torch.empty((cfg.m, HIDDEN), dtype=torch.int16, device="cuda")
    rout = torch.empty((cfg.m, HIDDEN), dtype=torch.int16, device="cuda")

    def call(i):
        assert lib.arnorm_push_reduce_norm(parts[i % 2], res, gamma, box, i % cfg.parities, EPS, out, rout,
                                           norm_box=nbox) is True

    for i in range(4):
        call(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(chunk):
            call(i)
    for _ in range(3):  # a new graph's first replays run slower
        g.replay()

    def timed():
        for _ in range(calls // chunk):
            g.replay()

    us = gpu_span_us(torch, timed) / (calls // chunk * chunk)
    assert lib.status() == lib.OK
    return cfg, us


def time_drafter_step(lib, torch, steps=400, layers=11):
    """µs per drafter decode step's collectives, graph-replayed: `layers` one-launch
    ArNorm calls at TP=8, M=4 (the first without a residual, the embedding case; the
    others with the new residual chained in place, as consecutive layers use it; parities
    alternating) and the two Gathers of a step, the context projection (M=64, S=448
    words) and the lm_head logits (M=4, S=10240 words)."""
    import dataclasses

    from tp_all_reduce_arnorm_amd import workloads as wl

    cfg = wl.CONFIGS["tp8_m4"]
    src = wl.ArNormInputs(dataclasses.replace(cfg, residual=True, sigma_residual=1.0))
    box = torch.empty((2, cfg.tp, cfg.cap, HIDDEN // 2), dtype=torch.int32, device="cuda")
    nbox = torch.empty((2, cfg.cap, 256), dtype=torch.int32, device="cuda")
    assert lib.lamport_arm(box) is True and lib.lamport_arm(nbox) is True
    parts = [torch.from_numpy(src.partials().view(np.int16)).cuda() for _ in range(layers)]
    gamma = torch.from_numpy(src.gamma.view(np.int16)).cuda()
    resid = torch.empty((cfg.m, HIDDEN), dtype=torch.int16, device="cuda")
    out = torch.empty((cfg.m, HIDDEN), dtype=torch.int16, device="cuda")
    gathers = []
    for name in ("ctx", "logits"):
        g = wl.CONFIGS[name]
        gbox = torch.empty((g.cap, g.tp * g.s), dtype=torch.int32, device="cuda")
        assert lib.lamport_arm(gbox) is True
        gathers.append((torch.from_numpy(wl.bf16_shards(g).view(np.int32)).cuda(), gbox,
                        torch.empty((g.m, g.tp * g.s), dtype=torch.int32, device="cuda")))

    def step(k):
        for layer in range(layers):
            parity = (k * layers + layer) % 2
            assert lib.arnorm_push_reduce_norm(parts[layer], resid if layer else None, gamma, box, parity, EPS,
                                               out, resid, norm_box=nbox) is True
        for shards, gbox, gout in gathers:
            assert lib.gather_push_poll(shards, gbox, out=gout, copy=True) is True

    for k in range(2):
        step(k)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for k in range(2):  # two steps: the parities line up again after an even number of calls
            step(k)
    for _ in range(3):  # a new graph's first replays run slower
        graph.replay()

    def timed():
        for _ in range(steps // 2):
            graph.replay()

    us = gpu_span_us(torch, timed) / (steps // 2 * 2)
    assert lib.status() == lib.OK
    return us


def gather_bytes(tp, m, s, copy=True):
    """Algorithmic bytes: gather_push of all TP slots reads and writes M*S words per
    slot; gather_poll reads the M*TP*S gathered words and, with copy, writes them out
    and writes the sentinel back."""
    words = tp * m * s
    return 2 * words * 4, (3 if copy else 1) * words * 4


def time_gather(lib, torch, calls=2000, chunk=200, name="gather_tp8_m32", one_launch=True, m=None):
    """µs per Gather call, graph-replayed: gather_push_poll (every rank's push and the
    copying poll, one launch for calls within 32 MiB of gathered rows), or with one_launch False the pair
    gather_push + gather_poll.  gather_tp8_m32 is TP=8, M=32, S=896; ctx and logits are the
    drafter's context-projection and lm_head shapes; m overrides the row count."""
    import dataclasses

    from tp_all_reduce_arnorm_amd import workloads as wl

    cfg = wl.CONFIGS[name] if m is None else dataclasses.replace(wl.CONFIGS[name], m=m)
    words = wl.gather_shards(cfg) if name == "gather_tp8_m32" else wl.bf16_shards(cfg)
    shards = torch.from_numpy(words.view(np.int32)).cuda()
    box = torch.empty((cfg.cap, cfg.tp * cfg.s), dtype=torch.int32, device="cuda")
    assert lib.lamport_arm(box) is True
    out = torch.empty((cfg.m, cfg.tp * cfg.s), dtype=torch.int32, device="cuda")

    def call():
        if one_launch:
            assert lib.gather_push_poll(shards, box, out=out, copy=True) is True
            return
        assert lib.gather_push(shards, box, cfg.tp, 0) is True
        assert lib.gather_poll(box, cfg.tp, cfg.m, out=out, copy=True) is True

    for _ in range(4):
        call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(chunk):
            call()
    for _ in range(3):  # a new graph's first replays run slower
        g.replay()

    def timed():
        for _ in range(calls // chunk):
            g.replay()

    us = gpu_span_us(torch, timed) / (calls // chunk * chunk)
    assert lib.status() == lib.OK
    return cfg, us


def twoshot_bytes(tp, m, width=HIDDEN):
    """Algorithmic bytes of the two-shot owner's reduce (TP slot reads, TP re-arm writes,
    the gather row) and of one read of the gather row (read, copy out, re-arm)."""
    row = width * 2
    return 2 * tp * m * row + m * row, 3 * m * row


def time_twoshot(lib, torch, calls=2000, chunk=200, launches=20, modes=("cold", "warm")):
    """Two-shot stand-in: µs per graph-replayed call at TP=8, M=4 (push of 8 slots,
    owner's reduce, read of the gather row) as one twoshot_push_reduce_read launch and
    as the three launches, and the reduce / read kernels at M=4096 (cold and warm, as
    in time_roofline)."""
    from tp_all_reduce_arnorm_amd import workloads as wl

    res = {}
    cfg = wl.CONFIGS["tp8_m4"]
    src = wl.ArNormInputs(cfg)
    recv = torch.empty((2, 8, cfg.cap, HIDDEN // 2), dtype=torch.int32, device="cuda")
    gath = torch.empty((2, 1, cfg.cap, HIDDEN // 2), dtype=torch.int32, device="cuda")
    assert lib.lamport_arm(recv) is True and lib.lamport_arm(gath) is True
    parts = [torch.from_numpy(src.partials().view(np.int16)).cuda() for _ in range(2)]
    outs = [torch.empty((cfg.m, HIDDEN), dtype=torch.int16, device="cuda") for _ in range(2)]

    def call(i, one_launch):
        p = i % 2
        if one_launch:
            assert lib.twoshot_push_reduce_read(parts[p], recv, gath, p, outs[p]) is True
            return
        assert lib.twoshot_push(parts[p], recv, p, 0) is True
        assert lib.twoshot_reduce(recv, gath, p, cfg.m) is True
        assert lib.twoshot_read(gath, p, outs[p]) is True

    for key, one_launch in (("us_per_call_m4", True), ("three_launch_us_per_call_m4", False)):
        for i in range(4):
            call(i, one_launch)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(chunk):
                call(i, one_launch)
        for _ in range(3):  # a new graph's first replays run slower
            g.replay()

        def timed():
            for _ in range(calls // chunk):
                g.replay()

        res[key] = gpu_span_us(torch, timed) / (calls // chunk * chunk)
        del g

    cfg = wl.CONFIGS["tp8_m4096"]
    p5 = torch.from_numpy(wl.ArNormInputs(cfg).partials().view(np.int16)).cuda()
    recv = torch.empty((1, 8, cfg.cap, HIDDEN // 2), dtype=torch.int32, device="cuda")
    gath = torch.empty((1, 1, cfg.cap, HIDDEN // 2), dtype=torch.int32, device="cuda")
    assert lib.lamport_arm(recv) is True and lib.lamport_arm(gath) is True
    out = torch.empty((cfg.m, HIDDEN), dtype=torch.int16, device="cuda")
    evict = torch.ones(1 << 28, dtype=torch.float32, device="cuda") if "cold" in modes else None
    for mode in modes:  # as time_roofline: "cold" evicts the last-level cache before each timed launch
        red, rd = [], []
        for i in range(launches + 3):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            assert lib.twoshot_push(p5, recv, 0, 0) is True
            if mode == "cold":
                evict.sum()
            e[0].record()
            assert lib.twoshot_reduce(recv, gath, 0, cfg.m) is True
            e[1].record()
            if mode == "cold":
                evict.sum()
            e[2].record()
            assert lib.twoshot_read(gath, 0, out) is True
            e[3].record()
            if i >= 3:
                red.append((e[0], e[1]))
                rd.append((e[2], e[3]))
        torch.cuda.synchronize()
        assert lib.status() == lib.OK
        sfx = "" if mode == "cold" else "_warm"
        res["reduce_us_m4096" + sfx] = float(np.mean([a.elapsed_time(b) for a, b in red])) * 1e3
        res["read_us_m4096" + sfx] = float(np.mean([a.elapsed_time(b) for a, b in rd])) * 1e3
    return res


def time_roofline(lib, torch, launches=20, modes=("cold", "warm"), steady_calls=0):
    """Consumer and producer kernels at TP=8, M=4096 with residual, each launch timed
    with HIP events on the launch stream.  "cold": before every timed launch a 1 GiB
    read-only pass over an unrelated buffer leaves MI355X's 256 MB last-level cache
    holding clean lines of that buffer, so the kernel's bytes come from HBM.  "warm": the
    push and the consumer back to back, as the call runs, where the consumer finds part of
    what the push just wrote still in that cache.  Returns cfg and {mode: (reduce_us,
    push_us)}; with steady_calls, also "steady": µs per call of that many push + consumer
    pairs back to back, timed as a whole (the stand-in call at this size as it repeats,
    each kernel paying for the lines the previous one left dirty in the cache)."""
    from tp_all_reduce_arnorm_amd import workloads as wl

    cfg = wl.CONFIGS["tp8_m4096"]
    src = wl.ArNormInputs(cfg)
    p, r = src.call()
    box = torch.empty((1, cfg.tp, cfg.cap, HIDDEN // 2), dtype=torch.int32, device="cuda")
    assert lib.lamport_arm(box) is True
    p_d = torch.from_numpy(p.view(np.int16)).cuda()
    r_d = torch.from_numpy(r.view(np.int16)).cuda()
    g_d = torch.from_numpy(src.gamma.view(np.int16)).cuda()
    del p, r
    out = torch.empty((cfg.m, HIDDEN), dtype=torch.int16, device="cuda")
    rout = torch.empty((cfg.m, HIDDEN), dtype=torch.int16, device="cuda")
    evict = torch.ones(1 << 28, dtype=torch.float32, device="cuda") if "cold" in modes else None
    res = {}
    for mode in modes:
        red, push = [], []
        for i in range(launches + 3):
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            if mode == "cold":
                evict.sum()
            a0.record()
            assert lib.arnorm_push(p_d, box, 0, 0) is True
            a1.record()
            if mode == "cold":
                evict.sum()
            b0.record()
            assert lib.arnorm_reduce_norm(r_d, g_d, box, 0, EPS, out, rout) is True
            b1.record()
            if i >= 3:
                push.append((a0, a1))
                red.append((b0, b1))
        torch.cuda.synchronize()
        assert lib.status() == lib.OK
        res[mode] = (float(np.mean([a.elapsed_time(b) for a, b in red])) * 1e3,
                     float(np.mean([a.elapsed_time(b) for a, b in push])) * 1e3)
    if steady_calls:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steady_calls):
            assert lib.arnorm_push(p_d, box, 0, 0) is True
            assert lib.arnorm_reduce_norm(r_d, g_d, box, 0, EPS, out, rout) is True
        e1.record()
        torch.cuda.synchronize()
        assert lib.status() == lib.OK
        res["steady"] = e0.elapsed_time(e1) * 1e3 / steady_calls
    return cfg, res


def pmc_workload(lib, torch, launches=3):
    """What the rocprofv3 counter runs profile: the consumer and producer kernels at
    TP=8, M=4096 with residual, and a plain 1 GiB device copy (torch's copy kernel)
    whose FETCH_SIZE / WRITE_SIZE calibrate the counters against known bytes."""
    cfg, t = time_roofline(lib, torch, launches=launches, modes=("warm",))
    red_us, push_us = t["warm"]
    # the two-shot owner's reduce and the gather-row read at the same size
    from tp_all_reduce_arnorm_amd import workloads as wl

    p5 = torch.from_numpy(wl.ArNormInputs(cfg).partials().view(np.int16)).cuda()
    recv = torch.empty((1, cfg.tp, cfg.cap, HIDDEN // 2), dtype=torch.int32, device="cuda")
    gath = torch.empty((1, 1, cfg.cap, HIDDEN // 2), dtype=torch.int32, device="cuda")
    out = torch.empty((cfg.m, HIDDEN), dtype=torch.int16, device="cuda")
    assert lib.lamport_arm(recv) is True and lib.lamport_arm(gath) is True
    for _ in range(launches):
        assert lib.twoshot_push(p5, recv, 0, 0) is True
        assert lib.twoshot_reduce(recv, gath, 0, cfg.m) is True
        assert lib.twoshot_read(gath, 0, out) is True
    torch.cuda.synchronize()
    assert lib.status() == lib.OK
    del p5, recv, gath, out
    n = 1 << 28  # int32 elements: 1 GiB
    a = torch.ones(n, dtype=torch.int32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(launches):
        b.copy_(a)
    torch.cuda.synchronize()
    return {"reduce_us": red_us, "push_us": push_us, "copy_bytes": n * 4}


def cpu_model():
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def _oracle_arnorm_call(oracle, box, p, r, gamma, parity, m):
    oracle.arnorm_push(box, p, parity, 0)
    oracle.arnorm_reduce_norm(box, parity, m, r, gamma, EPS)


def cpu_baseline(headline_s=3.0):
    """The oracle (numpy, one thread) timed on this host, per workload: the same calls
    the GPU runs, inputs drawn before each timed call (not timed).  ArNorm workloads
    time oracle.arnorm_push of every slot + oracle.arnorm_reduce_norm; gather_tp8_m32
    times oracle.gather_push of the 8 shards + oracle.gather_poll with copy.  Median of
    5 calls (3 at tp8_m4096, whole 4096-row calls), and for tp8_m4, the headline
    workload, of as many calls as fit in ``headline_s`` seconds (at least 5).  Returns
    {workload: {"us_per_call", "calls", "algorithmic_gbps"}}."""
    import oracle
    from tp_all_reduce_arnorm_amd import workloads as wl

    res = {}
    for name, runs in (("tp2_m1", 5), ("tp8_m4", 5), ("tp8_m64", 5), ("tp8_m4096", 3)):
        cfg = wl.CONFIGS[name]
        src = wl.ArNormInputs(cfg)
        box = oracle.arm(np.empty((cfg.parities, cfg.tp, cfg.cap, HIDDEN // 2), dtype=np.uint32))
        times = []
        start = time.perf_counter()
        i = 0
        while i < runs or (name == "tp8_m4" and time.perf_counter() - start < headline_s):
            p, r = src.call()
            t0 = time.perf_counter()
            _oracle_arnorm_call(oracle, box, p, r, src.gamma, i % cfg.parities, cfg.m)
            times.append(time.perf_counter() - t0)
            i += 1
        del box
        us = float(np.median(times)) * 1e6
        nbytes = push_bytes(cfg.tp, cfg.m) + reduce_bytes(cfg.tp, cfg.m, cfg.residual)
        res[name] = {"us_per_call": round(us, 1), "calls": len(times),
                     "algorithmic_gbps": round(nbytes / (us * 1e-6) / 1e9, 3)}
    cfg = wl.CONFIGS["gather_tp8_m32"]
    shards = wl.gather_shards(cfg)
    gbox = oracle.arm(np.empty((cfg.cap, cfg.tp * cfg.s), dtype=np.uint32))
    times = []
    for _ in range(5):
        t0 = time.perf_counter()
        oracle.gather_push(gbox, shards, 0)
        oracle.gather_poll(gbox, cfg.m, True)
        times.append(time.perf_counter() - t0)
    us = float(np.median(times)) * 1e6
    res["gather_tp8_m32"] = {"us_per_call": round(us, 1), "calls": len(times),
                             "algorithmic_gbps": round(sum(gather_bytes(cfg.tp, cfg.m, cfg.s)) / (us * 1e-6) / 1e9, 3)}
    return res


# -- rocprofv3 summaries (run on the CSVs a profiled run wrote) ----------------------

PROFILE_COMMANDS = {
    "lat": "rocprofv3 --kernel-trace --stats -f csv -d prof_out/prof_lat -o lat -- "
           "python bench.py --mode latency --steps 2000 > prof_out/prof_lat.log 2>&1",
    "roof": "rocprofv3 --kernel-trace --stats -f csv -d prof_out/prof_roof -o roof -- "
            "python bench.py --mode roofline > prof_out/prof_roof.log 2>&1",
    "gather": "rocprofv3 --kernel-trace --stats -f csv -d prof_out/prof_gather -o gather -- "
              "python bench.py --mode gather > prof_out/prof_gather.log 2>&1",
    "twoshot": "rocprofv3 --kernel-trace --stats -f csv -d prof_out/prof_twoshot -o twoshot -- "
               "python bench.py --mode twoshot > prof_out/prof_twoshot.log 2>&1",
    "fetch": "rocprofv3 --pmc FETCH_SIZE -f csv -d prof_out/pmc_fetch -o fetch -- "
             "python bench.py --mode pmc > prof_out/pmc_fetch.log 2>&1",
    "write": "rocprofv3 --pmc WRITE_SIZE -f csv -d prof_out/pmc_write -o write -- "
             "python bench.py --mode pmc > prof_out/pmc_write.log 2>&1",
}


def _profiled_record(log_path):
    """The JSON record that a profiled bench run printed (None if absent)."""
    try:
        for ln in open(log_path, errors="replace"):
            if ln.startswith('{"mode"'):
                return json.loads(ln)
    except OSError:
        pass
    return None


def _profiled_sha(log_path):
    """The kernel-sources hash that a profiled bench run printed (None if absent)."""
    rec = _profiled_record(log_path)
    return rec.get("sources_sha") if rec else None


def _short(name):
    return name.split("(")[0].replace("void ", "")


def _trace_medians(path):
    """Median duration in ns per kernel name from a rocprofv3 kernel-trace CSV (None if
    the file is absent)."""
    import csv

    if not os.path.exists(path):
        return None
    durs = {}
    with open(path) as f:
        rd = csv.DictReader(f)
        if not {"Kernel_Name", "Start_Timestamp", "End_Timestamp"} <= set(rd.fieldnames or ()):
            return None
        for r in rd:
            durs.setdefault(r["Kernel_Name"], []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return {k: float(np.median(v)) for k, v in durs.items()}


def _shape_table(trace_path):
    """Per launch shape (kernel, grid, workgroup) of this library's kernels: calls, median
    and average duration, from a rocprofv3 kernel-trace CSV; None without one."""
    import csv

    if not trace_path or not os.path.exists(trace_path):
        return None
    durs = {}
    with open(trace_path) as f:
        rd = csv.DictReader(f)
        need = {"Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Workgroup_Size_X"}
        if not need <= set(rd.fieldnames or ()):
            return None
        for r in rd:
            if "arn::" not in r["Kernel_Name"]:
                continue
            key = (_short(r["Kernel_Name"]), int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]))
            durs.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out = ["| kernel | grid (threads) | workgroup | calls | median µs | average µs |", "|---|---|---|---|---|---|"]
    for (name, grid, wg), v in sorted(durs.items(), key=lambda kv: (kv[0][0], kv[0][1])):
        out.append(f"| `{name}` | {grid} | {wg} | {len(v)} | {np.median(v) / 1e3:.2f} | {np.mean(v) / 1e3:.2f} |")
    return "\n".join(out)


def _stats_table(path, trace_path=None):
    import csv

    rows = list(csv.DictReader(open(path)))
    med = _trace_medians(trace_path) if trace_path else None
    head = "| kernel | calls | average µs | " + ("median µs | " if med else "") + "min µs | max µs | share of GPU time |"
    out = [head, "|---" * (head.count("|") - 1) + "|"]
    for r in rows:
        m = f"{med[r['Name']] / 1e3:.2f} | " if med and r["Name"] in med else ("– | " if med else "")
        out.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {m}"
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} % |")
    return rows, "\n".join(out)


def summarize_profiles(outdir):
    """Write profiles/*.md and profiles/hbm_traffic.json from the CSVs of the four
    profiled runs in PROFILE_COMMANDS (a directory laid out as those commands write)."""
    import csv

    prof = os.path.join(ROOT, "profiles")
    os.makedirs(prof, exist_ok=True)
    for key, title, fname in (
            ("lat", "Stand-in ArNorm call at TP=8, M=4, no residual, HIP-graph replay: 2000 calls of one "
                    "arnorm_push_reduce_norm launch each (the 8 ranks' pushes and the consumer, rows split "
                    "7 ways through the norm box), then 2000 calls as the pair arnorm_push of 8 slots + "
                    "arnorm_reduce_norm, then 2000 arnorm_push_reduce_norm calls at M=1 (one launch) and "
                    "2000 at M=64 (one launch, rows split 4 ways)", "arnorm_tp8_m4_kernel_stats.md"),
            ("roof", "ArNorm kernels at TP=8, M=4096, residual: one push of 8 slots + one consumer launch, "
                     "23 times, each launch after a 1 GiB read-only pass (torch's float32 sum) that evicts the "
                     "last-level cache", "arnorm_tp8_m4096_kernel_stats.md"),
            ("gather", "Gather at TP=8, S=896 words, cap=64, HIP-graph replay: 2000 gather_push_poll calls "
                       "at M=32 (917504 B, within the 32 MiB one-launch limit, so one launch each), 2000 calls "
                       "of the pair gather_push of 8 slots + gather_poll with copy at M=32, then 2000 "
                       "one-launch gather_push_poll calls at M=4",
             "gather_tp8_m32_s896_kernel_stats.md"),
            ("twoshot", "Two-shot all-reduce stand-in (owners = 1): TP=8, M=4 graph-replayed calls, 2000 as "
                        "one twoshot_push_reduce_read launch each, then 2000 as the three launches (push, "
                        "owner's reduce, read), then 23 calls at TP=8, M=4096 whose reduce and read each follow "
                        "a 1 GiB read-only pass (torch's float32 sum) that evicts the last-level cache",
             "twoshot_tp8_kernel_stats.md")):
        if not os.path.exists(os.path.join(outdir, f"prof_{key}", f"{key}_kernel_stats.csv")):
            continue
        rows, table = _stats_table(os.path.join(outdir, f"prof_{key}", f"{key}_kernel_stats.csv"),
                                   os.path.join(outdir, f"prof_{key}", f"{key}_kernel_trace.csv"))
        rec = _profiled_record(os.path.join(outdir, f"prof_{key}.log")) or {}
        sha = rec.get("sources_sha")
        shapes = _shape_table(os.path.join(outdir, f"prof_{key}", f"{key}_kernel_trace.csv")) \
            if key in ("lat", "gather") else None
        with open(os.path.join(prof, fname), "w") as f:
            f.write(f"# rocprofv3 kernel statistics: {title}\n\n"
                    f"Command, from the repository root on one MI355X:\n\n    {PROFILE_COMMANDS[key]}\n\n"
                    f"Kernel sources sha256[:16] = `{sha}`.\n\n{table}\n")
            if shapes:
                which = "M=1, 4 and 64" if key == "lat" else "M=32 and M=4"
                f.write(f"\nThe library's kernels by launch shape (grid size in threads; {which} launch "
                        f"different grids):\n\n{shapes}\n")
            if key == "lat" and rec:
                f.write("\nThe same profiled run's own figures, HIP events on the stream over the graph replays "
                        "(µs per call, the profiler attached): " +
                        ", ".join(f"{k} {v:.3f}" for k, v in rec.items() if k.endswith("per_call")) + "\n")

    def counters(key):
        path = os.path.join(outdir, f"pmc_{key}", f"{key}_counter_collection.csv")
        return list(csv.DictReader(open(path)))

    fetch, write = counters("fetch"), counters("write")
    sha = _profiled_sha(os.path.join(outdir, "pmc_fetch.log"))
    if sha is None or sha != _profiled_sha(os.path.join(outdir, "pmc_write.log")):
        raise SystemExit("the two counter runs do not name the same kernel sources")

    def calib(rows):
        copies = [r for r in rows if "copyBuffer" in r["Kernel_Name"]]
        big = max(int(r["Grid_Size"]) for r in copies)
        vals = [float(r["Counter_Value"]) for r in copies if int(r["Grid_Size"]) == big]
        return (1 << 30) / 1024 / float(np.mean(vals)), float(np.mean(vals))

    f_scale, f_raw = calib(fetch)
    w_scale, w_raw = calib(write)

    def per_launch(rows, pattern):
        vals = [float(r["Counter_Value"]) for r in rows if pattern in r["Kernel_Name"]]
        return float(np.mean(vals)), len(vals)

    kernels = (("reduce_norm_tp8_m4096_res", "reduce_norm_kernel<8, true, false, 896", reduce_bytes(8, 4096, True)),
               ("push_tp8_m4096", "push_kernel", push_bytes(8, 4096)),
               ("twoshot_reduce_tp8_m4096", "twoshot_reduce_kernel<8", twoshot_bytes(8, 4096)[0]),
               ("twoshot_read_m4096", "gather_poll_kernel", twoshot_bytes(8, 4096)[1]))
    rec, lines = {}, []
    for key, pat, alg in kernels:
        fr, n = per_launch(fetch, pat)
        wr, _ = per_launch(write, pat)
        rd, wt = fr * 1024 * f_scale, wr * 1024 * w_scale
        rec[key] = {"bytes_per_launch": round(rd + wt), "read_bytes": round(rd), "write_bytes": round(wt),
                    "algorithmic_bytes": alg, "sources_sha": sha, "launches": n}
        lines.append(f"| `{pat.split('<')[0]}` ({key}) | {fr:,.1f} | {rd / 1e6:,.1f} | {wr:,.1f} | {wt / 1e6:,.1f} | "
                     f"{(rd + wt) / 1e6:,.1f} | {alg / 1e6:,.1f} | {(rd + wt) / alg:.4f} |")
    with open(os.path.join(prof, "hbm_traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)
    with open(os.path.join(prof, "arnorm_tp8_m4096_hbm_traffic.md"), "w") as f:
        f.write("# HBM traffic per launch from rocprofv3 counters: TP=8, M=4096 (ArNorm with residual; "
                "the two-shot stand-in)\n\n"
                "Commands, from the repository root on one MI355X (two runs, one counter each):\n\n"
                f"    {PROFILE_COMMANDS['fetch']}\n    {PROFILE_COMMANDS['write']}\n\n"
                f"Kernel sources sha256[:16] = `{sha}`.\n\n"
                "Calibration: the same runs copy 1 GiB device to device (`__amd_rocclr_copyBuffer`, the largest "
                f"grid). It reads FETCH_SIZE = {f_raw:,.1f} KiB and WRITE_SIZE = {w_raw:,.1f} KiB for 1,048,576 KiB "
                f"moved each way, so bytes = FETCH_SIZE x 1024 x {f_scale:.4f} and WRITE_SIZE x 1024 x {w_scale:.4f}.\n\n"
                "| kernel | FETCH_SIZE KiB | read MB | WRITE_SIZE KiB | written MB | total MB | algorithmic MB | "
                "total / algorithmic |\n|---|---|---|---|---|---|---|---|\n" + "\n".join(lines) + "\n")
    print(json.dumps(rec))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20000)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--cpu-seconds", type=float, default=3.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", choices=["full", "latency", "roofline", "pmc", "gather", "twoshot"], default="full",
                    help="latency / roofline / pmc run one part only (for profiler runs)")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write profiles/ summaries from the CSVs of the profiled runs under DIR")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
    if args.gpus != 1:
        print(f"bench.py: this benchmark runs on one GPU; the TP ranks are mailbox slots of "
              f"one MI355X (--gpus {args.gpus} is not supported)", file=sys.stderr)
        sys.exit(2)

    import torch
    from tp_all_reduce_arnorm_amd import _lib as lib

    torch.cuda.set_device(0)
    sha = kernel_sources_hash()
    if args.mode == "latency":
        calls = max(args.steps, MIN_TIMED_CALLS)
        elapsed = time_latency(lib, torch, calls, args.warmup)
        pair = time_latency(lib, torch, calls, args.warmup, one_launch=False)
        m_us = {f"m{m}_us_per_call": time_latency(lib, torch, calls, args.warmup, m=m) / calls * 1e6
                for m in (1, 64)}
        print(json.dumps({"mode": "latency", "us_per_call": elapsed / calls * 1e6,
                          "two_launch_us_per_call": pair / calls * 1e6, **m_us, "sources_sha": sha}),
              flush=True)
        return
    if args.mode == "roofline":
        _, t = time_roofline(lib, torch, modes=("cold",))
        print(json.dumps({"mode": "roofline", "reduce_us": t["cold"][0], "push_us": t["cold"][1],
                          "sources_sha": sha}), flush=True)
        return
    if args.mode == "gather":
        _, us = time_gather(lib, torch)
        _, pair_us = time_gather(lib, torch, one_launch=False)
        _, m4_us = time_gather(lib, torch, m=4)
        print(json.dumps({"mode": "gather", "us_per_call": us, "two_launch_us_per_call": pair_us,
                          "m4_one_launch_us_per_call": m4_us, "sources_sha": sha}), flush=True)
        return
    if args.mode == "twoshot":
        print(json.dumps(dict(mode="twoshot", sources_sha=sha, **time_twoshot(lib, torch, modes=("cold",)))),
              flush=True)
        return
    if args.mode == "pmc":
        print(json.dumps(dict(mode="pmc", sources_sha=sha, **pmc_workload(lib, torch))), flush=True)
        return
    calls = max(args.steps, MIN_TIMED_CALLS)
    elapsed = time_latency(lib, torch, calls, args.warmup)
    pair_us = time_latency(lib, torch, calls, args.warmup, one_launch=False) / calls * 1e6
    m_us = {m: time_latency(lib, torch, calls, args.warmup, m=m) / calls * 1e6 for m in (1, 64)}
    cfg5, troof = time_roofline(lib, torch, steady_calls=20)
    red_us, push_us = troof["cold"]
    warm_red_us, warm_push_us = troof["warm"]
    cfg4, gather_us = time_gather(lib, torch)
    _, gather_pair_us = time_gather(lib, torch, one_launch=False)
    ts = time_twoshot(lib, torch)
    step_us = time_drafter_step(lib, torch)
    work = {}
    for name in ("tp2_m1", "tp8_m4", "tp8_m64"):
        c, us = time_config(lib, torch, name)
        nb = push_bytes(c.tp, c.m) + reduce_bytes(c.tp, c.m, c.residual)
        work[name] = {"tp": c.tp, "m": c.m, "residual": c.residual, "parities": c.parities, "cap": c.cap,
                      "us_per_call": round(us, 3), "algorithmic_bytes": nb,
                      "algorithmic_gbps": round(nb / (us * 1e-6) / 1e9, 1)}
    shapes = {}
    for name in ("ctx", "logits"):
        c, us = time_gather(lib, torch, name=name)
        _, pus = time_gather(lib, torch, name=name, one_launch=False)
        shapes[name] = {"tp": c.tp, "m": c.m, "s_words": c.s, "us_per_call": round(us, 3),
                        "two_launch_us_per_call": round(pus, 3),
                        "push_algorithmic_bytes": gather_bytes(c.tp, c.m, c.s)[0],
                        "poll_algorithmic_bytes": gather_bytes(c.tp, c.m, c.s)[1]}
    for key, name, m in (("gather_tp8_m4", "gather_tp8_m32", 4), ("logits_m1", "logits", 1)):  # one launch
        c, us = time_gather(lib, torch, name=name, m=m)
        _, pus = time_gather(lib, torch, name=name, m=m, one_launch=False)
        shapes[key] = {"tp": c.tp, "m": c.m, "s_words": c.s, "us_per_call": round(us, 3),
                                  "two_launch_us_per_call": round(pus, 3)}
    tsr, tsq = twoshot_bytes(8, 4096)
    gpb, gqb = gather_bytes(cfg4.tp, cfg4.m, cfg4.s)
    rb = reduce_bytes(cfg5.tp, cfg5.m, True)
    pb = push_bytes(cfg5.tp, cfg5.m)
    achieved = rb / (red_us * 1e-6) / 1e9
    traffic = committed_traffic("reduce_norm_tp8_m4096_res")
    cpu = None
    if not args.no_cpu_baseline:
        per = cpu_baseline(args.cpu_seconds)
        head = per["tp8_m4"]
        cpu = {"value": head["us_per_call"], "unit": "µs/call", "cores": 1, "kind": "oracle",
               "sample": f"{head['calls']} oracle calls (push of 8 slots + reduce_norm) at TP=8, M=4, no "
                         f"residual, median; and per workload in `workloads` (median of 5 calls, 3 whole "
                         f"4096-row calls at tp8_m4096); {os.cpu_count()} host CPUs visible ({cpu_model()}), "
                         f"numpy on one thread",
               "algorithmic_gbps": head["algorithmic_gbps"], "workloads": per}
    us_per_call = elapsed / calls * 1e6
    rec = {
        "metric": METRIC,
        "value": round(us_per_call, 3),
        "unit": "µs/call",
        "n_gpus": 1,
        "steps": args.steps,
        "timed_calls": calls,
        "warmup": args.warmup,
        "ms_per_step": round(us_per_call * 1e-3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "io_dtype": "bf16: BF16 rows in and out, FP32 adds, products and norm, one BF16 rounding per stage",
        "data": "synthetic",
        "config": {
            "workload": "ArNorm TP=8 M=4 width 7168, residual=False, 2 parities alternating: one "
                        "arnorm_push_reduce_norm per call (the 8 ranks' pushes and the consumer in one "
                        "launch, rows split over 7 workgroups through the norm box); HIP-graph replay, "
                        "max(steps, 2000) calls timed with HIP events on the stream",
            "tp": 8, "m": 4, "hidden": HIDDEN, "parities": 2, "residual": False,
            "two_launch_us_per_call": round(pair_us, 3),
            "m1_us_per_call": round(m_us[1], 3), "m64_us_per_call": round(m_us[64], 3),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
            "kernel": "arnorm_reduce_norm",
            "workload": "ArNorm TP=8 M=4096 width 7168, residual=True",
            "algorithmic_bytes": rb,
            "kernel_us": round(red_us, 2),
            "cache": "cold: before each timed launch a 1 GiB read of an unrelated buffer leaves the 256 MB "
                     "last-level cache holding none of the kernel's data, so its bytes come from HBM",
            "warm": {"kernel_us": round(warm_red_us, 2),
                     "algorithmic_frac_of_hbm_peak": round(rb / (warm_red_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
                     "note": "right after the push, as the call runs: part of the slots the push just wrote "
                             "are still in the last-level cache, so this is algorithmic bytes per time with "
                             "cache hits included, not a fraction of HBM bandwidth"},
            "call": {"us_per_call": round(troof["steady"], 2), "algorithmic_bytes": rb + pb,
                     "algorithmic_gbps": round((rb + pb) / (troof["steady"] * 1e-6) / 1e9, 1),
                     "algorithmic_frac_of_hbm_peak": round((rb + pb) / (troof["steady"] * 1e-6) / 1e9
                                                           / PEAK_HBM_GBPS, 4),
                     "note": "the whole stand-in call at this size, push of 8 slots + consumer, 20 calls back "
                             "to back timed as one span: algorithmic bytes per time, last-level cache hits "
                             "included (the consumer reads part of what the push just wrote from the 256 MB "
                             "cache), so not a fraction of HBM bandwidth; each kernel also writes back what "
                             "the previous one left dirty in the cache"},
        },
        "push": {
            "kernel": "arnorm_push", "workload": "8 slots, M=4096, cold as the roofline", "algorithmic_bytes": pb,
            "kernel_us": round(push_us, 2), "achieved_gbps": round(pb / (push_us * 1e-6) / 1e9, 1),
            "frac": round(pb / (push_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
            "warm": {"kernel_us": round(warm_push_us, 2),
                     "algorithmic_frac_of_hbm_peak": round(pb / (warm_push_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
                     "note": "right after the previous consumer, whose written lines the cache still holds"},
        },
        "gather": {
            "workload": "Gather TP=8 M=32 S=896 words cap=64: gather_push_poll with copy, HIP-graph replay "
                        "(917504 B of gathered rows, within the 32 MiB one-launch limit, so every rank's push "
                        "and the pollers run as one launch, as do all drafter_shapes entries); "
                        "two_launch_us_per_call is the pair gather_push + gather_poll",
            "us_per_call": round(gather_us, 3), "two_launch_us_per_call": round(gather_pair_us, 3),
            "push_algorithmic_bytes": gpb, "poll_algorithmic_bytes": gqb,
            "drafter_shapes": shapes,
        },
        "twoshot": {
            "workload": "two-shot all-reduce, owners = 1: push of 8 slots + owner's reduce + read of the "
                        "gather row; TP=8 M=4 graph-replayed as one twoshot_push_reduce_read launch per "
                        "call (and as the three launches), and the kernels at TP=8 M=4096, cold as the "
                        "roofline (warm: right after the push / the reduce)",
            "us_per_call_m4": round(ts["us_per_call_m4"], 3),
            "three_launch_us_per_call_m4": round(ts["three_launch_us_per_call_m4"], 3),
            "reduce_us_m4096": round(ts["reduce_us_m4096"], 2),
            "reduce_frac": round(tsr / (ts["reduce_us_m4096"] * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
            "read_us_m4096": round(ts["read_us_m4096"], 2),
            "read_frac": round(tsq / (ts["read_us_m4096"] * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
            "warm_reduce_frac": round(tsr / (ts["reduce_us_m4096_warm"] * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
            "warm_read_frac": round(tsq / (ts["read_us_m4096_warm"] * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
            "reduce_algorithmic_bytes": tsr, "read_algorithmic_bytes": tsq,
        },
        "drafter_step": {
            "workload": "the collectives of one drafter decode step at TP=8, HIP-graph replay: 11 one-launch "
                        "ArNorm calls at M=4 (the first without a residual, the others chaining the new "
                        "residual in place), the context-projection Gather (M=64, S=448 words) and the "
                        "lm_head logits Gather (M=4, S=10240 words)",
            "us_per_step": round(step_us, 2),
            "context": "the pages quote 6-9 us per stock one-shot all-reduce (11 per step) and 16-20 us per "
                       "stock all-gather (2 per step) on their NVLink hardware: another machine's figures",
        },
        "workloads": {
            "note": "the named configurations as they are stated (TP, M, residual, capacity, parities), one "
                    "arnorm_push_reduce_norm per call, graph-replayed, HIP events; algorithmic bytes are the "
                    "push of every slot plus the consumer's, per call; the Gather configuration is `gather`, "
                    "the M=4096 one `roofline` and `push`",
            **work,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
