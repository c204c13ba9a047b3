import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def read_golden(name):
    """Non-comment, non-empty lines of a golden fixture."""
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.rstrip("\n") for ln in f if ln.strip() and not ln.lstrip().startswith("#")]


@pytest.fixture(scope="session")
def lib():
    """The built HIP library through its Python binding (GPU tests only)."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tp_all_reduce_arnorm_amd import _lib

    return _lib


def _streams_overlap(lib, s_wait, s_push):
    """Whether work on the two streams runs side by side: a tiny Gather poll is queued
    first on s_wait, its push (after a short delay) on s_push.  If the streams share a
    hardware queue the poll runs alone and ends at a short spin limit (TIMEOUT)."""
    import torch

    from tests.gpu_util import armed_box

    old = lib.get_spin_limit()
    lib.set_spin_limit(1 << 13)
    try:
        box = armed_box((1, 8))  # TP=2 ranks of S=4 words, one row
        shard = torch.ones((2, 1, 4), dtype=torch.int32, device="cuda")
        cur = torch.cuda.current_stream()
        torch.cuda.synchronize()
        s_wait.wait_stream(cur)
        s_push.wait_stream(cur)
        with torch.cuda.stream(s_wait):
            assert lib.gather_poll(box, 2, 1, copy=False) is True
        with torch.cuda.stream(s_push):
            torch.cuda._sleep(20000)
            assert lib.gather_push(shard, box, 2, 0) is True
        cur.wait_stream(s_wait)
        cur.wait_stream(s_push)
        torch.cuda.synchronize()
        return lib.status() == lib.OK
    finally:
        lib.set_spin_limit(old)


@pytest.fixture(scope="session")
def side_streams(lib):
    """Three streams, pairwise side by side, for the concurrent-mode tests (producer,
    consumer, reader).  HIP runs streams on a few hardware queues, and two streams that
    share one run their work in submission order, which would serialize a consumer
    launched first with the producer it waits for; so candidates are checked pairwise."""
    import torch

    chosen = []
    for _ in range(12):
        s = torch.cuda.Stream()
        if all(_streams_overlap(lib, c, s) and _streams_overlap(lib, s, c) for c in chosen):
            chosen.append(s)
        if len(chosen) == 3:
            return tuple(chosen)
    pytest.skip("no three streams whose work overlaps")
