"""arnorm_push_reduce_norm_static, the entry point that allocates nothing (its norm box is
the library's static device array), against arnorm_push_reduce_norm with a norm box the
caller allocated: the same inputs give the same bits, on calls in a row with fewer rows
each time (M = 64, rows split 4 ways; M = 8 and 2, 7 ways; one launch each), and the
array's row limit is refused before anything is launched."""

import numpy as np
import pytest

from tests.gpu_util import armed_box, assert_bits_equal, dev16, empty16, host16, host32, say
from tp_all_reduce_arnorm_amd import workloads as wl

pytestmark = pytest.mark.gpu
W = 7168
EPS = 1e-6


def test_no_alloc_call_matches_the_call_with_a_norm_box(lib):
    import dataclasses

    say("[no-alloc] static-scratch ArNorm calls M=64, 8, 2 against the norm-box call")
    lib.set_reduce_split(0)
    shape = (2, 8, 64, W // 2)
    box_a, box_s = armed_box(shape), armed_box(shape)
    nbox = armed_box((2, 64, 256))
    for call, (m, residual) in enumerate(((64, True), (8, False), (2, True))):
        cfg = dataclasses.replace(wl.CONFIGS["tp8_m64"], m=m, residual=residual, seed=500 + call)
        src = wl.ArNormInputs(cfg)
        p, r = src.call()
        p_d, g_d = dev16(p), dev16(src.gamma)
        r_d = dev16(r) if residual else None
        parity = call % 2
        outs = [(empty16((m, W)), empty16((m, W))) for _ in range(2)]
        assert lib.arnorm_push_reduce_norm(p_d, r_d, g_d, box_a, parity, EPS, outs[0][0], outs[0][1],
                                           norm_box=nbox) is True
        assert lib.arnorm_push_reduce_norm_static(p_d, r_d, g_d, box_s, parity, EPS, outs[1][0], outs[1][1]) is True
        assert lib.status() == lib.OK
        assert_bits_equal(host16(outs[1][1]), host16(outs[0][1]), f"call {call} (M={m}) residual_out")
        assert_bits_equal(host16(outs[1][0]), host16(outs[0][0]), f"call {call} (M={m}) out")
        assert_bits_equal(host32(box_s), host32(box_a), f"call {call} (M={m}) mailbox")
    assert np.all(host32(nbox) == 0x80000000)


def test_no_alloc_call_refuses_rows_beyond_its_scratch(lib):
    say("[no-alloc] M=65 refused")
    box = armed_box((1, 8, 65, W // 2))
    p_d = dev16(np.zeros((8, 65, W), dtype=np.uint16))
    g_d = dev16(np.full(W, 0x3F80, dtype=np.uint16))
    with pytest.raises(lib.ArnormError) as e:
        lib.arnorm_push_reduce_norm_static(p_d, None, g_d, box, 0, EPS, empty16((65, W)), empty16((65, W)))
    assert e.value.code == lib.TOO_LARGE
    assert np.all(host32(box) == 0x80000000), "nothing was launched"
