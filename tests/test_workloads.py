"""The seeded workload generators produce the stated shapes, value distributions and
structure (sentinel words, rank-vs-tree rows)."""

import numpy as np

from oracle import bf16 as obf
from oracle import arnorm as oar
from tp_all_reduce_arnorm_amd import workloads as wl


def _tree_sum(slot_words):
    lanes = list(obf.widen(obf.unpack_pairs(slot_words)))
    while len(lanes) > 1:
        lanes = [(lanes[i] + lanes[i + 1]).astype(np.float32) for i in range(0, len(lanes), 2)]
    return obf.round_to_bf16(lanes[0])


def test_tp2_m1_shapes_and_distribution():
    cfg = wl.CONFIGS["tp2_m1"]
    src = wl.ArNormInputs(cfg)
    p, r = src.call()
    assert p.shape == (2, 1, 7168) and p.dtype == np.uint16
    assert r.shape == (1, 7168) and r.dtype == np.uint16
    v = obf.widen(p).astype(np.float64)
    assert abs(v.std() - 0.5) < 0.02
    g = obf.widen(src.gamma).astype(np.float64)
    assert abs(g.mean() - 1.0) < 0.01 and abs(g.std() - 0.1) < 0.01


def test_seeded_reproducible():
    a = wl.ArNormInputs(wl.CONFIGS["tp8_m4"]).call()[0]
    b = wl.ArNormInputs(wl.CONFIGS["tp8_m4"]).call()[0]
    assert np.array_equal(a, b)


def test_tp8_m4_no_residual():
    p, r = wl.ArNormInputs(wl.CONFIGS["tp8_m4"]).call()
    assert r is None and p.shape == (8, 4, 7168)
    assert abs(obf.widen(p).astype(np.float64).std() - 0.02) < 0.002


def test_tp8_m64_sentinel_and_tree_rows():
    cfg = wl.CONFIGS["tp8_m64"]
    src = wl.ArNormInputs(cfg)
    p, r = src.call()
    words = obf.pack_pairs(p)
    frac = np.mean(words == np.uint32(0x80000000))
    assert 0.04 < frac < 0.06
    assert np.all(r[48:64] == 0)
    slot_words = __import__("oracle").clean(words)
    rank = oar.allreduce_rows(slot_words)
    tree = _tree_sum(slot_words)
    for row in range(48, 64):
        assert np.any(rank[row] != tree[row]), row
    # rows outside the pattern are ordinary normals
    assert abs(obf.widen(p[:, :48]).astype(np.float64).std() - 0.5) < 0.05


def test_gather_tp8_m32_shards():
    cfg = wl.CONFIGS["gather_tp8_m32"]
    w = wl.gather_shards(cfg)
    assert w.shape == (8, 32, 896) and w.dtype == np.uint32
    assert 0.02 < np.mean(w == np.uint32(0x80000000)) < 0.04


def test_tp8_m4096_shape_metadata():
    cfg = wl.CONFIGS["tp8_m4096"]
    assert (cfg.tp, cfg.m, cfg.cap, cfg.parities) == (8, 4096, 4096, 1)
