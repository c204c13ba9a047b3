"""Seeded synthetic inputs for the ArNorm and Gather workloads.

This module holds none of the method's arithmetic: no rounding, no sums, no norm.
It draws numbers with ``numpy.random.default_rng(seed)`` and lays them out as the
kernels and the CPU oracle both expect them:

* BF16 values are uint16 bit patterns made by truncating float32 normals (the top
  half of the float32 pattern), so every drawn value is exactly a BF16 value and the
  distribution is the stated normal to within one BF16 step.
* Mailbox words are uint32; two BF16 values share a word, even column in the low half.
* The sentinel pair (+0, -0) is the word 0x80000000: +0 (0x0000) in the low half,
  -0 (0x8000) in the high half.

Workloads (the TP8 drafter shapes of the vLLM DSpark drafter pages: hidden 7168,
rows M = tokens in flight, TP slots playing the ranks of the one-GPU stand-in):

  tp2_m1          ArNorm TP=2, M=1, residual, one parity, seed 0
  tp8_m4          ArNorm TP=8, M=4, no residual (residual = AR(x)), 2 parities over 8
                  calls, seed 1
  tp8_m64         ArNorm TP=8, M=64 = cap, residual, 5 % of partial words set to the
                  sentinel pair, rows 48..63 built so that rank-order and pairwise-tree
                  sums differ, 61 calls over 2 parities, seed 2
  gather_tp8_m32  Gather TP=8, M=32, S=896 words, cap=64, uniform words with 3 %
                  sentinel, seed 3
  tp8_m4096       ArNorm TP=8, M=4096, residual, partials and residual N(0, 1), seed 4
  ctx             Gather of the context projection: TP=8, [M=64, 896] BF16 shards (448
                  words), N(0, 1) with 1 % of values -0, seed 5
  logits          Gather of the lm_head logits: TP=8, [M=4, 20480] BF16 shards (10240
                  words) of a synthetic V = 163840, N(0, 1) with 1 % of values -0, seed 6
"""

from dataclasses import dataclass, field

import numpy as np

HIDDEN = 7168
SENTINEL_WORD = 0x80000000


@dataclass(frozen=True)
class ArNormConfig:
    name: str
    tp: int
    m: int
    cap: int
    parities: int
    residual: bool
    sigma_partial: float
    sigma_residual: float
    seed: int
    calls: int = 1
    eps: float = 1e-6
    sentinel_frac: float = 0.0
    tree_rows: tuple = field(default=())
    description: str = ""


@dataclass(frozen=True)
class GatherConfig:
    name: str
    tp: int
    m: int
    s: int
    cap: int
    sentinel_frac: float
    seed: int
    description: str = ""


CONFIGS = {
    "tp2_m1": ArNormConfig(
        "tp2_m1", tp=2, m=1, cap=64, parities=1, residual=True, sigma_partial=0.5,
        sigma_residual=1.0, seed=0,
        description="ArNorm TP=2 slots, M=1 row, width 7168, residual, one parity"),
    "tp8_m4": ArNormConfig(
        "tp8_m4", tp=8, m=4, cap=64, parities=2, residual=False, sigma_partial=0.02,
        sigma_residual=0.0, seed=1, calls=8,
        description="ArNorm TP=8, M=4 rows, width 7168, residual=False, 2 parities x 8 calls"),
    "tp8_m64": ArNormConfig(
        "tp8_m64", tp=8, m=64, cap=64, parities=2, residual=True, sigma_partial=0.5,
        sigma_residual=1.0, seed=2, calls=61, sentinel_frac=0.05,
        tree_rows=tuple(range(48, 64)),
        description="ArNorm TP=8, M=64 (cap), residual, 5% sentinel words, "
                    "rank-vs-tree rows, 61 calls over 2 parities"),
    "gather_tp8_m32": GatherConfig(
        "gather_tp8_m32", tp=8, m=32, s=896, cap=64, sentinel_frac=0.03, seed=3,
        description="Gather TP=8, [M=32, S=896] word shards into [cap=64, 8*896]"),
    # the drafter's own gather shapes: the context projection's [M, 7168/TP] BF16 rows
    # and the lm_head's [M, V/TP] BF16 logits (V = 163840, a synthetic vocabulary: the
    # pages print none), as 32-bit words of BF16 pairs
    "ctx": GatherConfig(
        "ctx", tp=8, m=64, s=448, cap=64, sentinel_frac=0.0, seed=5,
        description="context-projection gather: TP=8, [M=64, 896] BF16 shards -> [M, 7168]"),
    "logits": GatherConfig(
        "logits", tp=8, m=4, s=10240, cap=64, sentinel_frac=0.0, seed=6,
        description="lm_head logits gather: TP=8, [M=4, 20480] BF16 shards -> [M, 163840]"),
    "tp8_m4096": ArNormConfig(
        "tp8_m4096", tp=8, m=4096, cap=4096, parities=1, residual=True, sigma_partial=1.0,
        sigma_residual=1.0, seed=4,
        description="ArNorm TP=8, M=4096 rows, width 7168, residual (HBM roofline run)"),
}


def bf16_normal(rng, shape, sigma):
    """BF16 patterns of sigma * N(0, 1), by truncating float32 draws."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_gamma(rng, width=HIDDEN):
    """RMSNorm weight 1 + 0.1 * N(0, 1) as BF16 patterns (truncated float32 draws)."""
    x = np.float32(1.0) + np.float32(0.1) * rng.standard_normal(size=width, dtype=np.float32)
    return (x.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def set_sentinel_words(rng, h, frac):
    """Set about ``frac`` of the 32-bit words of BF16 rows ``h`` (uint16 [..., 2n],
    modified in place) to the sentinel pair: low half +0, high half -0."""
    if frac <= 0:
        return h
    words_shape = h.shape[:-1] + (h.shape[-1] // 2,)
    hit = rng.random(size=words_shape) < frac
    lo = h[..., 0::2]
    hi = h[..., 1::2]
    lo[hit] = 0x0000
    hi[hit] = 0x8000
    return h


def _bf16_pow2(sign, exp):
    """BF16 pattern of sign * 2**exp for a normal exponent (bit layout only)."""
    return ((sign.astype(np.uint32) << 15) | ((exp + 127).astype(np.uint32) << 7)).astype(np.uint16)


def set_tree_rows(rng, partials, rows):
    """Rows whose rank-order sum differs from the pairwise tree: in every column the
    TP=8 slots hold s*2^e, s*2^(e-8) and six times s*2^(e-25) (random sign s and
    e in [-4, 4] per column); partials uint16 [8, M, 7168], modified in place."""
    tp = partials.shape[0]
    assert tp == 8, "the pattern needs eight slots"
    for r in rows:
        sign = rng.integers(0, 2, size=HIDDEN)
        e = rng.integers(-4, 5, size=HIDDEN)
        partials[0, r] = _bf16_pow2(sign, e)
        partials[1, r] = _bf16_pow2(sign, e - 8)
        for k in range(2, 8):
            partials[k, r] = _bf16_pow2(sign, e - 25)
    return partials


class ArNormInputs:
    """Seeded stream of one ArNorm workload's inputs: gamma once, then per call the
    TP partial rows (uint16 [TP, M, 7168]) and the residual (uint16 [M, 7168] or None).
    """

    def __init__(self, cfg: ArNormConfig):
        self.cfg = cfg
        self.rng = np.random.default_rng(cfg.seed)
        self.gamma = bf16_gamma(self.rng)

    def partials(self):
        c = self.cfg
        p = np.empty((c.tp, c.m, HIDDEN), dtype=np.uint16)
        for k in range(c.tp):  # slot by slot keeps the float32 temporary small
            p[k] = bf16_normal(self.rng, (c.m, HIDDEN), c.sigma_partial)
        if c.tree_rows:
            set_tree_rows(self.rng, p, [r for r in c.tree_rows if r < c.m])
        set_sentinel_words(self.rng, p, c.sentinel_frac)
        return p

    def residual(self):
        c = self.cfg
        if not c.residual:
            return None
        res = bf16_normal(self.rng, (c.m, HIDDEN), c.sigma_residual)
        for r in c.tree_rows:
            if r < c.m:
                res[r] = 0x0000  # +0, so the rank-vs-tree difference reaches res_out
        return res

    def call(self):
        p = self.partials()
        return p, self.residual()


def bf16_shards(cfg: GatherConfig, sigma=1.0, neg_zero_frac=0.01):
    """Seeded BF16 shards as uint32 [TP, M, S] words: sigma * N(0, 1) values, with about
    ``neg_zero_frac`` of the BF16 values set to -0 (so some words are the sentinel pair
    and others other -0 patterns, as real BF16 activations and logits can hold)."""
    rng = np.random.default_rng(cfg.seed)
    h = bf16_normal(rng, (cfg.tp, cfg.m, 2 * cfg.s), sigma)
    h[rng.random(size=h.shape) < neg_zero_frac] = 0x8000
    h[..., 0::2][rng.random(size=h[..., 0::2].shape) < neg_zero_frac] = 0x0000
    lo = h[..., 0::2].astype(np.uint32)
    hi = h[..., 1::2].astype(np.uint32)
    return lo | (hi << np.uint32(16))


def gather_shards(cfg: GatherConfig):
    """Seeded uint32 [TP, M, S] shards: uniform words, ``sentinel_frac`` of them the
    sentinel pair."""
    rng = np.random.default_rng(cfg.seed)
    w = rng.integers(0, 1 << 32, size=(cfg.tp, cfg.m, cfg.s), dtype=np.uint64).astype(np.uint32)
    hit = rng.random(size=w.shape) < cfg.sentinel_frac
    w[hit] = np.uint32(SENTINEL_WORD)
    return w
