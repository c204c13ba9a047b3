"""ArNorm oracle: Lamport-mailbox all-reduce + residual add + RMSNorm (test
infrastructure only).

Follows the drafter.comm page: the module prose (ArNorm bullet, "Exactness"
paragraph) and the ArNorm class entry (its docstring and kernel listing), read in
the pages' one-GPU stand-in form from the two-shot page's prose (owners = 1: the TP
local slots of one mailbox play the ranks).

Mailbox layout: uint32 [parities, TP, cap, 3584]; slot k of row m holds rank k's
partial row as 3584 words (BF16 pairs, even column in the low half).

Steps, in the page's order:
  push     rank r's partial row, each word cleaned, into slot [r]
  poll     every slot's fragments must be published (the oracle never spins)
  re-arm   the reader writes the sentinel over every slot it read (rows < M only)
  reduce   per BF16 column: start from slot 0's value, add slots 1..TP-1 in rank
           order with FP32 round-to-nearest adds, round once to BF16
  residual new residual = BF16(FP32(reduced) + FP32(residual)), one rounding; with
           no residual the new residual is the reduced row itself (residual = AR(x));
           stored as is (not cleaned)
  norm     out = x * rstd * w rounded once, rstd = 1 / sqrt(sum(x^2) / 7168 + eps)

The norm is the plain definition in float64 with one final BF16 rounding: the page
computes it in FP32 with a sum-of-squares order of its own, which makes ``out``
unique only to within one BF16 ulp (the tolerance the tests use).  eps is an FP32
kernel argument on the page (a Python float passed to an FP32 parameter), so the
oracle uses float64(float32(eps)).
"""

import numpy as np

from .bf16 import widen, round_to_bf16, pack_pairs, unpack_pairs
from .lamport import (
    SENTINEL,
    HIDDEN,
    WORDS_PER_ROW,
    clean,
    check_armed,
    check_published,
)


# -- the arithmetic, on BF16 patterns ---------------------------------------------


def allreduce_rows(slot_words):
    """Rank-order all-reduce of published slot words.

    slot_words: uint32 [TP, M, 3584] as read from the mailbox (already clean).
    Returns uint16 [M, 7168]: per column, FP32 sum starting from slot 0's value and
    adding slots 1..TP-1 in rank order (each add rounded to FP32), rounded once to BF16.
    """
    lanes = widen(unpack_pairs(slot_words))  # float32 [TP, M, 7168], exact
    total = lanes[0].copy()  # start from slot 0's value (not from +0.0)
    for k in range(1, lanes.shape[0]):
        total = (total + lanes[k]).astype(np.float32)  # one FP32 RN add per slot
    return round_to_bf16(total)


def add_residual(reduced, residual):
    """BF16(FP32(reduced) + FP32(residual)): one FP32 add, one BF16 rounding.
    ``residual`` None: the reduced row is the new residual (the embedding case)."""
    if residual is None:
        return np.asarray(reduced, dtype=np.uint16).copy()
    s = (widen(reduced) + widen(residual)).astype(np.float32)
    return round_to_bf16(s)


def rms_norm(x, gamma, eps):
    """x * w / sqrt(mean(x^2) + eps) per row, float64, one BF16 rounding at the end.

    x: uint16 [M, 7168]; gamma: uint16 [7168]; eps: the FP32 value of the argument.
    The page accumulates the sum of squares in FP32, so a total beyond the FP32 range
    is +inf there (rstd = 0: out is +-0, or NaN where x is infinite); the float64 total
    is taken through float32 to keep that range, which changes no finite total by more
    than half an FP32 ulp.
    """
    v = widen(x).astype(np.float64)
    g = widen(gamma).astype(np.float64)
    e = float(np.float32(eps))
    with np.errstate(over="ignore", invalid="ignore"):
        total = np.sum(v * v, axis=-1, keepdims=True)  # squares of BF16 values are exact
        total = total.astype(np.float32).astype(np.float64)  # the FP32 range of the page's sum
        rstd = 1.0 / np.sqrt(total / HIDDEN + e)
        return round_to_bf16(v * rstd * g)


def arnorm_rows(slot_words, residual, gamma, eps):
    """The stateless result of one ArNorm call on already-published slot words:
    (out, residual_out), both uint16 [M, 7168]."""
    reduced = allreduce_rows(slot_words)
    new_residual = add_residual(reduced, residual)
    return rms_norm(new_residual, gamma, eps), new_residual


# -- the mailbox calls (the stand-in's producer and consumer) ----------------------


def arnorm_push(box, partial, parity, rank):
    """Producer: rank ``rank + s``'s partial row into slot [rank + s] of ``box[parity]``.

    box: uint32 [P, TP, cap, 3584] (modified in place); partial: uint16 [nslots, M, 7168].
    Raises ProtocolError when a target fragment is not armed.
    """
    partial = np.asarray(partial, dtype=np.uint16)
    nslots, m, width = partial.shape
    assert width == HIDDEN
    target = box[parity, rank : rank + nslots, :m, :]
    check_armed(target, f"parity {parity} slots {rank}..{rank + nslots - 1} rows <{m}")
    box[parity, rank : rank + nslots, :m, :] = clean(pack_pairs(partial))


def arnorm_reduce_norm(box, parity, m, residual, gamma, eps, partial=None, rank=0):
    """Consumer: poll, re-arm and reduce the TP slots of rows < m of ``box[parity]``.

    With ``partial`` (uint16 [m, 7168]) the call first pushes it as rank ``rank``
    (the page's one-kernel form, where each rank's kernel pushes its own row).
    Returns (out, residual_out), uint16 [m, 7168].  ``box`` is re-armed in place.
    """
    if partial is not None:
        arnorm_push(box, np.asarray(partial, dtype=np.uint16)[None], parity, rank)
    slots = box[parity, :, :m, :]
    check_published(slots, f"parity {parity} rows <{m}")
    raw = slots.copy()
    box[parity, :, :m, :] = np.uint32(SENTINEL)  # the reader re-arms every slot it read
    assert raw.shape[-1] == WORDS_PER_ROW
    return arnorm_rows(raw, residual, gamma, eps)
