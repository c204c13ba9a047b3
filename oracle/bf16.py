"""BF16 bit patterns for the oracle (test infrastructure only).

The drafter.comm page fixes the arithmetic of ArNorm as "BF16 partials, FP32
accumulation, one BF16 rounding" (module prose, "Exactness" paragraph).  BF16 values
travel as raw uint16 patterns; two BF16 values share one 32-bit mailbox word with the
even column in the low half and the odd column in the high half (the little-endian
pair layout that the ArNorm listing unpacks word by word).

``round_to_bf16`` is the definition of round-to-nearest, ties-to-even written out in
float64: pick the quantum of the binade (8 significant bits, never finer than the
BF16 subnormal quantum 2**-133), scale exactly, round half-to-even with ``np.rint``,
scale back.  It is deliberately not the usual integer bit trick, so that it can be
checked against that trick (torch's cast) as an independent pin.
"""

import numpy as np

BF16_QNAN = 0x7FC0


def widen(h):
    """BF16 patterns (uint16) -> float32 values; exact (the pattern is the high half)."""
    h = np.asarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_bf16(x):
    """Round float32/float64 values to the nearest BF16, ties to even; returns uint16.

    NaN becomes the canonical quiet NaN 0x7FC0 (no input on the path produces one).
    Values at or beyond the overflow midpoint round to +-inf, as IEEE RNE does.
    """
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        _, e = np.frexp(x)  # |x| = m * 2**e with 0.5 <= m < 1 (e = 0 for 0, inf, nan)
        q = np.maximum(e - 8, -133)  # quantum exponent: 8 significant bits, subnormal floor
        r = np.rint(np.ldexp(x, -q))  # exact scaling, then round half to even
        v = np.ldexp(r, q)  # the rounded value, exact in float64
        v = np.where(np.abs(v) >= 2.0**128, np.copysign(np.inf, x), v)
        bits = (v.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(np.isnan(x), np.uint16(BF16_QNAN), bits)
    return bits.astype(np.uint16)


def pack_pairs(h):
    """uint16 [..., 2n] -> uint32 [..., n]: element 2j in the low half of word j."""
    h = np.asarray(h, dtype=np.uint16)
    lo = h[..., 0::2].astype(np.uint32)
    hi = h[..., 1::2].astype(np.uint32)
    return lo | (hi << np.uint32(16))


def unpack_pairs(w):
    """uint32 [..., n] -> uint16 [..., 2n], inverse of ``pack_pairs``."""
    w = np.asarray(w, dtype=np.uint32)
    out = np.empty(w.shape[:-1] + (2 * w.shape[-1],), dtype=np.uint16)
    out[..., 0::2] = (w & np.uint32(0xFFFF)).astype(np.uint16)
    out[..., 1::2] = (w >> np.uint32(16)).astype(np.uint16)
    return out
