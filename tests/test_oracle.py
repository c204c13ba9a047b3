"""Pins for the CPU oracle: each check compares the oracle with something other than
itself -- hand cases derived from the pages' rules (tests/golden), exact rational
arithmetic, a library cast, closed forms and invariants.  Every check is written as a
function of the implementation under test, so that ``test_mutants_are_caught`` can
run the same checks against copies of the oracle with a planted mistake and show that
each mistake is caught.
"""

import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import bf16 as obf
from oracle import arnorm as oar
from oracle import gather as oga
from oracle import lamport as olp
from oracle import twoshot as ots
from tests.conftest import read_golden

S0 = 0x80000000
W = 7168


# -- independent references ---------------------------------------------------------


def bf16_bits_to_fraction(h):
    """Exact rational value of a finite BF16 pattern, from its fields."""
    h = int(h)
    sign = -1 if h & 0x8000 else 1
    e = (h >> 7) & 0xFF
    m = h & 0x7F
    assert e != 0xFF
    if e == 0:
        return sign * Fraction(m, 1 << 7) * Fraction(2) ** -126
    return sign * (1 + Fraction(m, 1 << 7)) * Fraction(2) ** (e - 127)


def exact_rne_bf16(q, negative_zero=False):
    """Nearest BF16 (ties to even) of an exact rational, as a bit pattern."""
    if q == 0:
        return 0x8000 if negative_zero else 0x0000
    sign = 0x8000 if q < 0 else 0
    a = abs(Fraction(q))
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    qe = max(e - 7, -133)
    scaled = a / Fraction(2) ** qe
    n = math.floor(scaled)
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = n * Fraction(2) ** qe
    if v >= Fraction(2) ** 128:
        return sign | 0x7F80
    bits = int(np.array([float(v)], dtype=np.float64).astype(np.float32).view(np.uint32)[0]) >> 16
    return sign | bits


def random_finite_bf16(rng, n, emin=-30, emax=30):
    """Random BF16 patterns with exponents spread over [emin, emax] (plus some
    subnormals and zeros)."""
    sign = rng.integers(0, 2, n).astype(np.uint32)
    e = rng.integers(emin, emax + 1, n) + 127
    m = rng.integers(0, 128, n).astype(np.uint32)
    h = (sign << 15) | (e.astype(np.uint32) << 7) | m
    sub = rng.random(n) < 0.03
    h[sub] = (sign[sub] << 15) | m[sub]  # subnormals and signed zeros
    return h.astype(np.uint16)


# -- checks, each a function of the implementation under test -----------------------


def check_clean(clean):
    for ln in read_golden("clean_words.txt"):
        src, want = ln.split()[:2]
        got = int(np.asarray(clean(np.array([int(src, 16)], dtype=np.uint32)))[0])
        assert got == int(want, 16), f"clean({src}) = {got:08X}, want {want}"


def check_rounding_vs_torch(round_fn):
    """Against torch's CPU float32 -> bfloat16 cast (a library RNE) on random float32
    patterns and on hand-picked ties, subnormals and overflow."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    u = rng.integers(0, 1 << 32, size=1 << 18, dtype=np.uint64).astype(np.uint32)
    special = np.array(
        [0x00000000, 0x80000000, 0x3F808000, 0x3F818000, 0x3F807FFF, 0x3F808001,
         0x00008000, 0x00018000, 0x00007FFF, 0x807F8000, 0x7F7F8000, 0x7F7F7FFF,
         0x7F800000, 0xFF800000, 0x007FFFFF, 0x00800000, 0x33800000, 0xB3808000],
        dtype=np.uint32)
    u = np.concatenate([u, special])
    f = u.view(np.float32)
    f = f[~np.isnan(f)]
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.asarray(round_fn(f))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(hex(f.view(np.uint32)[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]


def check_rounding_vs_fraction(round_fn):
    """Against exact rational nearest-even on float64 inputs across the whole BF16
    range (the oracle's norm rounds float64 values once)."""
    rng = np.random.default_rng(12)
    e = rng.integers(-140, 128, 3000)
    x = rng.uniform(1.0, 2.0, 3000) * np.power(2.0, e) * rng.choice([-1.0, 1.0], 3000)
    # exact BF16 midpoints (ties) at several binades, and values next to them
    mids = []
    for k in (-130, -20, 0, 7, 100):
        for mant in (0, 1, 2, 127):
            base = (1 + mant / 128.0) * 2.0**k
            mids += [base + 2.0 ** (k - 8), np.nextafter(base + 2.0 ** (k - 8), 0)]
    x = np.concatenate([x, np.array(mids)])
    got = np.asarray(round_fn(x))
    for i, v in enumerate(x):
        want = exact_rne_bf16(Fraction(float(v)))
        assert int(got[i]) == want, (v, hex(int(got[i])), hex(want))
    assert int(np.asarray(round_fn(np.array([np.nan])))[0]) == 0x7FC0


def golden_allreduce_cases():
    cases = []
    for ln in read_golden("allreduce_words.txt"):
        name, slots, want = [p.strip() for p in ln.split("|")]
        words = [int(s, 16) for s in slots.split(",")]
        cases.append((name, words, int(want, 16)))
    return cases


def run_ar_words(push_fn, reduce_fn, words):
    """Drive a (push, reduce) pair on one word per slot: the golden words are padded
    into a full 7168-column row (the rest zero)."""
    tp = len(words)
    box = np.full((1, tp, 1, W // 2), S0, dtype=np.uint32)
    partial = np.zeros((tp, 1, W), dtype=np.uint16)
    for k, w in enumerate(words):
        partial[k, 0, 0] = w & 0xFFFF
        partial[k, 0, 1] = w >> 16
    push_fn(box, partial, 0, 0)
    gamma = np.full(W, 0x3F80, dtype=np.uint16)
    out, res_out = reduce_fn(box, 0, 1, None, gamma, 1e-6)
    return int(res_out[0, 0]) | (int(res_out[0, 1]) << 16), box


def check_allreduce_golden(push_fn, reduce_fn):
    for name, words, want in golden_allreduce_cases():
        got, box = run_ar_words(push_fn, reduce_fn, words)
        assert got == want, f"{name}: got {got:08X}, want {want:08X}"
        assert np.all(box == S0), f"{name}: mailbox not re-armed"


def golden_residual_cases():
    cases = []
    for ln in read_golden("residual_words.txt"):
        name, slots, res, want = [p.strip() for p in ln.split("|")]
        cases.append((name, [int(x, 16) for x in slots.split(",")], int(res, 16), int(want, 16)))
    return cases


def check_residual_golden(push_fn, reduce_fn):
    """The all-reduced word rounded, then the residual added and rounded again."""
    for name, words, res_word, want in golden_residual_cases():
        tp = len(words)
        box = np.full((1, tp, 1, W // 2), S0, dtype=np.uint32)
        partial = np.zeros((tp, 1, W), dtype=np.uint16)
        for k, w in enumerate(words):
            partial[k, 0, 0], partial[k, 0, 1] = w & 0xFFFF, w >> 16
        residual = np.zeros((1, W), dtype=np.uint16)
        residual[0, 0], residual[0, 1] = res_word & 0xFFFF, res_word >> 16
        push_fn(box, partial, 0, 0)
        _, res_out = reduce_fn(box, 0, 1, residual, np.full(W, 0x3F80, dtype=np.uint16), 1e-6)
        got = int(res_out[0, 0]) | (int(res_out[0, 1]) << 16)
        assert got == want, f"{name}: got {got:08X}, want {want:08X}"


def check_tp2_theorem(allreduce_fn):
    """TP=2: the FP32 sum of two BF16 values rounded to BF16 equals the correctly
    rounded BF16 of the exact sum (double rounding is innocuous: 24 >= 2*8 + 2)."""
    rng = np.random.default_rng(13)
    n = 4000
    a = random_finite_bf16(rng, n)
    b = random_finite_bf16(rng, n)
    # a third of the pairs with close exponents (cancellation, carries)
    b[: n // 3] = (a[: n // 3] ^ rng.integers(0, 1 << 7, n // 3).astype(np.uint16)) ^ np.uint16(0x8000)
    words = np.stack([obf.pack_pairs(a), obf.pack_pairs(b)])[:, None, :]  # [2, 1, n/2]
    got = np.asarray(allreduce_fn(words))[0]
    for i in range(n):
        qa, qb = bf16_bits_to_fraction(a[i]), bf16_bits_to_fraction(b[i])
        negz = bool(a[i] & 0x8000) and bool(b[i] & 0x8000)  # -0 + -0 = -0
        want = exact_rne_bf16(qa + qb, negative_zero=negz)
        assert int(got[i]) == want, (hex(a[i]), hex(b[i]), hex(int(got[i])), hex(want))


def check_exact_prefix_tp8(allreduce_fn):
    """TP=8 on values k * 2^-4 (|k| < 128): every FP32 prefix sum is exact, so the
    result is the correctly rounded BF16 of the exact sum, whatever the order."""
    rng = np.random.default_rng(14)
    n = 2048
    k = rng.integers(-127, 128, size=(8, n))
    vals = k.astype(np.float32) * np.float32(2.0**-4)
    h = (vals.view(np.uint32) >> np.uint32(16)).astype(np.uint16)  # exact: 8 bits
    words = obf.pack_pairs(h)[:, None, :]  # [8, 1, n/2]
    got = np.asarray(allreduce_fn(words))[0]
    for i in range(n):
        want = exact_rne_bf16(Fraction(int(k[:, i].sum()), 16),
                              negative_zero=False)
        if k[:, i].sum() == 0:
            assert int(got[i]) in (0x0000,), (i, hex(int(got[i])))
        else:
            assert int(got[i]) == want, (i, k[:, i], hex(int(got[i])), hex(want))


def check_residual_add(add_fn):
    """One FP32 add and one BF16 rounding equal the correctly rounded exact sum;
    residual None leaves the reduced row as the new residual."""
    rng = np.random.default_rng(15)
    n = 3000
    r = random_finite_bf16(rng, n, -12, 12)
    c = random_finite_bf16(rng, n, -12, 12)
    got = np.asarray(add_fn(r, c))
    for i in range(n):
        negz = bool(r[i] & 0x8000) and bool(c[i] & 0x8000)
        want = exact_rne_bf16(bf16_bits_to_fraction(r[i]) + bf16_bits_to_fraction(c[i]), negz)
        assert int(got[i]) == want, (hex(r[i]), hex(c[i]), hex(int(got[i])), hex(want))
    assert np.array_equal(np.asarray(add_fn(r, None)), r)


def decimal_norm_bits(x_bits, g_bits, eps):
    """RMSNorm of one row in 60-digit decimal arithmetic, rounded once to BF16."""
    getcontext().prec = 60
    xs = [bf16_bits_to_fraction(h) for h in x_bits]
    gs = [bf16_bits_to_fraction(h) for h in g_bits]
    total = sum(v * v for v in xs)  # exact rational
    mean = total / len(xs) + Fraction(float(np.float32(eps)))
    dm = Decimal(mean.numerator) / Decimal(mean.denominator)
    rstd = Fraction(Decimal(1) / dm.sqrt())
    out = []
    for h, v, g in zip(x_bits, xs, gs):
        out.append(exact_rne_bf16(v * rstd * g, negative_zero=bool(h & 0x8000) and v == 0))
    return out


def check_norm_closed_forms(norm_fn):
    eps = 1e-6
    one = np.full(W, 0x3F80, dtype=np.uint16)
    # all-zero row: every output is zero
    z = np.zeros((1, W), dtype=np.uint16)
    assert np.all(np.asarray(norm_fn(z, one, eps)) == 0)
    # constant row 1.0, gamma 1: rstd = 1/sqrt(1 + eps) rounds to 1.0
    assert np.all(np.asarray(norm_fn(one[None], one, eps)) == 0x3F80)
    # one-hot row: out = rstd = 1/sqrt(1/7168 + eps) = 84.36..., BF16 84.5 = 0x42A9
    x = np.zeros((1, W), dtype=np.uint16)
    x[0, 123] = 0x3F80
    got = np.asarray(norm_fn(x, one, eps))[0]
    getcontext().prec = 60
    want = exact_rne_bf16(Fraction(Decimal(1) / (Decimal(1) / Decimal(W) + Decimal(float(np.float32(eps)))).sqrt()))
    assert want == 0x42A9
    assert int(got[123]) == want and np.all(np.delete(got, 123) == 0)
    # eps-dominated row: all 2^-10, mean 2^-20 ~ eps; without eps the output is 1.0
    t = np.full((1, W), 0x3A80, dtype=np.uint16)
    got = np.asarray(norm_fn(t, one, eps))[0]
    mean = Fraction(1, 2**20) + Fraction(float(np.float32(eps)))
    getcontext().prec = 60
    rstd = Fraction(Decimal(1) / (Decimal(mean.numerator) / Decimal(mean.denominator)).sqrt())
    want = exact_rne_bf16(Fraction(1, 1024) * rstd)
    assert want != 0x3F80
    assert np.all(got == want), (hex(int(got[0])), hex(want))


def check_norm_fp32_range(norm_fn):
    """The page's FP32 sum of squares: a row whose total exceeds the FP32 range has
    rstd = 0, so finite values give +-0 and infinite values NaN."""
    one = np.full(W, 0x3F80, dtype=np.uint16)
    big = np.full((1, W), 0x7F00, dtype=np.uint16)  # 2^127: squares overflow FP32
    big[0, 1::2] = 0xFF00  # -2^127
    got = np.asarray(norm_fn(big, one, 1e-6))[0]
    assert np.all((got & 0x7FFF) == 0), hex(int(got[0]))
    assert np.all(got[1::2] == 0x8000) and np.all(got[0::2] == 0x0000)
    inf = big.copy()
    inf[0, 5] = 0x7F80
    got = np.asarray(norm_fn(inf, one, 1e-6))[0]
    assert (int(got[5]) & 0x7F80) == 0x7F80 and (int(got[5]) & 0x7F) != 0  # NaN
    # inside the range nothing changes: 2^50 everywhere (total 7168 * 2^100) gives 1.0
    mid = np.full((1, W), 0x5880, dtype=np.uint16)
    assert np.all(np.asarray(norm_fn(mid, one, 1e-6)) == 0x3F80)


def check_norm_random_rows(norm_fn):
    rng = np.random.default_rng(16)
    for sigma in (1.0, 0.02):
        x = (rng.standard_normal((2, W), dtype=np.float32) * np.float32(sigma))
        xb = (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
        g = (np.float32(1) + np.float32(0.1) * rng.standard_normal(W, dtype=np.float32))
        gb = (g.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
        got = np.asarray(norm_fn(xb, gb, 1e-6))
        for r in range(2):
            want = decimal_norm_bits(xb[r], gb, 1e-6)
            assert [int(v) for v in got[r]] == want


def check_protocol(push_fn, reduce_fn):
    """Arm / push / poll / re-arm over alternating parities (TP=4, M=3 of cap 5)."""
    rng = np.random.default_rng(17)
    tp, m, cap = 4, 3, 5
    box = np.full((2, tp, cap, W // 2), S0, dtype=np.uint32)
    gamma = np.full(W, 0x3F80, dtype=np.uint16)
    for call in range(6):
        parity = call % 2
        partial = random_finite_bf16(rng, tp * m * W, -3, 3).reshape(tp, m, W)
        other = box[1 - parity].copy()
        push_fn(box, partial, parity, 0)
        assert not np.any(box[parity, :, :m] == S0), "pushed words never equal the sentinel"
        # a second push into the same parity before its read breaks the protocol
        with pytest.raises(olp.ProtocolError):
            push_fn(box, partial[:1], parity, 0)
        reduce_fn(box, parity, m, None, gamma, 1e-6)
        assert np.all(box[parity] == S0), "reader re-arms every slot it read"
        assert np.array_equal(box[1 - parity], other), "the other parity is untouched"
    # a poll of a slot nobody pushed is a protocol error (the oracle never spins)
    push_fn(box, random_finite_bf16(rng, (tp - 1) * m * W, -3, 3).reshape(tp - 1, m, W), 0, 0)
    with pytest.raises(olp.ProtocolError):
        reduce_fn(box, 0, m, None, gamma, 1e-6)


def check_gather(push_fn, poll_fn):
    tp, m, s, cap = 2, 2, 4, 3
    shards = np.array([[[1, S0, 3, 0x80008000], [5, 6, 7, 8]],
                       [[S0, S0, S0, S0], [0xFFFFFFFF, 0, 0x8000, 9]]], dtype=np.uint32)
    want = np.array([[1, 0, 3, 0x80008000, 0, 0, 0, 0],
                     [5, 6, 7, 8, 0xFFFFFFFF, 0, 0x8000, 9]], dtype=np.uint32)
    gbox = np.full((cap, tp * s), S0, dtype=np.uint32)
    push_fn(gbox, shards[:1], 0)
    push_fn(gbox, shards[1:], 1)
    assert poll_fn(gbox, m, False) is None
    assert np.array_equal(gbox[:m], want), "no copy leaves the published rows in place"
    out = poll_fn(gbox, m, True)
    assert np.array_equal(out, want)
    assert np.all(gbox == S0), "copy re-arms the rows it read"
    with pytest.raises(olp.ProtocolError):
        poll_fn(gbox, m, True)  # nothing published


def run_twoshot_words(push_fn, reduce_fn, words):
    tp = len(words)
    recv = np.full((1, tp, 1, 4), S0, dtype=np.uint32)
    gath = np.full((1, 1, 1, 4), S0, dtype=np.uint32)
    part = np.zeros((tp, 1, 8), dtype=np.uint16)
    for k, w in enumerate(words):
        part[k, 0, 0] = w & 0xFFFF
        part[k, 0, 1] = w >> 16
    push_fn(recv, part, 0, 0)
    red = reduce_fn(recv, gath, 0, 1)
    return int(red[0, 0]) | (int(red[0, 1]) << 16), recv, gath


def check_twoshot_golden(push_fn, reduce_fn):
    for ln in read_golden("twoshot_words.txt"):
        name, slots, want = [p.strip() for p in ln.split("|")]
        got, recv, gath = run_twoshot_words(push_fn, reduce_fn, [int(x, 16) for x in slots.split(",")])
        assert got == int(want, 16), f"{name}: got {got:08X}, want {want}"
        assert np.all(recv == S0), f"{name}: recv not re-armed"
        assert gath[0, 0, 0, 0] == got, f"{name}: gather row does not hold the result"


def check_twoshot_theorem(reduce_rows_fn):
    """TP=2: correctly rounded exact sum, with -0 turned into +0."""
    rng = np.random.default_rng(19)
    n = 3000
    a = random_finite_bf16(rng, n)
    b = random_finite_bf16(rng, n)
    b[: n // 3] = (a[: n // 3] ^ rng.integers(0, 1 << 7, n // 3).astype(np.uint16)) ^ np.uint16(0x8000)
    a[-20:] = 0x8000  # -0 + -0: the one sum whose exact result is a negative zero
    b[-20:] = 0x8000
    got = np.asarray(reduce_rows_fn(np.stack([obf.pack_pairs(a), obf.pack_pairs(b)])[:, None, :]))[0]
    for i in range(n):
        want = exact_rne_bf16(bf16_bits_to_fraction(a[i]) + bf16_bits_to_fraction(b[i]))
        want = 0 if want == 0x8000 else want
        assert int(got[i]) == want, (hex(a[i]), hex(b[i]), hex(int(got[i])), hex(want))


def check_twoshot_protocol(push_fn, reduce_fn, read_fn):
    rng = np.random.default_rng(20)
    tp, m, cap, width = 4, 3, 5, 64
    recv = np.full((2, tp, cap, width // 2), S0, dtype=np.uint32)
    gath = np.full((2, 1, cap, width // 2), S0, dtype=np.uint32)
    for call in range(4):
        parity = call % 2
        other_r, other_g = recv[1 - parity].copy(), gath[1 - parity].copy()
        part = random_finite_bf16(rng, tp * m * width, -3, 3).reshape(tp, m, width)
        push_fn(recv, part, parity, 0)
        red = reduce_fn(recv, gath, parity, m)
        assert np.all(recv[parity] == S0), "the owner re-arms its slots"
        assert not np.any(gath[parity, 0, :m] == S0), "the reduced row is published"
        with pytest.raises(olp.ProtocolError):
            reduce_fn(recv, gath, parity, m)  # nothing pushed any more
        got = read_fn(gath, parity, m)
        assert np.array_equal(got, red)
        assert np.all(gath[parity] == S0), "the reader re-arms the gather row"
        assert np.array_equal(recv[1 - parity], other_r) and np.array_equal(gath[1 - parity], other_g)


# -- the pins, run on the oracle ---------------------------------------------------


def test_clean():
    check_clean(olp.clean)


def test_published():
    w = np.array([1, 2, 3, 4, 5, S0, 7, 8], dtype=np.uint32)
    assert list(olp.published(w)) == [True, False]


def test_rounding_vs_torch():
    check_rounding_vs_torch(obf.round_to_bf16)


def test_rounding_vs_fraction():
    check_rounding_vs_fraction(obf.round_to_bf16)


def test_pack_roundtrip():
    rng = np.random.default_rng(0)
    h = rng.integers(0, 1 << 16, size=(3, 10)).astype(np.uint16)
    w = obf.pack_pairs(h)
    assert w[0, 0] == (int(h[0, 0]) | (int(h[0, 1]) << 16))
    assert np.array_equal(obf.unpack_pairs(w), h)


def test_allreduce_golden():
    check_allreduce_golden(oar.arnorm_push, oar.arnorm_reduce_norm)


def test_allreduce_tp2_theorem():
    check_tp2_theorem(oar.allreduce_rows)


def test_allreduce_exact_prefix_tp8():
    check_exact_prefix_tp8(oar.allreduce_rows)


def test_residual_add():
    check_residual_add(oar.add_residual)


def test_norm_closed_forms():
    check_norm_closed_forms(oar.rms_norm)


def test_norm_fp32_range():
    check_norm_fp32_range(oar.rms_norm)


def test_norm_random_rows():
    check_norm_random_rows(oar.rms_norm)


def test_protocol():
    check_protocol(oar.arnorm_push, oar.arnorm_reduce_norm)


def test_gather():
    check_gather(oga.gather_push, oga.gather_poll)


def test_residual_golden():
    """All-reduce rounded once, residual added and rounded again (hand cases)."""
    check_residual_golden(oar.arnorm_push, oar.arnorm_reduce_norm)


def test_twoshot_golden():
    check_twoshot_golden(ots.twoshot_push, ots.twoshot_reduce)


def test_twoshot_theorem():
    check_twoshot_theorem(ots.reduce_no_negative_zero)


def test_twoshot_protocol():
    check_twoshot_protocol(ots.twoshot_push, ots.twoshot_reduce, ots.twoshot_read)


def test_twoshot_matches_arnorm_sum_off_negative_zero():
    """Away from -0 the two-shot sum is ArNorm's all-reduced row, bit for bit."""
    rng = np.random.default_rng(21)
    words = obf.pack_pairs(random_finite_bf16(rng, 8 * 2 * 512, -5, 5).reshape(8, 2, 512))
    a = oar.allreduce_rows(words)
    b = ots.reduce_no_negative_zero(words)
    assert np.array_equal(np.where(a == 0x8000, 0, a), b)


def test_fused_push_matches_separate_push():
    rng = np.random.default_rng(18)
    tp, m = 4, 2
    partial = random_finite_bf16(rng, tp * m * W, -3, 3).reshape(tp, m, W)
    res = random_finite_bf16(rng, m * W, -3, 3).reshape(m, W)
    gamma = random_finite_bf16(rng, W, -1, 1)
    a = np.full((1, tp, m, W // 2), S0, dtype=np.uint32)
    b = a.copy()
    oar.arnorm_push(a, partial, 0, 0)
    ra = oar.arnorm_reduce_norm(a, 0, m, res, gamma, 1e-6)
    oar.arnorm_push(b, np.delete(partial, 2, axis=0)[:2], 0, 0)
    oar.arnorm_push(b, partial[3:], 0, 3)
    rb = oar.arnorm_reduce_norm(b, 0, m, res, gamma, 1e-6, partial=partial[2], rank=2)
    assert np.array_equal(ra[0], rb[0]) and np.array_equal(ra[1], rb[1])
    assert np.all(a == S0) and np.all(b == S0)


# -- mutants: plausible mistakes planted in copies of the oracle must fail a pin ----


def _mut_tree(slot_words):
    lanes = list(obf.widen(obf.unpack_pairs(slot_words)))
    while len(lanes) > 1:
        nxt = [(lanes[i] + lanes[i + 1]).astype(np.float32) for i in range(0, len(lanes) - 1, 2)]
        if len(lanes) % 2:
            nxt.append(lanes[-1])
        lanes = nxt
    return obf.round_to_bf16(lanes[0])


def _mut_reverse(slot_words):
    return oar.allreduce_rows(slot_words[::-1])


def _mut_from_zero(slot_words):
    lanes = obf.widen(obf.unpack_pairs(slot_words))
    t = np.zeros_like(lanes[0])
    for k in range(lanes.shape[0]):
        t = (t + lanes[k]).astype(np.float32)
    return obf.round_to_bf16(t)


def _mut_drop_last(slot_words):
    return oar.allreduce_rows(slot_words[:-1])


def _mut_f64_accumulate(slot_words):
    lanes = obf.widen(obf.unpack_pairs(slot_words)).astype(np.float64)
    return obf.round_to_bf16(lanes.sum(axis=0))


def _mut_truncate(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _mut_round_half_up(x):
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x8000)) >> np.uint32(16)).astype(np.uint16)


def _mut_no_clean(w):
    return np.asarray(w, dtype=np.uint32)


def _mut_clean_lanes(w):
    # cleans every -0 lane instead of only the exact sentinel word
    w = np.asarray(w, dtype=np.uint32)
    lo, hi = w & 0xFFFF, w >> 16
    lo = np.where(lo == 0x8000, 0, lo)
    hi = np.where(hi == 0x8000, 0, hi)
    return (lo | (hi << 16)).astype(np.uint32)


def _mut_norm_no_eps(x, gamma, eps):
    return oar.rms_norm(x, gamma, 0.0)


def _mut_norm_sum_not_mean(x, gamma, eps):
    v = obf.widen(x).astype(np.float64)
    g = obf.widen(gamma).astype(np.float64)
    rstd = 1.0 / np.sqrt(np.sum(v * v, axis=-1, keepdims=True) + float(np.float32(eps)))
    return obf.round_to_bf16(v * rstd * g)


def _mut_norm_no_gamma(x, gamma, eps):
    return oar.rms_norm(x, np.full_like(gamma, 0x3F80), eps)


def _mut_norm_wrong_width(x, gamma, eps):
    v = obf.widen(x).astype(np.float64)
    g = obf.widen(gamma).astype(np.float64)
    rstd = 1.0 / np.sqrt(np.sum(v * v, axis=-1, keepdims=True) / 7167 + float(np.float32(eps)))
    return obf.round_to_bf16(v * rstd * g)


def _mut_norm_f64_range(x, gamma, eps):
    v = obf.widen(x).astype(np.float64)
    g = obf.widen(gamma).astype(np.float64)
    rstd = 1.0 / np.sqrt(np.sum(v * v, axis=-1, keepdims=True) / 7168 + float(np.float32(eps)))
    return obf.round_to_bf16(v * rstd * g)


def _mut_residual_double_round(r, c):
    if c is None:
        return np.asarray(r).copy()
    s = obf.widen(r).astype(np.float64) + obf.widen(c).astype(np.float64)
    return _mut_truncate(s.astype(np.float32))


def _reduce_residual_one_rounding(box, parity, m, residual, gamma, eps):
    # the residual added to the unrounded FP32 all-reduce: one rounding instead of two
    slots = box[parity, :, :m, :]
    olp.check_published(slots, "mutant")
    lanes = obf.widen(obf.unpack_pairs(slots.copy()))
    box[parity, :, :m, :] = S0
    total = lanes[0].copy()
    for k in range(1, lanes.shape[0]):
        total = (total + lanes[k]).astype(np.float32)
    if residual is not None:
        total = (total + obf.widen(residual)).astype(np.float32)
    new_res = obf.round_to_bf16(total)
    return oar.rms_norm(new_res, gamma, eps), new_res


def _with_allreduce(fn):
    def reduce_fn(box, parity, m, residual, gamma, eps):
        slots = box[parity, :, :m, :]
        olp.check_published(slots, "mutant")
        raw = slots.copy()
        box[parity, :, :m, :] = S0
        red = fn(raw)
        return oar.rms_norm(oar.add_residual(red, residual), gamma, eps), oar.add_residual(red, residual)
    return reduce_fn


def _push_with_clean(clean_fn):
    def push(box, partial, parity, rank):
        nslots, m, _ = partial.shape
        olp.check_armed(box[parity, rank:rank + nslots, :m], "mutant")
        box[parity, rank:rank + nslots, :m] = clean_fn(obf.pack_pairs(partial))
    return push


def _push_no_check(box, partial, parity, rank):
    nslots, m, _ = partial.shape
    box[parity, rank:rank + nslots, :m] = olp.clean(obf.pack_pairs(partial))


def _reduce_no_rearm(box, parity, m, residual, gamma, eps):
    return oar.arnorm_rows(box[parity, :, :m, :].copy(), residual, gamma, eps)


def _reduce_rearm_all_parities(box, parity, m, residual, gamma, eps):
    raw = box[parity, :, :m, :].copy()
    box[...] = S0
    return oar.arnorm_rows(raw, residual, gamma, eps)


def _gather_poll_no_rearm(gbox, m, copy):
    return gbox[:m].copy() if copy else None


def _gather_push_no_clean(gbox, shard, rank):
    nslots, m, s = shard.shape
    for k in range(nslots):
        gbox[:m, (rank + k) * s:(rank + k + 1) * s] = shard[k]


def _ts_keep_negative_zero(recv, gath, parity, m):
    slots = recv[parity, :, :m]
    olp.check_published(slots, "mutant")
    raw = slots.copy()
    recv[parity, :, :m] = S0
    red = oar.allreduce_rows(raw)
    gath[parity, 0, :m] = obf.pack_pairs(red)
    return red


def _ts_reader_keeps_row(gath, parity, m):
    return obf.unpack_pairs(gath[parity, 0, :m].copy())


def _ts_owner_keeps_slots(recv, gath, parity, m):
    raw = recv[parity, :, :m].copy()
    red = ots.reduce_no_negative_zero(raw)
    gath[parity, 0, :m] = obf.pack_pairs(red)
    return red


MUTANTS = {
    "two-shot keeps -0": lambda: check_twoshot_golden(ots.twoshot_push, _ts_keep_negative_zero),
    "two-shot -0 kept (theorem)": lambda: check_twoshot_theorem(oar.allreduce_rows),
    "two-shot reader keeps row": lambda: check_twoshot_protocol(ots.twoshot_push, ots.twoshot_reduce,
                                                                _ts_reader_keeps_row),
    "two-shot owner keeps slots": lambda: check_twoshot_protocol(ots.twoshot_push, _ts_owner_keeps_slots,
                                                                 ots.twoshot_read),
    "tree order": lambda: check_allreduce_golden(oar.arnorm_push, _with_allreduce(_mut_tree)),
    "reverse order": lambda: check_allreduce_golden(oar.arnorm_push, _with_allreduce(_mut_reverse)),
    "sum from +0": lambda: check_allreduce_golden(oar.arnorm_push, _with_allreduce(_mut_from_zero)),
    "dropped slot": lambda: check_exact_prefix_tp8(_mut_drop_last),
    "float64 accumulate": lambda: check_allreduce_golden(oar.arnorm_push, _with_allreduce(_mut_f64_accumulate)),
    "truncating round": lambda: check_rounding_vs_torch(_mut_truncate),
    "round half up": lambda: check_rounding_vs_torch(_mut_round_half_up),
    "no clean": lambda: check_clean(_mut_no_clean),
    "clean per lane": lambda: check_clean(_mut_clean_lanes),
    "push without clean": lambda: check_allreduce_golden(_push_with_clean(_mut_no_clean), oar.arnorm_reduce_norm),
    "push cleans lanes": lambda: check_allreduce_golden(_push_with_clean(_mut_clean_lanes), oar.arnorm_reduce_norm),
    "push ignores arming": lambda: check_protocol(_push_no_check, oar.arnorm_reduce_norm),
    "reader skips re-arm": lambda: check_protocol(oar.arnorm_push, _reduce_no_rearm),
    "re-arm both parities": lambda: check_protocol(oar.arnorm_push, _reduce_rearm_all_parities),
    "norm without eps": lambda: check_norm_closed_forms(_mut_norm_no_eps),
    "norm sum not mean": lambda: check_norm_closed_forms(_mut_norm_sum_not_mean),
    "norm without gamma": lambda: check_norm_random_rows(_mut_norm_no_gamma),
    "norm over 7167": lambda: check_norm_random_rows(_mut_norm_wrong_width),
    "norm sum in float64 range": lambda: check_norm_fp32_range(_mut_norm_f64_range),
    "residual truncated": lambda: check_residual_add(_mut_residual_double_round),
    "residual before the all-reduce rounding": lambda: check_residual_golden(oar.arnorm_push,
                                                                             _reduce_residual_one_rounding),
    "gather keeps rows": lambda: check_gather(oga.gather_push, _gather_poll_no_rearm),
    "gather no clean": lambda: check_gather(_gather_push_no_clean, oga.gather_poll),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutants_are_caught(name):
    with pytest.raises((AssertionError, olp.ProtocolError, pytest.fail.Exception)):
        MUTANTS[name]()
