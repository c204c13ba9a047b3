"""ctypes binding of libarnorm.so (include/arnorm.h), with the same entry-point names.

Argument marshalling only: torch tensors become device pointers and sizes, the
stream becomes torch's current HIP stream, return codes become None (NOT_SERVED,
the pages' "shape not served" answer) or an exception.  Every step of the method
runs in the HIP kernels of the library; importing this module fails loudly when the
library is not built.
"""

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libarnorm.so")

OK, NOT_SERVED, BAD_ARG, HIP_ERROR, TIMEOUT, TOO_LARGE = 0, 1, 2, 3, 4, 5
SENTINEL = 0x80000000
HIDDEN = 7168
ROW_WORDS = 3584
NORM_BOX_ROW_WORDS = 256

_c_int, _c_ptr, _c_size, _c_u32, _c_u64, _c_float = (
    ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_float)

_SIGNATURES = {
    "lamport_arm": (_c_int, [_c_ptr, _c_size, _c_u32, _c_ptr]),
    "arnorm_push": (_c_int, [_c_ptr, _c_ptr, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_ptr]),
    "arnorm_reduce_norm": (_c_int, [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_int, _c_int,
                                    _c_int, _c_int, _c_int, _c_int, _c_float, _c_ptr]),
    "arnorm_push_reduce_norm": (_c_int, [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_int, _c_int,
                                         _c_int, _c_int, _c_int, _c_float, _c_ptr]),
    "arnorm_push_reduce_norm_static": (_c_int, [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_int, _c_int,
                                                _c_int, _c_int, _c_int, _c_float, _c_ptr]),
    "gather_push": (_c_int, [_c_ptr, _c_ptr, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_ptr]),
    "gather_poll": (_c_int, [_c_ptr, _c_ptr, _c_int, _c_int, _c_int, _c_int, _c_int, _c_ptr]),
    "gather_push_poll": (_c_int, [_c_ptr, _c_ptr, _c_ptr, _c_int, _c_int, _c_int, _c_int, _c_int, _c_ptr]),
    "twoshot_push": (_c_int, [_c_ptr, _c_ptr, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                              _c_ptr]),
    "twoshot_reduce": (_c_int, [_c_ptr, _c_ptr, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_ptr]),
    "twoshot_read": (_c_int, [_c_ptr, _c_ptr, _c_int, _c_int, _c_int, _c_int, _c_int, _c_ptr]),
    "twoshot_push_reduce_read": (_c_int, [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_int, _c_int, _c_int, _c_int, _c_int,
                                          _c_int, _c_ptr]),
    "arnorm_set_spin_limit": (_c_int, [_c_u64]),
    "arnorm_get_spin_limit": (_c_u64, []),
    "arnorm_set_reduce_threads": (_c_int, [_c_int]),
    "arnorm_set_reduce_split": (_c_int, [_c_int]),
    "arnorm_set_poll": (_c_int, [_c_int, _c_int]),
    "arnorm_status": (_c_int, [ctypes.POINTER(_c_int), _c_ptr]),
    "arnorm_strerror": (ctypes.c_char_p, [_c_int]),
}


def load_library(path=LIB_PATH):
    """dlopen libarnorm.so and declare the C signatures (no GPU call is made)."""
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built: run `python -m tp_all_reduce_arnorm_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


LIB = load_library()


class ArnormError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn}: {LIB.arnorm_strerror(code).decode()} (code {code})")
        self.code = code


def _check(fn, code):
    if code == OK:
        return True
    if code == NOT_SERVED:
        return None
    raise ArnormError(fn, code)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    elif stream.device.index != torch.cuda.current_device():
        raise ValueError(f"stream is on {stream.device}, the current device is cuda:{torch.cuda.current_device()}")
    return ctypes.c_void_p(stream.cuda_stream)


def _shape(t, shape, what):
    """Raise ValueError unless tensor t has this shape: the kernels index the caller's
    buffers by the sizes passed, so a short buffer would be read or written past its
    end."""
    if t is None or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} must have shape {tuple(shape)}, got {None if t is None else tuple(t.shape)}")


# BF16 arguments: bfloat16 tensors, or int16 / uint16 tensors holding BF16 bit patterns.
BF16_DTYPES = (torch.bfloat16, torch.int16, torch.uint16)
# Mailboxes, shards and gathered rows: 32-bit words.
WORD_DTYPES = (torch.int32, torch.uint32)
_DTYPES = {2: BF16_DTYPES, 4: WORD_DTYPES}


def bf16_served(*tensors):
    """Whether every given BF16 argument is BF16 (None entries are absent arguments).
    drafter.comm, DrafterComm.ar_norm: the front-end serves BF16 rows only and returns None
    otherwise; a float16 or float32 tensor would otherwise be read as BF16 bits."""
    return all(t is None or t.dtype in BF16_DTYPES for t in tensors)


def _words(t, what):
    if t is not None and t.dtype not in WORD_DTYPES:
        raise ValueError(f"{what} must hold 32-bit words (int32), got {t.dtype}")


def _ptr(t, nbytes_per_elem=None, what="tensor"):
    if t is None:
        return None
    if nbytes_per_elem is not None and t.dtype not in _DTYPES[nbytes_per_elem]:
        raise ValueError(f"{what} must be one of {', '.join(str(d) for d in _DTYPES[nbytes_per_elem])}, got {t.dtype}")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{what} must be a contiguous device tensor")
    if t.device.index != torch.cuda.current_device():
        # the kernels run on the current device, which must own every buffer they touch
        raise ValueError(f"{what} is on {t.device}, the current device is cuda:{torch.cuda.current_device()}")
    return ctypes.c_void_p(t.data_ptr())


def lamport_arm(buf, sentinel=SENTINEL, stream=None):
    """Fill a mailbox (a contiguous int32 tensor) with the sentinel."""
    _words(buf, "buf")
    return _check("lamport_arm", LIB.lamport_arm(_ptr(buf, 4, "buf"), buf.numel(), sentinel, _stream(stream)))


def arnorm_push(partial, mailbox, parity, rank, stream=None):
    """partial: BF16 [nslots, M, 7168] (bfloat16/int16/uint16); mailbox: int32
    [parities, tp, cap, 3584].  Pushes slots rank .. rank+nslots-1 of mailbox[parity].
    None (not served) for a partial of another dtype or width."""
    if not bf16_served(partial):
        return None
    _words(mailbox, "mailbox")
    nslots, m, width = partial.shape
    if width != HIDDEN:
        return None
    p, tp, cap, words = mailbox.shape
    if words != ROW_WORDS:
        raise ValueError(f"mailbox rows must be {ROW_WORDS} words, got {words}")
    return _check("arnorm_push", LIB.arnorm_push(
        _ptr(partial, 2, "partial"), _ptr(mailbox, 4, "mailbox"), p, tp, cap, parity, rank, nslots, m,
        _stream(stream)))


def arnorm_reduce_norm(residual, gamma, mailbox, parity, eps, out, residual_out, partial=None, rank=0,
                       norm_box=None, stream=None):
    """Poll, re-arm and reduce rows < M (M = out.shape[0]) of mailbox[parity]; writes
    out and residual_out (BF16 [M, 7168]).  residual None: residual = AR(x).
    partial (BF16 [M, 7168]) is the fused own-rank push of rank `rank`.  norm_box
    (int32 [parities, cap, 256], sentinel-armed) lets small-M calls split rows.
    None (not served) when a BF16 argument has another dtype (as the pages' ar_norm)."""
    if not bf16_served(residual, gamma, out, residual_out, partial):
        return None
    _words(mailbox, "mailbox")
    _words(norm_box, "norm_box")
    m, width = out.shape
    if width != HIDDEN:
        return None
    p, tp, cap, words = mailbox.shape
    if words != ROW_WORDS:
        raise ValueError(f"mailbox rows must be {ROW_WORDS} words, got {words}")
    _shape(residual_out, (m, HIDDEN), "residual_out")
    _shape(gamma, (HIDDEN,), "gamma")
    if residual is not None:
        _shape(residual, (m, HIDDEN), "residual")
    if partial is not None:
        _shape(partial, (m, HIDDEN), "partial")
    if norm_box is not None:
        _shape(norm_box, (p, cap, NORM_BOX_ROW_WORDS), "norm_box")
    return _check("arnorm_reduce_norm", LIB.arnorm_reduce_norm(
        _ptr(partial, 2, "partial"), _ptr(residual, 2, "residual"), _ptr(gamma, 2, "gamma"),
        _ptr(out, 2, "out"), _ptr(residual_out, 2, "residual_out"), _ptr(mailbox, 4, "mailbox"),
        _ptr(norm_box, 4, "norm_box"), p, tp, cap, parity, rank, m, float(eps), _stream(stream)))


def arnorm_push_reduce_norm(partials, residual, gamma, mailbox, parity, eps, out, residual_out, norm_box=None,
                            stream=None):
    """One stand-in call: every rank's push (partials BF16 [tp, M, 7168]) and the
    consumer.  One launch when norm_box is given and the TP slots of rows < M total at
    most 1 MiB (M <= 9 at TP=8); otherwise the pair arnorm_push + arnorm_reduce_norm.
    None (not served) when a BF16 argument has another dtype (as the pages' ar_norm)."""
    if not bf16_served(partials, residual, gamma, out, residual_out):
        return None
    _words(mailbox, "mailbox")
    _words(norm_box, "norm_box")
    tp_, m, width = partials.shape
    if width != HIDDEN:
        return None
    p, tp, cap, words = mailbox.shape
    if words != ROW_WORDS:
        raise ValueError(f"mailbox rows must be {ROW_WORDS} words, got {words}")
    if tp_ != tp:
        raise ValueError(f"partials hold {tp_} ranks, the mailbox {tp} slots")
    _shape(out, (m, HIDDEN), "out")
    _shape(residual_out, (m, HIDDEN), "residual_out")
    _shape(gamma, (HIDDEN,), "gamma")
    if residual is not None:
        _shape(residual, (m, HIDDEN), "residual")
    if norm_box is not None:
        _shape(norm_box, (p, cap, NORM_BOX_ROW_WORDS), "norm_box")
    return _check("arnorm_push_reduce_norm", LIB.arnorm_push_reduce_norm(
        _ptr(partials, 2, "partials"), _ptr(residual, 2, "residual"), _ptr(gamma, 2, "gamma"),
        _ptr(out, 2, "out"), _ptr(residual_out, 2, "residual_out"), _ptr(mailbox, 4, "mailbox"),
        _ptr(norm_box, 4, "norm_box"), p, tp, cap, parity, m, float(eps), _stream(stream)))


def arnorm_push_reduce_norm_static(partials, residual, gamma, mailbox, parity, eps, out, residual_out,
                                   stream=None):
    """arnorm_push_reduce_norm whose norm box is the library's own static array: no
    workspace argument and no allocation, for M <= 64 rows (ArnormError TOO_LARGE above).
    Calls that overlap on one device race on that array."""
    if not bf16_served(partials, residual, gamma, out, residual_out):
        return None
    _words(mailbox, "mailbox")
    tp_, m, width = partials.shape
    if width != HIDDEN:
        return None
    p, tp, cap, words = mailbox.shape
    if words != ROW_WORDS:
        raise ValueError(f"mailbox rows must be {ROW_WORDS} words, got {words}")
    if tp_ != tp:
        raise ValueError(f"partials hold {tp_} ranks, the mailbox {tp} slots")
    _shape(out, (m, HIDDEN), "out")
    _shape(residual_out, (m, HIDDEN), "residual_out")
    _shape(gamma, (HIDDEN,), "gamma")
    if residual is not None:
        _shape(residual, (m, HIDDEN), "residual")
    return _check("arnorm_push_reduce_norm_static", LIB.arnorm_push_reduce_norm_static(
        _ptr(partials, 2, "partials"), _ptr(residual, 2, "residual"), _ptr(gamma, 2, "gamma"),
        _ptr(out, 2, "out"), _ptr(residual_out, 2, "residual_out"), _ptr(mailbox, 4, "mailbox"), p, tp, cap, parity,
        m, float(eps), _stream(stream)))


def gather_push(shard, mailbox, tp, rank, stream=None):
    """shard: int32 [nslots, M, S]; mailbox: int32 [cap, tp*S]."""
    _words(shard, "shard")
    _words(mailbox, "mailbox")
    nslots, m, s = shard.shape
    cap, width = mailbox.shape
    if width != tp * s:
        raise ValueError(f"mailbox rows must be tp*S = {tp * s} words, got {width}")
    return _check("gather_push", LIB.gather_push(
        _ptr(shard, 4, "shard"), _ptr(mailbox, 4, "mailbox"), tp, cap, s, rank, nslots, m, _stream(stream)))


def gather_poll(mailbox, tp, m, out=None, copy=True, stream=None):
    """Poll rows < m of mailbox (int32 [cap, tp*S]); copy: into out (int32 [m, tp*S])
    and re-arm; no copy: leave the published rows in place."""
    _words(mailbox, "mailbox")
    _words(out, "out")
    cap, width = mailbox.shape
    if tp < 1 or width % tp:
        raise ValueError(f"mailbox rows of {width} words do not split over tp = {tp}")
    s = width // tp
    if copy:
        _shape(out, (m, width), "out")
    return _check("gather_poll", LIB.gather_poll(
        _ptr(mailbox, 4, "mailbox"), _ptr(out, 4, "out") if copy else None, tp, cap, s, m, 1 if copy else 0,
        _stream(stream)))


def gather_push_poll(shard, mailbox, out=None, copy=True, stream=None):
    """One Gather call: every rank's shard (int32 [tp, M, S]) pushed and the M gathered
    rows polled (copied into out and re-armed, or left published), in one launch for
    small calls."""
    _words(shard, "shard")
    _words(mailbox, "mailbox")
    _words(out, "out")
    tp, m, s = shard.shape
    cap, width = mailbox.shape
    if width != tp * s:
        raise ValueError(f"mailbox rows must be tp*S = {tp * s} words, got {width}")
    if copy:
        _shape(out, (m, width), "out")
    return _check("gather_push_poll", LIB.gather_push_poll(
        _ptr(shard, 4, "shard"), _ptr(mailbox, 4, "mailbox"), _ptr(out, 4, "out") if copy else None, tp, cap, s, m,
        1 if copy else 0, _stream(stream)))


def twoshot_push(partial, recv, parity, rank, stream=None):
    """partial: BF16 [nslots, M, width]; recv: int32 [parities, tp, cap, width/2].  None
    (not served) for a partial of another dtype."""
    if not bf16_served(partial):
        return None
    _words(recv, "recv")
    nslots, m, width = partial.shape
    p, tp, cap, words = recv.shape
    if words * 2 != width:
        raise ValueError(f"recv rows of {words} words do not hold {width} BF16 columns")
    return _check("twoshot_push", LIB.twoshot_push(
        _ptr(partial, 2, "partial"), _ptr(recv, 4, "recv"), p, tp, cap, width, parity, rank, nslots, m,
        _stream(stream)))


def twoshot_reduce(recv, gather, parity, m, stream=None):
    """The owner's reduce of rows < m: recv int32 [parities, tp, cap, width/2] into the
    gather row int32 [parities, 1, cap, width/2]."""
    _words(recv, "recv")
    _words(gather, "gather")
    p, tp, cap, words = recv.shape
    _shape(gather, (p, 1, cap, words), "gather")
    return _check("twoshot_reduce", LIB.twoshot_reduce(
        _ptr(recv, 4, "recv"), _ptr(gather, 4, "gather"), p, tp, cap, 2 * words, parity, m, _stream(stream)))


def twoshot_read(gather, parity, out, stream=None):
    """A reader of the gather row: rows < M (M = out.shape[0]) into out (BF16 [M, width]).
    None (not served) for an out of another dtype."""
    if not bf16_served(out):
        return None
    _words(gather, "gather")
    p, one, cap, words = gather.shape
    m, width = out.shape
    if one != 1 or width != 2 * words:
        raise ValueError(f"gather must be [parities, 1, cap, width/2] for out [M, {width}]")
    return _check("twoshot_read", LIB.twoshot_read(
        _ptr(gather, 4, "gather"), _ptr(out, 2, "out"), p, cap, width, parity, m, _stream(stream)))


def twoshot_push_reduce_read(partial, recv, gather, parity, out, stream=None):
    """One two-shot call of every rank: partial BF16 [tp, M, width] pushed into recv,
    reduced by the owner into the gather row, read into out (BF16 [M, width]); one
    launch for small calls.  None (not served) when partial or out has another dtype."""
    if not bf16_served(partial, out):
        return None
    _words(recv, "recv")
    _words(gather, "gather")
    tp, m, width = partial.shape
    p, tp2, cap, words = recv.shape
    if tp2 != tp or words * 2 != width:
        raise ValueError(f"recv must be [parities, {tp}, cap, {width // 2}], got {tuple(recv.shape)}")
    _shape(gather, (p, 1, cap, words), "gather")
    _shape(out, (m, width), "out")
    return _check("twoshot_push_reduce_read", LIB.twoshot_push_reduce_read(
        _ptr(partial, 2, "partial"), _ptr(recv, 4, "recv"), _ptr(gather, 4, "gather"), _ptr(out, 2, "out"), p, tp,
        cap, width, parity, m, _stream(stream)))


def set_spin_limit(polls):
    return _check("arnorm_set_spin_limit", LIB.arnorm_set_spin_limit(polls))


def get_spin_limit():
    return int(LIB.arnorm_get_spin_limit())


def set_reduce_split(workgroups_per_row):
    return _check("arnorm_set_reduce_split", LIB.arnorm_set_reduce_split(workgroups_per_row))


def set_poll(frags_per_thread=0, mode=0):
    """Gather poll layout: fragments per thread in flight (0 auto, 1, 4) and the wait
    (0 auto, 1 re-read every pending fragment, 2 one witness per wave)."""
    return _check("arnorm_set_poll", LIB.arnorm_set_poll(frags_per_thread, mode))


def set_reduce_threads(threads):
    return _check("arnorm_set_reduce_threads", LIB.arnorm_set_reduce_threads(threads))


def status(stream=None):
    """Synchronize the stream; read and clear the device status (OK or TIMEOUT)."""
    v = ctypes.c_int(-1)
    _check("arnorm_status", LIB.arnorm_status(ctypes.byref(v), _stream(stream)))
    return v.value
