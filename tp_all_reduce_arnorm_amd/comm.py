"""The drafter's collective front-end in its one-GPU stand-in: mailboxes built once,
and the three calls of drafter.comm's DrafterComm (ar_norm, gather_context,
gather_logits) with the pages' gates, each returning None for what it does not serve
(the caller then runs its stock collective).

drafter.comm, DrafterComm: the drafter's TP all-reduces and gathers own two parities of
the [TP, ROWS_CAP, 7168] all-reduce mailbox, a [CONTEXT_ROWS_CAP, 7168] context-
projection gather row and a [ROWS_CAP, vocab_padded] logits gather row, all BF16 and
armed once at model load.  On one GPU the TP ranks are slots of these mailboxes, so
each call takes every rank's input at once (a leading TP dimension) where the pages'
call takes one rank's.  Host logic only: the buffers are torch allocations, and every
step of each call runs in the library's kernels through the binding in _lib.
"""

import torch

from . import _lib

HIDDEN = _lib.HIDDEN


def ar_norm_served(x, residual, weight, tp, rows_cap):
    """drafter.comm, DrafterComm.ar_norm's gate: x of every rank [TP, M, 7168] with
    1 <= M <= ROWS_CAP, and x, the norm weight and the residual (when given) BF16."""
    return (x.dim() == 3 and x.shape[0] == tp and x.shape[2] == HIDDEN and 1 <= x.shape[1] <= rows_cap
            and x.dtype == torch.bfloat16 and weight.dtype == torch.bfloat16
            and (residual is None or residual.dtype == torch.bfloat16))


def context_served(shards, tp):
    """drafter.comm, DrafterComm.gather_context's gate: BF16 shards of every rank [TP, M,
    S] with S * TP = 7168."""
    return shards.dim() == 3 and shards.shape[0] == tp and shards.dtype == torch.bfloat16 and \
        shards.shape[2] * tp == HIDDEN


def logits_served(shards, tp, vocab_shard):
    """drafter.comm, DrafterComm.gather_logits's gate: a logits row was built (vocab_shard
    given, a multiple of 8) and the shards are BF16 [TP, M, vocab_shard]."""
    return bool(vocab_shard) and vocab_shard % 8 == 0 and shards.dim() == 3 and shards.shape[0] == tp and \
        shards.dtype == torch.bfloat16 and shards.shape[2] == vocab_shard


def rows_served(shards, cap):
    """drafter.comm, DrafterComm._gather's gate: 1 <= rows <= cap and contiguous shards
    (here also an even shard width, so that the BF16 rows are whole 32-bit words)."""
    return 1 <= shards.shape[1] <= cap and shards.is_contiguous() and shards.shape[2] % 2 == 0


class StandInComm:
    """Mailboxes of one TP group on the current device, armed once.

    tp               ranks (2..8), the slots of every mailbox
    rows_cap         the pages' ROWS_CAP: most rows an ar_norm or gather_logits call serves
    context_rows_cap the pages' CONTEXT_ROWS_CAP: most rows of a gather_context call
    vocab_shard      columns of one rank's logits (V / TP); the logits row exists only when
                     it is given and a multiple of 8, as on the pages
    """

    def __init__(self, tp, rows_cap=64, context_rows_cap=64, vocab_shard=None, device=None):
        dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        words = HIDDEN // 2
        self.tp, self.rows_cap, self.context_rows_cap = tp, rows_cap, context_rows_cap
        self.ar = torch.empty((2, tp, rows_cap, words), dtype=torch.int32, device=dev)
        self.norm_box = torch.empty((2, rows_cap, _lib.NORM_BOX_ROW_WORDS), dtype=torch.int32, device=dev)
        self.context = torch.empty((context_rows_cap, words), dtype=torch.int32, device=dev)
        self.logits = None
        self.vocab_shard = vocab_shard
        if vocab_shard and vocab_shard % 8 == 0:
            self.logits = torch.empty((rows_cap, vocab_shard * tp // 2), dtype=torch.int32, device=dev)
        for box in (self.ar, self.norm_box, self.context, self.logits):
            if box is not None:
                assert _lib.lamport_arm(box) is True

    # -- all-reduce + residual + RMSNorm ------------------------------------------

    def ar_norm(self, x, residual, weight, eps, parity):
        """fused all-reduce + residual add + RMSNorm of the TP ranks' partial rows x
        (BF16 [TP, M, 7168]); residual None: the new residual is AR(x).  Returns (out,
        residual_out), BF16 [M, 7168], or None when the shape is not served.  The caller
        alternates `parity` (0, 1) from call to call, as the pages' layers do."""
        if not ar_norm_served(x, residual, weight, self.tp, self.rows_cap):
            return None
        m = x.shape[1]
        x = x.contiguous()
        res = None if residual is None else residual.contiguous()
        out = torch.empty((m, HIDDEN), dtype=torch.bfloat16, device=x.device)
        res_out = torch.empty_like(out)
        if _lib.arnorm_push_reduce_norm(x, res, weight.contiguous(), self.ar, parity, float(eps), out, res_out,
                                        norm_box=self.norm_box) is None:
            return None
        return out, res_out

    # -- gathers --------------------------------------------------------------------

    def _gather(self, box, shards, cap, width):
        """The rows' words gathered into box and copied out (BF16 [M, width]), or None
        (rows_served)."""
        if not rows_served(shards, cap):
            return None
        rows = shards.shape[1]
        out = torch.empty((rows, width), dtype=torch.bfloat16, device=shards.device)
        if _lib.gather_push_poll(shards.view(torch.int32), box, out=out.view(torch.int32), copy=True) is None:
            return None
        return out

    def gather_context(self, shards):
        """The column-parallel context projection's [M, 7168 / TP] rows of every rank
        (BF16 [TP, M, 7168 / TP]) -> [M, 7168]; None unless BF16 and shard width * TP =
        7168 (drafter.comm, DrafterComm.gather_context)."""
        if not context_served(shards, self.tp):
            return None
        return self._gather(self.context, shards, self.context_rows_cap, HIDDEN)

    def gather_logits(self, shards):
        """The vocab-parallel lm_head's [M, V / TP] logits of every rank (BF16 [TP, M,
        V / TP]) -> [M, V]; None unless the logits row exists, the shards are BF16 and
        their width is vocab_shard (drafter.comm, DrafterComm.gather_logits)."""
        if self.logits is None or not logits_served(shards, self.tp, self.vocab_shard):
            return None
        return self._gather(self.logits, shards, self.rows_cap, shards.shape[2] * self.tp)
