"""CPU oracle for the Lamport-mailbox ArNorm and Gather — TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously correct statement of what the hot path
computes, written from the vLLM API-doc pages for the DSpark drafter's TP collectives
(page "drafter.comm": the module prose, the ArNorm / Gather / clean / LamportRows
entries) and the two-shot all-reduce page ("cutedsl.common.twoshot": its module
prose and the push / reduce entries).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The product path (the HIP library and its Python
binding) never imports, calls or links anything here, and this package imports
nothing from the product path: the two share no code.  Inputs for both come from
``tp_all_reduce_arnorm_amd.workloads``, which holds no arithmetic of the method.

Everything is numpy on the CPU, single-threaded, bit-level where the pages fix the
bits (BF16 patterns as uint16, mailbox words as uint32) and float64 where they leave
the order open (the RMS sum of squares).

Pins (what the oracle is checked against, in ``tests/test_oracle.py``):
  * clean            -- hand cases of the sentinel pair (tests/golden/clean_words.txt)
  * round_to_bf16    -- torch's CPU float->bfloat16 cast and exact Fraction rounding
  * rank-order sum   -- TP=2 double-rounding theorem (exact Fraction sum), exact-prefix
                        TP=8 cases, the rank-vs-tree hand case, signed-zero hand cases
  * residual add     -- exact Fraction sum rounded once; hand cases of the all-reduce
                        rounded before the residual is added (tests/golden/residual_words.txt)
  * RMSNorm          -- closed forms (zero row, one-hot row, constant row, eps-dominated
                        row, a row past the FP32 range) and a 60-digit decimal reference
                        on random rows
  * mailbox protocol -- arm / push / poll / re-arm invariants, parity reuse
  * gather           -- hand case, byte movement, state after copy / no-copy
  * two-shot         -- the no-negative-zero hand cases (tests/golden/twoshot_words.txt),
                        the TP=2 theorem with -0 mapped to +0, and its protocol
Parity unpinned: the pages' kernel's exact sum-of-squares bit pattern (its tree order
is not something the oracle reproduces); ``out`` is pinned to 1 BF16 ulp, and the GPU
tests also bound how many of its values may differ from the oracle's bits at all
(``tests/gpu_util.assert_out_close``, itself pinned in ``tests/test_compare_contract.py``).
"""

from .bf16 import (  # noqa: F401
    widen,
    round_to_bf16,
    pack_pairs,
    unpack_pairs,
)
from .lamport import (  # noqa: F401
    SENTINEL,
    HIDDEN,
    WORDS_PER_ROW,
    ProtocolError,
    clean,
    published,
    arm,
)
from .arnorm import (  # noqa: F401
    arnorm_push,
    arnorm_reduce_norm,
    allreduce_rows,
    add_residual,
    rms_norm,
    arnorm_rows,
)
from .gather import gather_push, gather_poll  # noqa: F401
from .twoshot import twoshot_push, twoshot_reduce, twoshot_read, reduce_no_negative_zero  # noqa: F401
