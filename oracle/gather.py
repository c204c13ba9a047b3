"""Gather oracle: every rank's [M, S] word shard into the [cap, TP * S] mailbox rows
(test infrastructure only).

drafter.comm page: module prose (Gather bullet, "Exactness" paragraph: the gathers
move bytes, the sentinel pair is the only word that changes) and the Gather class
entry (rank r's shard at columns r*S ..; with copy the row goes to a dense output and
is re-armed; without copy it is left in place for a later reader, who re-arms it).
One-GPU stand-in: the ranks are local column blocks of one buffer.
"""

import numpy as np

from .lamport import SENTINEL, clean, check_armed, check_published


def gather_push(gbox, shard, rank):
    """Shards of ranks rank .. rank+nslots-1 (uint32 [nslots, M, S]) into ``gbox``
    (uint32 [cap, TP * S], modified in place), each word cleaned."""
    shard = np.asarray(shard, dtype=np.uint32)
    nslots, m, s = shard.shape
    assert s % 4 == 0
    for k in range(nslots):
        cols = slice((rank + k) * s, (rank + k + 1) * s)
        check_armed(gbox[:m, cols], f"gather rank {rank + k} rows <{m}")
        gbox[:m, cols] = clean(shard[k])


def gather_poll(gbox, m, copy):
    """Poll rows < m of ``gbox``.  copy: return the rows (uint32 [m, TP * S]) and
    re-arm them; no copy: return None and leave the published rows in place."""
    rows = gbox[:m]
    check_published(rows, f"gather rows <{m}")
    if not copy:
        return None
    out = rows.copy()
    gbox[:m] = np.uint32(SENTINEL)
    return out
