"""Model of appending a decoded token's K/V into the COLD pool (TEST INFRASTRUCTURE).

The COLD pool holds suffix tokens and decoded tokens one token per slot
(paperlayer.ai summary §1 "Design" and §3 "Asymmetric KV-cache paging").
Appending the new token of request i writes its K (and V) row, all KV heads,
into pool row slots[i]; every other row is left as it was.
"""

from __future__ import annotations

import numpy as np


def append_model(pool, slots, rows):
    """Return a copy of ``pool`` [C, n_kv, d] with pool[slots[i]] = rows[i].

    Byte-exact: no arithmetic, only a scatter.  With repeated slots the last
    write wins (the order rows are given in).
    """
    out = np.array(pool, copy=True)
    for i, s in enumerate(np.asarray(slots).tolist()):
        out[s] = rows[i]
    return out
