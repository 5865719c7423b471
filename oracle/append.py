"""Model of appending a decoded token's K/V into the COLD pool (TEST INFRASTRUCTURE).

The COLD pool holds suffix tokens and decoded tokens one token per slot
(paperlayer.ai summary §1 "Design" and §3 "Asymmetric KV-cache paging").
Appending the new token of request i writes its K (and V) row, all KV heads,
into pool slot slots[i]; every other slot is left as it was.

Inside a slot the pages fix no order of the KV heads.  The library's layout
(a reading of its own, stated with the pool format): the row of KV head g
sits at position g XOR (slot mod P), where P is the largest power of two
that divides n_kv; so P = 1 (odd n_kv) keeps head g at position g.
"""

from __future__ import annotations

import numpy as np


def slot_position(g: int, slot: int, n_kv: int) -> int:
    """In-slot position of KV head g's row in COLD slot ``slot``."""
    p = 1
    while n_kv % (2 * p) == 0:
        p *= 2
    return g ^ (slot % p)


def append_model(pool, slots, rows):
    """Return a copy of ``pool`` [C, n_kv, d] with slot slots[i] holding token
    row rows[i] [n_kv, d], head g at position slot_position(g, slots[i]).

    Byte-exact: no arithmetic, only a scatter.  With repeated slots the last
    write wins (the order rows are given in).
    """
    out = np.array(pool, copy=True)
    n_kv = out.shape[1]
    for i, s in enumerate(np.asarray(slots).tolist()):
        for g in range(n_kv):
            out[s, slot_position(g, s, n_kv)] = rows[i][g]
    return out
