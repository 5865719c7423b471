"""Model of the shared-prefix registry and its admission policy (TEST INFRASTRUCTURE).

What the pages fix:

* Admission is HOT-first: a prefix goes to the contiguous HOT pool when a
  contiguous extent of its length exists, otherwise to COLD; the HOT attempt
  fails when the pool is full or when every free fragment is shorter than the
  prefix (paperlayer.ai Appendix B.10 "Cross-pool admission and promotion
  policy").
* Prefixes already in HOT are never demoted to make room (same appendix):
  while a prefix is resident its slab does not move.
* The HOT share of the KV budget, f_p, is fixed when the server starts and
  defaults to 0.2 (paperlayer.ai "Limitations", static HOT/COLD pool
  fraction).
* Each distinct prefix is tagged on its own and gets a slab of its own
  (paperlayer.ai Appendix B.8, heterogeneous multi-prefix serving); the engine
  integrates admission and eviction (paperlayer.ai §1 "Design").

Readings where the pages are silent (each listed in the design notes):

* A prefix is identified by a caller-chosen 64-bit key and carries a
  reference count; ``acquire`` adds a reference (admitting the prefix if it is
  not resident), ``release`` drops one.
* A prefix whose count reaches zero stays resident (a cached prefix) and
  becomes evictable.  Cached prefixes are evicted least recently released
  first, and only when an admission needs their space, or on an explicit
  ``evict`` / ``reclaim_cold``.  Evicting frees the prefix's storage; it is not
  a demotion (nothing that is referenced moves or changes pool).
* HOT capacity for an admission counts the free extents and the slabs of
  cached HOT prefixes.  If evicting cached HOT prefixes in that order makes a
  contiguous extent appear, exactly that many (the shortest such prefix of
  the order) are evicted and the prefix goes to HOT.  Otherwise COLD is tried
  the same way with the cached COLD prefixes.  If neither can hold it, the
  call fails and nothing changes (no eviction happens).
* Admission places the prefix with the pools' own rules: first fit in HOT,
  LIFO pops in COLD (``oracle.alloc``).
"""

from __future__ import annotations

import copy
from dataclasses import dataclass, field
from typing import Dict, List, Optional

from .alloc import ColdAllocModel, HotAllocModel, NoSpace, NotFound

HOT, COLD = 0, 1


class InvalidArg(Exception):
    """A call that the registry's rules reject (wrong length, count underflow,
    evicting a referenced prefix)."""


def partition(total_tokens: int, f_p: float, block: int = 32):
    """(hot, cold) token capacities for a KV budget of ``total_tokens``: the
    HOT pool takes the fraction f_p, rounded down to whole blocks."""
    if total_tokens < 0 or not (0.0 <= f_p <= 1.0) or block < 1:
        raise InvalidArg("total_tokens >= 0, 0 <= f_p <= 1, block >= 1")
    hot = int(f_p * total_tokens) // block * block
    return hot, total_tokens - hot


@dataclass
class Entry:
    pool: int
    n: int
    refs: int
    hot_id: int = -1
    offset: int = -1
    slots: List[int] = field(default_factory=list)
    tick: int = 0     # release order while cached


class RegistryModel:
    def __init__(self, hot_capacity: int, cold_capacity: int, block: int = 32):
        self.hot = HotAllocModel(hot_capacity, block)
        self.cold = ColdAllocModel(cold_capacity)
        self.block = block
        self.entries: Dict[int, Entry] = {}
        self.clock = 0
        self.hits = self.hot_admits = self.cold_admits = self.evictions = 0

    # ------------------------------------------------------------ helpers
    def _cached(self, pool: int) -> List[int]:
        keys = [k for k, e in self.entries.items() if e.pool == pool and e.refs == 0]
        return sorted(keys, key=lambda k: self.entries[k].tick)

    def _drop(self, key: int):
        e = self.entries.pop(key)
        if e.pool == HOT:
            self.hot.free(e.hot_id)
        else:
            self.cold.free(e.slots)
        self.evictions += 1

    def _hot_evictions_needed(self, n: int) -> Optional[int]:
        """Fewest cached HOT prefixes (in eviction order) whose removal lets a
        slab of n tokens fit; None if even all of them do not suffice."""
        trial = copy.deepcopy(self.hot)
        order = self._cached(HOT)
        span = -(-n // self.block) * self.block
        for j in range(len(order) + 1):
            if trial.largest_hole() >= span:
                return j
            if j < len(order):
                trial.free(self.entries[order[j]].hot_id)
        return None

    def _cold_evictions_needed(self, n: int) -> Optional[int]:
        free = self.cold.free_count()
        order = self._cached(COLD)
        for j in range(len(order) + 1):
            if free >= n:
                return j
            if j < len(order):
                free += self.entries[order[j]].n
        return None

    # ------------------------------------------------------------ calls
    def acquire(self, key: int, n: int):
        """Returns (entry, fresh)."""
        if n < 1:
            raise InvalidArg("n must be >= 1")
        e = self.entries.get(key)
        if e is not None:
            if e.n != n:
                raise InvalidArg(f"key {key} is resident with {e.n} tokens, not {n}")
            e.refs += 1
            self.hits += 1
            return e, False
        j = self._hot_evictions_needed(n)
        if j is not None:
            for k in self._cached(HOT)[:j]:
                self._drop(k)
            pid, off = self.hot.alloc(n)
            e = Entry(HOT, n, 1, hot_id=pid, offset=off)
            self.hot_admits += 1
        else:
            j = self._cold_evictions_needed(n)
            if j is None:
                raise NoSpace(f"no room for a prefix of {n} tokens in HOT or COLD")
            for k in self._cached(COLD)[:j]:
                self._drop(k)
            e = Entry(COLD, n, 1, slots=self.cold.alloc(n))
            self.cold_admits += 1
        self.entries[key] = e
        return e, True

    def release(self, key: int):
        e = self.entries.get(key)
        if e is None:
            raise NotFound(f"key {key} is not resident")
        if e.refs == 0:
            raise InvalidArg(f"key {key} holds no reference")
        e.refs -= 1
        if e.refs == 0:
            self.clock += 1
            e.tick = self.clock

    def evict(self, key: int):
        e = self.entries.get(key)
        if e is None:
            raise NotFound(f"key {key} is not resident")
        if e.refs > 0:
            raise InvalidArg(f"key {key} is referenced")
        self._drop(key)

    def reclaim_cold(self, n_free: int):
        """Evict cached COLD prefixes (eviction order) until at least n_free
        COLD slots are free; NoSpace, with nothing changed, if impossible."""
        if n_free < 0:
            raise InvalidArg("n_free must be >= 0")
        j = self._cold_evictions_needed(n_free)
        if j is None:
            raise NoSpace(f"cannot free {n_free} COLD slots")
        for k in self._cached(COLD)[:j]:
            self._drop(k)

    def stats(self):
        es = list(self.entries.values())
        return dict(resident_hot=sum(e.pool == HOT for e in es), resident_cold=sum(e.pool == COLD for e in es),
                    referenced=sum(e.refs > 0 for e in es), cached=sum(e.refs == 0 for e in es),
                    hits=self.hits, hot_admits=self.hot_admits, cold_admits=self.cold_admits,
                    evictions=self.evictions)
