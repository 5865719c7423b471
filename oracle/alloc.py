"""Models of the two KV pools' allocators (TEST INFRASTRUCTURE).

HOT pool (paperlayer.ai summary §3 "Asymmetric KV-cache paging"; reading card
"Key ideas": one contiguous slab per prefix node, bump-pointer allocated;
Appendix B.8: mixed slab sizes use first-fit packing; Appendix B.10: admission
fails when no contiguous extent fits, either because the pool is full or
because the free fragments are all smaller than the prefix, and existing slabs
are never demoted).

Reading adopted (the pages mix "bump pointer" and "first fit"): free space is
a list of extents ordered by address; the last one reaches the end of the pool
and plays the bump region.  An allocation of n tokens takes the LOWEST-address
free extent of length >= n and carves the slab from that extent's start.
Freeing a slab merges it with free neighbours.  With no frees the offsets are
the running sum of the lengths, i.e. a plain bump allocator.  A failed
allocation changes nothing.  Prefix ids are the smallest unused non-negative
integers.

Granularity (``block``): the pages fix none.  With block = b, space is
counted in blocks of b tokens: a prefix of n tokens occupies ceil(n / b)
blocks starting on a block boundary, and a pool of C tokens holds floor(C / b)
blocks.  block = 1 is the plain reading above; the HIP library allocates in
blocks of its attention kernels' K/V tile (32 tokens).

COLD pool (paperlayer.ai §3: page size one token; reading card: token-level
free list).  Reading adopted: a LIFO stack of free slots.  A fresh pool hands
out 0, 1, 2, ...; ``free(slots)`` pushes the slots in the order given, so the
last one freed is the first one handed out again; ``alloc(n)`` pops n slots
in sequence and is all-or-nothing.
"""

from __future__ import annotations


class NoSpace(Exception):
    """No extent (HOT) or not enough slots (COLD) for the request."""


class NotFound(Exception):
    """Unknown or already-freed prefix id / slot."""


class HotAllocModel:
    def __init__(self, capacity: int, block: int = 1):
        if capacity < 0 or block < 1:
            raise ValueError("capacity must be >= 0 and block >= 1")
        self.block = int(block)
        self.capacity = int(capacity) // self.block * self.block
        # [offset, length] in tokens (multiples of block), address order
        self.free_extents = [[0, self.capacity]] if self.capacity > 0 else []
        self.live = {}  # id -> (offset, length in tokens as requested)

    def _next_id(self) -> int:
        i = 0
        while i in self.live:
            i += 1
        return i

    def alloc(self, n: int):
        """Return (prefix_id, token_offset) or raise NoSpace (state unchanged)."""
        if n <= 0:
            raise ValueError("n must be >= 1")
        span = -(-n // self.block) * self.block   # whole blocks
        for ext in self.free_extents:          # lowest address first
            if ext[1] >= span:
                off = ext[0]
                ext[0] += span
                ext[1] -= span
                if ext[1] == 0:
                    self.free_extents.remove(ext)
                pid = self._next_id()
                self.live[pid] = (off, n)
                return pid, off
        raise NoSpace(f"no contiguous extent of {n} tokens")

    def free(self, pid: int):
        if pid not in self.live:
            raise NotFound(f"prefix id {pid} is not live")
        off, n = self.live.pop(pid)
        exts = self.free_extents + [[off, -(-n // self.block) * self.block]]
        exts.sort()
        merged = []
        for o, ln in exts:
            if merged and merged[-1][0] + merged[-1][1] == o:
                merged[-1][1] += ln
            else:
                merged.append([o, ln])
        self.free_extents = merged

    def free_tokens(self) -> int:
        return sum(ln for _, ln in self.free_extents)

    def largest_hole(self) -> int:
        return max((ln for _, ln in self.free_extents), default=0)


class ColdAllocModel:
    def __init__(self, capacity: int):
        if capacity < 0:
            raise ValueError("capacity must be >= 0")
        self.capacity = int(capacity)
        self.stack = list(range(self.capacity - 1, -1, -1))  # top of stack = last element = slot 0
        self.allocated = set()

    def alloc(self, n: int):
        if n < 0:
            raise ValueError("n must be >= 0")
        if n > len(self.stack):
            raise NoSpace(f"{n} slots requested, {len(self.stack)} free")
        out = [self.stack.pop() for _ in range(n)]
        self.allocated.update(out)
        return out

    def free(self, slots):
        seen = set()
        for s in slots:
            if s not in self.allocated or s in seen:
                raise NotFound(f"slot {s} is not allocated")
            seen.add(s)
        for s in slots:
            self.allocated.remove(s)
            self.stack.append(s)

    def free_count(self) -> int:
        return len(self.stack)
