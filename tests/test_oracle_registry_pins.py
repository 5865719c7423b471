"""Pins for the oracle's prefix-registry model (oracle/registry.py).

A trace worked by hand from the admission rules (paperlayer.ai Appendix B.10:
HOT first, COLD when no contiguous HOT extent fits, no demotion; the cached-
prefix readings in the model's header), the f_p partition, and invariants
checked on random operation sequences against brute-force restatements that
do not reuse the model's own search.
"""

import copy

import pytest
from hypothesis import example, given, settings
from hypothesis import strategies as st

from oracle.alloc import HotAllocModel, NoSpace, NotFound
from oracle.registry import COLD, HOT, InvalidArg, RegistryModel, partition


def placement(e):
    return (e.pool, e.hot_id, e.offset, tuple(e.slots), e.n)


def test_registry_hand_trace():
    r = RegistryModel(hot_capacity=128, cold_capacity=100, block=32)   # 4 HOT blocks
    a, fresh = r.acquire(0xA, 64)
    assert fresh and placement(a) == (HOT, 0, 0, (), 64)
    b, fresh = r.acquire(0xB, 64)
    assert fresh and placement(b) == (HOT, 1, 64, (), 64)
    c, fresh = r.acquire(0xC, 32)                     # HOT full, nothing cached -> COLD
    assert fresh and placement(c) == (COLD, -1, -1, tuple(range(32)), 32)
    a2, fresh = r.acquire(0xA, 64)                    # resident: a second reference
    assert not fresh and a2 is a and a.refs == 2
    r.release(0xB)                                    # B cached
    d, fresh = r.acquire(0xD, 64)                     # evicts the cached B, takes its blocks
    assert fresh and placement(d) == (HOT, 1, 64, (), 64)
    assert 0xB not in r.entries and r.evictions == 1
    r.release(0xC)                                    # C cached (COLD)
    r.release(0xA)
    r.release(0xA)                                    # A cached (HOT), released after C
    # 96 tokens: evicting A would leave a 64-token hole -> HOT cannot hold it
    # and A stays; COLD has 68 free, evicting C gives 100 -> C goes, E in COLD
    e, fresh = r.acquire(0xE, 96)
    assert fresh and e.pool == COLD
    assert 0xA in r.entries and r.entries[0xA].pool == HOT and r.entries[0xA].offset == 0
    assert 0xC not in r.entries
    # C's slots were pushed back 0..31 (top 31), then the untouched 32..99 remain
    assert e.slots == list(range(31, -1, -1)) + list(range(32, 96))
    before = copy.deepcopy(r.__dict__)
    with pytest.raises(NoSpace):
        r.acquire(0xF, 200)                           # larger than both pools' room
    assert r.__dict__.keys() == before.keys()
    assert {k: placement(v) for k, v in r.entries.items()} == {k: placement(v) for k, v in before["entries"].items()}
    assert r.stats() == dict(resident_hot=2, resident_cold=1, referenced=2, cached=1,
                             hits=1, hot_admits=3, cold_admits=2, evictions=2)
    with pytest.raises(InvalidArg):
        r.acquire(0xD, 32)                            # resident with another length
    with pytest.raises(InvalidArg):
        r.evict(0xD)                                  # referenced
    r.evict(0xA)
    assert r.hot.free_extents == [[0, 64]]
    with pytest.raises(NotFound):
        r.release(0xA)
    r.release(0xE)
    r.reclaim_cold(100)                               # evicts E: every COLD slot free
    assert r.cold.free_count() == 100 and 0xE not in r.entries
    with pytest.raises(NoSpace):
        r.reclaim_cold(101)


def test_partition_values():
    assert partition(1000, 0.2) == (192, 808)        # 200 tokens -> 6 whole blocks
    assert partition(1000, 0.0) == (0, 1000)
    assert partition(100, 1.0) == (96, 4)
    assert partition(1 << 20, 0.2, block=1) == (209715, (1 << 20) - 209715)
    for bad in ((-1, 0.2), (10, -0.1), (10, 1.5)):
        with pytest.raises(InvalidArg):
            partition(*bad)


def _largest_hole_after_freeing(hot: HotAllocModel, ids):
    h = copy.deepcopy(hot)
    for i in ids:
        h.free(i)
    return h.largest_hole()


ops = st.lists(st.tuples(st.sampled_from(["acq", "acq", "acq", "rel", "rel", "evict", "reclaim"]),
                         st.integers(0, 9), st.integers(1, 200)), min_size=1, max_size=60)


@settings(max_examples=150, deadline=None)
@given(ops, st.integers(0, 12), st.integers(0, 400))
@example([("acq", 1, 1), ("acq", 2, 65), ("acq", 4, 1), ("acq", 0, 1), ("rel", 0, 1), ("rel", 2, 1), ("acq", 3, 33)],
         6, 0)   # two cached slabs evicted, released in the opposite order of their admission
def test_registry_invariants(seq, hot_blocks, cold_cap):
    r = RegistryModel(hot_capacity=32 * hot_blocks, cold_capacity=cold_cap, block=32)
    for op, key, n in seq:
        pre = copy.deepcopy(r)
        pre_place = {k: placement(e) for k, e in r.entries.items()}
        cached_order = [k for k in sorted(r.entries, key=lambda k: r.entries[k].tick)
                        if r.entries[k].refs == 0]
        try:
            if op == "acq":
                e, fresh = r.acquire(key, n if key not in r.entries else r.entries[key].n)
                if fresh:
                    span = -(-e.n // 32) * 32
                    cached_hot = [k for k in cached_order if pre.entries[k].pool == HOT]
                    all_hot = _largest_hole_after_freeing(pre.hot, [pre.entries[k].hot_id for k in cached_hot])
                    gone = [k for k in pre.entries if k not in r.entries]
                    if e.pool == COLD:
                        # HOT-first: even every cached HOT slab freed leaves no extent
                        assert all_hot < span
                        assert pre.cold.free_count() + sum(pre.entries[k].n for k in gone) >= e.n
                    else:
                        assert all_hot >= span
                        # the evicted ones are the first of the order (as a set: `gone`
                        # follows admission order), and no fewer would do
                        assert set(gone) == set(cached_hot[:len(gone)])
                        if gone:
                            fewer = [pre.entries[k].hot_id for k in cached_hot[:len(gone) - 1]]
                            assert _largest_hole_after_freeing(pre.hot, fewer) < span
                    for k in gone:
                        assert pre.entries[k].refs == 0
            elif op == "rel":
                r.release(key)
            elif op == "evict":
                r.evict(key)
            else:
                r.reclaim_cold(n)
        except (NoSpace, NotFound, InvalidArg):
            # a rejected call changes nothing
            assert {k: placement(e) for k, e in r.entries.items()} == pre_place
            assert r.hot.free_extents == pre.hot.free_extents and r.cold.stack == pre.cold.stack
            continue
        # no demotion: every prefix still resident kept its placement
        for k, p in pre_place.items():
            if k in r.entries:
                assert placement(r.entries[k]) == p
            else:
                assert pre.entries[k].refs == 0         # only cached prefixes leave
        # storage accounting: pools hold exactly the registry's prefixes
        hot_ids = {e.hot_id for e in r.entries.values() if e.pool == HOT}
        assert hot_ids == set(r.hot.live)
        cold_slots = [s for e in r.entries.values() if e.pool == COLD for s in e.slots]
        assert len(cold_slots) == len(set(cold_slots)) and set(cold_slots) == r.cold.allocated
        assert all(e.refs >= 0 for e in r.entries.values())
