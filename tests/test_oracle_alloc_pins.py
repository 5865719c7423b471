"""Pins for the oracle's allocator, append and dispatch models.

Hand-derived traces (worked by hand from the reading of the pages, written
here as literals), invariants that must hold for any operation sequence, and
the routing the pages state for the Llama-3.1-8B / TP=1 grid
(tests/golden/dispatch_llama8b_tp1_a100.txt).
"""

import os

import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

from oracle.alloc import ColdAllocModel, HotAllocModel, NoSpace, NotFound
from oracle.append import append_model, slot_position
from oracle.dispatch import BACKEND_CASCADE, BACKEND_DENSE, choose_backend, m_eff

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ HOT pool
def test_hot_hand_trace():
    h = HotAllocModel(100)
    assert h.alloc(30) == (0, 0)
    assert h.alloc(20) == (1, 30)
    assert h.alloc(40) == (2, 50)         # no frees so far: offsets are running sums
    h.free(1)                             # holes [30,50) and [90,100): 30 tokens free
    with pytest.raises(NoSpace):          # 25 <= 30 free, but no single hole of 25 (B.10)
        h.alloc(25)
    assert h.free_extents == [[30, 20], [90, 10]]   # failed alloc changed nothing
    assert h.alloc(15) == (1, 30)         # smallest unused id; lowest hole that fits
    assert h.alloc(10) == (3, 90)         # [45,50) too small, [90,100) fits
    h.free(0)                             # [0,30) free
    h.free(2)                             # [50,90) joins [45,50): [45,90)
    assert h.free_extents == [[0, 30], [45, 45]]
    assert h.alloc(31) == (0, 45)         # first hole too small -> second
    h.free(1)                             # [30,45) joins [0,30): [0,45)
    assert h.free_extents == [[0, 45], [76, 14]]
    with pytest.raises(NotFound):
        h.free(1)
    h.free(3)                             # [90,100) joins [76,90): [76,100)
    assert h.free_extents == [[0, 45], [76, 24]]
    assert h.largest_hole() == 45 and h.free_tokens() == 69


def test_hot_block_granularity_hand_trace():
    # blocks of 32 tokens: a 100-token pool holds 3 blocks (96 tokens)
    h = HotAllocModel(100, block=32)
    assert h.free_extents == [[0, 96]]
    assert h.alloc(33) == (0, 0)          # 2 blocks
    assert h.alloc(1) == (1, 64)          # 1 block, block-aligned
    with pytest.raises(NoSpace):
        h.alloc(1)                        # 96 of 96 tokens taken
    h.free(0)
    assert h.free_extents == [[0, 64]]
    assert h.alloc(64) == (0, 0)          # exactly the freed 2 blocks
    assert h.live == {0: (0, 64), 1: (64, 1)}
    h.free(1)
    h.free(0)
    assert h.free_extents == [[0, 96]] and h.largest_hole() == 96


def test_hot_exact_fit_and_full_pool():
    h = HotAllocModel(10)
    assert h.alloc(10) == (0, 0)
    assert h.free_extents == []
    with pytest.raises(NoSpace):
        h.alloc(1)
    h.free(0)
    assert h.free_extents == [[0, 10]]
    with pytest.raises(ValueError):
        h.alloc(0)


ops = st.lists(st.tuples(st.sampled_from(["a", "f"]), st.integers(1, 40)), max_size=60)


@settings(max_examples=200, deadline=None)
@given(ops, st.sampled_from([1, 4, 32]))
def test_hot_invariants(seq, block):
    cap = 128
    h = HotAllocModel(cap, block=block)
    no_free_yet, running = True, 0
    for kind, n in seq:
        if kind == "a":
            before = ([e[:] for e in h.free_extents], dict(h.live))
            fits = [e[:] for e in h.free_extents]
            try:
                pid, off = h.alloc(n)
            except NoSpace:
                assert h.largest_hole() < -(-n // block) * block  # NOSPACE iff no hole fits
                assert (h.free_extents, h.live) == before        # and nothing changed
                continue
            span = -(-n // block) * block
            assert off % block == 0
            assert [e for e in fits if e[1] >= span][0][0] == off    # lowest-address fitting hole
            assert pid == min(set(range(len(h.live) + 1)) - (set(h.live) - {pid}))
            if no_free_yet:
                assert off == running
                running += span
        else:
            if not h.live:
                continue
            pid = sorted(h.live)[n % len(h.live)]
            h.free(pid)
            no_free_yet = False
        # live slabs and free extents tile [0, cap) exactly, without overlap
        spans = sorted([[o, -(-ln // block) * block] for o, ln in h.live.values()] +
                       [e[:] for e in h.free_extents])
        pos = 0
        for o, ln in spans:
            assert o == pos and ln > 0
            pos += ln
        assert pos == cap
        # free extents are maximal (coalesced)
        for a, b in zip(h.free_extents, h.free_extents[1:]):
            assert a[0] + a[1] < b[0]


# ----------------------------------------------------------------- COLD pool
def test_cold_hand_trace():
    c = ColdAllocModel(6)
    assert c.alloc(3) == [0, 1, 2]        # fresh pool pops ascending
    c.free([2, 0])                        # push 2, then 0: 0 is on top
    assert c.alloc(2) == [0, 2]
    assert c.alloc(2) == [3, 4]
    with pytest.raises(NoSpace):          # 1 free, 2 asked: all or nothing
        c.alloc(2)
    assert c.free_count() == 1
    with pytest.raises(NotFound):         # 5 was never handed out
        c.free([1, 5])
    with pytest.raises(NotFound):         # duplicate inside one call
        c.free([1, 1])
    assert c.free_count() == 1            # failed frees changed nothing
    c.free([4, 1, 3])
    assert c.alloc(4) == [3, 1, 4, 5]
    assert c.alloc(0) == []


@settings(max_examples=200, deadline=None)
@given(st.lists(st.tuples(st.sampled_from(["a", "f"]), st.integers(0, 9)), max_size=60))
def test_cold_invariants(seq):
    cap = 24
    c = ColdAllocModel(cap)
    live = []
    for kind, n in seq:
        if kind == "a":
            try:
                got = c.alloc(n)
            except NoSpace:
                assert n > c.free_count()
                continue
            assert len(got) == n and not (set(got) & set(live))
            live += got
        else:
            k = min(n, len(live))
            out, live = live[:k], live[k:]
            c.free(out)
            if out:
                assert c.stack[-len(out):] == out      # pushed in the order given
        assert c.free_count() + len(live) == cap
        assert sorted(c.stack + live) == list(range(cap))


def test_cold_lifo_after_permuted_free():
    # the workload placement: take everything, free in a permuted order, then
    # allocation returns the permutation reversed
    c = ColdAllocModel(8)
    c.alloc(8)
    perm = [5, 2, 7, 0, 3, 6, 1, 4]
    c.free(perm)
    assert c.alloc(3) == [4, 1, 6]
    assert c.alloc(5) == [3, 0, 7, 2, 5]


# -------------------------------------------------------------------- append
def test_append_scatter():
    pool = np.arange(5 * 2 * 3, dtype=np.float32).reshape(5, 2, 3)
    rows = -np.arange(2 * 2 * 3, dtype=np.float32).reshape(2, 2, 3) - 1
    out = append_model(pool, [3, 1], rows)
    # n_kv = 2: odd slots hold their two heads swapped
    assert out[3].tolist() == [[-4.0, -5.0, -6.0], [-1.0, -2.0, -3.0]]
    assert out[1].tolist() == [[-10.0, -11.0, -12.0], [-7.0, -8.0, -9.0]]
    for r in (0, 2, 4):
        assert out[r].tobytes() == pool[r].tobytes()
    assert pool[3, 0, 0] == 18.0          # input untouched
    out = append_model(pool, [2, 2], rows)  # repeated slot: last write wins; even slot: in order
    assert np.array_equal(out[2], rows[1])


# in-slot position of head g, tabulated by hand from the layout's statement
# (head g at g XOR (slot mod P), P the largest power of two dividing n_kv)
SLOT_POSITIONS = {
    # (n_kv, slot): positions of heads 0, 1, ...
    (1, 7): [0],
    (3, 5): [0, 1, 2],                     # odd n_kv: P = 1
    (2, 4): [0, 1],
    (2, 9): [1, 0],
    (4, 6): [2, 3, 0, 1],                  # 6 mod 4 = 2
    (4, 8): [0, 1, 2, 3],
    (6, 3): [1, 0, 3, 2, 5, 4],            # P = 2
    (8, 13): [5, 4, 7, 6, 1, 0, 3, 2],     # 13 mod 8 = 5
    (12, 7): [3, 2, 1, 0, 7, 6, 5, 4, 11, 10, 9, 8],   # P = 4, 7 mod 4 = 3
    (16, 21): [5, 4, 7, 6, 1, 0, 3, 2, 13, 12, 15, 14, 9, 8, 11, 10],
    # slots where a mask of n_kv - 1 would differ from P - 1
    (6, 4): [0, 1, 2, 3, 4, 5],
    (12, 8): [0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11],
    (10, 3): [1, 0, 3, 2, 5, 4, 7, 6, 9, 8],
}


@pytest.mark.parametrize("key", sorted(SLOT_POSITIONS))
def test_slot_positions_tabulated(key):
    n_kv, slot = key
    assert [slot_position(g, slot, n_kv) for g in range(n_kv)] == SLOT_POSITIONS[key]


def test_append_places_each_head_once():
    """Every slot holds each head's row exactly once, at the tabulated
    positions (4 KV heads), and reading back through the positions restores
    the rows."""
    rng = np.random.default_rng(3)
    n_kv, d, cap = 4, 5, 16
    pool = rng.standard_normal((cap, n_kv, d))
    slots = [6, 0, 13, 8]
    rows = rng.standard_normal((len(slots), n_kv, d))
    out = append_model(pool, slots, rows)
    assert out[6, 2].tolist() == rows[0, 0].tolist() and out[6, 0].tolist() == rows[0, 2].tolist()
    for i, s in enumerate(slots):
        got = sorted(map(tuple, out[s].tolist()))
        assert got == sorted(map(tuple, rows[i].tolist()))
        for g in range(n_kv):
            assert np.array_equal(out[s, slot_position(g, s, n_kv)], rows[i, g])
    untouched = [r for r in range(cap) if r not in slots]
    assert np.array_equal(out[untouched], pool[untouched])


# ------------------------------------------------------------------ dispatch
def test_dispatch_golden_from_pages():
    with open(os.path.join(GOLDEN, "dispatch_llama8b_tp1_a100.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 4
    for b, nq, nkv, msat, me, backend in rows:
        assert m_eff(int(b), int(nq), int(nkv)) == int(me)
        want = BACKEND_DENSE if backend == "dense" else BACKEND_CASCADE
        assert choose_backend(int(b), int(nq), int(nkv), int(msat)) == want


def test_dispatch_tie_and_neighbours():
    assert choose_backend(256, 32, 8, 1024) == BACKEND_DENSE      # M_eff == M_sat
    assert choose_backend(255, 32, 8, 1024) == BACKEND_CASCADE
    assert choose_backend(205, 20, 4, 1024) == BACKEND_DENSE       # 1025
    with pytest.raises(ValueError):
        m_eff(4, 10, 4)
