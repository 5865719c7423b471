"""The library's prefix registry (gkv_prefix_* / gkv_partition_capacity) against
the oracle's RegistryModel: every call's status, placement, COLD slots and
the counters are compared bit-exactly on seeded and generated operation
sequences.  Host-only calls: no GPU needed.
"""

import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

from oracle.alloc import NoSpace as ModelNoSpace
from oracle.alloc import NotFound as ModelNotFound
from oracle.registry import COLD, HOT, InvalidArg, RegistryModel, partition
from shared_prefix_paged_contiguous_amd import binding


def make_ctx(hot_cap, cold_cap):
    return binding.Context(8, 2, 64, "f32", hot_cap, cold_cap)


def model_ref(e, fresh):
    return dict(pool=HOT if e.pool == HOT else COLD, prefix_id=e.hot_id if e.pool == HOT else -1,
                hot_offset=e.offset if e.pool == HOT else -1, n_tokens=e.n, fresh=int(fresh), refs=e.refs)


def outcome(fn):
    """('ok', value) or the error class name, for both sides alike."""
    try:
        return "ok", fn()
    except (binding.NoSpace, ModelNoSpace):
        return "nospace", None
    except (binding.NotFound, ModelNotFound):
        return "notfound", None
    except (binding.GkvError, InvalidArg):
        return "invalid", None


def run_both(ctx, model, op, key, n):
    if op == "acq":
        lib = outcome(lambda: ctx.prefix_acquire(key, n))
        mod = outcome(lambda: model_ref(*model.acquire(key, n)))
        assert lib == mod, (op, key, n)
        if lib[0] == "ok" and lib[1]["pool"] == binding.POOL_COLD:
            assert list(ctx.prefix_cold_slots(key, n)) == model.entries[key].slots
    elif op == "rel":
        assert outcome(lambda: ctx.prefix_release(key)) == outcome(lambda: model.release(key))
    elif op == "evict":
        assert outcome(lambda: ctx.prefix_evict(key)) == outcome(lambda: model.evict(key))
    else:
        assert outcome(lambda: ctx.prefix_reclaim_cold(n)) == outcome(lambda: model.reclaim_cold(n))
    assert ctx.registry_stats() == model.stats()
    ps = ctx.pool_stats()
    assert ps["hot_free_tokens"] == model.hot.free_tokens()
    assert ps["hot_largest_hole"] == model.hot.largest_hole()
    assert ps["cold_free_slots"] == model.cold.free_count()


def test_registry_hand_trace_through_the_abi():
    ctx, model = make_ctx(128, 100), RegistryModel(128, 100, block=32)
    trace = [("acq", 0xA, 64), ("acq", 0xB, 64), ("acq", 0xC, 32), ("acq", 0xA, 64), ("rel", 0xB, 0),
             ("acq", 0xD, 64), ("rel", 0xC, 0), ("rel", 0xA, 0), ("rel", 0xA, 0), ("acq", 0xE, 96),
             ("acq", 0xF, 200), ("acq", 0xD, 32), ("evict", 0xD, 0), ("evict", 0xA, 0), ("rel", 0xA, 0),
             ("rel", 0xE, 0), ("reclaim", 0, 100), ("reclaim", 0, 101)]
    for op, key, n in trace:
        run_both(ctx, model, op, key, n)
    e = ctx.prefix_lookup(0xD)
    assert (e["pool"], e["prefix_id"], e["hot_offset"], e["refs"]) == (binding.POOL_HOT, 1, 64, 1)


@pytest.mark.parametrize("seed", range(6))
def test_registry_bit_exact_vs_model_seeded(seed):
    rng = np.random.default_rng(seed)
    hot_cap, cold_cap = int(rng.integers(0, 16)) * 32 + int(rng.integers(0, 32)), int(rng.integers(0, 600))
    ctx, model = make_ctx(hot_cap, cold_cap), RegistryModel(hot_cap, cold_cap, block=32)
    for _ in range(400):
        op = rng.choice(["acq", "acq", "acq", "rel", "rel", "evict", "reclaim"])
        key = int(rng.integers(0, 24)) * 0x9E3779B97F4A7C15 % (1 << 64)
        n = model.entries[key].n if (key in model.entries and rng.random() < 0.9) else int(rng.integers(1, 260))
        run_both(ctx, model, op, key, n)


@settings(max_examples=60, deadline=None)
@given(st.lists(st.tuples(st.sampled_from(["acq", "acq", "rel", "evict", "reclaim"]), st.integers(0, 7),
                          st.integers(0, 150)), max_size=50),
       st.integers(0, 8), st.integers(0, 300))
def test_registry_bit_exact_vs_model_generated(seq, hot_blocks, cold_cap):
    ctx, model = make_ctx(hot_blocks * 32, cold_cap), RegistryModel(hot_blocks * 32, cold_cap, block=32)
    for op, key, n in seq:
        run_both(ctx, model, op, key, max(n, 1) if op == "acq" else n)


def test_registry_owned_storage_is_refused_by_the_raw_pool_calls():
    ctx = make_ctx(64, 64)
    h = ctx.prefix_acquire(1, 64)                      # fills HOT
    c = ctx.prefix_acquire(2, 10)                      # COLD
    with pytest.raises(binding.GkvError) as ei:
        ctx.hot_pool_free(h["prefix_id"])
    assert ei.value.code == binding.GKV_ERR_INVALID
    slots = ctx.prefix_cold_slots(2, 10)
    free_before = ctx.pool_stats()["cold_free_slots"]
    with pytest.raises(binding.GkvError):
        ctx.cold_pool_free(slots[:3])
    assert ctx.pool_stats()["cold_free_slots"] == free_before
    raw = ctx.cold_pool_alloc(4)                       # raw slots stay freeable
    ctx.cold_pool_free(raw)
    assert c["fresh"] == 1 and c["pool"] == binding.POOL_COLD
    with pytest.raises(binding.GkvError):
        ctx.prefix_cold_slots(1, 64)                   # a HOT prefix has no slots


@pytest.mark.parametrize("total,f_p", [(0, 0.2), (1000, 0.2), (1000, 0.0), (100, 1.0), (1 << 21, 0.2),
                                       (1_850_000, 0.2), (12345, 0.37)])
def test_partition_matches_model(total, f_p):
    assert binding.partition_capacity(total, f_p) == partition(total, f_p, block=32)


@pytest.mark.parametrize("total,f_p", [(-1, 0.2), (10, -0.01), (10, 1.01), (10, float("nan")), (1 << 40, 0.0)])
def test_partition_rejects_bad_arguments(total, f_p):
    with pytest.raises(binding.GkvError):
        binding.partition_capacity(total, f_p)


def test_registry_placement_of_a_workload_bit_exact_vs_model():
    """place_through_registry (the library) and the same steps replayed on the
    model: identical prefix placements (HOT ids/offsets, COLD slots) and
    suffix slots, with some prefixes pushed to COLD."""
    import dataclasses

    from shared_prefix_paged_contiguous_amd import workloads
    from shared_prefix_paged_contiguous_amd.harness import place_through_registry, prefix_key

    s = workloads.Spec("reg", n_q=8, n_kv=2, head_dim=64, dtype="f32", batch=0, prefix_len=0, suffix_lo=1,
                       suffix_hi=60, hot_capacity=1024, cold_capacity=6000, n_prefixes=7, prefix_len_lo=100,
                       prefix_len_hi=500, class_lo=1, class_hi=3)
    w = workloads.make(s)
    ctx = make_ctx(s.hot_capacity, s.cold_capacity)
    got = place_through_registry(w, ctx)
    m = RegistryModel(s.hot_capacity, s.cold_capacity, block=32)
    m.cold.alloc(s.cold_capacity)
    m.cold.free([int(x) for x in w.cold_perm])
    for b in range(w.batch):
        p = int(w.request_prefix[b])
        e, fresh = m.acquire(prefix_key(p), w.prefix_lens[p])
        if fresh and e.pool == HOT:
            assert (got["prefix_id"][p], got["prefix_offset"][p]) == (e.hot_id, e.offset)
        elif fresh:
            assert list(got["prefix_slots"][p]) == e.slots and got["prefix_id"][p] == -1
    for b in range(w.batch):
        assert list(got["req_slots"][b]) == m.cold.alloc(int(w.suffix_lens[b]))
    st = ctx.registry_stats()
    assert st == m.stats() and st["cold_admits"] >= 1 and st["hot_admits"] >= 1
    assert dataclasses.asdict(s)["n_prefixes"] == st["resident_hot"] + st["resident_cold"]
