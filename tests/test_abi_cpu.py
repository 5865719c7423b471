"""CPU tests of libgkv: the shared library loads, exports every symbol the
header declares, and its host-side logic (pool bookkeeping, dispatcher rule,
argument checks) matches the oracle's models bit for bit.  No device call is
made: these run without a GPU."""

import ctypes
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle
from oracle.alloc import ColdAllocModel, HotAllocModel
from shared_prefix_paged_contiguous_amd import binding, workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib_or_skip():
    try:
        return binding.load_library()
    except ImportError as e:
        pytest.skip(str(e))


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "gkv.h")).read()
    return sorted(set(re.findall(r"^\s*(?:[a-z_0-9]+\s*\*?\s+)+\*?\s*(gkv_[a-z_0-9]+)\s*\(", src, re.M)))


def test_header_declares_the_binding_signatures():
    names = declared_symbols()
    assert len(names) >= 18
    assert set(names) == set(binding.SIGNATURES)


def test_library_exports_every_declared_symbol():
    lib = _lib_or_skip()
    for name in declared_symbols():
        assert hasattr(lib, name), name


def _ctx(**kw):
    _lib_or_skip()
    args = dict(n_q_heads=8, n_kv_heads=2, head_dim=64, dtype="f32", hot_capacity_tokens=100,
                cold_capacity_tokens=6)
    args.update(kw)
    return binding.Context(**args)


def test_create_rejects_bad_configs():
    _lib_or_skip()
    for kw in [dict(n_q_heads=10, n_kv_heads=4), dict(head_dim=96), dict(n_q_heads=34, n_kv_heads=2),
               dict(n_q_heads=264, n_kv_heads=33), dict(hot_capacity_tokens=-1), dict(cold_capacity_tokens=2 ** 31),
               dict(dtype="f32", force_backend=binding.BACKEND_DENSE), dict(dtype="f32", partial_dtype="bf16"),
               dict(partial_dtype="f16")]:
        with pytest.raises(binding.GkvError):
            _ctx(**kw)


BLOCK = 32   # the library's HOT slab granularity (its kernels' K/V block)


def test_hot_pool_matches_hand_trace_and_model():
    # the model's hand trace scaled to whole blocks: same decisions, offsets x 32
    c = _ctx(hot_capacity_tokens=100 * BLOCK)
    m = HotAllocModel(100 * BLOCK, block=BLOCK)
    seq = [("a", 30 * BLOCK), ("a", 20 * BLOCK), ("a", 40 * BLOCK), ("f", 1), ("a", 25 * BLOCK),
           ("a", 15 * BLOCK - 7), ("a", 10 * BLOCK), ("f", 0), ("f", 2), ("a", 31 * BLOCK), ("f", 1), ("f", 1),
           ("f", 3)]
    for op, x in seq:
        if op == "a":
            try:
                want = m.alloc(x)
            except oracle.NoSpace:
                with pytest.raises(binding.NoSpace):
                    c.hot_pool_alloc(x)
                continue
            assert c.hot_pool_alloc(x) == want
            assert c.hot_prefix_info(want[0]) == (want[1], x)
        else:
            try:
                m.free(x)
            except oracle.NotFound:
                with pytest.raises(binding.NotFound):
                    c.hot_pool_free(x)
                continue
            c.hot_pool_free(x)
        s = c.pool_stats()
        assert s["hot_free_tokens"] == m.free_tokens()
        assert s["hot_largest_hole"] == m.largest_hole()
        assert s["hot_free_extents"] == len(m.free_extents)
        assert s["hot_live_prefixes"] == len(m.live)


@settings(max_examples=150, deadline=None)
@given(st.lists(st.tuples(st.sampled_from(["a", "f"]), st.integers(1, 200)), max_size=80))
def test_hot_pool_bit_exact_vs_model(seq):
    c = _ctx(hot_capacity_tokens=160 * 4 + 17)
    m = HotAllocModel(160 * 4 + 17, block=BLOCK)
    for op, x in seq:
        if op == "a":
            try:
                want = m.alloc(x)
            except oracle.NoSpace:
                with pytest.raises(binding.NoSpace):
                    c.hot_pool_alloc(x)
                continue
            assert c.hot_pool_alloc(x) == want
        else:
            pid = sorted(m.live)[x % len(m.live)] if m.live else x
            if pid in m.live:
                m.free(pid)
                c.hot_pool_free(pid)
            else:
                with pytest.raises(binding.NotFound):
                    c.hot_pool_free(pid)
    s = c.pool_stats()
    assert (s["hot_free_tokens"], s["hot_largest_hole"]) == (m.free_tokens(), m.largest_hole())


def test_cold_pool_matches_hand_trace():
    c = _ctx(cold_capacity_tokens=6)
    assert c.cold_pool_alloc(3).tolist() == [0, 1, 2]
    c.cold_pool_free([2, 0])
    assert c.cold_pool_alloc(2).tolist() == [0, 2]
    assert c.cold_pool_alloc(2).tolist() == [3, 4]
    with pytest.raises(binding.NoSpace):
        c.cold_pool_alloc(2)
    for bad in ([1, 5], [1, 1], [7], [-1]):
        with pytest.raises(binding.NotFound):
            c.cold_pool_free(bad)
    assert c.pool_stats()["cold_free_slots"] == 1
    c.cold_pool_free([4, 1, 3])
    assert c.cold_pool_alloc(4).tolist() == [3, 1, 4, 5]
    assert c.cold_pool_alloc(0).tolist() == []


@settings(max_examples=150, deadline=None)
@given(st.lists(st.tuples(st.sampled_from(["a", "f"]), st.integers(0, 9)), max_size=80))
def test_cold_pool_bit_exact_vs_model(seq):
    c = _ctx(cold_capacity_tokens=30)
    m = ColdAllocModel(30)
    live = []
    for op, x in seq:
        if op == "a":
            try:
                want = m.alloc(x)
            except oracle.NoSpace:
                with pytest.raises(binding.NoSpace):
                    c.cold_pool_alloc(x)
                continue
            assert c.cold_pool_alloc(x).tolist() == want
            live += want
        else:
            k = min(x, len(live))
            out, live = live[-k:][::-1] if k else [], live[:-k] if k else live
            m.free(out)
            c.cold_pool_free(out)
    assert c.pool_stats()["cold_free_slots"] == m.free_count()


@pytest.mark.parametrize("name", ["tiny", "hetero8"])
def test_workload_placement_bit_exact_vs_models(name):
    """The slot maps and HOT offsets the C allocators give for a workload's
    placement equal the oracle models' (the GPU tests read these slots)."""
    _lib_or_skip()
    w = workloads.make(name)
    s = w.spec
    c = binding.Context(s.n_q, s.n_kv, s.head_dim, s.dtype, s.hot_capacity, s.cold_capacity)

    def c_hot(n):
        try:
            return c.hot_pool_alloc(n)
        except binding.NoSpace:
            return None

    hm, cm = HotAllocModel(s.hot_capacity, block=BLOCK), ColdAllocModel(s.cold_capacity)

    def m_hot(n):
        try:
            return hm.alloc(n)
        except oracle.NoSpace:
            return None

    a = workloads.place(w, c_hot, c.hot_pool_free, c.cold_pool_alloc, c.cold_pool_free)
    b = workloads.place(w, m_hot, hm.free, cm.alloc, cm.free)
    assert a["prefix_id"] == b["prefix_id"] and a["prefix_offset"] == b["prefix_offset"]
    for x, y in zip(a["req_slots"], b["req_slots"]):
        assert np.array_equal(x, np.asarray(y, dtype=np.int32))
    if name == "hetero8":
        # churn left holes: some slab landed below the running sum of lengths
        assert min(o for o in a["prefix_offset"] if o >= 0) < sum(w.hot_churn[:1])


def test_step_status_and_spin_limit_host_checks():
    c = _ctx()
    with pytest.raises(binding.GkvError, match="no workspace"):
        c.step_status(stream=0)
    c.bind_workspace(256, 1 << 20)
    assert c.step_status(stream=0) == 0        # nothing has run on the workspace yet: no device call
    c.set_join_spin_limit(0)
    c.set_join_spin_limit(-1)
    with pytest.raises(binding.GkvError):
        c.set_join_spin_limit(-2)


def test_dispatch_rule_matches_model_and_pages():
    c = _ctx(n_q_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16", m_sat=1024)
    for bsz in [1, 8, 32, 128, 255, 256, 257, 512]:
        assert c.select_backend(bsz) == oracle.choose_backend(bsz, 32, 8, 1024)
    c.set_dispatch(binding.BACKEND_CASCADE)
    assert c.select_backend(512) == binding.BACKEND_CASCADE
    c.set_dispatch(binding.BACKEND_AUTO, 64)
    assert c.select_backend(16) == binding.BACKEND_DENSE
    assert c.select_backend(15) == binding.BACKEND_CASCADE
    f = _ctx(m_sat=1)   # fp32: the dense kernel is bf16 only, AUTO stays on cascade
    assert f.select_backend(64) == binding.BACKEND_CASCADE
    with pytest.raises(binding.GkvError):
        f.set_dispatch(binding.BACKEND_DENSE)
    assert binding.default_m_sat() > 0


def test_attn_decode_rejects_bad_steps_before_any_device_work():
    c = _ctx()
    pid, _ = c.hot_pool_alloc(10)
    assert c.hot_pool_bytes() == 2 * (100 // BLOCK) * BLOCK * 64 * 4
    # nothing bound yet
    with pytest.raises(binding.GkvError, match="not bound"):
        c.attn_decode(0, 16, [pid], [0, 0], 0, 0, 16, 16, stream=0)
    c.bind_layer(0, 16, 16, 16, 16)   # fake aligned addresses: only host checks run below
    with pytest.raises(binding.GkvError, match="workspace"):
        c.attn_decode(0, 16, [pid], [0, 0], 0, 0, 16, 16, stream=0)
    c.bind_workspace(256, 1 << 20)
    cases = [([-1], [0, 0], "neither"), ([pid + 7], [0, 1], "not live"), ([pid, pid], [0, 2, 1], "decreases"),
             ([-2], [0, 1], "< -1")]
    for ids, indptr, msg in cases:
        with pytest.raises(binding.GkvError, match=msg):
            c.attn_decode(0, 16, ids, indptr, 16, 16, 16, 16, batch=len(ids), stream=0)
    with pytest.raises(binding.GkvError, match="too small"):
        c2 = _ctx()
        pid2, _ = c2.hot_pool_alloc(50)          # prefix partials need workspace
        c2.bind_layer(0, 16, 16, 16, 16)
        c2.bind_workspace(256, 256)
        c2.attn_decode(0, 16, [pid2], [0, 3], 16, 16, 16, 16, stream=0)


def test_decode_step_rejects_bad_steps_before_any_device_work():
    c = _ctx()
    pid, _ = c.hot_pool_alloc(10)
    c.bind_layer(0, 16, 16, 16, 16)   # fake aligned addresses: only host checks run below
    c.bind_workspace(256, 1 << 20)
    # layer, q, k_new, v_new, new slots, ids, indptr, indices, out, lse
    with pytest.raises(binding.GkvError, match="null pointer"):
        c.decode_step(0, 16, 0, 16, 16, [pid], [0, 1], 16, 16, 16, stream=0)
    with pytest.raises(binding.GkvError, match="null pointer"):
        c.decode_step(0, 16, 16, 16, 0, [pid], [0, 1], 16, 16, 16, stream=0)
    with pytest.raises(binding.GkvError, match="16-byte aligned"):
        c.decode_step(0, 16, 24, 16, 16, [pid], [0, 1], 16, 16, 16, stream=0)
    # every request's new token is the last entry of its table: none may be empty
    with pytest.raises(binding.GkvError, match="empty slot table"):
        c.decode_step(0, 16, 16, 16, 16, [pid, pid], [0, 1, 1], 16, 16, 16, batch=2, stream=0)


def test_workspace_bound_covers_plans():
    c = _ctx(n_q_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16", hot_capacity_tokens=16384,
             cold_capacity_tokens=65536)
    assert c.workspace_size(64, 65536) > c.workspace_size(4, 100) > 0


def test_step_rejects_more_than_64_hot_classes_before_any_device_work():
    c = _ctx(hot_capacity_tokens=65 * BLOCK)
    ids = [c.hot_pool_alloc(BLOCK)[0] for _ in range(65)]
    c.bind_layer(0, 16, 16, 16, 16)   # fake aligned addresses: only host checks run below
    c.bind_workspace(256, 1 << 24)
    indptr = list(range(66))
    with pytest.raises(binding.GkvError, match="more than 64 distinct HOT prefixes"):
        c.attn_decode(0, 16, ids, indptr, 16, 16, 16, 16, batch=65, stream=0)


# ------------------------------------------------------------------ planner
# gkv_plan_step runs the step's planner alone (host only).  Without a GPU it
# plans for gfx950's 256 compute units in 8 XCDs: 512 workgroup slots (two per
# CU), grid ranges padded to 32 workgroups.
def _llama_ctx(hot=16384, cold=1 << 20):
    return _ctx(n_q_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16", hot_capacity_tokens=hot,
                cold_capacity_tokens=cold)


def test_plan_of_the_bench_step():
    """Llama-3.1-8B shape, one 16K HOT prefix, 64 requests of 128..1024 suffix
    tokens: cascade (M_eff 256 < 4096); 16K tokens x 8 KV heads x 2 M-tiles
    of 32 requests = 262144 units over 256 target workgroups gives 1024-token
    splits, 16 per (KV head, M-tile): 256 prefix workgroups.  64 parts x 8 KV
    heads = 512 workgroups overflow the 256 slots left, 32 folded pairs x 8 =
    256 fit: folded.  Every slot table is one part, so the suffix workgroups
    join their requests themselves: no join workgroups."""
    c = _llama_ctx()
    pid, _ = c.hot_pool_alloc(16384)
    lens = np.random.default_rng(5).integers(128, 1025, size=64)
    indptr = np.concatenate([[0], np.cumsum(lens)])
    p = c.plan_step([pid] * 64, indptr)
    assert p["backend"] == binding.BACKEND_CASCADE and p["m_eff"] == 256 and p["n_classes"] == 1
    assert (p["n_prefix_blocks"], p["n_suffix_blocks"], p["n_join_blocks"]) == (256, 256, 0)
    assert p["folded_parts"] == 1 and p["n_suffix_parts"] == 64 and p["n_short_requests"] == 0
    assert p["joins_partials"] == 1 and p["workspace_bytes"] > 0
    # the grid does not depend on the order the requests come in
    q = c.plan_step([pid] * 64, np.concatenate([[0], np.cumsum(lens[::-1])]))
    assert {k: v for k, v in q.items() if not k.startswith("host")} == {k: v for k, v in p.items() if not k.startswith("host")}


@pytest.mark.parametrize("batch,joins", [(256, 256), (512, 512), (513, 257), (1024, 512)])
def test_plan_groups_short_requests_beyond_the_slots(batch, joins):
    """One-token requests on a HOT prefix are short requests: no suffix part,
    one join workgroup each, or k = ceil(n / 512) consecutive ones per join
    workgroup when there are more than the 512 slots."""
    c = _llama_ctx(hot=2048)
    pid, _ = c.hot_pool_alloc(2048)
    p = c.plan_step([pid] * batch, np.arange(batch + 1))
    assert p["n_short_requests"] == batch and p["n_suffix_parts"] == 0 and p["n_suffix_blocks"] == 0
    assert p["n_join_blocks"] == joins


def test_plan_dense_split_rule():
    """Forced dense, 1024 one-token requests on a 16K prefix: 32 M-tiles x 8 KV
    heads = 256 (M-tile, head) pairs.  The rule's time, with k = ceil(blocks /
    256 CUs) workgroups per CU of one split each (two at a time 1.25x as fast,
    plus eight blocks' fixed cost): 1 split 16384 + 256 = 16640; 2 splits
    (k = 2) 2 x 8448 / 1.25 = 13517; 3 (k = 3) 2 x 5718 / 1.25 + 5718 = 14867;
    4 (k = 4) 4 x 4352 / 1.25 = 13926: two splits, 512 prefix workgroups."""
    c = _llama_ctx()
    pid, _ = c.hot_pool_alloc(16384)
    c.set_dispatch(binding.BACKEND_DENSE)
    p = c.plan_step([pid] * 1024, np.arange(1025))
    assert p["backend"] == binding.BACKEND_DENSE and p["m_eff"] == 4096
    assert p["n_prefix_blocks"] == 512 and p["n_join_blocks"] == 512 and p["n_suffix_blocks"] == 0


def test_plan_step_checks_like_the_step():
    c = _llama_ctx()
    pid, _ = c.hot_pool_alloc(100)
    with pytest.raises(binding.GkvError, match="not live"):
        c.plan_step([pid + 3], [0, 1])
    with pytest.raises(binding.GkvError, match="decreases"):
        c.plan_step([pid, pid], [0, 2, 1])
    with pytest.raises(binding.GkvError, match="exceeds the per-call limit"):
        c.plan_step([pid] * 1025, np.arange(1026))
    with pytest.raises(binding.GkvError, match="batch"):
        c.plan_step([], [0], batch=0)
