"""GPU parity of libgkv against the float64 oracle, through the C ABI.

Every case draws a seeded synthetic workload, places it with the library's
own allocators, appends the suffix tokens with gkv_cold_append, runs
gkv_attn_decode on the GPU and compares out / lse with the oracle's softmax
attention over the logical context (prefix || suffix) element by element.
"""

import dataclasses

import numpy as np
import pytest
import torch

from oracle.append import append_model
from shared_prefix_paged_contiguous_amd import binding, workloads
from shared_prefix_paged_contiguous_amd.harness import DecodeState
from tests.gpu_helpers import check, f64, oracle_ref

pytestmark = pytest.mark.gpu

CASCADE, DENSE, AUTO = binding.BACKEND_CASCADE, binding.BACKEND_DENSE, binding.BACKEND_AUTO
FP32_TOL = dict(atol=1e-4, rtol=1e-4, norm_rel=1e-4, lse_abs=1e-4, max_abs=1e-4)


def run(w, force=AUTO, **kw):
    st = DecodeState(w, force_backend=force, **kw)
    out, lse = st.new_outputs()
    backend = st.run(out, lse)
    torch.cuda.synchronize()
    return st, out, lse, backend


def spec(**kw):
    base = dict(name="case", n_q=32, n_kv=8, head_dim=128, dtype="bf16", batch=8, prefix_len=1000,
                suffix_lo=0, suffix_hi=0, hot_capacity=1200, cold_capacity=8192)
    base.update(kw)
    return workloads.Spec(**base)


# --------------------------------------------------------------- cold append
@pytest.mark.parametrize("n_kv,d", [(2, 64), (3, 64), (8, 128), (12, 64)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_cold_append_bit_exact(dtype, n_kv, d):
    """Whole pools after gkv_cold_append against the oracle's model of the
    COLD slot layout (heads permuted within a slot by its index)."""
    torch.manual_seed(0)
    cap = 300
    ctx = binding.Context(2 * n_kv, n_kv, d, dtype, 0, cap)
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    k_cold = torch.randn(cap, n_kv, d).to(td).cuda()
    v_cold = torch.randn(cap, n_kv, d).to(td).cuda()
    before_k, before_v = k_cold.cpu().clone(), v_cold.cpu().clone()
    ctx.bind_layer(0, None, None, k_cold, v_cold)
    slots = ctx.cold_pool_alloc(40)[np.random.default_rng(1).permutation(40)]
    slots_ext = np.concatenate([slots, [cap, -5]]).astype(np.int32)   # out of range: skipped
    k_new = torch.randn(len(slots_ext), n_kv, d).to(td)
    v_new = torch.randn(len(slots_ext), n_kv, d).to(td)
    ctx.cold_append(0, k_new.cuda(), v_new.cuda(), torch.from_numpy(slots_ext).cuda())
    torch.cuda.synchronize()
    want_k = append_model(before_k.view(torch.int16 if dtype == "bf16" else torch.int32).numpy(), slots,
                          k_new[:40].view(torch.int16 if dtype == "bf16" else torch.int32).numpy())
    want_v = append_model(before_v.view(torch.int16 if dtype == "bf16" else torch.int32).numpy(), slots,
                          v_new[:40].view(torch.int16 if dtype == "bf16" else torch.int32).numpy())
    got_k = k_cold.cpu().view(torch.int16 if dtype == "bf16" else torch.int32).numpy()
    got_v = v_cold.cpu().view(torch.int16 if dtype == "bf16" else torch.int32).numpy()
    assert got_k.tobytes() == want_k.tobytes()
    assert got_v.tobytes() == want_v.tobytes()


# --------------------------------------------------------- HOT block layout
def hot_layout_model(rows_k, rows_v, tok0, n_kv, d, blocks, bf16):
    """Expected HOT pool contents (element-indexed) after writing token rows
    [tok0, tok0 + n) of every KV head, from the layout definition: per KV
    head, blocks of 32 tokens; K image [half h][k-group s][lane n + 16 g][e],
    V image (bf16) [j][lane][e] with token tau(g, e) = 4g + e (e < 4) or
    16 + 4g + e - 4, element d = (d/16) n + j; (fp32) [e][lane][j]."""
    img = 32 * d
    k = np.zeros(n_kv * blocks * img, dtype=rows_k.dtype)
    v = np.zeros_like(k)
    epb = d // 16
    for t in range(rows_k.shape[0]):
        tok = tok0 + t
        blk, tt = divmod(tok, 32)
        h, nk = divmod(tt, 16)
        gl, e = (tt // 4, tt % 4) if tt < 16 else ((tt - 16) // 4, 4 + (tt - 16) % 4)
        for g in range(n_kv):
            base = (g * blocks + blk) * img
            for dd in range(d):
                nv, j = divmod(dd, epb)
                if bf16:
                    s, r = divmod(dd, 32)
                    ko = ((h * (d // 32) + s) * 64 + nk + 16 * (r // 8)) * 8 + r % 8
                    vo = (j * 64 + nv + 16 * gl) * 8 + e
                else:
                    gk, w_ = divmod(dd, d // 4)
                    ko = ((h * (d // 16) + w_ // 4) * 64 + nk + 16 * gk) * 4 + w_ % 4
                    vo = (e * 64 + nv + 16 * gl) * epb + j
                k[base + ko] = rows_k[t, g, dd]
                v[base + vo] = rows_v[t, g, dd]
    return k, v


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_hot_write_layout_bit_exact(dtype, d):
    n_kv, cap = 2, 4 * 32
    ctx = binding.Context(4, n_kv, d, dtype, cap, 0)
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    it = torch.int32 if dtype == "f32" else torch.int16
    elems = ctx.hot_pool_bytes() // (4 if dtype == "f32" else 2)
    k_hot = torch.zeros(elems, dtype=td, device="cuda")
    v_hot = torch.zeros_like(k_hot)
    ctx.bind_layer(0, k_hot, v_hot, None, None)
    ctx.hot_pool_alloc(20)                       # block 0
    pid, off = ctx.hot_pool_alloc(70)            # blocks 1..3
    assert off == 32
    g = torch.Generator().manual_seed(3)
    rk = torch.randn(70, n_kv, d, generator=g).to(td)
    rv = torch.randn(70, n_kv, d, generator=g).to(td)
    ctx.hot_write(0, pid, 0, rk[:45].cuda(), rv[:45].cuda())     # two writes, 45 + 25 rows
    ctx.hot_write(0, pid, 45, rk[45:].cuda(), rv[45:].cuda())
    torch.cuda.synchronize()
    want_k, want_v = hot_layout_model(rk.view(it).numpy(), rv.view(it).numpy(), off, n_kv, d, cap // 32,
                                      dtype == "bf16")
    assert k_hot.cpu().view(it).numpy().tobytes() == want_k.tobytes()
    assert v_hot.cpu().view(it).numpy().tobytes() == want_v.tobytes()
    with pytest.raises(binding.GkvError):
        ctx.hot_write(0, pid, 60, rk[:11].cuda(), rv[:11].cuda())   # past the slab end


# ------------------------------------------------------------- tiny configs
def test_tiny_fp32_parity():
    w = workloads.make("tiny")
    st, out, lse, backend = run(w)
    assert backend == CASCADE        # M_eff = 16 < M_sat, and fp32 has no dense kernel
    ref_o, ref_l = oracle_ref(w)
    check(out, lse, ref_o, ref_l, **FP32_TOL)


@pytest.mark.parametrize("force", [CASCADE, DENSE])
def test_tiny_bf16_parity(force):
    w = workloads.make("tiny", dtype="bf16")
    st, out, lse, backend = run(w, force=force)
    assert backend == force
    check(out, lse, *oracle_ref(w))


# --------------------------------------------------- several tiles, ragged
@pytest.mark.parametrize("force", [CASCADE, DENSE])
def test_ragged_multi_tile_parity(force):
    # prefix 1000 = 15 full 64-token tiles + 40; suffixes cover empty, single
    # token, tile-1, tile, tile+1, several chunks
    s = spec(batch=8, fixed_suffix=(0, 1, 31, 32, 33, 257, 700, 1500))
    w = workloads.make(s)
    st, out, lse, backend = run(w, force=force)
    assert backend == force
    check(out, lse, *oracle_ref(w))


@pytest.mark.parametrize("n_q,n_kv,d", [(8, 8, 128), (16, 1, 128), (10, 2, 128), (32, 8, 64), (20, 4, 64),
                                         (6, 3, 128), (24, 12, 64)])
@pytest.mark.parametrize("force", [CASCADE, DENSE])
def test_group_and_head_dim_parity(n_q, n_kv, d, force):
    s = spec(n_q=n_q, n_kv=n_kv, head_dim=d, batch=5, prefix_len=333, hot_capacity=400,
             fixed_suffix=(5, 64, 0, 100, 190))
    w = workloads.make(s)
    _, out, lse, _ = run(w, force=force)
    check(out, lse, *oracle_ref(w))


@pytest.mark.parametrize("d", [64, 128])
def test_fp32_head_dims(d):
    s = spec(dtype="f32", head_dim=d, batch=3, prefix_len=200, hot_capacity=256, fixed_suffix=(0, 77, 300))
    w = workloads.make(s)
    _, out, lse, _ = run(w)
    check(out, lse, *oracle_ref(w), **FP32_TOL)


def _spike(w, rows, toks, b, h, lam):
    """Sets key rows toks of `rows` ([tokens, n_kv, d]) for KV head h // G to
    lam * q[b, h] / |q[b, h]|: that query's score there is about lam."""
    G = w.spec.n_q // w.spec.n_kv
    q = w.q[b, h].float()
    k = (lam * q / q.norm()).to(rows.dtype)
    for t in toks:
        rows[t, h // G] = k


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("force", [CASCADE, DENSE])
def test_score_jumps_move_the_reference_points(dtype, force):
    """Scores that jump far above the running maximum in the middle of a
    prefix split, in its last partial block and inside suffix parts, and
    queries whose scores climb block after block: the lazily moved reference
    points of the online softmax (a move is rare with N(0,1) data) against
    the oracle."""
    if dtype == "f32" and force == DENSE:
        pytest.skip("fp32 runs the cascade backend only")
    s = spec(n_q=8, n_kv=2, head_dim=128, dtype=dtype, batch=6, prefix_len=3000, hot_capacity=3008,
             fixed_suffix=(0, 40, 300, 900, 33, 2000))
    w = workloads.make(s)
    pk = w.prefix_k[0]
    # upward jumps mid-split (split lengths are multiples of 64 tokens), in the
    # last partial block, and late in a long range
    _spike(w, pk, [100, 700], b=0, h=1, lam=30.0)
    _spike(w, pk, [2990], b=1, h=4, lam=60.0)
    _spike(w, pk, [1500, 1501], b=2, h=7, lam=15.0)
    # queries scaled up: their scores spread over tens of units, so the
    # running maximum climbs by more than the lazy threshold again and again
    # over the blocks of every split
    w.q[4, 3] = (w.q[4, 3].float() * 8.0).to(w.q.dtype)
    w.q[5, 6] = (w.q[5, 6].float() * 10.0).to(w.q.dtype)
    # suffix parts: a jump mid-part and one on the last (current) token
    for b, toks in ((3, [500]), (5, [10, 1999]), (4, [32])):
        lo = int(w.suffix_offsets[b])
        sk = w.suffix_k[lo:int(w.suffix_offsets[b + 1])]
        _spike(w, sk, toks, b=b, h=2 * b % w.spec.n_q, lam=40.0)
    _, out, lse, backend = run(w, force=force)
    assert backend == force
    ref_o, ref_l = oracle_ref(w)
    assert float(np.abs(ref_l).max()) > 20.0   # the jumps are in the reference
    if dtype == "f32":
        check(out, lse, ref_o, ref_l, **FP32_TOL)
    else:
        check(out, lse, ref_o, ref_l)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_suffix_joins_with_many_prefix_splits(dtype):
    """Every slot table is one part, so the suffix workgroups join their
    requests themselves; a 16K prefix over 2 KV heads and three requests is
    cut into 64 splits, more than the one-batch join of 32 partials takes,
    and a suffix-only request and an empty table share the step."""
    s = spec(n_q=8, n_kv=2, head_dim=128, dtype=dtype, batch=4, prefix_len=16384, hot_capacity=16384,
             fixed_suffix=(700, 40, 2000, 0))
    w = workloads.make(s)
    w.request_prefix[2] = -1          # suffix only: finished by its part
    st, out, lse, _ = run(w, force=CASCADE)
    plan = st.ctx.last_plan()
    assert plan["n_join_blocks"] == 1 and plan["n_short_requests"] == 1   # the empty table is short
    assert plan["n_prefix_blocks"] >= 2 * 33
    check(out, lse, *oracle_ref(w), **(FP32_TOL if dtype == "f32" else {}))


@pytest.mark.parametrize("group", [1, 5, 6, 8, 16])
def test_suffix_joins_deal_heads_over_waves(group):
    """Suffix workgroups that join their own requests deal the (query head,
    request) joins over their four waves, each wave holding up to three
    joins' loads at once: G = 1 (two waves idle), 5 and 6 (one round), 8 and
    16 (two rounds).  The 64 requests fold into pairs; two of them have no
    HOT prefix, so their pairs join one request."""
    lens = tuple(100 + (i * 53) % 700 for i in range(64))
    s = spec(n_q=8 * group, n_kv=8, head_dim=128, batch=64, prefix_len=2048, hot_capacity=2048,
             fixed_suffix=lens, cold_capacity=65536)
    w = workloads.make(s)
    w.request_prefix[5] = -1
    w.request_prefix[40] = -1
    st, out, lse, _ = run(w, force=CASCADE)
    plan = st.ctx.last_plan()
    # folded pairs, every slot table one part, no short request: the suffix
    # workgroups do every join (no join workgroups)
    assert plan["folded_parts"] == 1 and plan["n_short_requests"] == 0 and plan["n_join_blocks"] == 0
    check(out, lse, *oracle_ref(w))


@pytest.mark.parametrize("force", [CASCADE, DENSE])
def test_largest_batch_parity(force):
    """The largest batch one step takes (1024 requests): one shared prefix,
    slot tables of 0..8 tokens, so many requests are prefix-only and many
    suffix parts are one token long."""
    s = spec(n_q=8, n_kv=2, head_dim=64, batch=1024, prefix_len=200, hot_capacity=256, suffix_lo=0,
             suffix_hi=8, cold_capacity=16384)
    w = workloads.make(s)
    st, out, lse, _ = run(w, force=force)
    check(out, lse, *oracle_ref(w))
    # every request is short; more of them than workgroup slots (two per CU):
    # each join workgroup takes several consecutive ones
    plan = st.ctx.last_plan()
    slots = 2 * torch.cuda.get_device_properties(0).multi_processor_count
    per = -(-1024 // slots)
    assert plan["n_short_requests"] == 1024 and plan["n_suffix_blocks"] == 0
    assert plan["n_join_blocks"] == -(-1024 // per)


@pytest.mark.parametrize("batch", [127, 128, 129])
@pytest.mark.parametrize("force", [CASCADE, DENSE])
def test_argument_forms_at_their_edge(batch, force):
    """Steps of up to 128 requests launch with the small argument block, larger
    ones with the full one: both sides of the edge, with every table entry in
    use (short, long and prefix-only requests, last request long)."""
    lens = [(i * 37) % 90 for i in range(batch)]
    lens[-1] = 300
    s = spec(n_q=16, n_kv=4, head_dim=128, batch=batch, prefix_len=500, hot_capacity=512,
             fixed_suffix=tuple(lens), cold_capacity=16384)
    w = workloads.make(s)
    st, out, lse, backend = run(w, force=force)
    assert backend == force
    check(out, lse, *oracle_ref(w))
    # gkv_plan_step gives the plan of the step that ran
    ran = st.ctx.last_plan()
    planned = st.ctx.plan_step(st.hot_ids, st.indptr_h)
    assert {k: v for k, v in planned.items() if not k.startswith("host")} == \
        {k: v for k, v in ran.items() if not k.startswith("host")}


@pytest.mark.parametrize("force", [CASCADE, DENSE])
def test_most_query_heads_parity(force):
    """The most query heads a context takes (256), 16 per KV head."""
    s = spec(n_q=256, n_kv=16, head_dim=64, batch=3, prefix_len=100, hot_capacity=128, suffix_lo=0,
             suffix_hi=40, cold_capacity=4096)
    w = workloads.make(s)
    _, out, lse, _ = run(w, force=force)
    check(out, lse, *oracle_ref(w))


def test_single_request_single_token():
    s = spec(batch=1, prefix_len=0, hot_capacity=0, fixed_suffix=(1,))
    w = workloads.make(s)
    _, out, lse, _ = run(w)
    ref_o, ref_l = oracle_ref(w)
    check(out, lse, ref_o, ref_l)
    # one token: the output is that token's V row (exactly, up to bf16 output rounding)
    v = f64(w.suffix_v[0])
    g = np.arange(32) // 4
    assert np.abs(f64(out)[0] - v[g]).max() <= 2 ** -8 * np.abs(v).max()


# ------------------------------------------------ paged fallback & classes
@pytest.mark.parametrize("force", [CASCADE, DENSE])
def test_cold_fallback_equals_hot(force):
    """The same logical step with the prefix in HOT and, with a HOT pool too
    small for it, in COLD at the front of every slot table (the admission
    fallback): both match the oracle, and the HOT run's output is unchanged
    by the slot placement."""
    s = spec(batch=6, prefix_len=900, fixed_suffix=(3, 50, 0, 129, 64, 400))
    w = workloads.make(s)
    _, out_hot, lse_hot, _ = run(w, force=force)
    st, out_cold, lse_cold, _ = run(w, force=force, hot_capacity=512)   # 900 does not fit
    assert all(i == -1 for i in st.hot_ids)
    ref = oracle_ref(w)
    check(out_hot, lse_hot, *ref)
    check(out_cold, lse_cold, *ref)


def test_mixed_prefix_and_suffix_only_requests():
    s = spec(batch=6, prefix_len=700, fixed_suffix=(10, 0, 40, 1, 300, 64))
    w = workloads.make(s)
    w.request_prefix[[2, 4]] = -1     # two requests without a HOT prefix
    _, out, lse, _ = run(w)
    check(out, lse, *oracle_ref(w))


# ------------------------------------------------------- short requests
@pytest.mark.parametrize("n_q,n_kv,d,dtype,force",
                         [(n_q, n_kv, d, "bf16", f) for n_q, n_kv, d in ((32, 8, 128), (20, 4, 64), (16, 2, 128),
                                                                         (8, 8, 64)) for f in (CASCADE, DENSE)]
                         + [(32, 8, 64, "f32", AUTO), (8, 2, 128, "f32", AUTO)])   # fp32: cascade only
def test_short_requests_join_their_own_tiles(n_q, n_kv, d, dtype, force):
    """Requests with a HOT prefix and at most 32 slot-table tokens (0, 1, 2,
    17, 31 and 32 here; 33 is not short) get no suffix part: one join
    workgroup per request attends each KV head's tile (waves take KV heads
    w, w + 4, ...; fewer than four KV heads leave waves idle; G from 1 to 5)
    and joins it with the prefix splits."""
    lens = (0, 1, 2, 17, 31, 32, 33, 1)
    s = spec(n_q=n_q, n_kv=n_kv, head_dim=d, dtype=dtype, batch=len(lens), prefix_len=700, fixed_suffix=lens)
    w = workloads.make(s)
    st, out, lse, _ = run(w, force=force)
    plan = st.ctx.last_plan()
    assert plan["n_short_requests"] == 7 and plan["n_suffix_parts"] == 1
    # the one request with a suffix part is joined by its suffix workgroups
    assert plan["n_join_blocks"] == 7
    check(out, lse, *oracle_ref(w), **(FP32_TOL if dtype == "f32" else {}))


@pytest.mark.parametrize("prefix_len", [1000, 2048, 4096])
@pytest.mark.parametrize("force", [CASCADE, DENSE])
def test_short_request_joins_by_partial_count(prefix_len, force):
    """Short requests of the Llama-3.1-8B attention shape whose joins take
    each of their three forms: at most 8 partials (1000-token prefix), 9
    (2048: 8 prefix splits and the request's tile) and 17 (4096: 16 splits);
    tables of 0..32 tokens, so some requests have no tile of their own."""
    lens = tuple((i * 7) % 33 for i in range(64))
    s = spec(batch=64, prefix_len=prefix_len, hot_capacity=-(-prefix_len // 32) * 32, cold_capacity=4096,
             fixed_suffix=lens)
    w = workloads.make(s)
    st, out, lse, backend = run(w, force=force)
    assert backend == force and st.ctx.last_plan()["n_short_requests"] == 64
    check(out, lse, *oracle_ref(w))
    assert st.ctx.step_status() == 0


@pytest.mark.parametrize("force", [CASCADE, DENSE])
def test_prefix_bound_step_of_short_requests(force):
    """A prefix-bound step: 256 requests of the Llama-3.1-8B attention shape
    on one 2K prefix, each with its current token only: no suffix workgroup,
    one join workgroup per request, and every request matches the oracle on
    two calls in a row (the join counters return to zero)."""
    s = spec(batch=256, prefix_len=2048, hot_capacity=2048, cold_capacity=512, fixed_suffix=(1,) * 256)
    w = workloads.make(s)
    st, out, lse, _ = run(w, force=force)
    plan = st.ctx.last_plan()
    assert plan["n_suffix_blocks"] == 0 and plan["n_short_requests"] == 256 and plan["n_join_blocks"] == 256
    ref = oracle_ref(w)
    check(out, lse, *ref)
    out, lse = st.new_outputs()
    st.run(out, lse)
    torch.cuda.synchronize()
    check(out, lse, *ref)
    assert st.ctx.step_status() == 0


@pytest.mark.parametrize("force", [CASCADE, DENSE])
def test_heterogeneous_classes(force):
    s = dataclasses.replace(workloads.SPECS["hetero8"], n_prefixes=3, prefix_len_lo=100, prefix_len_hi=1100,
                            class_lo=1, class_hi=4, suffix_lo=0, suffix_hi=300, hot_capacity=4096,
                            cold_capacity=8192)
    w = workloads.make(s)
    st, out, lse, _ = run(w, force=force)
    assert st.ctx.last_plan()["n_classes"] == len(set(w.request_prefix.tolist()))
    check(out, lse, *oracle_ref(w))


def test_placement_invariance_is_bitwise():
    """Moving the slab and permuting the COLD slots changes no output bit:
    the kernels sum in an order set by the logical sequence alone."""
    s = spec(batch=4, prefix_len=600, hot_capacity=2000, fixed_suffix=(100, 33, 0, 500))
    w1 = workloads.make(s)
    _, o1, l1, _ = run(w1)
    w2 = dataclasses.replace(w1, cold_perm=np.random.default_rng(5).permutation(s.cold_capacity).astype(np.int32),
                             hot_churn=[300, 500])   # hole [0,320) too small: slab moves to 832
    st2, o2, l2, _ = run(w2)
    assert st2.placement["prefix_offset"][0] == 832   # 300 and 500 tokens take 10 and 16 blocks of 32
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_repeated_calls_identical_and_failed_call_writes_nothing():
    w = workloads.make(spec(batch=3, fixed_suffix=(10, 20, 30)))
    st = DecodeState(w)
    out, lse = st.new_outputs()
    st.run(out, lse)
    out2, lse2 = st.new_outputs()
    st.run(out2, lse2)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    sentinel = torch.full_like(out, 7.0)
    with pytest.raises(binding.GkvError):
        st.ctx.attn_decode(0, st.q, [st.hot_ids[0] + 9] * 3, st.indptr_h, st.indptr_d, st.indices_d,
                           sentinel, lse)
    torch.cuda.synchronize()
    assert bool((sentinel == 7.0).all())


def test_join_counters_survive_rebinds_and_batch_changes():
    """The step kernel coordinates its partial joins through counters in the
    workspace.  A freshly bound workspace full of garbage is cleared by the
    first call; later calls (same batch, a smaller batch, a rebind to a
    second garbage workspace) must all stay exact."""
    s = spec(batch=6, prefix_len=700, hot_capacity=1024, cold_capacity=30000,
             fixed_suffix=(5000, 3, 0, 4100, 17, 9000))
    w = workloads.make(s)
    st = DecodeState(w)
    ref_o, ref_l = oracle_ref(w)
    for fill in (0xFF, 0x7F):
        ws = torch.full_like(st.workspace, fill)
        st.ctx.bind_workspace(ws)
        st.workspace = ws
        for _ in range(2):
            out, lse = st.new_outputs()
            st.run(out, lse)
            torch.cuda.synchronize()
            check(out, lse, ref_o, ref_l)
        # the first three requests alone (indptr prefix of the same tables)
        out3, lse3 = st.new_outputs()
        st.ctx.attn_decode(0, st.q[:3], st.hot_ids[:3], st.indptr_h[:4], st.indptr_d[:4], st.indices_d,
                           out3[:3], lse3[:3])
        torch.cuda.synchronize()
        check(out3, lse3, ref_o, ref_l, requests=[0, 1, 2])
    out, lse = st.new_outputs()
    st.run(out, lse)
    torch.cuda.synchronize()
    check(out, lse, ref_o, ref_l)


def test_dispatch_follows_m_eff():
    s = spec(batch=16, n_q=32, n_kv=8, fixed_suffix=tuple([8] * 16))
    w = workloads.make(s)
    st = DecodeState(w, m_sat=64)              # M_eff = 16 * 4 = 64 >= 64: dense
    out, lse = st.new_outputs()
    assert st.run(out, lse) == DENSE
    st.ctx.set_dispatch(AUTO, 65)              # 64 < 65: cascade
    assert st.run(out, lse) == CASCADE
    torch.cuda.synchronize()
    check(out, lse, *oracle_ref(w))


@pytest.mark.parametrize("force", [CASCADE, DENSE])
def test_long_suffixes_span_several_parts(force):
    """Slot tables longer than one suffix part are split into parts joined
    inside the step kernel; mixed with single-part requests and a prefix-only
    request.  The part length follows the step's total work."""
    s = spec(batch=4, prefix_len=300, hot_capacity=512, cold_capacity=20000,
             fixed_suffix=(5000, 10, 0, 9000))
    w = workloads.make(s)
    st, out, lse, _ = run(w, force=force)
    plan = st.ctx.last_plan()
    pt = plan["suffix_part_tokens"]
    assert pt % 32 == 0 and 64 <= pt <= 4096
    assert plan["joins_partials"] == 1
    # the 10- and 0-token tables are short requests (joined with their tiles, no part)
    assert plan["n_short_requests"] == 2
    assert plan["n_suffix_parts"] == sum(max(1, -(-n // pt)) for n in (5000, 9000))
    check(out, lse, *oracle_ref(w))


def _fold_lengths(batch):
    # tables of 33..199 tokens, one prefix-only request, two more short
    # requests (1 and 32 tokens) and one two-part table
    lens = np.random.default_rng(batch).integers(33, 200, batch)
    lens[3], lens[7], lens[11], lens[12] = 0, 5000, 1, 32
    return tuple(int(x) for x in lens)


def _parts(lens, short=32, part=4096):
    """Suffix parts of a step whose requests all have a HOT prefix."""
    return sum(max(1, -(-n // part)) for n in lens if n > short)


@pytest.mark.parametrize("batch,dtype", [(64, "bf16"), (65, "bf16"), (65, "f32")])
def test_folded_suffix_parts_parity(batch, dtype):
    """When the suffix parts' workgroups overflow the slots the prefix leaves
    and half as many fit, each suffix workgroup runs two parts (short, then
    long).  An odd part count leaves the middle part alone; a two-part table
    and a prefix-only request ride along."""
    s = spec(n_q=32, n_kv=8, head_dim=64, dtype=dtype, batch=batch, prefix_len=256, hot_capacity=256,
             cold_capacity=24000, fixed_suffix=_fold_lengths(batch))
    w = workloads.make(s)
    st, out, lse, backend = run(w, force=CASCADE)
    plan = st.ctx.last_plan()
    parts = _parts(_fold_lengths(batch))
    assert parts == batch - 2 and plan["n_short_requests"] == 3
    assert plan["folded_parts"] == 1 and plan["n_suffix_parts"] == parts
    assert plan["n_suffix_blocks"] == -(-(-(-parts // 2) * 8) // 32) * 32
    tol = FP32_TOL if dtype == "f32" else {}
    ref = oracle_ref(w)
    check(out, lse, *ref, **tol)
    # repeated calls: each part is counted once per call (padding workgroups
    # of the folded grid do nothing), so the join counters start at zero
    for _ in range(3):
        out, lse = st.new_outputs()
        st.run(out, lse)
        torch.cuda.synchronize()
        check(out, lse, *ref, **tol)


def test_fold_rule():
    """No folding when the parts fit beside the prefix, when even half as
    many would not, for suffix-only steps whose parts fill the slots exactly,
    or under the dense backend."""
    few = workloads.make(spec(n_kv=8, batch=40, prefix_len=256, hot_capacity=256, fixed_suffix=(40,) * 40))
    st, *_ = run(few, force=CASCADE)
    assert st.ctx.last_plan()["folded_parts"] == 0
    only = workloads.make(spec(n_kv=8, batch=64, prefix_len=0, hot_capacity=0, fixed_suffix=(9,) * 64))
    st, *_ = run(only, force=CASCADE)
    assert st.ctx.last_plan()["folded_parts"] == 0 and st.ctx.last_plan()["n_suffix_blocks"] == 512
    many = workloads.make(spec(n_q=32, n_kv=8, head_dim=64, batch=128, prefix_len=256, hot_capacity=256,
                               cold_capacity=8192, fixed_suffix=(40,) * 128))
    for force in (CASCADE, DENSE):              # 1024 part workgroups, 480 free slots
        st, out, lse, _ = run(many, force=force)
        assert st.ctx.last_plan()["folded_parts"] == 0
        check(out, lse, *oracle_ref(many))


def test_prefix_splits_lengthen_so_pairs_fit():
    """Qwen-2.5-14B TP=2 slice (128 requests, 4 KV heads, a 16K prefix): the
    first split length makes 288 prefix workgroups, beside which the 256
    folded suffix workgroups would not fit; the splits are lengthened until
    they do (256 prefix workgroups).  Every request matches the oracle (the
    full-size tests run the same plan under AUTO dispatch)."""
    w = workloads.make("qwen14b_tp2_lp16k_b128")
    st, out, lse, backend = run(w, force=CASCADE)
    plan = st.ctx.last_plan()
    assert plan["folded_parts"] == 1 and plan["n_suffix_blocks"] == 256
    assert plan["n_prefix_blocks"] == 256
    check(out, lse, *oracle_ref(w))


# ------------------------------------------------------- fused decode step
def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _fused_cases():
    tiny = workloads.SPECS["tiny"]
    return {
        "tiny_f32": (tiny, AUTO, None),
        "ragged_cascade": (spec(batch=6, fixed_suffix=(1, 31, 32, 33, 257, 700)), CASCADE, None),
        "ragged_dense": (spec(batch=6, fixed_suffix=(1, 31, 32, 33, 257, 700)), DENSE, None),
        "group5_d64": (spec(n_q=20, n_kv=4, head_dim=64, batch=5, fixed_suffix=(2, 64, 65, 129, 3)), AUTO, None),
        "suffix_only_requests": (spec(batch=6, prefix_len=700, fixed_suffix=(10, 1, 40, 1, 300, 64)), AUTO, [2, 4]),
        "fallback_to_cold": (spec(batch=4, prefix_len=900, fixed_suffix=(3, 50, 129, 400)), AUTO, "cold"),
        "multi_part": (spec(batch=4, prefix_len=300, hot_capacity=512, cold_capacity=20000,
                            fixed_suffix=(5000, 10, 1, 9000)), AUTO, None),
        "short_only": (spec(batch=16, prefix_len=500, fixed_suffix=(1,) * 8 + (5,) * 7 + (32,)), AUTO, None),
        "folded": (spec(n_q=32, n_kv=8, head_dim=64, batch=65, prefix_len=256, hot_capacity=256,
                        cold_capacity=24000, fixed_suffix=tuple(max(1, n) for n in _fold_lengths(65))),
                   CASCADE, None),
    }


@pytest.mark.parametrize("case", list(_fused_cases()))
def test_fused_step_equals_append_then_attend(case):
    """gkv_decode_step (append the batch's new tokens and attend, one launch)
    against gkv_cold_append followed by gkv_attn_decode on an identical
    placement: out, lse and both COLD pools agree bit for bit.  The new rows
    are fresh random values, so reading a stale pool row would show."""
    s, force, variant = _fused_cases()[case]
    w = workloads.make(s)
    kw = {}
    if isinstance(variant, list):
        w.request_prefix[variant] = -1            # some requests without a HOT prefix
    elif variant == "cold":
        kw["hot_capacity"] = 512                  # the prefix falls back to COLD slots
    sa = DecodeState(w, force_backend=force, **kw)
    sb = DecodeState(w, force_backend=force, **kw)
    if variant == "cold":
        assert all(i == -1 for i in sa.hot_ids)
    slots = torch.from_numpy(sa.last_slots()).cuda()
    assert np.array_equal(sa.last_slots(), sb.last_slots())
    g = torch.Generator().manual_seed(7)
    shape = (w.batch, w.spec.n_kv, w.spec.head_dim)
    k_new = torch.randn(shape, generator=g).to(w.torch_dtype).cuda()
    v_new = torch.randn(shape, generator=g).to(w.torch_dtype).cuda()

    out_a, lse_a = sa.new_outputs()
    sa.append(0, k_new, v_new, slots)
    ba = sa.run(out_a, lse_a)
    out_b, lse_b = sb.new_outputs()
    bb = sb.step(out_b, lse_b, k_new, v_new, slots)
    torch.cuda.synchronize()
    assert ba == bb
    assert sb.ctx.last_plan()["folded_parts"] == (case == "folded")
    assert torch.equal(_bits(out_a), _bits(out_b))
    assert torch.equal(lse_a.view(torch.int32), lse_b.view(torch.int32))
    for i in (2, 3):                                  # k_cold, v_cold
        assert torch.equal(_bits(sa.pools[0][i]), _bits(sb.pools[0][i]))
    # the appended slots hold the new rows, each KV head at its in-slot
    # position (the oracle's model of the COLD layout)
    for i, new in ((2, k_new), (3, v_new)):
        pool = _bits(sb.pools[0][i]).cpu().numpy()
        want = append_model(pool, sa.last_slots(), _bits(new).cpu().numpy())
        assert pool.tobytes() == want.tobytes()


def test_fused_step_repeats_and_matches_the_oracle():
    """Repeated fused steps on one state (the pool already holds the new
    rows from the previous step) stay equal to the oracle."""
    w = workloads.make(spec(batch=5, fixed_suffix=(7, 70, 700, 1, 33)))
    st = DecodeState(w)
    slots = torch.from_numpy(st.last_slots()).cuda()
    last = torch.from_numpy(w.suffix_offsets[1:] - 1)
    k_new = w.suffix_k[last].cuda().contiguous()
    v_new = w.suffix_v[last].cuda().contiguous()
    ref = oracle_ref(w)
    for _ in range(3):
        out, lse = st.new_outputs()
        st.step(out, lse, k_new, v_new, slots)
        torch.cuda.synchronize()
        check(out, lse, *ref)


# ------------------------------------------------------- join give-up path
def test_join_give_up_is_reported_and_counters_recover():
    """The join of a step's partials waits with a bounded wait.  With the
    bound set to zero polls from the host, joins whose partials have not
    arrived (a 16K prefix: its splits take far longer than a join's first
    look) give up at once, every kernel still ends, and gkv_step_status
    reports them.  With the default bound back, the next steps are exact:
    the counters came back to zero when the late partials arrived."""
    s = spec(batch=4, prefix_len=16384, hot_capacity=16384, cold_capacity=20000,
             fixed_suffix=(10, 300, 5000, 9000))
    w = workloads.make(s)
    st = DecodeState(w)
    ref = oracle_ref(w)
    st.ctx.set_join_spin_limit(0)
    out, lse = st.new_outputs()
    st.run(out, lse)
    torch.cuda.synchronize()
    gave_up = st.ctx.step_status()
    assert 0 < gave_up <= w.batch * s.n_kv
    assert st.ctx.step_status() == 0           # read and cleared
    st.ctx.set_join_spin_limit(-1)
    for _ in range(2):
        out, lse = st.new_outputs()
        st.run(out, lse)
        torch.cuda.synchronize()
        check(out, lse, *ref)
    assert st.ctx.step_status() == 0


# ---------------------------------------------- uniform-page prefix copies
def test_paged_prefix_copies_match_the_oracle():
    """The baseline layout of the kernel-mechanism comparison: each request
    holds its own copy of the shared prefix in 16-token pages of the COLD pool
    (pages in random order) plus its current token, read through its slot
    table (no HOT prefix).  Output equals the oracle's attention over prefix
    || current token, as does the same step with the prefix in one HOT slab."""
    from shared_prefix_paged_contiguous_amd.harness import paged_copies

    bsz, plen, page, n_q, n_kv, d = 8, 512, 16, 32, 8, 128
    rng = np.random.default_rng(21)

    def vals(shape):
        return torch.from_numpy(rng.standard_normal(size=shape, dtype=np.float32)).to(torch.bfloat16)

    q, pk, pv = vals((bsz, n_q, d)), vals((plen, n_kv, d)), vals((plen, n_kv, d))
    ck, cv = vals((bsz, n_kv, d)), vals((bsz, n_kv, d))
    ref_o, ref_l = decode_ref(q, pk, pv, ck, cv)

    ctx = binding.Context(n_q, n_kv, d, "bf16", 0, bsz * (plen + 1))
    k_cold = torch.zeros((bsz * (plen + 1), n_kv, d), dtype=torch.bfloat16, device="cuda")
    v_cold = torch.zeros_like(k_cold)
    ctx.bind_layer(0, None, None, k_cold, v_cold)
    indptr, indices = paged_copies(ctx, 0, pk.cuda(), pv.cuda(), ck.cuda(), cv.cuda(), page, rng)
    assert len(set(indices.tolist())) == bsz * (plen + 1)      # every request's copy is its own
    ws = torch.empty(ctx.workspace_size(bsz, len(indices)), dtype=torch.uint8, device="cuda")
    ctx.bind_workspace(ws)
    out = torch.empty((bsz, n_q, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((bsz, n_q), dtype=torch.float32, device="cuda")
    ctx.attn_decode(0, q.cuda(), [-1] * bsz, indptr, None, torch.from_numpy(indices).cuda(), out, lse)
    torch.cuda.synchronize()
    check(out, lse, ref_o, ref_l)

    # the same logical step over one HOT slab shared by the batch
    hc = binding.Context(n_q, n_kv, d, "bf16", plen, bsz)
    pid, _ = hc.hot_pool_alloc(plen)
    k_hot = torch.zeros(hc.hot_pool_bytes() // 2, dtype=torch.bfloat16, device="cuda")
    v_hot = torch.zeros_like(k_hot)
    k_c2 = torch.zeros((bsz, n_kv, d), dtype=torch.bfloat16, device="cuda")
    v_c2 = torch.zeros_like(k_c2)
    hc.bind_layer(0, k_hot, v_hot, k_c2, v_c2)
    hc.hot_write(0, pid, 0, pk.cuda(), pv.cuda())
    cur = torch.arange(bsz, dtype=torch.int32, device="cuda")
    hc.cold_append(0, ck.cuda(), cv.cuda(), cur)
    ws2 = torch.empty(hc.workspace_size(bsz, bsz), dtype=torch.uint8, device="cuda")
    hc.bind_workspace(ws2)
    out2, lse2 = torch.empty_like(out), torch.empty_like(lse)
    hc.attn_decode(0, q.cuda(), [pid] * bsz, np.arange(bsz + 1, dtype=np.int32), None, cur, out2, lse2)
    torch.cuda.synchronize()
    check(out2, lse2, ref_o, ref_l)


def decode_ref(q, pk, pv, ck, cv):
    """Oracle of a step whose requests share prefix (pk, pv) and each have one
    suffix token (ck[b], cv[b])."""
    from oracle.attention import decode_step

    bsz = q.shape[0]
    return decode_step(f64(q), [f64(pk)], [f64(pv)], np.zeros(bsz, dtype=np.int32),
                       [f64(ck[b:b + 1]) for b in range(bsz)], [f64(cv[b:b + 1]) for b in range(bsz)])
