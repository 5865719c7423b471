"""Device-side set-up of a synthetic decode step (used by tests and bench.py).

Given a ``workloads.Workload`` it creates a library context, replays the
workload's placement through the context's own allocators (HOT first, COLD
fallback for prefixes that do not fit, permuted COLD free order for the
suffix slots) - or through its prefix registry (``registry=True``) - writes the prefix slabs into the HOT pool with ``hot_write``
(the caller's prefill, outside the decode path), appends every suffix token
into the COLD pool with ``cold_append``, and builds the per-request CSR slot
table.
"""

from __future__ import annotations

from typing import List, Optional

import numpy as np
import torch

from . import binding, workloads


def prefix_key(p: int) -> int:
    """Registry key of the workload's prefix p (any distinct 64-bit values do)."""
    return (0x9E3779B97F4A7C15 * (p + 1)) % (1 << 64)


def place_through_registry(w: workloads.Workload, ctx: binding.Context):
    """Place a workload with the library's prefix registry instead of raw
    allocations: the COLD free order is scattered as the workload's recipe
    says, then every request takes a reference to its prefix in request order
    (the first one admits it: HOT first, COLD when no HOT extent fits, no
    demotion), then each request's suffix slots are popped.  Same result
    format as ``workloads.place`` ('prefix_slots' holds the prefixes the
    registry put in COLD)."""
    n_p = len(w.prefix_lens)
    out = {"prefix_id": [-1] * n_p, "prefix_offset": [-1] * n_p, "prefix_slots": {},
           "req_slots": [None] * w.batch, "refs": {}}
    ctx.cold_pool_alloc(w.spec.cold_capacity)
    ctx.cold_pool_free(w.cold_perm)
    for b in range(w.batch):
        p = int(w.request_prefix[b])
        if p < 0:
            continue
        r = ctx.prefix_acquire(prefix_key(p), w.prefix_lens[p])
        out["refs"][p] = out["refs"].get(p, 0) + 1
        if r["fresh"]:
            if r["pool"] == binding.POOL_HOT:
                out["prefix_id"][p], out["prefix_offset"][p] = r["prefix_id"], r["hot_offset"]
            else:
                out["prefix_slots"][p] = ctx.prefix_cold_slots(prefix_key(p), w.prefix_lens[p])
    for b in range(w.batch):
        out["req_slots"][b] = ctx.cold_pool_alloc(int(w.suffix_lens[b]))
    return out


def paged_copies(ctx: binding.Context, layer: int, prefix_k, prefix_v, cur_k, cur_v, page: int,
                 rng: np.random.Generator, base_slot: int = 0):
    """The uniform-page layout of a shared prefix (the baseline the pages
    compare the HOT slab with): every request gets a copy of its own of the
    prefix in pages of `page` consecutive COLD slots, the pages in random
    order, followed by one slot holding the request's current token.

    prefix_k/v: dev [L, n_kv, d] (L a multiple of `page`); cur_k/v: dev
    [B, n_kv, d].  Writes the rows with gkv_cold_append into slots
    [base_slot, base_slot + B * (L + 1)) of `layer` and returns the CSR slot
    table (indptr [B+1] int32 host, indices int32 host), request b's table
    being its L prefix slots in token order, then its current-token slot."""
    plen = int(prefix_k.shape[0])
    bsz = int(cur_k.shape[0])
    if plen % page:
        raise ValueError("prefix length must be a whole number of pages")
    per = plen // page
    pages = rng.permutation(bsz * per).astype(np.int64)
    tables = []
    for b in range(bsz):
        slots = base_slot + (pages[b * per:(b + 1) * per, None] * page + np.arange(page)[None, :]).reshape(-1)
        ctx.cold_append(layer, prefix_k, prefix_v, torch.from_numpy(slots.astype(np.int32)).to(prefix_k.device))
        tables.append(np.concatenate([slots, [base_slot + bsz * plen + b]]).astype(np.int32))
    cur = torch.arange(base_slot + bsz * plen, base_slot + bsz * plen + bsz, dtype=torch.int32,
                       device=prefix_k.device)
    ctx.cold_append(layer, cur_k, cur_v, cur)
    indptr = (np.arange(bsz + 1, dtype=np.int64) * (plen + 1)).astype(np.int32)
    return indptr, np.concatenate(tables)


class DecodeState:
    def __init__(self, w: workloads.Workload, device: str = "cuda", n_layers: int = 1,
                 m_sat: int = 0, force_backend: int = binding.BACKEND_AUTO,
                 hot_capacity: Optional[int] = None, cold_capacity: Optional[int] = None,
                 registry: bool = False, partial_dtype: str = "input", bind_workspace: bool = True):
        s = w.spec
        self.w = w
        self.device = device
        self.dtype = w.torch_dtype
        self.hot_cap = s.hot_capacity if hot_capacity is None else hot_capacity
        self.cold_cap = s.cold_capacity if cold_capacity is None else cold_capacity
        self.n_layers = n_layers
        self.ctx = binding.Context(s.n_q, s.n_kv, s.head_dim, s.dtype, self.hot_cap, self.cold_cap,
                                   n_layers=n_layers, m_sat=m_sat, force_backend=force_backend,
                                   partial_dtype=partial_dtype if s.dtype == "bf16" else "input")
        ctx = self.ctx

        def hot_alloc(n):
            try:
                return ctx.hot_pool_alloc(n)
            except binding.NoSpace:
                return None

        if registry:
            self.placement = place_through_registry(w, ctx)
        else:
            self.placement = workloads.place(w, hot_alloc, ctx.hot_pool_free, ctx.cold_pool_alloc,
                                             ctx.cold_pool_free)
        pl = self.placement

        n_kv, d = s.n_kv, s.head_dim
        dev = torch.device(device)
        hot_elems = max(ctx.hot_pool_bytes() // w.q.element_size(), 16)
        k_hot = torch.zeros(hot_elems, dtype=self.dtype, device=dev)
        v_hot = torch.zeros_like(k_hot)
        k_cold = torch.zeros((max(self.cold_cap, 1), n_kv, d), dtype=self.dtype, device=dev)
        v_cold = torch.zeros_like(k_cold)
        self.pools = [(k_hot, v_hot, k_cold, v_cold)]
        ctx.bind_layer(0, k_hot, v_hot, k_cold, v_cold)
        # the prefill of each HOT prefix: rows into the slab (blocked layout)
        for p, ln in enumerate(w.prefix_lens):
            if pl["prefix_offset"][p] >= 0:
                ctx.hot_write(0, pl["prefix_id"][p], 0, w.prefix_k[p].to(dev).contiguous(),
                              w.prefix_v[p].to(dev).contiguous())

        # COLD rows: fallen-back prefixes, then every suffix token, via cold_append
        rows_k, rows_v, slots = [], [], []
        for p, sl in pl["prefix_slots"].items():
            rows_k.append(w.prefix_k[p]); rows_v.append(w.prefix_v[p]); slots.append(sl)
        rows_k.append(w.suffix_k); rows_v.append(w.suffix_v)
        slots.append(np.concatenate([pl["req_slots"][b] for b in range(w.batch)]) if w.batch else
                     np.zeros(0, np.int32))
        all_slots = np.concatenate(slots).astype(np.int32)
        if len(all_slots):
            self.append(0, torch.cat(rows_k).to(dev), torch.cat(rows_v).to(dev),
                        torch.from_numpy(all_slots).to(dev))

        # per-request context: HOT id (or -1 and the prefix slots up front), then suffix slots
        ids: List[int] = []
        tables = []
        for b in range(w.batch):
            p = int(w.request_prefix[b])
            t = []
            if p >= 0 and pl["prefix_id"][p] >= 0:
                ids.append(pl["prefix_id"][p])
            else:
                ids.append(-1)
                if p >= 0:
                    t.append(pl["prefix_slots"][p])
            t.append(pl["req_slots"][b])
            tables.append(np.concatenate(t))
        self.hot_ids = np.asarray(ids, dtype=np.int32)
        lens = np.asarray([len(t) for t in tables], dtype=np.int64)
        indptr = np.zeros(w.batch + 1, dtype=np.int64)
        np.cumsum(lens, out=indptr[1:])
        assert indptr[-1] < 2 ** 31
        self.indptr_h = indptr.astype(np.int32)
        self.indices_h = (np.concatenate(tables) if tables else np.zeros(0)).astype(np.int32)
        self.indptr_d = torch.from_numpy(self.indptr_h).to(dev)
        self.indices_d = torch.from_numpy(self.indices_h).to(dev)
        self.q = w.q.to(dev)
        self.workspace = None
        if bind_workspace:
            ws_bytes = ctx.workspace_size(w.batch, int(self.indptr_h[-1]))
            self.workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
            ctx.bind_workspace(self.workspace)
        for layer in range(1, n_layers):
            self.add_layer_copy(layer)

    def append(self, layer, k_rows, v_rows, slots_dev):
        self.ctx.cold_append(layer, k_rows.contiguous(), v_rows.contiguous(), slots_dev)

    def add_layer_copy(self, layer: int):
        """Bind a copy of layer 0's pools as `layer` (distinct memory, same data)."""
        k_hot, v_hot, k_cold, v_cold = (t.clone() for t in self.pools[0])
        self.pools.append((k_hot, v_hot, k_cold, v_cold))
        self.ctx.bind_layer(layer, k_hot, v_hot, k_cold, v_cold)

    def new_outputs(self):
        s = self.w.spec
        out = torch.empty((self.w.batch, s.n_q, s.head_dim), dtype=self.dtype, device=self.device)
        lse = torch.empty((self.w.batch, s.n_q), dtype=torch.float32, device=self.device)
        return out, lse

    def run(self, out, lse, layer: int = 0, stream=None) -> int:
        return self.ctx.attn_decode(layer, self.q, self.hot_ids, self.indptr_h, self.indptr_d,
                                    self.indices_d, out, lse, stream=stream)

    def last_slots(self) -> np.ndarray:
        """Slot of each request's last slot-table entry (its decode token)."""
        if not np.all(np.diff(self.indptr_h) > 0):
            raise ValueError("a request has an empty slot table")
        return self.indices_h[self.indptr_h[1:] - 1].astype(np.int32)

    def step(self, out, lse, k_new, v_new, slots_dev, layer: int = 0, stream=None) -> int:
        """One fused decode step (gkv_decode_step): request b's new token
        (k_new[b], v_new[b]) goes into slots_dev[b], its last table entry."""
        return self.ctx.decode_step(layer, self.q, k_new, v_new, slots_dev, self.hot_ids, self.indptr_h,
                                    self.indices_d, out, lse, stream=stream)
