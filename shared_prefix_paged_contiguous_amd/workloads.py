"""Seeded synthetic decode-step workloads (input generation only).

This module draws random numbers and nothing else: it holds none of the
attention arithmetic, so both the HIP path and the CPU oracle can take their
inputs from it.  It describes each workload *logically* (per-request prefix
index, suffix lengths, Q/K/V token rows in context order) plus the random
draws the storage placement needs (a COLD free-order permutation, HOT churn
lengths).  Where the rows land in the pools is decided by whichever allocator
replays ``placement_ops`` - the C library on the GPU side, the allocator
models on the oracle side.

The shapes follow the attention shapes of the models the GraniKV pages
evaluate (Llama-3.1-8B at TP=1, Qwen-2.5-14B at TP=2, Qwen-2.5-32B at TP=4,
one GPU's head slice each) with a long shared prefix and short per-request
suffixes; the pages measure on ShareGPT-V3 conversations, for which these
N(0,1) tensors stand in.

Draw order (numpy PCG64, one generator per workload, seed 0 by default):
  a) heterogeneous workloads only: prefix lengths, class sizes, then the
     request order (a permutation interleaving the classes), then HOT churn
     lengths;
  b) suffix lengths, integers(lo, hi + 1);
  c) COLD free-order permutation of all C_cold slots;
  d) Q;
  e) for each prefix in order: K then V;
  f) suffix K for all requests in request order, then suffix V.
All values are float32 standard normals, rounded to bfloat16 (round to
nearest even, by torch) for bf16 workloads.
"""

from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Spec:
    name: str
    n_q: int
    n_kv: int
    head_dim: int
    dtype: str                      # "f32" | "bf16"
    batch: int                      # requests (heterogeneous: drawn, this is ignored)
    prefix_len: int                 # single-prefix workloads; 0 = no prefix
    suffix_lo: int
    suffix_hi: int
    hot_capacity: int
    cold_capacity: int
    n_prefixes: int = 1
    prefix_len_lo: int = 0          # heterogeneous prefix lengths
    prefix_len_hi: int = 0
    class_lo: int = 0               # heterogeneous class sizes
    class_hi: int = 0
    fixed_suffix: Optional[tuple] = None
    seed: int = 0
    description: str = ""


SPECS = {
    "tiny": Spec(
        "tiny", n_q=8, n_kv=2, head_dim=64, dtype="f32", batch=4, prefix_len=512,
        suffix_lo=16, suffix_hi=64, hot_capacity=512, cold_capacity=1024,
        fixed_suffix=(16, 32, 48, 64),
        description="tiny decode step: B=4, 8q/2kv, d=64, fp32, L_p=512, suffixes 16/32/48/64"),
    "llama8b_lp16k_b64": Spec(
        "llama8b_lp16k_b64", n_q=32, n_kv=8, head_dim=128, dtype="bf16", batch=64,
        prefix_len=16384, suffix_lo=128, suffix_hi=1024, hot_capacity=16384,
        cold_capacity=65536,
        description="Llama-3.1-8B attention shape, 32q/8kv, d=128, bf16, L_p=16384, B=64, "
                    "suffixes U{128..1024}"),
    "qwen14b_tp2_lp16k_b128": Spec(
        "qwen14b_tp2_lp16k_b128", n_q=20, n_kv=4, head_dim=128, dtype="bf16", batch=128,
        prefix_len=16384, suffix_lo=64, suffix_hi=2048, hot_capacity=16384,
        cold_capacity=262144,
        description="Qwen-2.5-14B TP=2 one-GPU head slice, 20q/4kv, d=128, bf16, L_p=16384, "
                    "B=128, suffixes U{64..2048}"),
    "hetero8": Spec(
        "hetero8", n_q=32, n_kv=8, head_dim=128, dtype="bf16", batch=0, prefix_len=0,
        suffix_lo=128, suffix_hi=1024, hot_capacity=131072, cold_capacity=131072,
        n_prefixes=8, prefix_len_lo=2048, prefix_len_hi=16384, class_lo=8, class_hi=16,
        description="8 distinct HOT prefixes U{2K..16K}, 8-16 requests each, 32q/8kv, d=128, "
                    "bf16, suffixes U{128..1024}"),
    "qwen32b_tp4_lp1k_b256": Spec(
        "qwen32b_tp4_lp1k_b256", n_q=10, n_kv=2, head_dim=128, dtype="bf16", batch=256,
        prefix_len=1024, suffix_lo=256, suffix_hi=4096, hot_capacity=1024,
        cold_capacity=1048576,
        description="Qwen-2.5-32B TP=4 one-GPU head slice, 10q/2kv, d=128, bf16, L_p=1024, "
                    "B=256, suffixes U{256..4096}"),
}


@dataclasses.dataclass
class Workload:
    spec: Spec
    prefix_lens: List[int]
    request_prefix: np.ndarray      # [B] int32, prefix index, -1 = none
    suffix_lens: np.ndarray         # [B] int64
    cold_perm: np.ndarray           # [C_cold] int32, COLD free order
    hot_churn: List[int]            # lengths of throw-away HOT slabs (heterogeneous only)
    q: torch.Tensor                 # [B, n_q, d] cpu
    prefix_k: List[torch.Tensor]    # [L_p, n_kv, d] cpu, per prefix
    prefix_v: List[torch.Tensor]
    suffix_k: torch.Tensor          # [sum S_b, n_kv, d] cpu, request order then token order
    suffix_v: torch.Tensor
    suffix_offsets: np.ndarray      # [B+1] int64 into suffix_k/v

    @property
    def batch(self) -> int:
        return int(self.q.shape[0])

    @property
    def torch_dtype(self):
        return torch.float32 if self.spec.dtype == "f32" else torch.bfloat16

    def suffix_rows(self, b: int):
        lo, hi = int(self.suffix_offsets[b]), int(self.suffix_offsets[b + 1])
        return self.suffix_k[lo:hi], self.suffix_v[lo:hi]


def _values(rng, shape, dtype: str) -> torch.Tensor:
    x = torch.from_numpy(rng.standard_normal(size=shape, dtype=np.float32))
    return x if dtype == "f32" else x.to(torch.bfloat16)


def make(name_or_spec, *, seed: Optional[int] = None, dtype: Optional[str] = None,
         batch: Optional[int] = None, suffix_range: Optional[tuple] = None,
         prefix_len: Optional[int] = None) -> Workload:
    """Draw a workload.  Overrides derive variants (a bf16 copy of the tiny
    step, an M_eff sweep point with another batch, prefix-only steps)."""
    spec = SPECS[name_or_spec] if isinstance(name_or_spec, str) else name_or_spec
    repl = {}
    if seed is not None:
        repl["seed"] = seed
    if dtype is not None:
        repl["dtype"] = dtype
    if batch is not None:
        repl["batch"] = batch
        repl["fixed_suffix"] = None
    if suffix_range is not None:
        repl["suffix_lo"], repl["suffix_hi"] = suffix_range
        repl["fixed_suffix"] = None
    if prefix_len is not None:
        repl["prefix_len"] = prefix_len
    if repl:
        spec = dataclasses.replace(spec, **repl)

    rng = np.random.default_rng(spec.seed)
    d, n_kv, n_q = spec.head_dim, spec.n_kv, spec.n_q

    hot_churn: List[int] = []
    if spec.n_prefixes > 1:
        prefix_lens = rng.integers(spec.prefix_len_lo, spec.prefix_len_hi + 1,
                                   size=spec.n_prefixes).tolist()
        class_sizes = rng.integers(spec.class_lo, spec.class_hi + 1, size=spec.n_prefixes)
        request_prefix = np.repeat(np.arange(spec.n_prefixes), class_sizes)
        request_prefix = request_prefix[rng.permutation(len(request_prefix))].astype(np.int32)
        hot_churn = rng.integers(4096, 16384 + 1, size=4).tolist()
        n_b = len(request_prefix)
    else:
        n_b = spec.batch
        prefix_lens = [spec.prefix_len] if spec.prefix_len > 0 else []
        request_prefix = np.full(n_b, 0 if prefix_lens else -1, dtype=np.int32)

    if spec.fixed_suffix is not None:
        suffix_lens = np.asarray(spec.fixed_suffix, dtype=np.int64)
        assert len(suffix_lens) == n_b
    elif spec.suffix_hi <= 0:
        suffix_lens = np.zeros(n_b, dtype=np.int64)
    else:
        suffix_lens = rng.integers(spec.suffix_lo, spec.suffix_hi + 1, size=n_b).astype(np.int64)

    # a larger batch than the spec's (an M_eff sweep point) may need a larger
    # COLD pool; specs that fit draw exactly as before
    need = int(suffix_lens.sum()) + n_b
    if need > spec.cold_capacity:
        spec = dataclasses.replace(spec, cold_capacity=-(-need * 5 // 4 // 4096) * 4096)
    cold_perm = rng.permutation(spec.cold_capacity).astype(np.int32)

    q = _values(rng, (n_b, n_q, d), spec.dtype)
    prefix_k, prefix_v = [], []
    for ln in prefix_lens:
        prefix_k.append(_values(rng, (ln, n_kv, d), spec.dtype))
        prefix_v.append(_values(rng, (ln, n_kv, d), spec.dtype))
    total = int(suffix_lens.sum())
    suffix_k = _values(rng, (total, n_kv, d), spec.dtype)
    suffix_v = _values(rng, (total, n_kv, d), spec.dtype)
    offsets = np.zeros(n_b + 1, dtype=np.int64)
    np.cumsum(suffix_lens, out=offsets[1:])
    return Workload(spec, prefix_lens, request_prefix, suffix_lens, cold_perm, hot_churn,
                    q, prefix_k, prefix_v, suffix_k, suffix_v, offsets)


def make_uniform_multi_prefix(k: int, *, prefix_len: int = 8192, batch: int = 256,
                              suffix_range: tuple = (128, 1024), hot_capacity: int,
                              cold_capacity: int, seed: int = 0, device: str = "cpu") -> Workload:
    """k distinct prefixes of prefix_len tokens at the Llama-3.1-8B attention
    shape (32q/8kv, d=128, bf16), request b on prefix b % k (batch / k
    requests each), suffix lengths U{lo..hi}: the uniform-length multi-prefix
    sweep of paperlayer.ai Appendix B.8 (k in {1, 4, 16, 64}, L_p = 8K,
    B = 256).

    Integer draws (numpy PCG64, seeded): suffix lengths, then the COLD free
    order.  Values: standard normals from torch's generator on `device`
    seeded with `seed` (Q, then each prefix's K and V, then suffix K and V),
    rounded to bf16; drawing them on the GPU keeps multi-gigabyte prefix sets
    off the host."""
    import torch

    spec = Spec(f"uniform_k{k}_lp{prefix_len}_b{batch}", n_q=32, n_kv=8, head_dim=128, dtype="bf16",
                batch=batch, prefix_len=prefix_len, suffix_lo=suffix_range[0], suffix_hi=suffix_range[1],
                hot_capacity=hot_capacity, cold_capacity=cold_capacity, n_prefixes=k,
                prefix_len_lo=prefix_len, prefix_len_hi=prefix_len, class_lo=batch // k,
                class_hi=batch // k, seed=seed,
                description=f"{k} distinct prefixes of {prefix_len} tokens, B={batch} (request b on "
                            f"prefix b % {k}), 32q/8kv, d=128, bf16, suffixes U{{{suffix_range[0]}.."
                            f"{suffix_range[1]}}}")
    rng = np.random.default_rng(seed)
    suffix_lens = rng.integers(suffix_range[0], suffix_range[1] + 1, size=batch).astype(np.int64)
    cold_perm = rng.permutation(cold_capacity).astype(np.int32)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)

    def vals(shape):
        return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)

    q = vals((batch, 32, 128))
    prefix_k, prefix_v = [], []
    for _ in range(k):
        prefix_k.append(vals((prefix_len, 8, 128)))
        prefix_v.append(vals((prefix_len, 8, 128)))
    total = int(suffix_lens.sum())
    suffix_k, suffix_v = vals((total, 8, 128)), vals((total, 8, 128))
    offsets = np.zeros(batch + 1, dtype=np.int64)
    np.cumsum(suffix_lens, out=offsets[1:])
    request_prefix = (np.arange(batch) % k).astype(np.int32)
    return Workload(spec, [prefix_len] * k, request_prefix, suffix_lens, cold_perm, [],
                    q, prefix_k, prefix_v, suffix_k, suffix_v, offsets)


def placement_ops(w: Workload):
    """The allocator calls that place a workload, in order.

    Yields tuples both allocator implementations replay:
      ("hot_alloc", tag, n)      tag names the slab ("churn<i>" or "prefix<p>")
      ("hot_free", tag)
      ("cold_alloc", tag, n)     tag: "all", "prefix<p>" (COLD fallback), "req<b>"
      ("cold_free", tag, slots)  slots: int32 array
    The churn leaves two holes at the low end of the HOT pool so mixed slab
    sizes go through first fit.  A prefix whose HOT allocation fails falls
    back to COLD (the caller decides that; see ``place``).
    """
    for i, n in enumerate(w.hot_churn):
        yield ("hot_alloc", f"churn{i}", n)
    for i in (0, 2):
        if i < len(w.hot_churn):
            yield ("hot_free", f"churn{i}")
    for p, ln in enumerate(w.prefix_lens):
        yield ("hot_alloc", f"prefix{p}", ln)
    yield ("cold_alloc", "all", w.spec.cold_capacity)
    yield ("cold_free", "all", w.cold_perm)
    for b in range(w.batch):
        yield ("cold_alloc", f"req{b}", int(w.suffix_lens[b]))


def place(w: Workload, hot_alloc, hot_free, cold_alloc, cold_free):
    """Replay ``placement_ops`` on an allocator given as four callables.

    hot_alloc(n) -> (id, offset) or None on NOSPACE; hot_free(id);
    cold_alloc(n) -> int32 array; cold_free(slots).
    Returns dict with 'prefix_id' [P], 'prefix_offset' [P] (-1 when the prefix
    fell back to COLD), 'prefix_slots' {p: slots} for fallen-back prefixes and
    'req_slots' [B] arrays.
    """
    ids = {}
    out = {"prefix_id": [-1] * len(w.prefix_lens), "prefix_offset": [-1] * len(w.prefix_lens),
           "prefix_slots": {}, "req_slots": [None] * w.batch}
    fallen = []
    for op in placement_ops(w):
        kind, tag = op[0], op[1]
        if kind == "hot_alloc":
            r = hot_alloc(op[2])
            if r is None:
                if tag.startswith("prefix"):
                    fallen.append(int(tag[6:]))
                continue
            ids[tag] = r[0]
            if tag.startswith("prefix"):
                p = int(tag[6:])
                out["prefix_id"][p], out["prefix_offset"][p] = r
        elif kind == "hot_free":
            if tag in ids:
                hot_free(ids.pop(tag))
        elif kind == "cold_alloc":
            slots = np.asarray(cold_alloc(op[2]), dtype=np.int32)
            if tag.startswith("req"):
                out["req_slots"][int(tag[3:])] = slots
        elif kind == "cold_free":
            cold_free(np.asarray(op[2], dtype=np.int32))
    # COLD fallback of prefixes that did not fit in HOT: allocated after the
    # suffixes so the suffix placement does not depend on HOT occupancy.
    for p in fallen:
        out["prefix_slots"][p] = np.asarray(cold_alloc(w.prefix_lens[p]), dtype=np.int32)
    return out
