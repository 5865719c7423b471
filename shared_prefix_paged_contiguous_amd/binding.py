"""ctypes binding of libgkv (include/gkv.h): argument marshalling only.

Each method has the name of the C entry point without its ``gkv_`` prefix.
Device buffers are passed as torch tensors (their data pointers) or as raw
integer addresses; streams default to torch's current stream.  Every step of
the decode path runs in the library's HIP kernels; there is no fallback: if
libgkv.so is missing, loading raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgkv.so")

GKV_OK, GKV_ERR_INVALID, GKV_ERR_NOSPACE, GKV_ERR_NOTFOUND, GKV_ERR_DEVICE = 0, -1, -2, -3, -4
GKV_F32, GKV_BF16 = 0, 1
BACKEND_AUTO, BACKEND_CASCADE, BACKEND_DENSE = 0, 1, 2
BACKEND_NAMES = {BACKEND_AUTO: "auto", BACKEND_CASCADE: "cascade", BACKEND_DENSE: "dense"}
PARTIALS_INPUT, PARTIALS_F32 = 0, 1


class GkvError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"gkv error {code}: {msg}")
        self.code = code


class NoSpace(GkvError):
    pass


class NotFound(GkvError):
    pass


class _Config(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("n_layers", ctypes.c_int32), ("hot_capacity_tokens", ctypes.c_int64),
                ("cold_capacity_tokens", ctypes.c_int64), ("m_sat", ctypes.c_int32),
                ("force_backend", ctypes.c_int32), ("partials", ctypes.c_int32)]


class _Stats(ctypes.Structure):
    _fields_ = [("hot_free_tokens", ctypes.c_int64), ("hot_largest_hole", ctypes.c_int64),
                ("hot_live_prefixes", ctypes.c_int32), ("hot_free_extents", ctypes.c_int32),
                ("cold_free_slots", ctypes.c_int64)]


class _PlanInfo(ctypes.Structure):
    _fields_ = [("backend", ctypes.c_int32), ("m_eff", ctypes.c_int32),
                ("n_classes", ctypes.c_int32), ("n_prefix_blocks", ctypes.c_int32),
                ("n_suffix_blocks", ctypes.c_int32), ("n_suffix_parts", ctypes.c_int32),
                ("joins_partials", ctypes.c_int32), ("suffix_part_tokens", ctypes.c_int32),
                ("folded_parts", ctypes.c_int32), ("n_join_blocks", ctypes.c_int32),
                ("n_short_requests", ctypes.c_int32), ("workspace_bytes", ctypes.c_int64), ("host_plan_us", ctypes.c_double),
                ("host_call_us", ctypes.c_double)]


class _PrefixRef(ctypes.Structure):
    _fields_ = [("pool", ctypes.c_int32), ("prefix_id", ctypes.c_int32), ("hot_offset", ctypes.c_int64),
                ("n_tokens", ctypes.c_int32), ("fresh", ctypes.c_int32), ("refs", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class _RegistryCounts(ctypes.Structure):
    _fields_ = [("resident_hot", ctypes.c_int32), ("resident_cold", ctypes.c_int32),
                ("referenced", ctypes.c_int32), ("cached", ctypes.c_int32), ("hits", ctypes.c_int64),
                ("hot_admits", ctypes.c_int64), ("cold_admits", ctypes.c_int64), ("evictions", ctypes.c_int64)]


POOL_HOT, POOL_COLD = 0, 1

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_PI32 = ctypes.POINTER(ctypes.c_int32)

# name -> (restype, argtypes); the exported symbols of include/gkv.h
SIGNATURES = {
    "gkv_default_m_sat": (_I32, []),
    "gkv_create": (ctypes.c_int, [ctypes.POINTER(_Config), ctypes.POINTER(_P)]),
    "gkv_destroy": (None, [_P]),
    "gkv_last_error": (ctypes.c_char_p, [_P]),
    "gkv_bind_layer": (ctypes.c_int, [_P, _I32, _P, _P, _P, _P]),
    "gkv_workspace_size": (ctypes.c_int, [_P, _I32, _I64, ctypes.POINTER(ctypes.c_size_t)]),
    "gkv_bind_workspace": (ctypes.c_int, [_P, _P, ctypes.c_size_t]),
    "gkv_hot_pool_bytes": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_size_t)]),
    "gkv_hot_write": (ctypes.c_int, [_P, _I32, _I32, _I32, _I32, _P, _P, _P]),
    "gkv_hot_pool_alloc": (ctypes.c_int, [_P, _I32, _PI32, ctypes.POINTER(_I64)]),
    "gkv_hot_pool_free": (ctypes.c_int, [_P, _I32]),
    "gkv_hot_prefix_info": (ctypes.c_int, [_P, _I32, ctypes.POINTER(_I64), _PI32]),
    "gkv_cold_pool_alloc": (ctypes.c_int, [_P, _I32, _PI32]),
    "gkv_cold_pool_free": (ctypes.c_int, [_P, _PI32, _I32]),
    "gkv_pool_stats": (ctypes.c_int, [_P, ctypes.POINTER(_Stats)]),
    "gkv_partition_capacity": (ctypes.c_int, [_I64, ctypes.c_double, ctypes.POINTER(_I64), ctypes.POINTER(_I64)]),
    "gkv_prefix_acquire": (ctypes.c_int, [_P, ctypes.c_uint64, _I32, ctypes.POINTER(_PrefixRef)]),
    "gkv_prefix_lookup": (ctypes.c_int, [_P, ctypes.c_uint64, ctypes.POINTER(_PrefixRef)]),
    "gkv_prefix_cold_slots": (ctypes.c_int, [_P, ctypes.c_uint64, _PI32, _I32]),
    "gkv_prefix_release": (ctypes.c_int, [_P, ctypes.c_uint64]),
    "gkv_prefix_evict": (ctypes.c_int, [_P, ctypes.c_uint64]),
    "gkv_prefix_reclaim_cold": (ctypes.c_int, [_P, _I32]),
    "gkv_registry_stats": (ctypes.c_int, [_P, ctypes.POINTER(_RegistryCounts)]),
    "gkv_cold_append": (ctypes.c_int, [_P, _I32, _P, _P, _P, _I32, _P]),
    "gkv_attn_decode": (ctypes.c_int, [_P, _I32, _P, _I32, _PI32, _PI32, _P, _P, _P, _P, _P, _P]),
    "gkv_decode_step": (ctypes.c_int, [_P, _I32, _P, _P, _P, _P, _I32, _PI32, _PI32, _P, _P, _P, _P, _P]),
    "gkv_decode_step_static": (ctypes.c_int, [_P, _I32, _P, _P, _P, _P, _I32, _PI32, _PI32, _P, _P, _P, _P, _P]),
    "gkv_select_backend": (ctypes.c_int, [_P, _I32, _PI32]),
    "gkv_set_dispatch": (ctypes.c_int, [_P, _I32, _I32]),
    "gkv_last_plan": (ctypes.c_int, [_P, ctypes.POINTER(_PlanInfo)]),
    "gkv_plan_step": (ctypes.c_int, [_P, _I32, _PI32, _PI32, ctypes.POINTER(_PlanInfo)]),
    "gkv_step_status": (ctypes.c_int, [_P, _P, _PI32]),
    "gkv_stream_read": (ctypes.c_int, [_P, ctypes.c_size_t, _I32, _P, _P]),
    "gkv_step_trace": (ctypes.c_int, [_P, _P, ctypes.c_size_t]),
    "gkv_set_join_spin_limit": (ctypes.c_int, [_P, _I32]),
    "gkv_kernel_timing": (ctypes.c_int, [_P, _I32]),
    "gkv_kernel_timing_read": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_float), _I32, _PI32]),
}

_lib = None


def load_library(path: str = LIB_PATH):
    """Load libgkv.so (built by ``python -m shared_prefix_paged_contiguous_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m shared_prefix_paged_contiguous_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def partition_capacity(total_tokens: int, f_p: float = 0.2):
    """gkv_partition_capacity: (hot, cold) token capacities of a KV budget."""
    lib = load_library()
    hot, cold = _I64(), _I64()
    rc = lib.gkv_partition_capacity(total_tokens, f_p, ctypes.byref(hot), ctypes.byref(cold))
    if rc != GKV_OK:
        raise GkvError(rc, "partition_capacity: total < 0, f_p outside [0, 1] or COLD above 2^31 - 1 slots")
    return hot.value, cold.value


def stream_read(dev, nbytes: int, workgroups: int, sink_dev, stream=None):
    """gkv_stream_read: a plain streaming read of nbytes at dev (measurement)."""
    rc = load_library().gkv_stream_read(_ptr(dev), nbytes, workgroups, _ptr(sink_dev), _stream(stream))
    if rc != GKV_OK:
        raise GkvError(rc, "stream_read: bad arguments or launch failure")


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


class Context:
    """One gkv_ctx: pools bookkeeping, layer bindings, workspace, dispatcher."""

    def __init__(self, n_q_heads: int, n_kv_heads: int, head_dim: int, dtype: str,
                 hot_capacity_tokens: int, cold_capacity_tokens: int, n_layers: int = 1,
                 m_sat: int = 0, force_backend: int = BACKEND_AUTO, partial_dtype: str = "input"):
        """partial_dtype: element type of the step's partial results before
        their join: "input" (the input dtype, the default), "f32", or "bf16"
        (bf16 inputs only: the same as "input")."""
        self._lib = load_library()
        self.dtype = dtype
        if partial_dtype not in ("input", "f32", "bf16") or (partial_dtype == "bf16" and dtype != "bf16"):
            raise GkvError(GKV_ERR_INVALID, f"partial dtype {partial_dtype!r} with {dtype} inputs")
        self.partial_dtype = "f32" if partial_dtype == "f32" or dtype == "f32" else "bf16"
        cfg = _Config(n_q_heads, n_kv_heads, head_dim, GKV_BF16 if dtype == "bf16" else GKV_F32,
                      n_layers, hot_capacity_tokens, cold_capacity_tokens, m_sat, force_backend,
                      PARTIALS_F32 if partial_dtype == "f32" else PARTIALS_INPUT)
        h = _P()
        rc = self._lib.gkv_create(ctypes.byref(cfg), ctypes.byref(h))
        if rc != GKV_OK:
            raise GkvError(rc, "gkv_create rejected the configuration")
        self._h = h
        self.cfg = cfg

    # ------------------------------------------------------------ lifecycle
    def destroy(self):
        if getattr(self, "_h", None):
            self._lib.gkv_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass

    def _check(self, rc: int, what: str):
        if rc == GKV_OK:
            return
        msg = f"{what}: {self._lib.gkv_last_error(self._h).decode()}"
        if rc == GKV_ERR_NOSPACE:
            raise NoSpace(rc, msg)
        if rc == GKV_ERR_NOTFOUND:
            raise NotFound(rc, msg)
        raise GkvError(rc, msg)

    # ---------------------------------------------------------------- pools
    def hot_pool_alloc(self, n_tokens: int):
        pid, off = ctypes.c_int32(), ctypes.c_int64()
        self._check(self._lib.gkv_hot_pool_alloc(self._h, n_tokens, ctypes.byref(pid), ctypes.byref(off)),
                    "hot_pool_alloc")
        return pid.value, off.value

    def hot_pool_free(self, prefix_id: int):
        self._check(self._lib.gkv_hot_pool_free(self._h, prefix_id), "hot_pool_free")

    def hot_prefix_info(self, prefix_id: int):
        off, n = ctypes.c_int64(), ctypes.c_int32()
        self._check(self._lib.gkv_hot_prefix_info(self._h, prefix_id, ctypes.byref(off), ctypes.byref(n)),
                    "hot_prefix_info")
        return off.value, n.value

    def cold_pool_alloc(self, n: int) -> np.ndarray:
        out = np.empty(max(n, 0), dtype=np.int32)
        self._check(self._lib.gkv_cold_pool_alloc(self._h, n, out.ctypes.data_as(_PI32)), "cold_pool_alloc")
        return out

    def cold_pool_free(self, slots):
        s = _i32(slots)
        self._check(self._lib.gkv_cold_pool_free(self._h, s.ctypes.data_as(_PI32), len(s)), "cold_pool_free")

    def pool_stats(self) -> dict:
        st = _Stats()
        self._check(self._lib.gkv_pool_stats(self._h, ctypes.byref(st)), "pool_stats")
        return {f: getattr(st, f) for f, _ in _Stats._fields_}

    # ------------------------------------------------------------- prefixes
    def prefix_acquire(self, key: int, n_tokens: int) -> dict:
        r = _PrefixRef()
        self._check(self._lib.gkv_prefix_acquire(self._h, key, n_tokens, ctypes.byref(r)), "prefix_acquire")
        return {f: getattr(r, f) for f, _ in _PrefixRef._fields_ if f != "reserved"}

    def prefix_lookup(self, key: int) -> dict:
        r = _PrefixRef()
        self._check(self._lib.gkv_prefix_lookup(self._h, key, ctypes.byref(r)), "prefix_lookup")
        return {f: getattr(r, f) for f, _ in _PrefixRef._fields_ if f != "reserved"}

    def prefix_cold_slots(self, key: int, n_tokens: int) -> np.ndarray:
        out = np.empty(n_tokens, dtype=np.int32)
        self._check(self._lib.gkv_prefix_cold_slots(self._h, key, out.ctypes.data_as(_PI32), n_tokens),
                    "prefix_cold_slots")
        return out

    def prefix_release(self, key: int):
        self._check(self._lib.gkv_prefix_release(self._h, key), "prefix_release")

    def prefix_evict(self, key: int):
        self._check(self._lib.gkv_prefix_evict(self._h, key), "prefix_evict")

    def prefix_reclaim_cold(self, n_free_slots: int):
        self._check(self._lib.gkv_prefix_reclaim_cold(self._h, n_free_slots), "prefix_reclaim_cold")

    def registry_stats(self) -> dict:
        c = _RegistryCounts()
        self._check(self._lib.gkv_registry_stats(self._h, ctypes.byref(c)), "registry_stats")
        return {f: getattr(c, f) for f, _ in _RegistryCounts._fields_}

    # --------------------------------------------------------------- memory
    def bind_layer(self, layer: int, k_hot, v_hot, k_cold, v_cold):
        self._check(self._lib.gkv_bind_layer(self._h, layer, _ptr(k_hot), _ptr(v_hot), _ptr(k_cold),
                                             _ptr(v_cold)), "bind_layer")

    def workspace_size(self, max_batch: int, max_suffix_tokens: int) -> int:
        b = ctypes.c_size_t()
        self._check(self._lib.gkv_workspace_size(self._h, max_batch, max_suffix_tokens, ctypes.byref(b)),
                    "workspace_size")
        return b.value

    def bind_workspace(self, dev, nbytes: Optional[int] = None):
        if nbytes is None:
            nbytes = dev.numel() * dev.element_size()
        self._check(self._lib.gkv_bind_workspace(self._h, _ptr(dev), nbytes), "bind_workspace")

    def hot_pool_bytes(self) -> int:
        b = ctypes.c_size_t()
        self._check(self._lib.gkv_hot_pool_bytes(self._h, ctypes.byref(b)), "hot_pool_bytes")
        return b.value

    # ------------------------------------------------------------- device ops
    def hot_write(self, layer: int, prefix_id: int, token_begin: int, k_rows, v_rows,
                  n: Optional[int] = None, stream=None):
        if n is None:
            n = k_rows.shape[0]
        self._check(self._lib.gkv_hot_write(self._h, layer, prefix_id, token_begin, n, _ptr(k_rows),
                                            _ptr(v_rows), _stream(stream)), "hot_write")

    def cold_append(self, layer: int, k_new, v_new, slots_dev, n: Optional[int] = None, stream=None):
        if n is None:
            n = slots_dev.numel()
        self._check(self._lib.gkv_cold_append(self._h, layer, _ptr(k_new), _ptr(v_new), _ptr(slots_dev), n,
                                              _stream(stream)), "cold_append")

    def attn_decode(self, layer: int, q, hot_prefix_ids, cold_indptr_h, cold_indptr_d, cold_indices_d,
                    out, lse, batch: Optional[int] = None, stream=None) -> int:
        ids = _i32(hot_prefix_ids)
        ind = _i32(cold_indptr_h)
        if batch is None:
            batch = len(ids)
        backend = ctypes.c_int32()
        self._check(self._lib.gkv_attn_decode(
            self._h, layer, _ptr(q), batch, ids.ctypes.data_as(_PI32), ind.ctypes.data_as(_PI32),
            _ptr(cold_indptr_d), _ptr(cold_indices_d), _ptr(out), _ptr(lse), _stream(stream),
            ctypes.byref(backend)), "attn_decode")
        return backend.value

    def decode_step(self, layer: int, q, k_new, v_new, new_slots_dev, hot_prefix_ids, cold_indptr_h,
                    cold_indices_d, out, lse, batch: Optional[int] = None, stream=None) -> int:
        """gkv_decode_step: append request b's new token (k_new[b], v_new[b]) into
        slot new_slots_dev[b], the last entry of its slot table, and attend, in
        one launch."""
        ids = _i32(hot_prefix_ids)
        ind = _i32(cold_indptr_h)
        if batch is None:
            batch = len(ids)
        backend = ctypes.c_int32()
        self._check(self._lib.gkv_decode_step(
            self._h, layer, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(new_slots_dev), batch,
            ids.ctypes.data_as(_PI32), ind.ctypes.data_as(_PI32), _ptr(cold_indices_d), _ptr(out), _ptr(lse),
            _stream(stream), ctypes.byref(backend)), "decode_step")
        return backend.value

    def decode_step_static(self, layer: int, q, k_new, v_new, new_slots_dev, hot_prefix_ids, cold_indptr_h,
                           cold_indices_d, out, lse, batch: Optional[int] = None, stream=None) -> int:
        """gkv_decode_step_static: decode_step with its scratch in the
        library's static device array (no workspace, no allocation)."""
        ids = _i32(hot_prefix_ids)
        ind = _i32(cold_indptr_h)
        if batch is None:
            batch = len(ids)
        backend = ctypes.c_int32()
        self._check(self._lib.gkv_decode_step_static(
            self._h, layer, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(new_slots_dev), batch,
            ids.ctypes.data_as(_PI32), ind.ctypes.data_as(_PI32), _ptr(cold_indices_d), _ptr(out), _ptr(lse),
            _stream(stream), ctypes.byref(backend)), "decode_step_static")
        return backend.value

    # ------------------------------------------------------------ dispatcher
    def select_backend(self, batch: int) -> int:
        b = ctypes.c_int32()
        self._check(self._lib.gkv_select_backend(self._h, batch, ctypes.byref(b)), "select_backend")
        return b.value

    def set_dispatch(self, force_backend: int = BACKEND_AUTO, m_sat: int = 0):
        self._check(self._lib.gkv_set_dispatch(self._h, force_backend, m_sat), "set_dispatch")

    def kernel_timing(self, capacity: int):
        self._check(self._lib.gkv_kernel_timing(self._h, capacity), "kernel_timing")

    def kernel_timing_read(self, max_calls: int) -> np.ndarray:
        """[calls] milliseconds of each recorded call's step kernel."""
        ms = np.zeros(max(max_calls, 1), dtype=np.float32)
        n = ctypes.c_int32()
        self._check(self._lib.gkv_kernel_timing_read(
            self._h, ms.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), max_calls, ctypes.byref(n)),
            "kernel_timing_read")
        return ms[:n.value]

    def step_status(self, stream=None) -> int:
        """gkv_step_status: joins that gave up waiting since the last read
        (synchronises the stream)."""
        n = ctypes.c_int32()
        self._check(self._lib.gkv_step_status(self._h, _stream(stream), ctypes.byref(n)), "step_status")
        return n.value

    def step_trace(self, trace_dev=None, nbytes: Optional[int] = None):
        """gkv_step_trace: per-workgroup timeline records of the following
        steps into trace_dev (a device tensor), or off with None."""
        if trace_dev is not None and nbytes is None:
            nbytes = trace_dev.numel() * trace_dev.element_size()
        self._check(self._lib.gkv_step_trace(self._h, _ptr(trace_dev), nbytes or 0), "step_trace")

    def set_join_spin_limit(self, polls: int):
        self._check(self._lib.gkv_set_join_spin_limit(self._h, polls), "set_join_spin_limit")

    def last_plan(self) -> dict:
        p = _PlanInfo()
        self._check(self._lib.gkv_last_plan(self._h, ctypes.byref(p)), "last_plan")
        return {f: getattr(p, f) for f, _ in _PlanInfo._fields_ if f not in ("pad_", "reserved")}

    def plan_step(self, hot_prefix_ids, cold_indptr_h, batch: Optional[int] = None) -> dict:
        """gkv_plan_step: the plan a step of these requests would use (host only)."""
        ids = _i32(hot_prefix_ids)
        ind = _i32(cold_indptr_h)
        if batch is None:
            batch = len(ids)
        p = _PlanInfo()
        self._check(self._lib.gkv_plan_step(self._h, batch, ids.ctypes.data_as(_PI32), ind.ctypes.data_as(_PI32),
                                            ctypes.byref(p)), "plan_step")
        return {f: getattr(p, f) for f, _ in _PlanInfo._fields_ if f not in ("pad_", "reserved")}


def default_m_sat() -> int:
    return load_library().gkv_default_m_sat()
