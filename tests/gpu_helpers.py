"""Shared helpers of the GPU parity tests: oracle references on the logical
workload, the tolerance gate, and diagnostics."""

from __future__ import annotations

import numpy as np
import torch

from oracle.attention import decode_step

# The gate: elementwise |x - r| <= ATOL + RTOL * |r| on out and lse (bf16
# inputs, fp32 accumulation, bf16 output), and on its own max |out - ref| <=
# MAX_ABS (the stated bound on the absolute error).
ATOL, RTOL = 1e-2, 2e-2
MAX_ABS = 1e-2
# Diagnostics held as well (the gate alone is weak when outputs are ~1e-2).
NORM_REL_MAX = 1e-2       # ||out - ref||_2 / ||ref||_2
LSE_ABS_MAX = 1e-3


def f64(t) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def oracle_ref(w, requests=None):
    sk = [f64(w.suffix_rows(b)[0]) for b in range(w.batch)]
    sv = [f64(w.suffix_rows(b)[1]) for b in range(w.batch)]
    pk = [f64(x) for x in w.prefix_k]
    pv = [f64(x) for x in w.prefix_v]
    return decode_step(f64(w.q), pk, pv, w.request_prefix, sk, sv, requests=requests)


def check(out, lse, ref_out, ref_lse, requests=None, atol=ATOL, rtol=RTOL,
          norm_rel=NORM_REL_MAX, lse_abs=LSE_ABS_MAX, max_abs=MAX_ABS):
    o = f64(out)
    l = f64(lse)
    if requests is not None:
        o, l, ref_out, ref_lse = o[requests], l[requests], ref_out[requests], ref_lse[requests]
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l)), "non-finite output"
    err_o = np.abs(o - ref_out)
    err_l = np.abs(l - ref_lse)
    bad_o = err_o > atol + rtol * np.abs(ref_out)
    bad_l = err_l > atol + rtol * np.abs(ref_lse)
    stats = {
        "max_abs_out": float(err_o.max()),
        "max_abs_lse": float(err_l.max()),
        "norm_rel_out": float(np.linalg.norm(o - ref_out) / np.linalg.norm(ref_out)),
        "max_rel_out_big": float((err_o / np.abs(ref_out))[np.abs(ref_out) >= 1e-3].max()),
    }
    assert not bad_o.any(), f"out outside the gate at {np.argwhere(bad_o)[:5].tolist()} {stats}"
    assert not bad_l.any(), f"lse outside the gate at {np.argwhere(bad_l)[:5].tolist()} {stats}"
    assert stats["max_abs_out"] <= max_abs, stats
    assert stats["norm_rel_out"] <= norm_rel, stats
    assert stats["max_abs_lse"] <= lse_abs, stats
    return stats
