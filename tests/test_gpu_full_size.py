"""GPU parity at the workloads' full sizes, on every request.

The four large workloads (Llama-3.1-8B shape with a 16K prefix and 64
requests; the Qwen-2.5-14B TP=2 slice with 128 requests; eight heterogeneous
prefixes; the Qwen-2.5-32B TP=4 slice with a 1K prefix and 256 requests) run
through the C ABI in the launch configuration the benchmark uses (AUTO
dispatch), then with the other prefix backend forced, each with fp32 and with
bf16 partial results, and every output row is compared with the float64
oracle.  The fused call the benchmark times (gkv_decode_step at the Llama
shape) is compared the same way, and the rows it appends are compared bit for
bit.  Each run prints one PARITY line with its error statistics (pytest -s).
"""

import json

import numpy as np
import pytest
import torch

from shared_prefix_paged_contiguous_amd import binding, workloads
from shared_prefix_paged_contiguous_amd.harness import DecodeState
from tests.gpu_helpers import check, oracle_ref

pytestmark = pytest.mark.gpu

CASCADE, DENSE, AUTO = binding.BACKEND_CASCADE, binding.BACKEND_DENSE, binding.BACKEND_AUTO
FULL = ["llama8b_lp16k_b64", "qwen14b_tp2_lp16k_b128", "hetero8", "qwen32b_tp4_lp1k_b256"]

_cache = {}


def full_ref(name):
    """The workload and its oracle output on every request (one workload kept
    at a time: the largest holds about a gigabyte of inputs)."""
    if name not in _cache:
        _cache.clear()
        w = workloads.make(name)
        _cache[name] = (w, oracle_ref(w))
    return _cache[name]


def _report(**kw):
    print("PARITY " + json.dumps(kw), flush=True)


@pytest.mark.parametrize("partials", ["f32", "bf16"])
@pytest.mark.parametrize("name", FULL)
def test_full_size_all_requests(name, partials):
    w, (ref_o, ref_l) = full_ref(name)
    st = DecodeState(w, partial_dtype=partials)
    out, lse = st.new_outputs()
    auto = st.run(out, lse)
    torch.cuda.synchronize()
    plan = st.ctx.last_plan()
    stats = check(out, lse, ref_o, ref_l)
    _report(workload=name, partials=partials, backend=binding.BACKEND_NAMES[auto], dispatch="auto",
            folded=plan["folded_parts"], prefix_blocks=plan["n_prefix_blocks"],
            suffix_blocks=plan["n_suffix_blocks"], requests=w.batch, **stats)
    other = DENSE if auto == CASCADE else CASCADE
    st.ctx.set_dispatch(other)
    out2, lse2 = st.new_outputs()
    assert st.run(out2, lse2) == other
    torch.cuda.synchronize()
    stats = check(out2, lse2, ref_o, ref_l)
    _report(workload=name, partials=partials, backend=binding.BACKEND_NAMES[other], dispatch="forced",
            requests=w.batch, **stats)
    # no join of either step stopped waiting for its partials
    assert st.ctx.step_status() == 0


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_fused_step_at_the_bench_workload_all_requests():
    """gkv_decode_step at the Llama-3.1-8B shape (16K prefix, 64 requests),
    the call the benchmark times: cascade prefix, folded suffix pairs, the new
    tokens read from their input rows and appended inside the launch.  The
    new tokens' COLD rows are cleared first, so the appended rows must come
    from the step; the whole pools must then equal the original ones bit for
    bit, and every output row must match the oracle, on two calls in a row."""
    w, (ref_o, ref_l) = full_ref("llama8b_lp16k_b64")
    st = DecodeState(w)
    slots = torch.from_numpy(st.last_slots()).cuda()
    last = torch.from_numpy(w.suffix_offsets[1:] - 1)
    k_new = w.suffix_k[last].cuda().contiguous()
    v_new = w.suffix_v[last].cuda().contiguous()
    k_cold, v_cold = st.pools[0][2], st.pools[0][3]
    want_k, want_v = k_cold.clone(), v_cold.clone()   # the new tokens' rows are already in place
    k_cold[slots.long()] = 0
    v_cold[slots.long()] = 0
    torch.cuda.synchronize()
    assert not torch.equal(_bits(k_cold), _bits(want_k))
    for call in range(2):
        out, lse = st.new_outputs()
        backend = st.step(out, lse, k_new, v_new, slots)
        torch.cuda.synchronize()
        plan = st.ctx.last_plan()
        assert backend == CASCADE and plan["folded_parts"] == 1
        assert torch.equal(_bits(k_cold), _bits(want_k))
        assert torch.equal(_bits(v_cold), _bits(want_v))
        stats = check(out, lse, ref_o, ref_l)
        _report(workload="llama8b_lp16k_b64", call="gkv_decode_step", repeat=call, requests=w.batch, **stats)
    assert st.ctx.step_status() == 0
