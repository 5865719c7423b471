"""GPU parity of decode steps whose prefixes were admitted through the
library's prefix registry (gkv_prefix_acquire: HOT first, COLD fallback, no
demotion), and of steps with many distinct HOT prefixes, against the float64
oracle on the logical context."""

import pytest
import torch

from shared_prefix_paged_contiguous_amd import binding, workloads
from shared_prefix_paged_contiguous_amd.harness import DecodeState
from tests.gpu_helpers import check, oracle_ref

pytestmark = pytest.mark.gpu

CASCADE, DENSE = binding.BACKEND_CASCADE, binding.BACKEND_DENSE


def multi_spec(**kw):
    base = dict(name="reg", n_q=32, n_kv=8, head_dim=128, dtype="bf16", batch=0, prefix_len=0,
                suffix_lo=1, suffix_hi=80, hot_capacity=2048, cold_capacity=16384, n_prefixes=6,
                prefix_len_lo=200, prefix_len_hi=900, class_lo=1, class_hi=3)
    base.update(kw)
    return workloads.Spec(**base)


def run_registry(w, force):
    st = DecodeState(w, force_backend=force, registry=True)
    out, lse = st.new_outputs()
    st.run(out, lse)
    torch.cuda.synchronize()
    return st, out, lse


@pytest.mark.parametrize("force", [CASCADE, DENSE])
def test_registry_placement_with_cold_fallback_matches_oracle(force):
    w = workloads.make(multi_spec())
    st, out, lse = run_registry(w, force)
    pl = st.placement
    hot = [p for p in range(len(w.prefix_lens)) if pl["prefix_id"][p] >= 0]
    cold = sorted(pl["prefix_slots"])
    assert hot and cold and len(hot) + len(cold) == len(w.prefix_lens)
    rs = st.ctx.registry_stats()
    assert (rs["hot_admits"], rs["cold_admits"], rs["referenced"]) == (len(hot), len(cold), len(w.prefix_lens))
    ref_out, ref_lse = oracle_ref(w)
    check(out, lse, ref_out, ref_lse)


@pytest.mark.parametrize("n_prefixes,force", [(48, CASCADE), (64, CASCADE), (64, DENSE)])
def test_many_hot_classes_in_one_step_match_oracle(n_prefixes, force):
    w = workloads.make(multi_spec(n_prefixes=n_prefixes, prefix_len_lo=32, prefix_len_hi=160, class_lo=1,
                                  class_hi=2, hot_capacity=n_prefixes * 160, suffix_hi=40))
    st, out, lse = run_registry(w, force)
    assert st.ctx.last_plan()["n_classes"] == n_prefixes
    ref_out, ref_lse = oracle_ref(w)
    check(out, lse, ref_out, ref_lse)
