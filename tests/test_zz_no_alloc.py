"""The allocation-free decode step (gkv_decode_step_static) against the step
it mirrors (gkv_decode_step): same kernels, same plan, scratch in the
library's static device array instead of a bound workspace.  Compared bit for
bit (out, lse, both COLD pools) on two calls in a row, the second with a
smaller batch, and against the float64 oracle."""

import numpy as np
import pytest
import torch

from shared_prefix_paged_contiguous_amd import binding, workloads
from shared_prefix_paged_contiguous_amd.harness import DecodeState
from tests.gpu_helpers import check, oracle_ref

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _new_tokens(w, st, n):
    """The current tokens (last slot-table entries) of the first n requests."""
    last = torch.from_numpy(w.suffix_offsets[1:n + 1] - 1)
    slots = torch.from_numpy(st.last_slots()[:n]).cuda()
    return w.suffix_k[last].cuda().contiguous(), w.suffix_v[last].cuda().contiguous(), slots


@pytest.mark.parametrize("name", ["llama8b_lp16k_b64", "tiny"])
def test_static_scratch_step_equals_workspace_step(name):
    w = workloads.make(name)
    ref_o, ref_l = oracle_ref(w)
    sa = DecodeState(w)                          # gkv_decode_step with its bound workspace
    sb = DecodeState(w, bind_workspace=False)    # gkv_decode_step_static: no workspace at all
    assert np.array_equal(sa.indices_h, sb.indices_h) and np.array_equal(sa.hot_ids, sb.hot_ids)
    for n in (w.batch, max(1, w.batch // 3)):    # two calls in a row, the second smaller
        k_new, v_new, slots = _new_tokens(w, sa, n)
        out_a, lse_a = sa.new_outputs()
        out_b, lse_b = sb.new_outputs()
        ba = sa.ctx.decode_step(0, sa.q[:n], k_new, v_new, slots, sa.hot_ids[:n], sa.indptr_h[:n + 1],
                                sa.indices_d, out_a[:n], lse_a[:n], batch=n)
        bb = sb.ctx.decode_step_static(0, sb.q[:n], k_new, v_new, slots, sb.hot_ids[:n], sb.indptr_h[:n + 1],
                                       sb.indices_d, out_b[:n], lse_b[:n], batch=n)
        torch.cuda.synchronize()
        assert ba == bb
        assert torch.equal(_bits(out_a[:n]), _bits(out_b[:n]))
        assert torch.equal(lse_a[:n].view(torch.int32), lse_b[:n].view(torch.int32))
        for i in (2, 3):                         # k_cold, v_cold after the in-launch append
            assert torch.equal(_bits(sa.pools[0][i]), _bits(sb.pools[0][i]))
        check(out_b[:n], lse_b[:n], ref_o[:n], ref_l[:n],
              **({} if w.spec.dtype == "bf16" else dict(atol=1e-4, rtol=1e-4, norm_rel=1e-4, lse_abs=1e-4,
                                                        max_abs=1e-4)))
    assert sb.ctx.step_status() == 0


def test_static_scratch_refuses_a_step_that_does_not_fit():
    """A step whose partial results exceed the static scratch is refused on
    the host, before anything is enqueued, with a message naming both sizes."""
    c = binding.Context(32, 8, 128, "bf16", 16384, 2048, partial_dtype="f32")
    pid, _ = c.hot_pool_alloc(16384)
    c.bind_layer(0, 16, 16, 16, 16)   # never dereferenced: the call is refused on the host
    bsz = 1024                        # 1024 requests x 16 splits x 32 heads of fp32 partial rows
    with pytest.raises(binding.GkvError, match="static scratch"):
        c.decode_step_static(0, 16, 16, 16, 16, [pid] * bsz, np.arange(bsz + 1, dtype=np.int32), 16, 16, 16,
                             batch=bsz)
