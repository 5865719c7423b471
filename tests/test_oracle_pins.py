"""Pins for the float64 attention oracle, against things other than itself.

* closed forms of softmax attention (one token; zero query; equal keys;
  constant values);
* a pure-Python brute force (no numpy) on tiny inputs;
* torch's CPU float64 scaled_dot_product_attention with KV heads repeated per
  group (a library routine that computes the same definition) and
  torch.logsumexp for lse;
* the log-sum-exp merge invariant from the GraniKV pages (paperlayer.ai
  summary §2, "Prefix–suffix attention"): prefix part and suffix part merged
  by log-sum-exp equal attention over prefix || suffix.

Each pin is a function of the attention callable, and the last tests plant
plausible mistakes (wrong scale, wrong GQA mapping, swapped K/V, a dropped
max subtraction with large scores, a wrong merge sign) in copies of the oracle
to show that some pin fails for each.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import attend, decode_step, merge

TOL = 1e-12


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ----------------------------------------------------------------- pin checks
def pin_single_token(fn, rng):
    n_q, n_kv, d = 8, 2, 16
    q, k, v = _rand(rng, n_q, d), _rand(rng, 1, n_kv, d), _rand(rng, 1, n_kv, d)
    out, lse = fn(q, k, v)
    g = np.arange(n_q) // (n_q // n_kv)
    exp_out = v[0, g, :]
    exp_lse = np.einsum("hd,hd->h", q, k[0, g, :]) / math.sqrt(d)
    return max(np.abs(out - exp_out).max(), np.abs(lse - exp_lse).max())


def pin_zero_query(fn, rng):
    n_q, n_kv, d, n = 6, 3, 8, 37
    q = np.zeros((n_q, d))
    k, v = _rand(rng, n, n_kv, d), _rand(rng, n, n_kv, d)
    out, lse = fn(q, k, v)
    g = np.arange(n_q) // (n_q // n_kv)
    exp_out = v.mean(axis=0)[g]
    return max(np.abs(out - exp_out).max(), np.abs(lse - math.log(n)).max())


def pin_equal_keys(fn, rng):
    n_q, n_kv, d, n = 4, 1, 32, 11
    q = _rand(rng, n_q, d)
    k = np.repeat(_rand(rng, 1, n_kv, d), n, axis=0)
    v = _rand(rng, n, n_kv, d)
    out, lse = fn(q, k, v)
    s = q @ k[0, 0] / math.sqrt(d)
    return max(np.abs(out - v[:, 0, :].mean(axis=0)).max(),
               np.abs(lse - (s + math.log(n))).max())


def pin_constant_values(fn, rng):
    n_q, n_kv, d, n = 4, 2, 8, 19
    q, k = _rand(rng, n_q, d) * 3.0, _rand(rng, n, n_kv, d)
    c = _rand(rng, n_kv, d)
    v = np.broadcast_to(c, (n, n_kv, d)).copy()
    out, _ = fn(q, k, v)
    g = np.arange(n_q) // (n_q // n_kv)
    return np.abs(out - c[g]).max()


def brute_force(q, k, v):
    """Pure-Python loops, no numpy arithmetic."""
    q, k, v = q.tolist(), k.tolist(), v.tolist()
    n_q, d = len(q), len(q[0])
    n, n_kv = len(k), len(k[0])
    group = n_q // n_kv
    out, lse = [], []
    for h in range(n_q):
        g = h // group
        s = [sum(q[h][i] * k[j][g][i] for i in range(d)) / math.sqrt(d) for j in range(n)]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        tot = math.fsum(e)
        out.append([math.fsum(e[j] * v[j][g][i] for j in range(n)) / tot for i in range(d)])
        lse.append(m + math.log(tot))
    return np.array(out), np.array(lse)


def pin_brute_force(fn, rng, n_q=8, n_kv=2, d=16, n=40):
    q, k, v = _rand(rng, n_q, d), _rand(rng, n, n_kv, d), _rand(rng, n, n_kv, d)
    out, lse = fn(q, k, v)
    bo, bl = brute_force(q, k, v)
    return max(np.abs(out - bo).max(), np.abs(lse - bl).max())


def pin_sdpa(fn, rng, n_q=12, n_kv=3, d=32, n=300):
    q, k, v = _rand(rng, n_q, d), _rand(rng, n, n_kv, d), _rand(rng, n, n_kv, d)
    out, lse = fn(q, k, v)
    group = n_q // n_kv
    tq = torch.from_numpy(q)[:, None, :]                                  # [H, 1, d]
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(group, 0)  # [H, N, d]
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(group, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk.contiguous(), tv.contiguous())
    scores = torch.matmul(tq, tk.transpose(1, 2).contiguous()) * (1.0 / math.sqrt(d))
    ref_lse = torch.logsumexp(scores[:, 0, :], dim=-1)
    return max(np.abs(out - ref[:, 0, :].numpy()).max(), np.abs(lse - ref_lse.numpy()).max())


def pin_merge_invariant(fn, merge_fn, rng, n_q=8, n_kv=2, d=16, n1=50, n2=23):
    q = _rand(rng, n_q, d)
    k1, v1 = _rand(rng, n1, n_kv, d), _rand(rng, n1, n_kv, d)
    k2, v2 = _rand(rng, n2, n_kv, d), _rand(rng, n2, n_kv, d)
    o1, l1 = fn(q, k1, v1)
    o2, l2 = fn(q, k2, v2)
    om, lm = merge_fn(o1, l1, o2, l2)
    oc, lc = fn(q, np.concatenate([k1, k2]), np.concatenate([v1, v2]))
    return max(np.abs(om - oc).max(), np.abs(lm - lc).max())


def pin_large_scores(fn, rng):
    """Scores of several hundred: the exact result is finite and the lse is
    the max score plus the log of a small sum."""
    n_q, n_kv, d, n = 2, 1, 4, 3
    q = np.full((n_q, d), 20.0)
    k = np.zeros((n, n_kv, d))
    k[0, 0, :] = 20.0                     # score 20*20*4/2 = 800
    k[1, 0, :] = 19.0                     # score 760
    v = _rand(rng, n, n_kv, d)
    out, lse = fn(q, k, v)
    s = np.array([800.0, 760.0, 0.0])
    w = np.exp(s - 800.0)
    exp_out = (w[:, None] * v[:, 0, :]).sum(0) / w.sum()
    return max(np.abs(out - exp_out).max(), np.abs(lse - (800.0 + math.log(w.sum()))).max())


ALL_PINS = [pin_single_token, pin_zero_query, pin_equal_keys, pin_constant_values,
            pin_brute_force, pin_sdpa, pin_large_scores]


# --------------------------------------------------------------------- tests
@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_passes_pin(pin):
    assert pin(attend, np.random.default_rng(1)) <= TOL


def test_brute_force_shapes_of_tiny_config():
    # the tiny step's shape (8 q / 2 kv heads, d=64) at a context the loops finish quickly
    assert pin_brute_force(attend, np.random.default_rng(2), n_q=8, n_kv=2, d=64, n=96) <= TOL


def test_sdpa_llama_group():
    assert pin_sdpa(attend, np.random.default_rng(3), n_q=32, n_kv=8, d=128, n=700) <= TOL


def test_merge_invariant():
    rng = np.random.default_rng(4)
    for _ in range(5):
        assert pin_merge_invariant(attend, merge, rng) <= TOL


def test_merge_empty_part_has_zero_weight():
    rng = np.random.default_rng(5)
    o = rng.standard_normal((3, 8))
    lse = rng.standard_normal(3)
    neg = np.full(3, -np.inf)
    om, lm = merge(o, lse, np.full((3, 8), np.nan), neg)
    assert np.array_equal(om, o) and np.array_equal(lm, lse)
    om, lm = merge(np.full((3, 8), np.nan), neg, o, lse)
    assert np.array_equal(om, o) and np.array_equal(lm, lse)


def test_decode_step_matches_per_request_attention():
    """decode_step = attend over prefix || suffix per request, -1 = suffix only,
    S_b = 0 = prefix only, and both empty is rejected."""
    rng = np.random.default_rng(6)
    n_q, n_kv, d = 4, 2, 8
    pk = {0: rng.standard_normal((30, n_kv, d)), 1: rng.standard_normal((7, n_kv, d))}
    pv = {0: rng.standard_normal((30, n_kv, d)), 1: rng.standard_normal((7, n_kv, d))}
    prefix_of = [0, 1, -1, 0]
    sl = [5, 0, 9, 1]
    sk = [rng.standard_normal((s, n_kv, d)) for s in sl]
    sv = [rng.standard_normal((s, n_kv, d)) for s in sl]
    q = rng.standard_normal((4, n_q, d))
    out, lse = decode_step(q, pk, pv, prefix_of, sk, sv)
    for b in range(4):
        ks = ([pk[prefix_of[b]]] if prefix_of[b] >= 0 else []) + ([sk[b]] if sl[b] else [])
        vs = ([pv[prefix_of[b]]] if prefix_of[b] >= 0 else []) + ([sv[b]] if sl[b] else [])
        bo, bl = brute_force(q[b], np.concatenate(ks), np.concatenate(vs))
        assert np.abs(out[b] - bo).max() <= TOL and np.abs(lse[b] - bl).max() <= TOL
    with pytest.raises(ValueError):
        decode_step(q[:1], pk, pv, [-1], [np.zeros((0, n_kv, d))], [np.zeros((0, n_kv, d))])


def test_decode_step_storage_independent():
    """Serving a prefix from its own rows or inlined at the front of the
    suffix (the COLD fallback of Appendix B.10) gives the same result."""
    rng = np.random.default_rng(7)
    n_q, n_kv, d = 6, 3, 8
    pk, pv = rng.standard_normal((20, n_kv, d)), rng.standard_normal((20, n_kv, d))
    sk, sv = rng.standard_normal((5, n_kv, d)), rng.standard_normal((5, n_kv, d))
    q = rng.standard_normal((1, n_q, d))
    a = decode_step(q, [pk], [pv], [0], [sk], [sv])
    b = decode_step(q, [pk], [pv], [-1], [np.concatenate([pk, sk])], [np.concatenate([pv, sv])])
    assert np.abs(a[0] - b[0]).max() <= TOL and np.abs(a[1] - b[1]).max() <= TOL


# ------------------------------------------------------ planted mistakes fail
def _mut_scale(q, k, v):
    return attend(q * math.sqrt(q.shape[1]) / q.shape[1], k, v)   # 1/d instead of 1/sqrt(d)


def _mut_gqa(q, k, v):
    # head h -> KV head h % n_kv (interleaved groups instead of contiguous)
    n_q, n_kv = q.shape[0], k.shape[1]
    g = n_q // n_kv
    order = np.array([(h % n_kv) * g + h // n_kv for h in range(n_q)])
    inv = np.argsort(order)
    o, l = attend(q[inv], k, v)
    return o[order], l[order]


def _mut_swap_kv(q, k, v):
    return attend(q, v, k)


def _mut_no_max(q, k, v):
    # softmax without subtracting the max: overflows for large scores
    q = np.asarray(q, float); k = np.asarray(k, float); v = np.asarray(v, float)
    n_q, d = q.shape
    g = n_q // k.shape[1]
    out = np.empty((n_q, d)); lse = np.empty(n_q)
    with np.errstate(over="ignore", invalid="ignore"):
        for h in range(n_q):
            s = k[:, h // g, :] @ q[h] / math.sqrt(d)
            w = np.exp(s)
            out[h] = w @ v[:, h // g, :] / w.sum()
            lse[h] = math.log(w.sum()) if np.isfinite(w.sum()) else np.inf
    return out, lse


def _mut_lse_log2(q, k, v):
    o, l = attend(q, k, v)
    return o, l / math.log(2.0)


def _mut_merge_sign(o1, l1, o2, l2):
    m = np.maximum(l1, l2)
    w1, w2 = np.exp(l1 - m), np.exp(m - l2)      # sign slip in one weight
    return (w1[:, None] * o1 + w2[:, None] * o2) / (w1 + w2)[:, None], m + np.log(w1 + w2)


@pytest.mark.parametrize("mutant", [_mut_scale, _mut_gqa, _mut_swap_kv, _mut_no_max, _mut_lse_log2],
                         ids=lambda f: f.__name__)
def test_planted_mistake_is_caught(mutant):
    rng = np.random.default_rng(8)
    worst = 0.0
    for pin in ALL_PINS:
        with np.errstate(all="ignore"):
            e = pin(mutant, np.random.default_rng(9))
        worst = max(worst, e if np.isfinite(e) else np.inf)
    assert worst > 1e-6, "no pin noticed the planted mistake"
    del rng


def test_planted_merge_mistake_is_caught():
    assert pin_merge_invariant(attend, _mut_merge_sign, np.random.default_rng(10)) > 1e-6


def test_oracle_package_exports():
    assert oracle.softmax_scale(128) == 1.0 / math.sqrt(128)
