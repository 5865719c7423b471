"""Float64 softmax attention over the logical context (TEST INFRASTRUCTURE).

What the decode step computes, per the GraniKV paperlayer.ai summary (§2
Related Work, "Prefix–suffix attention"): both shared-prefix methods split the
attention of a decode query into a shared-prefix part and a per-request
suffix part and join the two partial softmaxes with a log-sum-exp merge.  The
merge is exact, so the result is ordinary softmax attention over the whole
context "prefix tokens, then suffix tokens".  This module writes that plain
definition out; it does not split or merge anything (``merge`` exists only so
tests can check the invariant).

Readings where the pages are silent:
* scale 1/sqrt(d);
* grouped-query attention maps query head h to KV head floor(h / G) with
  G = n_q / n_kv (contiguous groups);
* lse is the natural log of the sum of exp(scaled score);
* the context of request b is its HOT prefix (if any) followed by its suffix
  tokens in slot-table order; the current token is already in the suffix.
"""

from __future__ import annotations

import math

import numpy as np


def softmax_scale(head_dim: int) -> float:
    """1/sqrt(d): the pages give no scale; this is the Llama/Qwen convention."""
    return 1.0 / math.sqrt(head_dim)


def attend(q, k, v):
    """Softmax attention of one request's query heads over one token sequence.

    q: [n_q, d]; k, v: [N, n_kv, d] with N >= 1.  Returns (out [n_q, d],
    lse [n_q]) in float64.  For query head h with g = h // (n_q // n_kv):
    s_j = q[h] . k[j, g] / sqrt(d),  out[h] = sum_j softmax(s)_j v[j, g],
    lse[h] = log sum_j exp(s_j).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n_q, d = q.shape
    n_tok, n_kv, d_k = k.shape
    if n_tok < 1:
        raise ValueError("attention over an empty context is undefined")
    if d_k != d or v.shape != k.shape or n_q % n_kv != 0:
        raise ValueError("shape mismatch")
    group = n_q // n_kv
    scale = softmax_scale(d)
    out = np.empty((n_q, d), dtype=np.float64)
    lse = np.empty(n_q, dtype=np.float64)
    for g in range(n_kv):
        heads = slice(g * group, (g + 1) * group)
        s = (q[heads] @ k[:, g, :].T) * scale          # [G, N]
        m = s.max(axis=1, keepdims=True)
        w = np.exp(s - m)
        l = w.sum(axis=1, keepdims=True)
        out[heads] = (w @ v[:, g, :]) / l
        lse[heads] = (m + np.log(l))[:, 0]
    return out, lse


def decode_step(q, prefix_k, prefix_v, prefix_of, suffix_k, suffix_v, requests=None):
    """One decode step over a batch, on logical sequences.

    q:         [B, n_q, d]
    prefix_k/v: dict or list, prefix index -> [L, n_kv, d]
    prefix_of: [B] prefix index of each request, or -1 for "no HOT prefix"
               (the paged fallback of Appendix B.10: then the whole context is
               the suffix)
    suffix_k/v: list of [S_b, n_kv, d] (S_b may be 0)
    requests:  optional iterable of request indices to evaluate (sampling at
               large sizes); default all.
    Returns (out [B, n_q, d], lse [B, n_q]) float64; rows not requested are NaN.
    """
    q = np.asarray(q)
    n_b, n_q, d = q.shape
    out = np.full((n_b, n_q, d), np.nan)
    lse = np.full((n_b, n_q), np.nan)
    for b in (range(n_b) if requests is None else requests):
        parts_k, parts_v = [], []
        p = int(prefix_of[b])
        if p >= 0:
            parts_k.append(np.asarray(prefix_k[p], dtype=np.float64))
            parts_v.append(np.asarray(prefix_v[p], dtype=np.float64))
        if len(suffix_k[b]):
            parts_k.append(np.asarray(suffix_k[b], dtype=np.float64))
            parts_v.append(np.asarray(suffix_v[b], dtype=np.float64))
        if not parts_k:
            raise ValueError(f"request {b} has neither a prefix nor a suffix")
        k = parts_k[0] if len(parts_k) == 1 else np.concatenate(parts_k, axis=0)
        v = parts_v[0] if len(parts_v) == 1 else np.concatenate(parts_v, axis=0)
        out[b], lse[b] = attend(q[b], k, v)
    return out, lse


def merge(o1, lse1, o2, lse2):
    """Log-sum-exp join of two partial softmax results over disjoint token sets.

    With lse = log sum exp(scores) of each part and o the part's normalised
    output: lse = log(exp(lse1) + exp(lse2)) and
    o = (exp(lse1 - lse) o1 + exp(lse2 - lse) o2).  A part with lse = -inf
    (no tokens) has weight 0.
    """
    o1 = np.asarray(o1, dtype=np.float64)
    o2 = np.asarray(o2, dtype=np.float64)
    lse1 = np.asarray(lse1, dtype=np.float64)
    lse2 = np.asarray(lse2, dtype=np.float64)
    m = np.maximum(lse1, lse2)
    w1 = np.where(np.isneginf(lse1), 0.0, np.exp(lse1 - m))
    w2 = np.where(np.isneginf(lse2), 0.0, np.exp(lse2 - m))
    tot = w1 + w2
    lse = m + np.log(tot)
    o = (w1[..., None] * np.where(np.isneginf(lse1)[..., None], 0.0, o1)
         + w2[..., None] * np.where(np.isneginf(lse2)[..., None], 0.0, o2)) / tot[..., None]
    return o, lse
