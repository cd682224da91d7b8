"""Softmax attention, per-stripe partials, the exact LSE merge and own-token attention, in float64 numpy.

TEST INFRASTRUCTURE (see the package docstring): only tests, the smoke check and the CPU baseline use it.

Sources:
* mstar PR #1124, "Context / Sequence Parallel 1/5: split the KV cache by position across GPUs (DCP)", PR
  description: each rank attends the slots it holds and returns its partial output together with the partial's
  log-sum-exp; the partials are then merged exactly; a step with more than one token in a row also attends the row's
  own in-step tokens, taken from the K/V the layer hands over, and that result is merged in as well. The review
  thread on the padding test adds that padding tokens must come out as zero and must never influence a real row.
* vLLM compare view "[Core] Add explicit layer parallel plans", ``FlashAttentionImpl._forward_with_dcp``: context
  attention over the paged cache returns (out, lse); the own-token call uses the query offsets as key offsets; the
  two are merged by their LSEs; with no context anywhere only the own-token call runs.

Definitions used (plain softmax attention, natural log):
    s_j = scale * <q, k_j>;  lse = log sum_j exp(s_j);  out = sum_j exp(s_j - lse) * v_j
An empty key set gives out = 0 and lse = -inf. The merge of partials (o_i, lse_i) is
    lse = log sum_i exp(lse_i);  out = sum_i exp(lse_i - lse) * o_i,
with out = 0, lse = -inf when every lse_i is -inf.

Readings where the pages are silent: the GQA head group of query head h is kv head h // (Hq / Hkv); the own-token
mask is causal (in-step query i sees in-step keys 0..i) while the prior context is visible to every in-step query;
in the decode workloads the query attends every context token in the pool.
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def _f64(x):
    if hasattr(x, "detach"):          # torch tensor (any dtype, any device)
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def attention(q, k, v, scale: float, visible=None):
    """Softmax attention of queries over one key set.

    q [m, D], k [n, D], v [n, Dv]; ``visible`` is an optional bool [m, n] mask (True = key j is in query i's set).
    Returns out [m, Dv] and lse [m] (natural log). A query with no visible key gets out 0 and lse -inf.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    m, n, dv = q.shape[0], k.shape[0], v.shape[1]
    out = np.zeros((m, dv), dtype=np.float64)
    lse = np.full((m,), NEG_INF, dtype=np.float64)
    if m == 0 or n == 0:
        return out, lse
    s = scale * (q @ k.T)                                    # [m, n]
    if visible is not None:
        s = np.where(np.asarray(visible, dtype=bool), s, NEG_INF)
    mx = s.max(axis=1)
    live = np.isfinite(mx)
    if not live.any():
        return out, lse
    sl = s[live]
    e = np.exp(sl - mx[live][:, None])                       # exp(-inf) = 0 for masked keys
    tot = e.sum(axis=1)
    lse[live] = mx[live] + np.log(tot)
    out[live] = (e / tot[:, None]) @ v
    return out, lse


def gqa_attention(q, k, v, scale: float, visible=None):
    """Grouped-query attention: q [m, Hq, D], k [n, Hkv, D], v [n, Hkv, Dv] -> out [m, Hq, Dv], lse [m, Hq].

    Query head h reads kv head h // (Hq // Hkv). ``visible`` [m, n] applies to every head.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    m, hq = q.shape[0], q.shape[1]
    hkv = k.shape[1]
    if hq % hkv:
        raise ValueError(f"Hq={hq} is not a multiple of Hkv={hkv}")
    g = hq // hkv
    out = np.zeros((m, hq, v.shape[2]), dtype=np.float64)
    lse = np.full((m, hq), NEG_INF, dtype=np.float64)
    for h in range(hq):
        o, l = attention(q[:, h], k[:, h // g], v[:, h // g], scale, visible)
        out[:, h], lse[:, h] = o, l
    return out, lse


def stripe_partial(q, k_ctx, v_ctx, P: int, r: int, scale: float, interleave: int = 1):
    """Partner r's partial: attention of every query over the context positions t with floor(t / I) mod P == r
    (I = interleave; I = 1 is the PR's t mod P == r).

    q [m, Hq, D]; k_ctx [c, Hkv, D], v_ctx [c, Hkv, Dv] are the row's logical (unstriped) context.
    Returns out [m, Hq, Dv], lse [m, Hq]; an empty stripe gives (0, -inf).
    """
    k_ctx, v_ctx = _f64(k_ctx), _f64(v_ctx)
    keep = np.array([(t // interleave) % P == r for t in range(k_ctx.shape[0])], dtype=bool)
    return gqa_attention(q, k_ctx[keep], v_ctx[keep], scale)


def merge(outs, lses):
    """Exact merge of partials: outs is a list of [..., Dv], lses a list of [...] (natural-log LSEs)."""
    outs = [_f64(o) for o in outs]
    lses = [_f64(l) for l in lses]
    if not outs:
        raise ValueError("merge needs at least one partial")
    L = np.stack(lses)                                       # [N, ...]
    mx = L.max(axis=0)
    live = np.isfinite(mx)
    safe_mx = np.where(live, mx, 0.0)
    w = np.exp(L - safe_mx)                                  # exp(-inf) = 0: empty partials weigh nothing
    tot = w.sum(axis=0)
    lse = np.where(live, safe_mx + np.log(np.where(live, tot, 1.0)), NEG_INF)
    scale = np.where(live, 1.0 / np.where(live, tot, 1.0), 0.0)
    out = np.zeros_like(outs[0])
    for i, o in enumerate(outs):
        out = out + (w[i] * scale)[..., None] * o
    return out, lse


def own_token_partial(q, k_new, v_new, scale: float):
    """Own-token attention of one row's in-step queries over its in-step keys, causal (query i sees keys 0..i)."""
    n = _f64(q).shape[0]
    vis = np.tril(np.ones((n, n), dtype=bool))
    return gqa_attention(q, k_new, v_new, scale, visible=vis)


def row_attention(q, k_ctx, v_ctx, scale: float, k_new=None, v_new=None):
    """The whole row as plain attention over the unstriped logical KV.

    Every in-step query sees every context token; with own-token K/V it also sees its row's in-step keys 0..i.
    """
    q = _f64(q)
    n = q.shape[0]
    k_ctx, v_ctx = _f64(k_ctx), _f64(v_ctx)
    c = k_ctx.shape[0]
    if k_new is None:
        return gqa_attention(q, k_ctx, v_ctx, scale)
    k_all = np.concatenate([k_ctx, _f64(k_new)], axis=0)
    v_all = np.concatenate([v_ctx, _f64(v_new)], axis=0)
    vis = np.concatenate([np.ones((n, c), dtype=bool), np.tril(np.ones((n, n), dtype=bool))], axis=1)
    return gqa_attention(q, k_all, v_all, scale, visible=vis)


def row_partials(q, k_ctx, v_ctx, P: int, scale: float, k_new=None, v_new=None, interleave: int = 1):
    """The method's steps for one row: P stripe partials (plus the own-token partial), then the exact merge.

    Returns (partials, (out, lse)) where partials is a list of (out, lse) pairs in stripe order, the own-token
    partial last when present.
    """
    parts = [stripe_partial(q, k_ctx, v_ctx, P, r, scale, interleave) for r in range(P)]
    if k_new is not None:
        parts.append(own_token_partial(q, k_new, v_new, scale))
    merged = merge([p[0] for p in parts], [p[1] for p in parts])
    return parts, merged
