"""Gradients of exact attention: the plain chain rule through the softmax.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py for who may import it).

The cost guide notes that training keeps a score table per layer for the
backward pass, and that FlashAttention keeps only a few statistics per row
instead [cost-guide, "eager 어텐션 메모리, 길이에 따라 얼마나 커지나",
the paragraphs after the memory table]; its speed figures are training
figures [same page, "긴 입력에서 어텐션 연산이 차지하는 비중"].  The
gradients themselves are not printed on the pages; they follow from the
forward definition in ``oracle.reference`` by differentiation.  For one
query row i of head h (KV head h // G), with s_ij = scale <q_i, k_j> over the
visible keys, p_ij = softmax_j(s_ij), out_i = sum_j p_ij v_j, and an upstream
gradient dout_i of the loss with respect to out_i:

  dv_j  += p_ij dout_i                        (out is linear in v)
  dp_ij  = <dout_i, v_j>                      (d loss / d p_ij)
  ds_ij  = p_ij (dp_ij - sum_l p_il dp_il)    (softmax Jacobian)
  dq_i   = scale sum_j ds_ij k_j
  dk_j  += scale ds_ij q_i

and the KV-head gradients collect the contributions of all G query heads
that read that KV head.  sum_l p_il dp_il equals <dout_i, out_i>.
"""
from __future__ import annotations

import numpy as np

from .reference import _check, _softmax_rows, kv_head_of, visible_mask


def attention_backward(q, k, v, dout, causal: bool, scale: float, window: int = 0):
    """(dq [B,Hq,Lq,D], dk [B,Hkv,Lk,D], dv [B,Hkv,Lk,D]) in float64.

    Every row must see at least one key (always so for the bottom-right
    causal mask with Lq <= Lk)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, Hq, Hkv, Lq, Lk, D = _check(q, k, v)
    if dout.shape != q.shape:
        raise ValueError("dout must have the shape of q")
    keep = visible_mask(Lq, Lk, causal, "bottom_right", window)
    if not keep.any(axis=1).all():
        raise ValueError("a row sees no key")
    sc = np.float64(scale)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            hk = kv_head_of(h, Hq, Hkv)
            s = np.where(keep, sc * (q[b, h] @ k[b, hk].T), -np.inf)
            p, _ = _softmax_rows(s)
            dv[b, hk] += p.T @ dout[b, h]
            dp = dout[b, h] @ v[b, hk].T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dq[b, h] = sc * (ds @ k[b, hk])
            dk[b, hk] += sc * (ds.T @ q[b, h])
    return dq, dk, dv


def attention_backward_sampled(q, k, v, dout, causal: bool, scale: float, qrows, krows, window: int = 0,
                               heads=None):
    """The same gradients at selected positions only (for long sequences).

    qrows: query rows whose dq is wanted; krows: key positions whose dk and
    dv are wanted; heads: KV heads to evaluate (default all).  Returns
    dq [B, Hq, len(qrows), D] (rows of heads outside ``heads`` are NaN),
    dk and dv [B, Hkv, len(krows), D] (NaN outside ``heads``).  Each value is
    the formula above with all of its sums taken in full: the per-row
    statistics (the softmax normaliser and sum_l p_il dp_il) use every
    visible key of the row, and dk_j, dv_j sum over every row that sees j.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, Hq, Hkv, Lq, Lk, D = _check(q, k, v)
    G = Hq // Hkv
    qrows = np.asarray(qrows, dtype=np.int64)
    krows = np.asarray(krows, dtype=np.int64)
    heads = range(Hkv) if heads is None else heads
    sc = np.float64(scale)
    off = Lk - Lq
    j = np.arange(Lk)
    dq = np.full((B, Hq, len(qrows), D), np.nan)
    dk = np.full((B, Hkv, len(krows), D), np.nan)
    dv = np.full((B, Hkv, len(krows), D), np.nan)
    for b in range(B):
        for hk in heads:
            dk[b, hk] = 0.0
            dv[b, hk] = 0.0
            for h in range(hk * G, (hk + 1) * G):
                for i0 in range(0, Lq, 512):          # rows one slab at a time (memory only)
                    i = np.arange(i0, min(Lq, i0 + 512))
                    if causal:
                        keep = j[None, :] <= i[:, None] + off
                        if window:
                            keep &= j[None, :] > i[:, None] + off - window
                    else:
                        keep = np.ones((len(i), Lk), dtype=bool)
                    s = np.where(keep, sc * (q[b, h, i] @ k[b, hk].T), -np.inf)
                    p, _ = _softmax_rows(s)
                    dp = dout[b, h, i] @ v[b, hk].T
                    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                    dk[b, hk] += sc * (ds[:, krows].T @ q[b, h, i])
                    dv[b, hk] += p[:, krows].T @ dout[b, h, i]
                    sel = np.flatnonzero(np.isin(qrows, i))
                    if len(sel):
                        dq[b, h, sel] = sc * (ds[qrows[sel] - i0] @ k[b, hk])
    return dq, dk, dv


def attention_backward_from_forward(q, k, v, out, dout, lse, causal: bool, scale: float, window: int = 0):
    """The gradients as a backward pass computes them from a forward's saved
    out and lse: p_ij = exp(scale s_ij - lse_i) over the visible keys and
    delta_i = <dout_i, out_i> with the given out and lse (instead of the
    exact softmax and its own sum_l p_il dp_il).  With the exact out and lse
    this is ``attention_backward``; with an out rounded to bf16 it is what a
    kernel that receives that out computes, before its own rounding."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    out = np.asarray(out, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    B, Hq, Hkv, Lq, Lk, D = _check(q, k, v)
    keep = visible_mask(Lq, Lk, causal, "bottom_right", window)
    sc = np.float64(scale)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    delta = delta_rows(out, dout)
    for b in range(B):
        for h in range(Hq):
            hk = kv_head_of(h, Hq, Hkv)
            p = np.where(keep, np.exp(sc * (q[b, h] @ k[b, hk].T) - lse[b, h][:, None]), 0.0)
            dv[b, hk] += p.T @ dout[b, h]
            dp = dout[b, h] @ v[b, hk].T
            ds = p * (dp - delta[b, h][:, None])
            dq[b, h] = sc * (ds @ k[b, hk])
            dk[b, hk] += sc * (ds.T @ q[b, h])
    return dq, dk, dv


def attention_backward_from_forward_sampled(q, k, v, out, dout, lse, causal: bool, scale: float, qrows, krows,
                                            window: int = 0):
    """``attention_backward_from_forward`` at selected query rows (dq) and key
    positions (dk, dv) only.  With the saved out and lse given, every weight
    p_ij is known without a pass over the row, so dq_i needs row i only and
    dk_j, dv_j need column j only (over every row that sees key j)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    B, Hq, Hkv, Lq, Lk, D = _check(q, k, v)
    qrows = np.asarray(qrows, dtype=np.int64)
    krows = np.asarray(krows, dtype=np.int64)
    keep = visible_mask(Lq, Lk, causal, "bottom_right", window)
    sc = np.float64(scale)
    delta = delta_rows(out, dout)
    dq = np.zeros((B, Hq, len(qrows), D))
    dk = np.zeros((B, Hkv, len(krows), D))
    dv = np.zeros((B, Hkv, len(krows), D))
    for b in range(B):
        for h in range(Hq):
            hk = kv_head_of(h, Hq, Hkv)
            # rows qrows, all keys
            p = np.where(keep[qrows], np.exp(sc * (q[b, h, qrows] @ k[b, hk].T) - lse[b, h, qrows][:, None]), 0.0)
            ds = p * (dout[b, h, qrows] @ v[b, hk].T - delta[b, h, qrows][:, None])
            dq[b, h] = sc * (ds @ k[b, hk])
            # all rows, keys krows
            p = np.where(keep[:, krows], np.exp(sc * (q[b, h] @ k[b, hk, krows].T) - lse[b, h][:, None]), 0.0)
            ds = p * (dout[b, h] @ v[b, hk, krows].T - delta[b, h][:, None])
            dk[b, hk] += sc * (ds.T @ q[b, h])
            dv[b, hk] += p.T @ dout[b, h]
    return dq, dk, dv


def delta_rows(out, dout):
    """sum_l p_il dp_il written as <dout_i, out_i> (the same number)."""
    return (np.asarray(out, dtype=np.float64) * np.asarray(dout, dtype=np.float64)).sum(axis=-1)


__all__ = ["attention_backward", "attention_backward_sampled", "attention_backward_from_forward",
           "attention_backward_from_forward_sampled", "delta_rows", "kv_head_of"]
