"""Eager fp64 attention: the plain definition, computed with a full score table.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py for who may import it).

Definition followed (for every batch b, query head h, query row i):
  * the group size is G = Hq / Hkv and query head h reads KV head h // G
    (consecutive query heads share a KV head) [nvidia-long, section
    "Параметр первый: размер группы (group size)"; cost-guide, section
    "KV 캐시를 끄면 생기는 일, use_cache 비용" on GQA's 8 KV heads];
  * s_ij = scale * <q_i, k_j> for visible keys j; the caller passes 1/sqrt(D)
    as scale for the usual scaling [cost-guide, "is_causal 마스크 정렬, KV
    캐시와 쓸 때의 함정", numpy example: scores divided by sqrt(d)];
  * visible keys: all of them without a causal mask; with a causal mask,
    j <= i + (Lk - Lq), the mask anchored at the bottom-right corner of the
    Lq x Lk table, which is the alignment flash-attn uses from version 2.1;
    the top-left anchored mask (j <= i) is offered only so that tests can
    show it is the wrong one when Lq < Lk [cost-guide, same section];
  * softmax over the visible keys with the row maximum subtracted; lse is the
    natural log of the row's normaliser; out_i = sum_j p_ij v_j [cost-guide,
    "eager 어텐션 메모리, 길이에 따라 얼마나 커지나": the eager path builds
    the table, applies softmax in a wider type, then multiplies by V; here
    the wider type is float64 as the page's reproducibility advice suggests
    in "상황별 추천 구현"].

The split-KV combine is the identity lse = log(sum_c exp(lse_c)),
out = sum_c exp(lse_c - lse) out_c, obtained by splitting the visible set into
disjoint chunks; the pages only imply it through KV-cache sharding
[nvidia-long, "Параметр четвёртый: параллелизм и распределение по GPU", KVP].
"""
from __future__ import annotations

import numpy as np


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """KV head read by query head h: groups of G = Hq/Hkv consecutive heads."""
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return h // (Hq // Hkv)


def visible_mask(Lq: int, Lk: int, causal: bool, align: str = "bottom_right", window: int = 0) -> np.ndarray:
    """Boolean [Lq, Lk] table of the keys each query row may attend to.

    window > 0 (causal only) keeps, of the keys a row sees, only the `window`
    most recent ones: j > i + (Lk - Lq) - window.  This is the sliding-window
    (local) attention the pages name as a way to shorten the effective KV
    history [nvidia-long, "Параметр третий: длина последовательности"; the
    cost-guide's "상황별 추천 구현" lists sliding windows among the masks
    written for flex_attention].
    """
    if window < 0:
        raise ValueError("window must be >= 0")
    if not causal:
        if window:
            raise ValueError("a window needs the causal mask")
        return np.ones((Lq, Lk), dtype=bool)
    i = np.arange(Lq)[:, None]
    j = np.arange(Lk)[None, :]
    if align == "bottom_right":
        keep = j <= i + (Lk - Lq)
        if window:
            keep &= j > i + (Lk - Lq) - window
        return keep
    if align == "upper_left":
        if window:
            raise ValueError("windows are anchored like the bottom-right mask")
        return j <= i
    raise ValueError(align)


def _softmax_rows(s: np.ndarray):
    """Row softmax of a score block with -inf at hidden cells.

    Returns (p, lse).  A row with no visible key gets a -inf maximum and
    therefore NaN, as the page's own numpy helper would.
    """
    with np.errstate(invalid="ignore"):
        m = s.max(axis=-1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=-1, keepdims=True)
        p = e / z
        lse = (m + np.log(z))[..., 0]
    return p, lse


def _check(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.shape != k.shape:
        raise ValueError("expected q [B,Hq,Lq,D], k and v [B,Hkv,Lk,D]")
    B, Hq, Lq, D = q.shape
    if k.shape[0] != B or k.shape[3] != D or Hq % k.shape[1]:
        raise ValueError("shape mismatch")
    return B, Hq, k.shape[1], Lq, k.shape[2], D


def attention(q, k, v, causal: bool, scale: float, align: str = "bottom_right", window: int = 0):
    """Full eager attention.  q [B,Hq,Lq,D], k/v [B,Hkv,Lk,D] -> (out, lse).

    out is [B,Hq,Lq,D] float64, lse [B,Hq,Lq] float64 (natural log).
    window: see visible_mask.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Hkv, Lq, Lk, D = _check(q, k, v)
    keep = visible_mask(Lq, Lk, causal, align, window)
    out = np.empty((B, Hq, Lq, D))
    lse = np.empty((B, Hq, Lq))
    sc = np.float64(scale)
    for b in range(B):
        for h in range(Hq):
            hk = kv_head_of(h, Hq, Hkv)
            s = np.where(keep, sc * (q[b, h] @ k[b, hk].T), -np.inf)
            p, lse[b, h] = _softmax_rows(s)
            out[b, h] = p @ v[b, hk]
    return out, lse


def attention_probs(q, k, causal: bool, scale: float, align: str = "bottom_right"):
    """The softmax table P [B,Hq,Lq,Lk] itself, for tiny shapes."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    keep = visible_mask(Lq, Lk, causal, align)
    P = np.empty((B, Hq, Lq, Lk))
    for b in range(B):
        for h in range(Hq):
            hk = kv_head_of(h, Hq, Hkv)
            s = np.where(keep, np.float64(scale) * (q[b, h] @ k[b, hk].T), -np.inf)
            P[b, h], _ = _softmax_rows(s)
    return P


def attention_rows(q, k, v, rows, causal: bool, scale: float, window: int = 0):
    """Selected query rows only (sampled mode for long sequences).

    rows: int array [B, Hq, R] of query-row indices.  Each selected row is
    computed exactly as in ``attention`` (same definition, same mask); only
    the rows not asked for are skipped.  Returns out [B,Hq,R,D], lse [B,Hq,R].
    """
    if window and not causal:
        raise ValueError("a window needs the causal mask")
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    rows = np.asarray(rows)
    R = rows.shape[-1]
    out = np.empty((B, Hq, R, D))
    lse = np.empty((B, Hq, R))
    sc = np.float64(scale)
    j = np.arange(Lk)[None, :]
    for b in range(B):
        for h in range(Hq):
            hk = kv_head_of(h, Hq, Hkv)
            r = rows[b, h]
            qr = np.asarray(q[b, h, r], dtype=np.float64)
            kb = np.asarray(k[b, hk], dtype=np.float64)
            vb = np.asarray(v[b, hk], dtype=np.float64)
            s = sc * (qr @ kb.T)
            if causal:
                s = np.where(j <= r[:, None] + (Lk - Lq), s, -np.inf)
                if window:
                    s = np.where(j > r[:, None] + (Lk - Lq) - window, s, -np.inf)
            p, lse[b, h] = _softmax_rows(s)
            out[b, h] = p @ vb
    return out, lse


def decode(q, kcache, vcache, kv_lens, scale: float):
    """Single-token decode over a KV cache.

    q [B,Hq,D]; kcache/vcache [B,Hkv,Lmax,D]; kv_lens [B].  The new token's
    K/V is already in the cache, and the query sees keys [0, n) with
    n = min(kv_lens[b], Lmax) and no mask [cost-guide, "is_causal 마스크 정렬,
    KV 캐시와 쓸 때의 함정": one query row over the cache is called without a
    causal mask; "KV 캐시를 끄면 생기는 일": cached K/V do not change].
    n = 0 gives out = 0 and lse = -inf.  Returns out [B,Hq,D], lse [B,Hq].
    """
    B, Hq, D = q.shape
    Hkv, Lmax = kcache.shape[1], kcache.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    sc = np.float64(scale)
    for b in range(B):
        n = int(min(max(int(kv_lens[b]), 0), Lmax))
        if n == 0:
            continue
        for hk in range(Hkv):
            kb = np.asarray(kcache[b, hk, :n], dtype=np.float64)
            vb = np.asarray(vcache[b, hk, :n], dtype=np.float64)
            heads = [h for h in range(Hq) if kv_head_of(h, Hq, Hkv) == hk]
            qg = np.asarray(q[b, heads], dtype=np.float64)          # [G, D]
            p, l = _softmax_rows(sc * (qg @ kb.T))
            out[b, heads] = p @ vb
            lse[b, heads] = l
    assert G * Hkv == Hq
    return out, lse


def combine_partials(outs, lses):
    """Merge attention results over disjoint key chunks.

    outs [n, ..., D] (each chunk's normalised output), lses [n, ...].
    Chunks with lse = -inf (no keys) carry zero weight.
    """
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    top = lses.max(axis=0)
    safe = np.where(np.isfinite(top), top, 0.0)
    w = np.exp(lses - safe)                       # [n, ...]
    z = w.sum(axis=0)
    with np.errstate(invalid="ignore", divide="ignore"):
        out = (w[..., None] * outs).sum(axis=0) / z[..., None]
        lse = safe + np.log(z)
    out = np.where(np.isfinite(top)[..., None], out, 0.0)
    return out, lse
