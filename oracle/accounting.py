"""Closed-form sizes and operation counts.  TEST INFRASTRUCTURE ONLY.

These are the counting rules the measurement uses, written so that they
reproduce the tables the pages print:
  * score table cells = batch x query heads x length^2; bytes per cell 2 for a
    bf16 table and 6 at the softmax peak when a bf16 and an fp32 table coexist
    [cost-guide "어텐션 구현 고르기, SDPA·FlashAttention 메모리와 GPU 비용",
    section "eager 어텐션 메모리, 길이에 따라 얼마나 커지나", memory table];
  * KV cache bytes = tokens x layers x KV heads x head dim x 2 tensors x 2 B
    [same table, last column; section "KV 캐시를 끄면 생기는 일, use_cache 비용"
    for the per-token figure];
  * per-row statistics = query heads x rows x 4 B [section "eager 어텐션
    메모리…", the closing paragraph on row statistics];
  * attention FLOPs for a token at position t = 4 x query heads x head dim x t
    per layer (QK^T and PV, 2 FLOPs per multiply-add), and 2 FLOPs per weight
    for the matmuls [section "긴 입력에서 어텐션 연산이 차지하는 비중", chart
    and table];
  * exact causal work counts the visible (query, key) pairs of the bottom-right
    mask instead of the page's t = L/2 average.
"""
from __future__ import annotations

import numpy as np

GiB = 2 ** 30
KiB = 2 ** 10
MiB = 2 ** 20


def score_table_bytes(B: int, Hq: int, L: int, bytes_per_cell: int) -> int:
    return B * Hq * L * L * bytes_per_cell


def kv_cache_bytes(tokens: int, Hkv: int, D: int, layers: int, elem_bytes: int = 2) -> int:
    return tokens * layers * Hkv * D * 2 * elem_bytes


def row_stats_bytes(Hq: int, L: int, elem_bytes: int = 4) -> int:
    return Hq * L * elem_bytes


def attention_flops_at(Hq: int, D: int, t: float, layers: int) -> float:
    """FLOPs for one token that attends to t keys, summed over layers."""
    return 4.0 * Hq * D * t * layers


def weight_flops_per_token(params: float) -> float:
    return 2.0 * params


def visible_pairs(Lq: int, Lk: int, causal: bool) -> int:
    """Number of (query, key) cells the mask keeps (bottom-right alignment)."""
    if not causal:
        return Lq * Lk
    if Lq > Lk:
        raise ValueError("causal with Lq > Lk leaves rows with no key")
    return Lq * (Lk - Lq) + Lq * (Lq + 1) // 2


def prefill_flops(B: int, Hq: int, D: int, Lq: int, Lk: int, causal: bool) -> int:
    return 4 * B * Hq * D * visible_pairs(Lq, Lk, causal)


def decode_kv_bytes(kv_lens, Hkv: int, D: int, Lmax: int, elem_bytes: int = 2) -> int:
    n = np.minimum(np.maximum(np.asarray(kv_lens, dtype=np.int64), 0), Lmax)
    return int(n.sum()) * Hkv * D * 2 * elem_bytes


def decode_q8_kv_bytes(kv_lens, Hkv: int, D: int, Lmax: int) -> int:
    """int8 caches: per visible key and KV head, D one-byte codes and D / 32
    two-byte scales, for K and for V."""
    n = np.minimum(np.maximum(np.asarray(kv_lens, dtype=np.int64), 0), Lmax)
    return int(n.sum()) * Hkv * 2 * (D + 2 * (D // 32))


def decode_flops(kv_lens, Hq: int, D: int, Lmax: int) -> int:
    n = np.minimum(np.maximum(np.asarray(kv_lens, dtype=np.int64), 0), Lmax)
    return 4 * Hq * D * int(n.sum())
