"""Scalar-loop attention for tiny shapes.  TEST INFRASTRUCTURE ONLY.

An independent spelling of the same definition as ``oracle.reference``:
plain Python floats, ``math.exp`` and correctly rounded ``math.fsum`` sums, one
score at a time, with the visibility test written inline.  It is used to
check the vectorised oracle by exhaustive enumeration of tiny shapes.
Definition sources: [cost-guide] "어텐션 구현 고르기, SDPA·FlashAttention
메모리와 GPU 비용", section "is_causal 마스크 정렬, KV 캐시와 쓸 때의 함정"
(bottom-right mask, scores over sqrt(d)); [nvidia-long] "Как NVIDIA учит
нейросети думать быстрее…", section on group size G (Hq/Hkv heads share a
KV head).
"""
from __future__ import annotations

import math


def brute_attention(q, k, v, causal: bool, scale: float, window: int = 0):
    """q [B][Hq][Lq][D], k/v [B][Hkv][Lk][D] (nested sequences or arrays).

    window > 0 (causal): a row keeps only its `window` most recent visible
    keys (the diagonal key and the window - 1 before it).
    Returns (out, lse) as nested lists of Python floats.
    """
    B, Hq, Lq, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv, Lk = len(k[0]), len(k[0][0])
    group = Hq // Hkv
    out = [[[[0.0] * D for _ in range(Lq)] for _ in range(Hq)] for _ in range(B)]
    lse = [[[0.0] * Lq for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            kh = h // group
            for i in range(Lq):
                diag = i + (Lk - Lq)          # the row's own position among the keys
                keys = [j for j in range(Lk) if (not causal) or j <= diag]
                if causal and window:
                    keys = keys[max(0, len(keys) - window):]
                sc = []
                for j in keys:
                    dot = math.fsum(float(q[b][h][i][d]) * float(k[b][kh][j][d]) for d in range(D))
                    sc.append(float(scale) * dot)
                top = max(sc)
                ex = [math.exp(x - top) for x in sc]
                z = math.fsum(ex)
                lse[b][h][i] = top + math.log(z)
                for d in range(D):
                    out[b][h][i][d] = math.fsum(ex[t] * float(v[b][kh][j][d]) for t, j in enumerate(keys)) / z
    return out, lse
