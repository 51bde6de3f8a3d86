"""int8 (q8_0-style) KV caches: the element values attention sees.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py for who may import it).

The Attention Slack page (Gemma-4 26B) runs llama.cpp flash attention with
both the K and the V cache stored as q8_0 (its llama-server service
configuration); none of the pages defines that format.  Reading taken here:

  * a cache row of D elements is cut into D / 32 blocks of 32 consecutive
    elements; block j carries one IEEE binary16 scale s_j and 32 signed 8-bit
    codes c (all of -128..127 allowed);
  * the element's value is s_j * c, and, as with a bf16 cache, attention takes
    its K and V operands in bfloat16: the value enters attention rounded to
    the nearest bfloat16 (ties to even).  s_j * c needs at most 11 + 8
    significant bits, so it is exact in float32 and float64, and the one
    rounding is that to bfloat16.

Everything after the dequantization is the plain definition in
``oracle.reference`` applied to these values.
"""
from __future__ import annotations

import numpy as np

Q8_BLOCK = 32


def half_bits_to_f64(bits) -> np.ndarray:
    """IEEE binary16 bit patterns (uint16) to their float64 values (exact)."""
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def round_to_bf16(x) -> np.ndarray:
    """Nearest bfloat16 value of each float64 (ties to even), as float64.

    bfloat16 keeps 8 significant bits: write x = m * 2^e with 0.5 <= |m| < 1,
    round m * 2^8 to an integer (numpy's rint rounds halves to even) and scale
    back.  Zeros stay zeros; NaN stays NaN.  Inputs here are far from the
    bfloat16 overflow and subnormal ranges.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def dequantize_q8(codes, scale_bits) -> np.ndarray:
    """codes int8 [..., D], scale_bits uint16 [..., D / 32] -> values [..., D] (float64).

    Element i of a row belongs to block i // 32 and takes that block's scale.
    """
    c = np.asarray(codes)
    if c.dtype != np.int8:
        raise TypeError("codes must be int8")
    D = c.shape[-1]
    if D % Q8_BLOCK:
        raise ValueError("row length must be a multiple of 32")
    s = half_bits_to_f64(scale_bits)
    if s.shape != c.shape[:-1] + (D // Q8_BLOCK,):
        raise ValueError("one scale per 32-element block of each row")
    per_elem = np.repeat(s, Q8_BLOCK, axis=-1)
    return round_to_bf16(per_elem * c.astype(np.float64))
