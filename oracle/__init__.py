"""CPU oracle for exact grouped-query attention.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check of the package entry point and the CPU
baseline leg of the bench may import anything from this package.  The product
path (the HIP library and its Python binding) never imports it, and this
package imports nothing from the product path: the two share only the seeded
input generators of ``attn_inputs``.

Everything here is plain numpy in float64 on bf16-exact inputs, written from
the definition of scaled-dot-product attention, not from any kernel design.

Pages cited (by title):
  [cost-guide]   "어텐션 구현 고르기, SDPA·FlashAttention 메모리와 GPU 비용"
                 (tool.smithlab.co.kr; an SDPA / FlashAttention memory and
                 GPU-cost guide)
  [nvidia-long]  "Как NVIDIA учит нейросети думать быстрее: оптимизация
                 внимания для длинных контекстов" (iphoneandroid24.ru)
  [gqa-glossary] "grouped-query attention 그룹 쿼리 어텐션" (0to1log.com)
  [slack]        "Attention Slack (어텐션 슬랙): KV 캐시 크기가 추론 능력을
                 결정한다" (kiban.pages.dev; llama.cpp runs with q8_0 K/V
                 caches)

Pinned by tests/test_oracle.py (page example, closed forms, invariants,
brute force; the byte and FLOP counters of ``accounting`` against the cost
guide's per-token KV size and FLOP count and the int8 layout's own arrays),
tests/test_oracle_q8.py and tests/test_oracle_backward.py.  Every function
here has such a pin; none is "parity unpinned".
"""
from .reference import (visible_mask, kv_head_of, attention, attention_rows, decode, combine_partials,
                        attention_probs)
from .brute import brute_attention
from .quant import dequantize_q8, round_to_bf16, half_bits_to_f64
from .backward import (attention_backward, attention_backward_sampled, attention_backward_from_forward,
                       attention_backward_from_forward_sampled, delta_rows)
from . import accounting

__all__ = ["visible_mask", "kv_head_of", "attention", "attention_rows", "decode", "combine_partials",
           "attention_probs", "brute_attention", "dequantize_q8", "round_to_bf16", "half_bits_to_f64",
           "attention_backward", "attention_backward_sampled", "attention_backward_from_forward",
           "attention_backward_from_forward_sampled", "delta_rows",
           "accounting"]
