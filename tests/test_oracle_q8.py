"""Pins for the int8 (q8_0-style) cache reading of the oracle (oracle/quant.py).

Format read: blocks of 32 elements per cache row, one binary16 scale per
block, element = bfloat16 nearest (ties to even) of scale * code.  The pins
are hand-computed values, the rounding rule's ties, the block layout, an
independent float32 -> bfloat16 conversion (torch's, on the CPU), and the
rounding bound; the planted-mistake test shows that a wrong block index,
truncation instead of rounding, or codes read as unsigned each fail a pin.
"""
import numpy as np
import pytest
import torch

import attn_inputs as ai
import oracle
from oracle import quant

pytestmark = pytest.mark.filterwarnings("ignore")


def _half(x):
    return np.array(x, dtype=np.float16).view(np.uint16)


def _hand_case():
    """A D = 64 row: block 0 scale 0.5, block 1 scale -2; codes chosen so every
    product is a bfloat16 value, so the expected values are the products."""
    codes = np.zeros(64, dtype=np.int8)
    codes[:5] = [-128, -1, 0, 1, 127]
    codes[32:36] = [-128, 3, 127, -7]
    scales = _half([0.5, -2.0])
    expect = np.zeros(64)
    expect[:5] = [-64.0, -0.5, 0.0, 0.5, 63.5]
    expect[32:36] = [256.0, -6.0, -254.0, 14.0]
    return codes, scales, expect


def _tie_case():
    """Scales 1 + 2^-8 (a tie: down to the even 1), 1 + 3 * 2^-8 (a tie: up to
    the even 1 + 2^-6), 1 + 2^-8 + 2^-10 (above the tie: up to 1 + 2^-7) and
    1 + 2^-9 (below the tie: down to 1), each times code 1.  Block 4 has scale
    1 + 2^-8 and code 3: 3 + 3 * 2^-8 lies above the midpoint 3 + 2^-7 of the
    bfloat16 neighbours 3 and 3 + 2^-6, so it rounds up to 3 + 2^-6."""
    s = [1 + 2**-8, 1 + 3 * 2**-8, 1 + 2**-8 + 2**-10, 1 + 2**-9, 1 + 2**-8]
    codes = np.zeros(160, dtype=np.int8)
    for j in range(4):
        codes[32 * j] = 1
    codes[128] = 3
    expect = np.zeros(160)
    expect[0], expect[32], expect[64], expect[96] = 1.0, 1 + 2**-6, 1 + 2**-7, 1.0
    expect[128] = 3 + 2**-6
    return codes, _half(s), expect


def test_q8_hand_example():
    codes, scales, expect = _hand_case()
    assert np.array_equal(oracle.dequantize_q8(codes, scales), expect)


def test_q8_rounding_ties_to_even():
    codes, scales, expect = _tie_case()
    assert np.array_equal(half_f := quant.half_bits_to_f64(scales), [1 + 2**-8, 1 + 3 * 2**-8, 1 + 2**-8 + 2**-10,
                                                                    1 + 2**-9, 1 + 2**-8]), half_f
    assert np.array_equal(oracle.dequantize_q8(codes, scales), expect)


def test_q8_block_layout():
    """Block j of a row takes scale j: all-ones codes reproduce the scales
    (chosen as k / 16 with |k| < 64, so they are bfloat16 values), each
    repeated over its 32 elements, for every batch position."""
    rng = np.random.default_rng(5)
    for D in (32, 64, 128, 256):
        k = rng.integers(1, 64, size=(3, 2, D // 32)) * rng.choice([-1, 1], size=(3, 2, D // 32))
        sc = (k / 16.0).astype(np.float16)
        ones = np.ones((3, 2, D), dtype=np.int8)
        got = oracle.dequantize_q8(ones, sc.view(np.uint16))
        for j in range(D // 32):
            assert np.all(got[..., 32 * j:32 * (j + 1)] == sc[..., j:j + 1].astype(np.float64))


def test_q8_matches_an_independent_bf16_conversion():
    """scale * code is exact in float32; torch's float32 -> bfloat16 cast (round
    to nearest even) of that product must give the oracle's values."""
    codes, sbits = ai.q8_codes_scales((4, 37, 128), [90, 1])
    prod32 = np.repeat(sbits.view(np.float16).astype(np.float32), 32, axis=-1) * codes.astype(np.float32)
    assert np.array_equal(prod32.astype(np.float64),
                          np.repeat(quant.half_bits_to_f64(sbits), 32, axis=-1) * codes.astype(np.float64))
    ref = torch.from_numpy(prod32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.dequantize_q8(codes, sbits), ref)


def test_q8_rounding_bound_and_grid():
    codes, sbits = ai.q8_codes_scales((8, 64, 64), [90, 2])
    exact = np.repeat(quant.half_bits_to_f64(sbits), 32, axis=-1) * codes
    got = oracle.dequantize_q8(codes, sbits)
    # 8 significant bits: the unit roundoff is 2^-8
    assert np.all(np.abs(got - exact) <= 2.0**-8 * np.abs(exact))
    # every value is a bfloat16: its float32 pattern has no low 16 bits
    assert np.all((got.astype(np.float32).view(np.uint32) & 0xFFFF) == 0)
    # products that are bfloat16 values already come through unchanged
    small = (np.abs(codes.astype(np.int64)) < 2) | (codes == -128)
    pow2 = np.repeat(sbits.view(np.float16), 32, axis=-1).astype(np.float64)
    pow2_ok = (np.frexp(pow2)[0] == 0.5)
    m = small & pow2_ok
    assert np.array_equal(got[m], exact[m])


def test_q8_rejects_bad_shapes():
    with pytest.raises(TypeError):
        oracle.dequantize_q8(np.zeros(32, dtype=np.int16), _half([1.0]))
    with pytest.raises(ValueError):
        oracle.dequantize_q8(np.zeros(48, dtype=np.int8), _half([1.0]))
    with pytest.raises(ValueError):
        oracle.dequantize_q8(np.zeros(64, dtype=np.int8), _half([1.0]))


def test_q8_planted_mistakes_are_caught():
    """Each plausible mistake in a dequantizer fails the hand or the tie pin."""
    def blocks_of_64(c, s):
        sc = quant.half_bits_to_f64(s)
        per = np.repeat(sc, 64, axis=-1)[..., :c.shape[-1]]
        return quant.round_to_bf16(per * c.astype(np.float64))

    def truncating(c, s):
        x = np.repeat(quant.half_bits_to_f64(s), 32, axis=-1) * c.astype(np.float64)
        m, e = np.frexp(x)
        return np.ldexp(np.trunc(np.ldexp(m, 8)), e - 8)

    def unsigned_codes(c, s):
        return quant.round_to_bf16(np.repeat(quant.half_bits_to_f64(s), 32, axis=-1) * c.view(np.uint8))

    def round_half_up(c, s):
        x = np.repeat(quant.half_bits_to_f64(s), 32, axis=-1) * c.astype(np.float64)
        m, e = np.frexp(x)
        return np.ldexp(np.floor(np.ldexp(m, 8) + 0.5), e - 8)

    for wrong in (blocks_of_64, truncating, unsigned_codes, round_half_up):
        caught = False
        for codes, scales, expect in (_hand_case(), _tie_case()):
            if not np.array_equal(wrong(codes, scales), expect):
                caught = True
        assert caught, wrong.__name__


def test_q8_input_recipe():
    """The generator: codes span [-128, 127], scales lie in [0.5, 1.5) * sqrt(3)/127
    (up to binary16 rounding), values have about unit variance."""
    codes, sbits = ai.q8_codes_scales((16, 256, 128), [91, 0])
    assert codes.min() == -128 and codes.max() == 127
    s = quant.half_bits_to_f64(sbits)
    lo, hi = 0.5 * np.sqrt(3) / 127, 1.5 * np.sqrt(3) / 127
    assert s.min() >= lo * (1 - 2**-11) and s.max() <= hi * (1 + 2**-11)
    x = oracle.dequantize_q8(codes, sbits)
    # E[x^2] = E[u^2] * 3 E[c^2] / 127^2 = (13/12) * (5461.5 * 3 / 16129) = 1.1005
    assert abs(float(np.mean(x * x)) - 1.1005) < 0.01
