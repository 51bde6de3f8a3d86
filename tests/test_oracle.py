"""Pins for the CPU oracle: page values, closed forms, invariants, brute force.

Each test fixes the oracle against something other than itself: a value a
page prints, a closed form, an invariant of the mathematics, or an
independent scalar-loop spelling.  The mutation tests at the end plant a
plausible mistake into the oracle (on the CPU) and check that a pin catches it.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import accounting as acc
from oracle import reference as ref
import attn_inputs as ai


# ---------------------------------------------------------------------------
# 1. The worked example of the cost guide ("is_causal 마스크 정렬" section).
# ---------------------------------------------------------------------------
def _page_example_inputs():
    rng = np.random.default_rng(1)
    S, d = 5, 8
    q_all, k, v = (rng.standard_normal((S, d)) for _ in range(3))
    return S, d, q_all, k, v


def _as4(x):
    return np.asarray(x)[None, None]


def test_page_is_causal_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "cost_guide_is_causal_example.json")))
    S, d, q_all, k, v = _page_example_inputs()
    scale = 1.0 / np.sqrt(d)
    full, _ = oracle.attention(_as4(q_all), _as4(k), _as4(v), True, scale, align="upper_left")
    for line in g["printed"]:
        L, align = line["L"], line["align"]
        qL = _as4(q_all[-L:])
        out, _ = oracle.attention(qL, _as4(k), _as4(v), True, scale, align=align)
        P = oracle.attention_probs(qL, _as4(k), True, scale, align=align)
        w_last = np.round(P[0, 0, -1], 2)
        np.testing.assert_array_equal(w_last, np.array(line["last_row_weights_2dp"]))
        assert bool(np.allclose(out[0, 0], full[0, 0, -L:])) == line["allclose_to_full"]


def test_alignments_agree_when_square():
    S, d, q_all, k, v = _page_example_inputs()
    a, la = oracle.attention(_as4(q_all), _as4(k), _as4(v), True, 0.3, align="upper_left")
    b, lb = oracle.attention(_as4(q_all), _as4(k), _as4(v), True, 0.3, align="bottom_right")
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)


# ---------------------------------------------------------------------------
# 2. Closed-form tables of the cost guide.
# ---------------------------------------------------------------------------
def test_memory_table(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "cost_guide_memory_table.json")))
    m = g["model"]
    for row in g["rows"]:
        L = row["L"]
        assert acc.score_table_bytes(1, m["Hq"], L, 2) == row["bf16_table"] * acc.GiB
        assert acc.score_table_bytes(1, m["Hq"], L, 6) == row["peak_with_fp32"] * acc.GiB
        kv = acc.kv_cache_bytes(L, m["Hkv"], m["D"], m["layers"]) / acc.GiB
        # exact 0.5625 / 1.125 / 2.25 / 4.5 GiB, printed rounded half-up
        assert abs(kv - row["kv_cache"]) <= 0.005 + 1e-12
    rs = g["row_stats"]
    assert acc.row_stats_bytes(rs["heads"], rs["rows"]) == rs["MiB"] * acc.MiB
    # the cost guide's own example: one Qwen3-8B layer (32 query heads) at 16K tokens has a 16 GiB bf16 table
    assert acc.score_table_bytes(1, 32, 16384, 2) == 16 * acc.GiB


def test_kv_per_token(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "cost_guide_kv_per_token.json")))
    m = g["model"]
    for row in g["rows"]:
        assert acc.kv_cache_bytes(1, row["Hkv"], m["D"], m["layers"], m["elem_bytes"]) == row["KiB_per_token"] * acc.KiB


def test_compute_share(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "cost_guide_compute_share.json")))
    m = g["model"]
    w = acc.weight_flops_per_token(m["non_embedding_params"]) / 1e9
    shares = {}
    for row in g["rows_gflop"]:
        L = row["L"]
        a = acc.attention_flops_at(m["Hq"], m["D"], L / 2, m["layers"]) / 1e9
        assert round(a, 1) == row["attention"]
        assert round(w, 1) == row["weights"]
        shares[L] = 100 * a / (a + w)
    for s in g["attention_share_percent"]:
        assert round(shares[s["L"]]) == s["share"]


def test_visible_pairs_counts_the_mask():
    for Lq, Lk in [(1, 1), (1, 9), (3, 7), (8, 8), (5, 12)]:
        n = int(ref.visible_mask(Lq, Lk, True).sum())
        assert acc.visible_pairs(Lq, Lk, True) == n
        assert acc.visible_pairs(Lq, Lk, False) == Lq * Lk
    # exact counts used by the measurement
    assert acc.prefill_flops(1, 32, 128, 16384, 16384, True) == 4 * 32 * 128 * (16384 * 16385 // 2) == 2199157473280
    assert acc.prefill_flops(1, 32, 128, 512, 16384, True) == 4 * 32 * 128 * 8257792


def test_decode_kv_bytes_is_the_pages_per_token_size(golden_dir):
    """Decode KV bytes = the cost guide's KV bytes per token (use_cache
    section: 144 KiB at 8 KV heads, 576 KiB at 32, over 36 layers) divided by
    the layers, times the keys each sequence reads (lengths clamped to
    [0, Lmax])."""
    g = json.load(open(os.path.join(golden_dir, "cost_guide_kv_per_token.json")))
    m = g["model"]
    for row in g["rows"]:
        per_key = row["KiB_per_token"] * acc.KiB // m["layers"]          # one layer: 4 KiB at Hkv = 8
        assert acc.decode_kv_bytes([1], row["Hkv"], m["D"], 100) == per_key
        assert acc.decode_kv_bytes([37], row["Hkv"], m["D"], 100) == 37 * per_key
        # ragged batch by hand: 3 + 0 (empty) + 0 (negative) + 100 (clamped) + 99 keys
        assert acc.decode_kv_bytes([3, 0, -2, 10 ** 6, 99], row["Hkv"], m["D"], 100) == 202 * per_key
    assert acc.decode_kv_bytes([1], 8, 128, 10) == 4 * acc.KiB
    # the ragged workload's seeded lengths: 1,102,942 keys x 4 KiB
    lens = ai.RAGGED_DECODE.kv_lens()
    assert int(lens.sum()) == 1102942
    assert acc.decode_kv_bytes(lens, 8, 128, 32768) == 1102942 * 4096 == 4517650432


def test_decode_q8_kv_bytes_counts_the_int8_layout():
    """int8 caches: the bytes of the codes and binary16 scales the seeded
    generator actually lays out for those keys (K and V), counted from the
    arrays themselves; 272 B per key and KV head at D = 128 by hand
    (2 x (128 codes + 4 scales x 2 B))."""
    assert acc.decode_q8_kv_bytes([1], 1, 128, 10) == 2 * (128 + 4 * 2) == 272
    for D, Hkv, lens, Lmax in [(32, 1, [5], 8), (64, 2, [7, 0, 3], 10), (128, 8, [1, 9], 9), (256, 3, [4, 12], 6)]:
        case = ai.DecodeCase("q8_bytes", 90, B=len(lens), Hq=Hkv, Hkv=Hkv, Lmax=Lmax, D=D, lens_lo=0, lens_hi=0,
                             fixed_lens=lens)
        counted = 0
        for b, n, kq, vq in case.iter_q8_seqs():
            if n:
                counted += sum(x.nbytes for x in (*kq, *vq))
        assert acc.decode_q8_kv_bytes(lens, Hkv, D, Lmax) == counted, (D, Hkv, lens)


def test_decode_flops_is_the_pages_per_token_count():
    """A decode row over n keys costs the compute-share section's 4 Hq D t
    FLOPs (t = n), and equals a one-row causal prefill over the same n keys
    (bottom-right: the row sees them all)."""
    for lens, Hq, D, Lmax in [([1], 32, 128, 10), ([5, 0, 300, -4, 70000], 32, 128, 32768), ([17, 2], 64, 256, 16)]:
        n = np.minimum(np.maximum(np.asarray(lens), 0), Lmax)
        want = sum(acc.attention_flops_at(Hq, D, int(t), 1) for t in n)
        assert acc.decode_flops(lens, Hq, D, Lmax) == want
        assert acc.decode_flops(lens, Hq, D, Lmax) == sum(
            acc.prefill_flops(1, Hq, D, 1, int(t), True) for t in n if t > 0)


# ---------------------------------------------------------------------------
# 3. Closed form: zero scores.  lse_i = ln(#visible keys), out_i = mean of them.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("Lq,Lk,causal", [(16, 16, True), (5, 13, True), (7, 7, False), (1, 9, True)])
def test_zero_scores_closed_form(Lq, Lk, causal):
    rng = np.random.default_rng(11)
    q = rng.standard_normal((2, 4, Lq, 8))
    k = rng.standard_normal((2, 2, Lk, 8))
    v = rng.standard_normal((2, 2, Lk, 8))
    out, lse = oracle.attention(q, k, v, causal, 0.0)
    cnt = np.array([(i + 1 + Lk - Lq) if causal else Lk for i in range(Lq)], dtype=np.float64)
    np.testing.assert_allclose(lse, np.broadcast_to(np.log(cnt), lse.shape), rtol=0, atol=1e-14)
    csum = np.cumsum(v, axis=2)                          # prefix sums over keys
    for h in range(4):
        hk = h // 2
        want = csum[:, hk, (cnt - 1).astype(int), :] / cnt[None, :, None]
        np.testing.assert_allclose(out[:, h], want, rtol=0, atol=1e-13)
    out0, lse0 = oracle.attention(np.zeros_like(q), k, v, causal, 0.7)
    np.testing.assert_allclose(out0, out, atol=1e-14)
    np.testing.assert_allclose(lse0, lse, atol=1e-14)


# ---------------------------------------------------------------------------
# 4. Invariants.
# ---------------------------------------------------------------------------
def test_softmax_rows_sum_to_one_and_respect_the_mask():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 2, 6, 4))
    k = rng.standard_normal((1, 1, 9, 4))
    P = oracle.attention_probs(q, k, True, 0.9)
    np.testing.assert_allclose(P.sum(-1), 1.0, atol=1e-15)
    assert np.all(P[..., ~ref.visible_mask(6, 9, True)] == 0)
    assert np.all(P[..., ref.visible_mask(6, 9, True)] > 0)


def test_identical_v_rows_give_that_row():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 4, 10, 8))
    k = rng.standard_normal((1, 2, 10, 8))
    row = rng.standard_normal(8)
    v = np.broadcast_to(row, (1, 2, 10, 8)).copy()
    out, _ = oracle.attention(q, k, v, True, 0.5)
    np.testing.assert_allclose(out, np.broadcast_to(row, out.shape), atol=1e-14)


def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(4)
    G, Hkv = 3, 2
    q = rng.standard_normal((2, G * Hkv, 7, 8))
    k = rng.standard_normal((2, Hkv, 11, 8))
    v = rng.standard_normal((2, Hkv, 11, 8))
    o1, l1 = oracle.attention(q, k, v, True, 0.4)
    o2, l2 = oracle.attention(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), True, 0.4)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-14)


def test_two_key_row_is_logistic():
    # one query, two keys: weights (sigma(s0-s1), sigma(s1-s0)), also for huge scores
    for sc in (0.37, 50.0, 900.0):
        q = np.array([[[[1.0, 2.0]]]])
        k = np.array([[[[0.5, -1.0], [2.0, 0.25]]]])
        P = oracle.attention_probs(q, k, False, sc)
        s0, s1 = sc * (0.5 - 2.0), sc * (2.0 + 0.5)
        e = math.exp(-(s1 - s0))                      # s1 > s0 here
        np.testing.assert_allclose(P[0, 0, 0], [e / (1.0 + e), 1.0 / (1.0 + e)], rtol=1e-14, atol=1e-300)
        assert np.all(np.isfinite(P))


def test_decode_equals_last_row_of_prefill():
    rng = np.random.default_rng(5)
    B, Hq, Hkv, L, D = 3, 4, 2, 12, 8
    q_full = rng.standard_normal((B, Hq, L, D))
    k = rng.standard_normal((B, Hkv, L, D))
    v = rng.standard_normal((B, Hkv, L, D))
    out, lse = oracle.attention(q_full, k, v, True, 0.35)
    lens = np.array([L, L, L])
    od, ld = oracle.decode(q_full[:, :, -1], k, v, lens, 0.35)
    np.testing.assert_allclose(od, out[:, :, -1], atol=1e-14)
    np.testing.assert_allclose(ld, lse[:, :, -1], atol=1e-14)
    # ragged: sequence b sees its first n keys only, whatever follows in the cache
    lens = np.array([5, 12, 1])
    kc, vc = k.copy(), v.copy()
    kc[0, :, 5:] = np.nan
    vc[0, :, 5:] = np.nan
    kc[2, :, 1:] = np.nan
    vc[2, :, 1:] = np.nan
    od, ld = oracle.decode(q_full[:, :, 4], kc, vc, lens, 0.35)
    o5, l5 = oracle.attention(q_full[:1, :, :5], k[:1, :, :5], v[:1, :, :5], True, 0.35)
    np.testing.assert_allclose(od[0], o5[0, :, -1], atol=1e-14)
    np.testing.assert_allclose(od[2], np.repeat(v[2, :, 0], 2, axis=0), atol=1e-14)
    np.testing.assert_allclose(ld[2], 0.35 * np.einsum("hd,hd->h", q_full[2, :, 4], np.repeat(k[2, :, 0], 2, axis=0)),
                               atol=1e-14)


def test_decode_empty_and_clamped_lengths():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((2, 2, 4))
    k = rng.standard_normal((2, 1, 6, 4))
    v = rng.standard_normal((2, 1, 6, 4))
    od, ld = oracle.decode(q, k, v, np.array([0, 99]), 0.5)
    assert np.all(od[0] == 0) and np.all(np.isneginf(ld[0]))
    o6, l6 = oracle.decode(q, k, v, np.array([6, 6]), 0.5)
    np.testing.assert_array_equal(od[1], o6[1])
    np.testing.assert_array_equal(ld[1], l6[1])


def test_chunked_prefill_equals_tail_of_full():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, 2, 20, 8))
    k = rng.standard_normal((1, 1, 20, 8))
    v = rng.standard_normal((1, 1, 20, 8))
    full, lf = oracle.attention(q, k, v, True, 0.3)
    tail, lt = oracle.attention(q[:, :, -6:], k, v, True, 0.3)
    np.testing.assert_allclose(tail, full[:, :, -6:], atol=1e-14)
    np.testing.assert_allclose(lt, lf[:, :, -6:], atol=1e-14)


@pytest.mark.parametrize("chunk", [1, 3, 4, 7, 16])
def test_split_kv_combine_matches_unsplit(chunk):
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 2, 1, 8))
    k = rng.standard_normal((1, 2, 16, 8))
    v = rng.standard_normal((1, 2, 16, 8))
    want, lw = oracle.attention(q, k, v, False, 0.6)
    outs, lses = [], []
    for s in range(0, 16, chunk):
        o, l_ = oracle.attention(q, k[:, :, s:s + chunk], v[:, :, s:s + chunk], False, 0.6)
        outs.append(o)
        lses.append(l_)
    o, l_ = oracle.combine_partials(outs, lses)
    np.testing.assert_allclose(o, want, atol=1e-14)
    np.testing.assert_allclose(l_, lw, atol=1e-14)
    # an empty chunk (lse = -inf) changes nothing
    o2, l2 = oracle.combine_partials(outs + [np.zeros_like(outs[0])], lses + [np.full_like(lses[0], -np.inf)])
    np.testing.assert_allclose(o2, want, atol=1e-14)


def test_sampled_rows_equal_full_rows():
    rng = np.random.default_rng(9)
    B, Hq, Hkv, Lq, Lk, D = 1, 4, 2, 40, 64, 8
    q = rng.standard_normal((B, Hq, Lq, D))
    k = rng.standard_normal((B, Hkv, Lk, D))
    v = rng.standard_normal((B, Hkv, Lk, D))
    out, lse = oracle.attention(q, k, v, True, 0.3)
    rows = np.stack([np.stack([ai.rows_for_head(99, b, h, Lq, 9) for h in range(Hq)]) for b in range(B)])
    assert rows.shape == (B, Hq, 9)
    assert np.all(rows[..., 0] == 0) and np.all(rows[..., -1] == Lq - 1)
    o, l_ = oracle.attention_rows(q, k, v, rows, True, 0.3)
    for b in range(B):
        for h in range(Hq):
            np.testing.assert_allclose(o[b, h], out[b, h, rows[b, h]], atol=1e-14)
            np.testing.assert_allclose(l_[b, h], lse[b, h, rows[b, h]], atol=1e-14)


def test_causal_with_more_queries_than_keys_has_empty_rows():
    # the page's helper turns a row with no visible key into NaN; so does the oracle
    rng = np.random.default_rng(10)
    out, lse = oracle.attention(rng.standard_normal((1, 1, 4, 2)), rng.standard_normal((1, 1, 2, 2)),
                                rng.standard_normal((1, 1, 2, 2)), True, 1.0)
    assert np.all(np.isnan(out[0, 0, :2])) and np.all(np.isfinite(out[0, 0, 2:]))


# ---------------------------------------------------------------------------
# 5. Brute force on every tiny shape.
# ---------------------------------------------------------------------------
def test_brute_force_enumeration():
    rng = np.random.default_rng(12)
    n = 0
    for B, G, D, causal in itertools.product((1, 2), (1, 2, 4), (1, 2, 8), (False, True)):
        Hkv = 2 if G < 4 else 1
        Hq = G * Hkv
        for Lk in range(1, 9):
            for Lq in range(1, Lk + 1):
                if Lq not in (1, 2, Lk // 2 + 1, Lk):
                    continue
                q = rng.standard_normal((B, Hq, Lq, D))
                k = rng.standard_normal((B, Hkv, Lk, D))
                v = rng.standard_normal((B, Hkv, Lk, D))
                o1, l1 = oracle.attention(q, k, v, causal, 0.41)
                o2, l2 = oracle.brute_attention(q.tolist(), k.tolist(), v.tolist(), causal, 0.41)
                np.testing.assert_allclose(o1, np.array(o2), rtol=0, atol=1e-12)
                np.testing.assert_allclose(l1, np.array(l2), rtol=0, atol=1e-12)
                n += 1
    assert n > 300


# ---------------------------------------------------------------------------
# 5b. Sliding window (causal rows keep their `window` most recent keys).
# ---------------------------------------------------------------------------
def test_window_brute_force_enumeration():
    rng = np.random.default_rng(21)
    n = 0
    for B, G, D in itertools.product((1, 2), (1, 4), (1, 8)):
        Hkv = 2 if G < 4 else 1
        Hq = G * Hkv
        for Lk in range(1, 9):
            for Lq in (1, 2, Lk):
                if Lq > Lk:
                    continue
                for window in (1, 2, 3, 5):
                    q = rng.standard_normal((B, Hq, Lq, D))
                    k = rng.standard_normal((B, Hkv, Lk, D))
                    v = rng.standard_normal((B, Hkv, Lk, D))
                    o1, l1 = oracle.attention(q, k, v, True, 0.37, window=window)
                    o2, l2 = oracle.brute_attention(q.tolist(), k.tolist(), v.tolist(), True, 0.37, window=window)
                    np.testing.assert_allclose(o1, np.array(o2), rtol=0, atol=1e-12)
                    np.testing.assert_allclose(l1, np.array(l2), rtol=0, atol=1e-12)
                    n += 1
    assert n > 300


def _windowed_by_slices(q, k, v, scale, window):
    """Each row as full (unmasked) attention over its own slice of keys: the
    window's definition spelled without any mask."""
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    off = Lk - Lq
    out = np.empty((B, Hq, Lq, D))
    lse = np.empty((B, Hq, Lq))
    for i in range(Lq):
        hi = i + off + 1
        lo = max(0, hi - window)
        o, l_ = oracle.attention(q[:, :, i:i + 1], k[:, :, lo:hi], v[:, :, lo:hi], False, scale)
        out[:, :, i], lse[:, :, i] = o[:, :, 0], l_[:, :, 0]
    return out, lse


@pytest.mark.parametrize("Lq,Lk,window", [(40, 40, 7), (16, 100, 33), (1, 50, 50), (30, 30, 1), (64, 200, 64)])
def test_window_equals_attention_over_each_rows_slice(Lq, Lk, window):
    rng = np.random.default_rng([22, Lq, Lk, window])
    q = rng.standard_normal((1, 4, Lq, 8))
    k = rng.standard_normal((1, 2, Lk, 8))
    v = rng.standard_normal((1, 2, Lk, 8))
    o1, l1 = oracle.attention(q, k, v, True, 0.3, window=window)
    o2, l2 = _windowed_by_slices(q, k, v, 0.3, window)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)
    rows = np.stack([np.stack([np.arange(0, Lq, 3) for _ in range(4)])])
    o3, l3 = oracle.attention_rows(q, k, v, rows, True, 0.3, window=window)
    np.testing.assert_allclose(o3, o1[:, :, ::3], rtol=0, atol=1e-12)
    np.testing.assert_allclose(l3, l1[:, :, ::3], rtol=0, atol=1e-12)


def test_window_special_cases():
    rng = np.random.default_rng(23)
    q = rng.standard_normal((1, 2, 20, 8))
    k = rng.standard_normal((1, 1, 50, 8))
    v = rng.standard_normal((1, 1, 50, 8))
    off = 30
    # a window at least as long as the keys is the plain causal mask
    full = oracle.attention(q, k, v, True, 0.5)
    for w in (50, 51, 1000):
        o, l_ = oracle.attention(q, k, v, True, 0.5, window=w)
        assert np.array_equal(o, full[0]) and np.array_equal(l_, full[1])
    # a window of one key: the row's own position, weight 1
    o, l_ = oracle.attention(q, k, v, True, 0.5, window=1)
    for i in range(20):
        np.testing.assert_allclose(o[0, :, i], np.repeat(v[0, :, i + off], 2, axis=0), rtol=0, atol=1e-15)
        np.testing.assert_allclose(l_[0, :, i], 0.5 * (q[0, :, i] @ k[0, 0, i + off]), rtol=0, atol=1e-12)
    # the window is anchored bottom-right: row i's keys end at i + Lk - Lq
    keep = oracle.visible_mask(20, 50, True, window=4)
    assert [int(np.flatnonzero(r)[0]) for r in keep] == [i + off - 3 for i in range(20)]
    assert [int(np.flatnonzero(r)[-1]) for r in keep] == [i + off for i in range(20)]
    with pytest.raises(ValueError):
        oracle.visible_mask(4, 4, False, window=2)


def test_window_planted_off_by_one_is_caught():
    """A mask that keeps one key too many (j >= i + off - W) differs from the
    slice definition: the slice test above would catch it."""
    rng = np.random.default_rng(24)
    q = rng.standard_normal((1, 1, 12, 4))
    k = rng.standard_normal((1, 1, 30, 4))
    v = rng.standard_normal((1, 1, 30, 4))
    W, off = 5, 18
    i = np.arange(12)[:, None]
    j = np.arange(30)[None, :]
    wrong = (j <= i + off) & (j >= i + off - W)
    s = np.where(wrong, 0.3 * (q[0, 0] @ k[0, 0].T), -np.inf)
    p, _ = ref._softmax_rows(s)
    o_wrong = p @ v[0, 0]
    o_right, _ = _windowed_by_slices(q, k, v, 0.3, W)
    assert np.max(np.abs(o_wrong - o_right[0, 0])) > 1e-3


# ---------------------------------------------------------------------------
# 6. Input recipe.
# ---------------------------------------------------------------------------
def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.0e-3], dtype=np.float32)
    bits = ai.f32_to_bf16_bits(x)
    back = ai.bf16_bits_to_f32(bits)
    # ties go to the even mantissa; others to the nearest representable value
    assert back[1] == 1.0 and back[2] == 1.0 + 2 ** -6 and back[3] == 1.0
    assert back[0] == 1.0 and back[4] == -2.5
    assert abs(back[5] - 3.0e-3) <= 3.0e-3 * 2 ** -8
    y = np.random.default_rng(0).standard_normal(10000, dtype=np.float32)
    yb = ai.bf16_bits_to_f32(ai.f32_to_bf16_bits(y))
    assert np.all(np.abs(yb - y) <= np.abs(y) * 2.0 ** -8)


def test_ragged_lengths_and_nan_tail():
    c = ai.RAGGED_DECODE
    lens = c.kv_lens()
    assert lens.shape == (64,) and lens.min() >= 1024 and lens.max() <= 32768
    small = ai.DecodeCase("t", 4, B=3, Hq=2, Hkv=1, Lmax=16, D=4, lens_lo=3, lens_hi=16)
    kb = small.cache_bits(ai.K_ID)
    ln = small.kv_lens()
    for b in range(3):
        assert not np.any(kb[b, :, :ln[b]] == ai.BF16_NAN_BITS)
        assert np.all(kb[b, :, ln[b]:] == ai.BF16_NAN_BITS)


# ---------------------------------------------------------------------------
# 7. Planted mistakes: each must be caught by one of the pins above.
# ---------------------------------------------------------------------------
def test_planted_wrong_alignment_is_caught(golden_dir, monkeypatch):
    orig = ref.visible_mask
    monkeypatch.setattr(ref, "visible_mask",
                        lambda Lq, Lk, causal, align="bottom_right", window=0: orig(Lq, Lk, causal, "upper_left"))
    with pytest.raises(AssertionError):
        test_page_is_causal_example(golden_dir)


def test_planted_off_by_one_mask_is_caught(monkeypatch):
    def shifted(Lq, Lk, causal, align="bottom_right", window=0):
        if not causal:
            return np.ones((Lq, Lk), bool)
        i = np.arange(Lq)[:, None]
        j = np.arange(Lk)[None, :]
        return j < i + (Lk - Lq)  # drops the diagonal
    monkeypatch.setattr(ref, "visible_mask", shifted)
    with pytest.raises(AssertionError):
        test_zero_scores_closed_form(5, 13, True)


def test_planted_wrong_head_map_is_caught(monkeypatch):
    monkeypatch.setattr(ref, "kv_head_of", lambda h, Hq, Hkv: h % Hkv)
    with pytest.raises(AssertionError):
        test_gqa_equals_mha_with_repeated_kv()


def test_planted_dropped_scale_is_caught(golden_dir, monkeypatch):
    orig = ref.attention_probs

    def noscale(q, k, causal, scale, align="bottom_right"):
        return orig(q, k, causal, 1.0, align)
    monkeypatch.setattr(oracle, "attention_probs", noscale)
    with pytest.raises(AssertionError):
        test_page_is_causal_example(golden_dir)


def test_planted_swapped_k_and_v_is_caught(monkeypatch):
    orig = ref.attention

    def swapped(q, k, v, causal, scale, align="bottom_right"):
        return orig(q, v, k, causal, scale, align)   # scores against V, values from K
    monkeypatch.setattr(oracle, "attention", swapped)
    with pytest.raises(AssertionError):
        test_identical_v_rows_give_that_row()


def test_planted_softmax_over_wrong_axis_is_caught(monkeypatch):
    def wrong_axis(s):
        with np.errstate(invalid="ignore"):
            m = s.max(axis=0, keepdims=True)          # over queries, not keys
            e = np.exp(s - m)
            z = e.sum(axis=0, keepdims=True)
            return e / z, (m + np.log(z))[0]
    monkeypatch.setattr(ref, "_softmax_rows", wrong_axis)
    with pytest.raises(AssertionError):
        test_softmax_rows_sum_to_one_and_respect_the_mask()


def test_planted_accounting_slips_are_caught(golden_dir, monkeypatch):
    """K/V factor of 2 dropped, a 4-byte element, the scales left out of the
    int8 count, one head's FLOPs instead of all heads': each fails a pin."""
    good_kv, good_q8, good_fl = acc.decode_kv_bytes, acc.decode_q8_kv_bytes, acc.decode_flops

    def clamp(lens, Lmax):
        return np.minimum(np.maximum(np.asarray(lens, dtype=np.int64), 0), Lmax)

    slips = [
        ("decode_kv_bytes", lambda l, Hkv, D, Lmax, e=2: int(clamp(l, Lmax).sum()) * Hkv * D * e,
         lambda: test_decode_kv_bytes_is_the_pages_per_token_size(golden_dir)),
        ("decode_kv_bytes", lambda l, Hkv, D, Lmax, e=2: int(clamp(l, Lmax).sum()) * Hkv * D * 2 * 4,
         lambda: test_decode_kv_bytes_is_the_pages_per_token_size(golden_dir)),
        ("decode_kv_bytes", lambda l, Hkv, D, Lmax, e=2: int(np.asarray(l).sum()) * Hkv * D * 2 * e,
         lambda: test_decode_kv_bytes_is_the_pages_per_token_size(golden_dir)),
        ("decode_q8_kv_bytes", lambda l, Hkv, D, Lmax: int(clamp(l, Lmax).sum()) * Hkv * 2 * D,
         test_decode_q8_kv_bytes_counts_the_int8_layout),
        ("decode_flops", lambda l, Hq, D, Lmax: 4 * D * int(clamp(l, Lmax).sum()),
         test_decode_flops_is_the_pages_per_token_count),
    ]
    for name, bad, pin in slips:
        monkeypatch.setattr(acc, name, bad)
        with pytest.raises(AssertionError):
            pin()
        monkeypatch.setattr(acc, "decode_kv_bytes", good_kv)
        monkeypatch.setattr(acc, "decode_q8_kv_bytes", good_q8)
        monkeypatch.setattr(acc, "decode_flops", good_fl)


def test_planted_log2_lse_is_caught(monkeypatch):
    orig = ref._softmax_rows

    def log2_lse(s):
        p, lse = orig(s)
        return p, lse / np.log(2.0)
    monkeypatch.setattr(ref, "_softmax_rows", log2_lse)
    with pytest.raises(AssertionError):
        test_zero_scores_closed_form(16, 16, True)
