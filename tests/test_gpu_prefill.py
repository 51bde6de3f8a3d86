"""GPU parity of attn_prefill against the CPU oracle (element by element).

Full-oracle cases cover every output; long sequences compare 64 seeded rows
per (batch, head) (rows 0 and Lq-1 included), computed one by one by the
oracle's row mode.  Shapes span several tiles and ragged tails, every head
dim, several group sizes, causal and full attention, Lq < Lk (bottom-right
mask) and the workloads used for measurement.
"""
import numpy as np
import pytest
import torch

import attn_inputs as ai
import oracle

pytestmark = pytest.mark.gpu

from gpu_util import DEV, PrefillData, check_lse, check_out, to_dev, to_np  # noqa: E402


@pytest.fixture(scope="module")
def attn():
    import exact_attention_30_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def run_full(attn, case, scale=None):
    d = PrefillData(case)
    sc = case.scale if scale is None else scale
    out, lse = attn.prefill(d.q, d.k, d.v, causal=case.causal, scale=sc)
    torch.cuda.synchronize()
    q, k, v = d.f64()
    ro, rl = oracle.attention(q, k, v, case.causal, sc)
    e = check_out(to_np(out), ro, case.name)
    check_lse(to_np(lse), rl, case.name)
    return e


def run_sampled(attn, case, nrows=64):
    d = PrefillData(case)
    out, lse = attn.prefill(d.q, d.k, d.v, causal=case.causal, scale=case.scale)
    torch.cuda.synchronize()
    rows = np.stack([np.stack([ai.rows_for_head(case.wid * 1000 + case.variant, b, h, case.Lq, nrows)
                               for h in range(case.Hq)]) for b in range(case.B)])
    q, k, v = d.f64()
    ro, rl = oracle.attention_rows(q, k, v, rows, case.causal, case.scale)
    go = to_np(out)
    gl = to_np(lse)
    bi = np.arange(case.B)[:, None, None]
    hi = np.arange(case.Hq)[None, :, None]
    check_out(go[bi, hi, rows], ro, case.name)
    check_lse(gl[bi, hi, rows], rl, case.name)


SMALL = [
    ai.TINY,
    ai.PrefillCase("ragged_G2_L100_D64", 11, B=2, Hq=4, Hkv=2, Lq=100, Lk=100, D=64),
    ai.PrefillCase("chunk_G3_Lq77_Lk200_D128", 12, B=1, Hq=6, Hkv=2, Lq=77, Lk=200, D=128),
    ai.PrefillCase("full_G1_Lq33_Lk129_D256", 13, B=1, Hq=2, Hkv=2, Lq=33, Lk=129, D=256, causal=False),
    ai.PrefillCase("causal_G8_L130_D128", 14, B=1, Hq=8, Hkv=1, Lq=130, Lk=130, D=128),
    ai.PrefillCase("one_row_Lk300_D128", 15, B=2, Hq=4, Hkv=1, Lq=1, Lk=300, D=128),
    ai.PrefillCase("one_by_one_D64", 16, B=1, Hq=1, Hkv=1, Lq=1, Lk=1, D=64),
    ai.PrefillCase("full_G4_Lq65_Lk65_D64", 17, B=3, Hq=8, Hkv=2, Lq=65, Lk=65, D=64, causal=False),
    ai.PrefillCase("chunk_G2_Lq40_Lk1000_D256", 18, B=1, Hq=4, Hkv=2, Lq=40, Lk=1000, D=256),
    ai.PrefillCase("causal_G16_L257_D128", 19, B=1, Hq=16, Hkv=1, Lq=257, Lk=257, D=128),
    ai.PrefillCase("causal_G6_L300_D64", 20, B=1, Hq=12, Hkv=2, Lq=300, Lk=300, D=64),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: c.name)
def test_prefill_small(attn, case):
    run_full(attn, case)


SPLIT_CASES = [SMALL[1], SMALL[2], SMALL[3], SMALL[8], SMALL[9], SMALL[10]]


@pytest.mark.parametrize("splits", [1, 2, 5, 13])
@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: c.name)
def test_prefill_forced_splits(attn, case, splits):
    """Every key-split count (including more ranges than tiles, which leaves
    some ranges empty) matches the oracle."""
    d = PrefillData(case)
    out, lse = attn.prefill_ex(d.q, d.k, d.v, causal=case.causal, scale=case.scale, splits=splits)
    torch.cuda.synchronize()
    q, k, v = d.f64()
    ro, rl = oracle.attention(q, k, v, case.causal, case.scale)
    check_out(to_np(out), ro, f"{case.name} splits={splits}")
    check_lse(to_np(lse), rl, f"{case.name} splits={splits}")


def test_prefill_split_independence_and_workspace(attn):
    """The merge of key ranges equals the single-range result up to fp32
    rounding; a caller workspace gives the same bits as the pool."""
    case = ai.PrefillCase("split_G4_Lq300_Lk2000_D128", 21, B=2, Hq=8, Hkv=2, Lq=300, Lk=2000, D=128)
    d = PrefillData(case)
    o1, l1 = attn.prefill_ex(d.q, d.k, d.v, causal=True, scale=case.scale, splits=1)
    o7, l7 = attn.prefill_ex(d.q, d.k, d.v, causal=True, scale=case.scale, splits=7)
    nb = attn.prefill_workspace_bytes(case.B, case.Hq, case.Hkv, case.Lq, case.Lk, case.D, True, 7)
    assert nb > 0
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    o7w, l7w = attn.prefill_ex(d.q, d.k, d.v, causal=True, scale=case.scale, splits=7, workspace=ws)
    torch.cuda.synchronize()
    a1, a7 = to_np(o1), to_np(o7)
    # Each range rounds its own weights to bf16 against its own maximum, so
    # the two results differ by a few weight roundings (absolute, not
    # relative to the output), well inside the oracle tolerance both meet.
    q, k, v = d.f64()
    ro, rl = oracle.attention(q, k, v, True, case.scale)
    for o, l in ((o1, l1), (o7, l7)):
        check_out(to_np(o), ro, case.name)
        check_lse(to_np(l), rl, case.name)
    assert float(np.abs(a1 - a7).max()) <= 4e-3
    assert float(np.abs(a1 - a7).mean()) <= 2e-4
    assert float(np.abs(to_np(l1) - to_np(l7)).max()) <= 1e-5
    assert torch.equal(o7, o7w) and torch.equal(l7, l7w)
    assert attn.prefill_splits(case.B, case.Hq, case.Hkv, case.Lq, case.Lk, case.D, True, 0) >= 1


def test_prefill_qwen_4k_full(attn):
    run_full(attn, ai.QWEN_4K)


def test_prefill_d256_full(attn):
    run_full(attn, ai.D256)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", [ai.QWEN_16K, ai.QWEN_32K, ai.QWEN_CHUNK], ids=lambda c: c.name)
def test_prefill_long_sampled(attn, case):
    run_sampled(attn, case)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("G", ai.G_SWEEP)
def test_prefill_gsweep_sampled(attn, G):
    run_sampled(attn, ai.gsweep_prefill(G))


# Grids of two or more device rounds run on resident workgroups that each take
# several work items (32-row query blocks here: G = 8 packs one head per wave;
# D = 128 on the two-group kernel, D = 64 on the in-wave kernel).
# 514 and 513 items are not multiples of the 8 XCDs, so the leftover items go
# one each to the first workgroups; one row of every item is checked (causal)
# or every row (full attention over a short key range).
RESIDENT_CASES = [
    ai.PrefillCase("resident_causal_G8_L16432_D128", 75, B=1, Hq=8, Hkv=1, Lq=16432, Lk=16432, D=128),
    ai.PrefillCase("resident_full_G8_Lq16400_Lk300_D128", 76, B=1, Hq=8, Hkv=1, Lq=16400, Lk=300, D=128,
                   causal=False),
    ai.PrefillCase("resident_causal_G8_L16432_D64", 77, B=1, Hq=8, Hkv=1, Lq=16432, Lk=16432, D=64),
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", RESIDENT_CASES, ids=lambda c: c.name)
def test_prefill_resident_workgroups_leftover_items(attn, case):
    assert attn.prefill_splits(case.B, case.Hq, case.Hkv, case.Lq, case.Lk, case.D, case.causal, 0) == 1
    d = PrefillData(case)
    out, lse = attn.prefill(d.q, d.k, d.v, causal=case.causal, scale=case.scale)
    torch.cuda.synchronize()
    q, k, v = d.f64()
    go, gl = to_np(out), to_np(lse)
    if not case.causal:
        ro, rl = oracle.attention(q, k, v, False, case.scale)
        check_out(go, ro, case.name)
        check_lse(gl, rl, case.name)
        return
    nblk = (case.Lq + 31) // 32
    rows1 = np.minimum(np.arange(nblk) * 32 + np.arange(nblk) % 32, case.Lq - 1)
    rows = np.broadcast_to(rows1, (case.B, case.Hq, nblk))
    ro, rl = oracle.attention_rows(q, k, v, rows, True, case.scale)
    bi = np.arange(case.B)[:, None, None]
    hi = np.arange(case.Hq)[None, :, None]
    check_out(go[bi, hi, rows], ro, case.name)
    check_lse(gl[bi, hi, rows], rl, case.name)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_prefill_scale_zero_closed_form(attn, D):
    # zero scores: lse_i = ln(#visible keys) and out_i = mean of the visible V rows
    c = ai.PrefillCase(f"scale0_chunk_D{D}", 21, B=1, Hq=4, Hkv=2, Lq=96, Lk=300, D=D)
    d = PrefillData(c)
    out, lse = attn.prefill(d.q, d.k, d.v, causal=True, scale=0.0)
    torch.cuda.synchronize()
    _, _, v = d.f64()
    cnt = np.arange(c.Lq) + 1 + (c.Lk - c.Lq)
    np.testing.assert_allclose(to_np(lse)[0], np.broadcast_to(np.log(cnt), (4, c.Lq)), atol=1e-5)
    csum = np.cumsum(v[0], axis=1)
    want = np.stack([csum[h // 2][cnt - 1] / cnt[:, None] for h in range(4)])
    check_out(to_np(out)[0], want, "scale0")


@pytest.mark.parametrize("D", [64, 128, 256])
def test_prefill_negative_scale(attn, D):
    # the same logit spread for every head dim (std 1.6, as -0.2 gives at D = 64):
    # the sign of the scale is under test, not a sharper temperature, at which
    # outputs near single V rows reach |out| in [2, 4) and bf16 output rounding
    # alone approaches the 1e-2 bound
    run_full(attn, ai.PrefillCase(f"neg_scale_D{D}", 22, B=1, Hq=4, Hkv=1, Lq=70, Lk=150, D=D),
             scale=-0.2 * (64 / D) ** 0.5)


def test_prefill_identical_v_rows(attn):
    c = ai.PrefillCase("same_v", 23, B=1, Hq=4, Hkv=1, Lq=200, Lk=200, D=128)
    d = PrefillData(c)
    v = d.v[:, :, :1].expand_as(d.v).contiguous()
    out, _ = attn.prefill(d.q, d.k, v, causal=True, scale=c.scale)
    torch.cuda.synchronize()
    want = np.broadcast_to(to_np(v[:, :, :1]), (1, 1, 200, 128))
    np.testing.assert_allclose(to_np(out), np.broadcast_to(want, (1, 4, 200, 128)), atol=1e-2, rtol=0)


def test_prefill_gqa_equals_replicated_mha(attn):
    c = ai.PrefillCase("gqa_vs_mha", 24, B=2, Hq=8, Hkv=2, Lq=190, Lk=190, D=128)
    d = PrefillData(c)
    o1, l1 = attn.prefill(d.q, d.k, d.v, causal=True, scale=c.scale)
    kr = d.k.repeat_interleave(4, dim=1).contiguous()
    vr = d.v.repeat_interleave(4, dim=1).contiguous()
    o2, l2 = attn.prefill(d.q, kr, vr, causal=True, scale=c.scale)
    torch.cuda.synchronize()
    np.testing.assert_allclose(to_np(o1), to_np(o2), atol=1e-2, rtol=0)
    np.testing.assert_allclose(to_np(l1), to_np(l2), atol=1e-4, rtol=0)


def test_prefill_chunk_equals_tail_of_full(attn):
    c = ai.PrefillCase("tail", 25, B=1, Hq=8, Hkv=2, Lq=2048, Lk=2048, D=128)
    d = PrefillData(c)
    full, lf = attn.prefill(d.q, d.k, d.v, causal=True, scale=c.scale)
    tail, lt = attn.prefill(d.q[:, :, -300:].contiguous(), d.k, d.v, causal=True, scale=c.scale)
    torch.cuda.synchronize()
    np.testing.assert_allclose(to_np(tail), to_np(full[:, :, -300:]), atol=1e-2, rtol=0)
    np.testing.assert_allclose(to_np(lt), to_np(lf[:, :, -300:]), atol=1e-4, rtol=0)


def test_prefill_deterministic(attn):
    d = PrefillData(ai.QWEN_4K)
    o1, l1 = attn.prefill(d.q, d.k, d.v, causal=True, scale=ai.QWEN_4K.scale)
    o2, l2 = attn.prefill(d.q, d.k, d.v, causal=True, scale=ai.QWEN_4K.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_prefill_empty_calls(attn):
    q = torch.empty((0, 4, 8, 64), dtype=torch.bfloat16, device=DEV)
    k = torch.empty((0, 1, 8, 64), dtype=torch.bfloat16, device=DEV)
    out, lse = attn.prefill(q, k, k)
    assert out.shape == q.shape
    q = torch.empty((1, 4, 0, 64), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16, device=DEV)
    out, lse = attn.prefill(q, k, k)
    assert out.numel() == 0


def test_prefill_lse_optional(attn):
    d = PrefillData(ai.TINY)
    out, lse = attn.prefill(d.q, d.k, d.v, causal=True, scale=ai.TINY.scale, return_lse=False)
    torch.cuda.synchronize()
    assert lse is None
    q, k, v = d.f64()
    ro, _ = oracle.attention(q, k, v, True, ai.TINY.scale)
    check_out(to_np(out), ro, "no-lse")


# ---- sliding window ------------------------------------------------------------

WINDOW_CASES = [
    (ai.PrefillCase("win37_G2_L300_D64", 41, B=1, Hq=4, Hkv=2, Lq=300, Lk=300, D=64), 37),
    (ai.PrefillCase("win64_chunk_G3_Lq77_Lk200_D128", 42, B=1, Hq=6, Hkv=2, Lq=77, Lk=200, D=128), 64),
    (ai.PrefillCase("win1_G1_L130_D128", 43, B=1, Hq=2, Hkv=2, Lq=130, Lk=130, D=128), 1),
    (ai.PrefillCase("win_ge_Lk_G1_Lq33_Lk129_D128", 44, B=1, Hq=2, Hkv=2, Lq=33, Lk=129, D=128), 200),
    (ai.PrefillCase("win50_G2_L100_D256", 45, B=2, Hq=4, Hkv=2, Lq=100, Lk=100, D=256), 50),
    (ai.PrefillCase("win100_G8_L257_D128", 46, B=1, Hq=8, Hkv=1, Lq=257, Lk=257, D=128), 100),
    (ai.PrefillCase("win65_G4_L1000_D128", 47, B=1, Hq=8, Hkv=2, Lq=1000, Lk=1000, D=128), 65),
]


@pytest.mark.parametrize("splits", [0, 3])
@pytest.mark.parametrize("case,window", WINDOW_CASES, ids=lambda x: x.name if hasattr(x, "name") else str(x))
def test_prefill_window(attn, case, window, splits):
    d = PrefillData(case)
    out, lse = attn.prefill_ex(d.q, d.k, d.v, causal=True, scale=case.scale, window=window, splits=splits)
    torch.cuda.synchronize()
    q, k, v = d.f64()
    ro, rl = oracle.attention(q, k, v, True, case.scale, window=window)
    check_out(to_np(out), ro, f"{case.name} splits={splits}")
    check_lse(to_np(lse), rl, f"{case.name} splits={splits}")


def test_prefill_window_long_sampled(attn):
    """Qwen3-8B heads at 16K with a 4096-key window, 64 sampled rows per head."""
    case, window = ai.QWEN_16K, 4096
    d = PrefillData(case)
    out, lse = attn.prefill_ex(d.q, d.k, d.v, causal=True, scale=case.scale, window=window)
    torch.cuda.synchronize()
    rows = np.stack([np.stack([ai.rows_for_head(case.wid * 1000 + case.variant, b, h, case.Lq, 64)
                               for h in range(case.Hq)]) for b in range(case.B)])
    q, k, v = d.f64()
    ro, rl = oracle.attention_rows(q, k, v, rows, True, case.scale, window=window)
    bi = np.arange(case.B)[:, None, None]
    hi = np.arange(case.Hq)[None, :, None]
    check_out(to_np(out)[bi, hi, rows], ro, "window 4096 at 16K")
    check_lse(to_np(lse)[bi, hi, rows], rl, "window 4096 at 16K")


def test_prefill_window_at_least_lk_is_causal(attn):
    case = WINDOW_CASES[0][0]
    d = PrefillData(case)
    o1, l1 = attn.prefill(d.q, d.k, d.v, causal=True, scale=case.scale)
    o2, l2 = attn.prefill_ex(d.q, d.k, d.v, causal=True, scale=case.scale, window=case.Lk)
    o3, l3 = attn.prefill_ex(d.q, d.k, d.v, causal=True, scale=case.scale, window=10 * case.Lk)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(o1, o3) and torch.equal(l1, l3)
