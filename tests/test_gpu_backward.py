"""GPU parity of attn_backward (dq, dk, dv) against the CPU oracle's gradients.

The kernel is given the forward's out (the oracle's, rounded to bf16) and lse
(the oracle's, as fp32), and is compared with the oracle's gradients computed
from those same saved values (oracle.attention_backward_from_forward: the
weights from the given lse, delta_i = <dout_i, out_i> from the given out).
The end-to-end test feeds the kernel the GPU forward's own out and lse
instead; there the reference keeps the oracle's out, and the bound grows by
what one bf16 step of each out element can move delta_i (see there).

Tolerance, from the arithmetic.  The kernel computes p and ds in fp32 and
rounds them to bf16 (8 significant bits: relative error <= 2^-8) before the
fp32 matrix products, and rounds each result to bf16 (<= 2^-8 of its size).
So every element obeys |gpu - oracle| <= 2^-8 (T + |oracle|) up to fp32
noise, where T is the sum of the absolute values of the terms the element
adds up: T(dq_i) = scale sum_j |ds_ij| |k_j|, T(dk_j) = scale sum_i |ds_ij|
|q_i| and T(dv_j) = sum_i p_ij |dout_i| (elementwise in d, over all G heads
for dk and dv); |ds_ij| is widened by p_ij times a bound on the fp32 error of
dp_ij - delta_i, which matters only where ds vanishes (a one-key window).  The checks, with rms the root mean square of that tensor's
oracle values:
  * every element: |gpu - oracle| <= 2^-7 (T + |oracle|) + 1e-4 rms
    (twice the rounding bound, plus a floor for the fp32 noise),
  * on average:   mean |gpu - oracle| <= 2^-8 rms.
"""
import numpy as np
import pytest
import torch

import attn_inputs as ai
import oracle

pytestmark = pytest.mark.gpu

from gpu_util import DEV, to_dev, to_np  # noqa: E402

GRAD_TERM_REL = 2.0 ** -7
GRAD_MEAN_REL = 2.0 ** -8


@pytest.fixture(scope="module")
def attn():
    import exact_attention_30_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def check_grad(gpu, ref, T, what, extra=0.0):
    """T: the per-element sums of absolute terms (see above); extra: a further
    allowance per element."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite gradient"
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = np.abs(gpu - ref)
    bound = GRAD_TERM_REL * (T + np.abs(ref)) + extra + 1e-4 * rms
    worst = float((err / np.where(bound > 0, bound, 1.0)).max()) if np.all(err[bound == 0] == 0) else np.inf
    assert worst <= 1.0, f"{what}: error reaches {worst:.3f} of its bound"
    mean = float(err.mean()) / rms if rms > 0 else 0.0
    assert mean <= GRAD_MEAN_REL, f"{what}: mean err / rms = {mean:.3e} > {GRAD_MEAN_REL:.3e}"
    return worst, mean


def term_sums(case, q64, k64, v64, g64, o64, lse64, window, qr=None, kr=None, one_step=False):
    """(Tq, Tk, Tv) of the tolerance for the saved out / lse given, at rows qr
    and keys kr (all when None); with one_step, also the allowance (aq, ak)
    for an out that is within one bf16 step (2^-8 of its size) of o64:
    |d delta_i| <= 2^-8 sum_d |dout_id out_id| moves ds_ij by p_ij |d delta_i|,
    so dq_i by scale |d delta_i| sum_j p_ij |k_j| and dk_j by
    scale sum_i p_ij |d delta_i| |q_i|; dv not at all."""
    B, Hq, Lq, D = q64.shape
    Hkv, Lk = k64.shape[1], k64.shape[2]
    G = Hq // Hkv
    qr = np.arange(Lq) if qr is None else np.asarray(qr)
    kr = np.arange(Lk) if kr is None else np.asarray(kr)
    keep = oracle.visible_mask(Lq, Lk, case.causal, window=window)
    delta = (o64 * g64).sum(-1)
    dd = 2.0 ** -8 * np.abs(o64 * g64).sum(-1)
    # fp32 noise of dp_ij - delta_i (two D-term fp32 sums, D <= 2^7 terms):
    # at most 2^-16 sum_d |dout_id| (|v_jd| + |out_id|); taken with max_j |v_jd|
    vmax = np.abs(v64).max(axis=2)                                  # [B, Hkv, D]
    Tq = np.zeros((B, Hq, len(qr), D))
    Tk = np.zeros((B, Hkv, len(kr), D))
    Tv = np.zeros((B, Hkv, len(kr), D))
    aq = np.zeros_like(Tq)
    ak = np.zeros_like(Tk)
    sc = case.scale
    for b in range(B):
        for h in range(Hq):
            hk = h // G
            kk, vv, qq, gg = k64[b, hk], v64[b, hk], q64[b, h], g64[b, h]
            nu = 2.0 ** -16 * (np.abs(gg) * (np.abs(o64[b, h]) + vmax[b, hk])).sum(-1)   # [Lq]
            p = np.where(keep[qr], np.exp(sc * (qq[qr] @ kk.T) - lse64[b, h, qr][:, None]), 0.0)
            ds = p * (gg[qr] @ vv.T - delta[b, h, qr][:, None])
            Tq[b, h] = sc * ((np.abs(ds) + p * nu[qr][:, None]) @ np.abs(kk))
            aq[b, h] = sc * dd[b, h, qr][:, None] * (p @ np.abs(kk))
            p = np.where(keep[:, kr], np.exp(sc * (qq @ kk[kr].T) - lse64[b, h][:, None]), 0.0)
            ds = p * (gg @ vv[kr].T - delta[b, h][:, None])
            Tk[b, hk] += sc * ((np.abs(ds) + p * nu[:, None]).T @ np.abs(qq))
            Tv[b, hk] += p.T @ np.abs(gg)
            ak[b, hk] += sc * (p.T @ (dd[b, h][:, None] * np.abs(qq)))
    if one_step:
        return Tq, Tk, Tv, aq, ak
    return Tq, Tk, Tv



def run(attn, case, window=0, forward_on_gpu=False):
    qb, kb, vb, gb = case.q_bits(), case.k_bits(), case.v_bits(), case.dout_bits()
    q64, k64, v64, g64 = (ai.bf16_bits_to_f64(x) for x in (qb, kb, vb, gb))
    q, k, v, g = to_dev(qb), to_dev(kb), to_dev(vb), to_dev(gb)
    ro, rl = oracle.attention(q64, k64, v64, case.causal, case.scale, window=window)
    ob = ai.f32_to_bf16_bits(ro.astype(np.float32))
    l32 = rl.astype(np.float32)
    if forward_on_gpu:
        out, lse = attn.prefill_ex(q, k, v, causal=case.causal, scale=case.scale, window=window)
    else:
        out = to_dev(ob)
        lse = torch.from_numpy(l32).to(DEV)
    dq, dk, dv = attn.backward(q, k, v, out, g, lse, causal=case.causal, scale=case.scale, window=window)
    torch.cuda.synchronize()
    if forward_on_gpu:
        # the exact gradient (exact out and lse), plus what the GPU out's
        # deviation from the exact out can move delta by
        o64, lse64 = ro, rl
    else:
        o64, lse64 = ai.bf16_bits_to_f64(ob), l32.astype(np.float64)
    wq, wk, wv = oracle.attention_backward_from_forward(q64, k64, v64, o64, g64, lse64, case.causal, case.scale,
                                                        window=window)
    Tq, Tk, Tv, aq, ak = term_sums(case, q64, k64, v64, g64, o64, lse64, window, one_step=True)
    if not forward_on_gpu:
        aq = ak = 0.0
    tag = f"{case.name} window={window}"
    check_grad(to_np(dq), wq, Tq, "dq " + tag, extra=aq)
    check_grad(to_np(dk), wk, Tk, "dk " + tag, extra=ak)
    check_grad(to_np(dv), wv, Tv, "dv " + tag)
    return dq, dk, dv


CASES = [
    ai.PrefillCase("bwd_tiny_G4_D64_L256", 61, B=1, Hq=4, Hkv=1, Lq=256, Lk=256, D=64),
    ai.PrefillCase("bwd_G4_D128_Lq200_Lk333", 62, B=2, Hq=8, Hkv=2, Lq=200, Lk=333, D=128),
    ai.PrefillCase("bwd_full_G1_D128_Lq100_Lk257", 63, B=1, Hq=2, Hkv=2, Lq=100, Lk=257, D=128, causal=False),
    ai.PrefillCase("bwd_G3_D64_L160", 64, B=1, Hq=6, Hkv=2, Lq=160, Lk=160, D=64),
    ai.PrefillCase("bwd_G2_D128_L97", 65, B=2, Hq=4, Hkv=2, Lq=97, Lk=97, D=128),
    ai.PrefillCase("bwd_one_row_D128_Lk300", 66, B=2, Hq=8, Hkv=2, Lq=1, Lk=300, D=128),
    ai.PrefillCase("bwd_G8_D128_L640", 67, B=1, Hq=8, Hkv=1, Lq=640, Lk=640, D=128),
    ai.PrefillCase("bwd_full_G4_D64_Lq33_Lk70", 68, B=1, Hq=4, Hkv=1, Lq=33, Lk=70, D=64, causal=False),
    ai.PrefillCase("bwd_full_G2_D128_Lq300_Lk50", 70, B=1, Hq=4, Hkv=2, Lq=300, Lk=50, D=128, causal=False),
    ai.PrefillCase("bwd_G2_D256_Lq150_Lk260", 71, B=1, Hq=4, Hkv=2, Lq=150, Lk=260, D=256),
    ai.PrefillCase("bwd_full_G1_D256_L70", 72, B=2, Hq=2, Hkv=2, Lq=70, Lk=70, D=256, causal=False),
    # eight heads per dq workgroup (G a multiple of 8), at D = 64 and with Lq < Lk
    ai.PrefillCase("bwd_G16_D64_L333", 73, B=1, Hq=16, Hkv=1, Lq=333, Lk=333, D=64),
    ai.PrefillCase("bwd_G8_D128_Lq200_Lk520", 74, B=2, Hq=16, Hkv=2, Lq=200, Lk=520, D=128),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c.name)
def test_backward_parity(attn, case):
    run(attn, case)


@pytest.mark.parametrize("window,idx", [(1, 0), (100, 1), (37, 3), (64, 6), (1000, 6), (40, 9)])
def test_backward_window(attn, window, idx):
    run(attn, CASES[idx], window=window)


def test_backward_after_gpu_forward(attn):
    """The usual pipeline: the GPU forward's own out and lse feed the backward."""
    run(attn, CASES[1], forward_on_gpu=True)
    run(attn, CASES[6], window=64, forward_on_gpu=True)


def test_backward_caller_workspace_and_determinism(attn):
    case = CASES[1]
    qb, kb, vb, gb = case.q_bits(), case.k_bits(), case.v_bits(), case.dout_bits()
    q, k, v, g = to_dev(qb), to_dev(kb), to_dev(vb), to_dev(gb)
    out, lse = attn.prefill(q, k, v, causal=True, scale=case.scale)
    ws = torch.empty(attn.backward_workspace_bytes(case.B, case.Hq, case.Lq), dtype=torch.uint8, device=DEV)
    a = attn.backward(q, k, v, out, g, lse, causal=True, scale=case.scale)
    b = attn.backward(q, k, v, out, g, lse, causal=True, scale=case.scale, workspace=ws)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


QWEN_BWD_4K = ai.PrefillCase("bwd_qwen3_8b_L4096", 69, B=1, Hq=32, Hkv=8, Lq=4096, Lk=4096, D=128)


def test_backward_stream_order_and_two_streams(attn):
    """The dq kernel runs on a stream of the library's own, forked from and joined back into the
    caller's stream: work enqueued on the caller's stream right after the call (no host
    synchronisation in between) sees the finished gradients, and calls on two streams at once give
    the results of a call on its own."""
    case = QWEN_BWD_4K
    q, k, v, g = to_dev(case.q_bits()), to_dev(case.k_bits()), to_dev(case.v_bits()), to_dev(case.dout_bits())
    out, lse = attn.prefill(q, k, v, causal=True, scale=case.scale)
    ref = attn.backward(q, k, v, out, g, lse, causal=True, scale=case.scale)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(s1):
        a = attn.backward(q, k, v, out, g, lse, causal=True, scale=case.scale)
        ca = [x.clone() for x in a]
    with torch.cuda.stream(s2):
        b = attn.backward(q, k, v, out, g, lse, causal=True, scale=case.scale)
        cb = [x.clone() for x in b]
    torch.cuda.synchronize()
    for name, x, y, z in zip(("dq", "dk", "dv"), ca, cb, ref):
        assert torch.equal(x, z), name + " (first stream)"
        assert torch.equal(y, z), name + " (second stream)"


def test_backward_qwen_4k_sampled(attn):
    """Qwen3-8B heads at L = 4096, in the launch configuration the bench
    times, after the GPU forward: 24 query rows and 24 keys (first, last and
    seeded others) of two KV heads (eight query heads) checked against the
    exact gradient with the one-bf16-step allowance of the end-to-end test;
    every dk and dv of all heads checked against the sum rules (the dk of a
    KV head sum to 0, its dv sum to the dout of its query heads)."""
    case = QWEN_BWD_4K
    qb, kb, vb, gb = case.q_bits(), case.k_bits(), case.v_bits(), case.dout_bits()
    q, k, v, g = to_dev(qb), to_dev(kb), to_dev(vb), to_dev(gb)
    out, lse = attn.prefill(q, k, v, causal=True, scale=case.scale)
    dq, dk, dv = attn.backward(q, k, v, out, g, lse, causal=True, scale=case.scale)
    torch.cuda.synchronize()
    qr = ai.sample_rows(case.Lq, 24, [case.wid, 7, 0])
    kr = ai.sample_rows(case.Lk, 24, [case.wid, 7, 1])
    G = case.Hq // case.Hkv
    heads = [0, 5]
    hq = [h for hk in heads for h in range(hk * G, (hk + 1) * G)]
    q64, k64, v64, g64 = (ai.bf16_bits_to_f64(x) for x in (qb, kb, vb, gb))
    q64, g64, k64, v64 = q64[:, hq], g64[:, hq], k64[:, heads], v64[:, heads]
    ro, rl = oracle.attention(q64, k64, v64, True, case.scale)
    wq, wk, wv = oracle.attention_backward_from_forward_sampled(q64, k64, v64, ro, g64, rl, True, case.scale, qr, kr)
    Tq, Tk, Tv, aq, ak = term_sums(case, q64, k64, v64, g64, ro, rl, 0, qr=qr, kr=kr, one_step=True)
    check_grad(to_np(dq[:, hq][:, :, qr]), wq, Tq, "dq sampled", extra=aq)
    check_grad(to_np(dk[:, heads][:, :, kr]), wk, Tk, "dk sampled", extra=ak)
    check_grad(to_np(dv[:, heads][:, :, kr]), wv, Tv, "dv sampled")
    # sum rules over every key of every KV head
    g_all = ai.bf16_bits_to_f64(gb)
    sk = dk.float().sum(dim=2).cpu().numpy()
    sv = dv.float().sum(dim=2).cpu().numpy()
    want_v = g_all.reshape(case.B, case.Hkv, G, case.Lq, case.D).sum(axis=(2, 3))
    size = np.sqrt(case.Lq * G)                        # typical size of those sums
    assert np.abs(sv - want_v).max() <= 2e-2 * size
    assert np.abs(sk).max() <= 2e-2 * size


QWEN_BWD_16K = ai.PrefillCase("bwd_qwen3_8b_L16384", 70, B=1, Hq=32, Hkv=8, Lq=16384, Lk=16384, D=128)


def test_backward_qwen_16k_sampled(attn):
    """Qwen3-8B heads at L = 16384, the length the backward is measured at,
    in the same launch configuration, after the GPU forward: 16 query rows and
    16 keys (first, last and seeded others) of one KV head (its four query
    heads) checked against the exact gradient with the one-bf16-step
    allowance, as at L = 4096 (the fp64 forward of those four heads is the
    oracle's cost here); every dk and dv of all heads checked against the sum
    rules."""
    case = QWEN_BWD_16K
    qb, kb, vb, gb = case.q_bits(), case.k_bits(), case.v_bits(), case.dout_bits()
    q, k, v, g = to_dev(qb), to_dev(kb), to_dev(vb), to_dev(gb)
    out, lse = attn.prefill(q, k, v, causal=True, scale=case.scale)
    dq, dk, dv = attn.backward(q, k, v, out, g, lse, causal=True, scale=case.scale)
    torch.cuda.synchronize()
    qr = ai.sample_rows(case.Lq, 16, [case.wid, 7, 0])
    kr = ai.sample_rows(case.Lk, 16, [case.wid, 7, 1])
    G = case.Hq // case.Hkv
    heads = [3]
    hq = [h for hk in heads for h in range(hk * G, (hk + 1) * G)]
    q64, k64, v64, g64 = (ai.bf16_bits_to_f64(x) for x in (qb, kb, vb, gb))
    q64, g64, k64, v64 = q64[:, hq], g64[:, hq], k64[:, heads], v64[:, heads]
    ro, rl = oracle.attention(q64, k64, v64, True, case.scale)
    wq, wk, wv = oracle.attention_backward_from_forward_sampled(q64, k64, v64, ro, g64, rl, True, case.scale, qr, kr)
    Tq, Tk, Tv, aq, ak = term_sums(case, q64, k64, v64, g64, ro, rl, 0, qr=qr, kr=kr, one_step=True)
    del ro, rl, q64, k64, v64, g64
    check_grad(to_np(dq[:, hq][:, :, qr]), wq, Tq, "dq sampled", extra=aq)
    check_grad(to_np(dk[:, heads][:, :, kr]), wk, Tk, "dk sampled", extra=ak)
    check_grad(to_np(dv[:, heads][:, :, kr]), wv, Tv, "dv sampled")
    g_all = ai.bf16_bits_to_f64(gb)
    sk = dk.float().sum(dim=2).cpu().numpy()
    sv = dv.float().sum(dim=2).cpu().numpy()
    want_v = g_all.reshape(case.B, case.Hkv, G, case.Lq, case.D).sum(axis=(2, 3))
    size = np.sqrt(case.Lq * G)
    assert np.abs(sv - want_v).max() <= 2e-2 * size
    assert np.abs(sk).max() <= 2e-2 * size
