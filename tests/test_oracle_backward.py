"""Pins for the attention gradients of the oracle (oracle/backward.py).

The gradients are pinned to things other than their own formulas: central
finite differences of the forward definition, PyTorch's autograd in float64
on the CPU (a separate implementation of the same forward), the closed form
of zero scale, the two sum rules that softmax attention obeys, and the
selective evaluation agreeing with the full one.  The planted-mistake test
shows that the finite-difference pin rejects the plausible slips (a dropped
softmax-Jacobian term, a missing scale, the wrong head grouping).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import backward as bw
from oracle import reference as ref


def _inputs(B, Hq, Hkv, Lq, Lk, D, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, Hq, Lq, D)), rng.standard_normal((B, Hkv, Lk, D)),
            rng.standard_normal((B, Hkv, Lk, D)), rng.standard_normal((B, Hq, Lq, D)))


def _loss(q, k, v, dout, causal, scale, window=0):
    out, _ = oracle.attention(q, k, v, causal, scale, window=window)
    return float((out * dout).sum())


def _finite_diff(q, k, v, dout, causal, scale, window=0, h=1e-6):
    grads = []
    for which in range(3):
        base = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(base[which])
        for idx in np.ndindex(*g.shape):
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[which][idx] += h
            minus[which][idx] -= h
            g[idx] = (_loss(*plus, dout, causal, scale, window) - _loss(*minus, dout, causal, scale, window)) / (2 * h)
        grads.append(g)
    return grads


CASES = [
    # (B, Hq, Hkv, Lq, Lk, D, causal, window)
    (1, 2, 1, 3, 5, 4, True, 0),
    (1, 2, 2, 4, 4, 3, False, 0),
    (2, 4, 2, 3, 6, 2, True, 2),
    (1, 3, 1, 1, 4, 3, True, 0),
]


@pytest.mark.parametrize("case", CASES)
def test_backward_matches_finite_differences(case):
    B, Hq, Hkv, Lq, Lk, D, causal, window = case
    q, k, v, dout = _inputs(B, Hq, Hkv, Lq, Lk, D, [40, Lq, Lk, D])
    dq, dk, dv = bw.attention_backward(q, k, v, dout, causal, 0.45, window=window)
    fq, fk, fv = _finite_diff(q, k, v, dout, causal, 0.45, window)
    for got, want in ((dq, fq), (dk, fk), (dv, fv)):
        np.testing.assert_allclose(got, want, rtol=0, atol=2e-7)


def _torch_grads(q, k, v, dout, causal, scale, window=0):
    """Autograd of an independent float64 PyTorch forward on the CPU."""
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v)]
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    kk = t[1].repeat_interleave(G, dim=1)
    vv = t[2].repeat_interleave(G, dim=1)
    s = scale * torch.matmul(t[0], kk.transpose(-1, -2))
    if causal:
        i = torch.arange(Lq)[:, None]
        j = torch.arange(Lk)[None, :]
        keep = j <= i + (Lk - Lq)
        if window:
            keep &= j > i + (Lk - Lq) - window
        s = s.masked_fill(~keep, float("-inf"))
    out = torch.matmul(torch.softmax(s, dim=-1), vv)
    (out * torch.tensor(dout, dtype=torch.float64)).sum().backward()
    return [x.grad.numpy() for x in t]


@pytest.mark.parametrize("shape,causal,window", [
    ((2, 4, 2, 33, 47, 16), True, 0),
    ((1, 8, 1, 20, 20, 8), False, 0),
    ((1, 4, 4, 17, 40, 8), True, 9),
    ((2, 6, 3, 64, 64, 32), True, 1),
])
def test_backward_matches_torch_autograd(shape, causal, window):
    q, k, v, dout = _inputs(*shape, [41, *shape])
    got = bw.attention_backward(q, k, v, dout, causal, 0.3, window=window)
    want = _torch_grads(q, k, v, dout, causal, 0.3, window)
    for g, w in zip(got, want):
        np.testing.assert_allclose(g, w, rtol=1e-10, atol=1e-11)


def test_backward_zero_scale_closed_form():
    """scale 0: every visible key has weight 1/n_i, so dq = dk = 0 and
    dv_j = sum over the rows i that see j of dout_i / n_i."""
    B, Hq, Hkv, Lq, Lk, D = 1, 4, 2, 5, 9, 3
    q, k, v, dout = _inputs(B, Hq, Hkv, Lq, Lk, D, 42)
    dq, dk, dv = bw.attention_backward(q, k, v, dout, True, 0.0)
    assert np.all(dq == 0) and np.all(dk == 0)
    want = np.zeros_like(v)
    for h in range(Hq):
        for i in range(Lq):
            n = i + (Lk - Lq) + 1
            for j in range(n):
                want[0, h // 2, j] += dout[0, h, i] / n
    np.testing.assert_allclose(dv, want, rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 5)])
def test_backward_sum_rules(causal, window):
    """Shifting every key by one vector leaves each row's softmax unchanged,
    so the dk of a KV head sum to zero; the weights of a row sum to one, so
    the dv of a KV head sum to the dout of its query heads."""
    B, Hq, Hkv, Lq, Lk, D = 2, 6, 2, 11, 19, 5
    q, k, v, dout = _inputs(B, Hq, Hkv, Lq, Lk, D, [43, causal, window])
    _, dk, dv = bw.attention_backward(q, k, v, dout, causal, 0.7, window=window)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    want = dout.reshape(B, Hkv, Hq // Hkv, Lq, D).sum(axis=(2, 3))
    np.testing.assert_allclose(dv.sum(axis=2), want, atol=1e-12)


def test_backward_delta_is_rowsum_of_out_times_dout():
    q, k, v, dout = _inputs(1, 2, 1, 7, 12, 4, 44)
    out, _ = oracle.attention(q, k, v, True, 0.5)
    P = oracle.attention_probs(q, k, True, 0.5)
    dp = np.stack([dout[0, h] @ v[0, 0].T for h in range(2)])[None]     # one KV head
    np.testing.assert_allclose(bw.delta_rows(out, dout), (P * dp).sum(-1), atol=1e-12)


@pytest.mark.parametrize("causal,window", [(True, 0), (False, 0), (True, 37)])
def test_backward_sampled_equals_full(causal, window):
    B, Hq, Hkv, Lq, Lk, D = 1, 4, 2, 600, 700, 8
    q, k, v, dout = _inputs(B, Hq, Hkv, Lq, Lk, D, [45, causal, window])
    dq, dk, dv = bw.attention_backward(q, k, v, dout, causal, 0.35, window=window)
    qr = np.array([0, 1, 255, 511, 512, 599])
    kr = np.array([0, 99, 100, 650, 699])
    sq, sk, sv = bw.attention_backward_sampled(q, k, v, dout, causal, 0.35, qr, kr, window=window)
    np.testing.assert_allclose(sq, dq[:, :, qr], rtol=0, atol=1e-12)
    np.testing.assert_allclose(sk, dk[:, :, kr], rtol=0, atol=1e-12)
    np.testing.assert_allclose(sv, dv[:, :, kr], rtol=0, atol=1e-12)
    # one KV head only: the other head's entries stay NaN
    sq1, sk1, _ = bw.attention_backward_sampled(q, k, v, dout, causal, 0.35, qr, kr, window=window, heads=[1])
    assert np.isnan(sq1[:, :2]).all() and np.isnan(sk1[:, 0]).all()
    np.testing.assert_allclose(sk1[:, 1], dk[:, 1, kr], rtol=0, atol=1e-12)


def test_backward_planted_mistakes_are_caught():
    """Each slip gives gradients that the finite differences reject."""
    q, k, v, dout = _inputs(1, 2, 1, 3, 5, 4, 46)
    sc = 0.45
    fq, fk, fv = _finite_diff(q, k, v, dout, True, sc)
    keep = ref.visible_mask(3, 5, True)

    def grads(no_delta=False, no_scale_dk=False, wrong_group=False):
        dq = np.zeros_like(q); dk = np.zeros_like(k); dv = np.zeros_like(v)
        for h in range(2):
            hk = 0
            s = np.where(keep, sc * (q[0, h] @ k[0, hk].T), -np.inf)
            p, _ = ref._softmax_rows(s)
            dp = dout[0, h] @ v[0, hk].T
            ds = p * dp if no_delta else p * (dp - (p * dp).sum(1, keepdims=True))
            dq[0, h] = sc * ds @ k[0, hk]
            if not (wrong_group and h == 1):
                dk[0, hk] += (1.0 if no_scale_dk else sc) * ds.T @ q[0, h]
                dv[0, hk] += p.T @ dout[0, h]
        return dq, dk, dv

    ok = grads()
    assert all(np.allclose(a, b, atol=2e-7) for a, b in zip(ok, (fq, fk, fv)))
    for slip in ({"no_delta": True}, {"no_scale_dk": True}, {"wrong_group": True}):
        bad = grads(**slip)
        assert not all(np.allclose(a, b, atol=2e-7) for a, b in zip(bad, (fq, fk, fv))), slip


@pytest.mark.parametrize("causal,window", [(True, 0), (False, 0), (True, 6)])
def test_backward_from_forward_with_exact_forward_is_the_gradient(causal, window):
    """Given the exact out and lse, the saved-statistics form equals the
    gradient pinned above; given a perturbed out, only dq and dk move."""
    q, k, v, dout = _inputs(2, 4, 2, 13, 21, 6, [47, causal, window])
    out, lse = oracle.attention(q, k, v, causal, 0.4, window=window)
    want = bw.attention_backward(q, k, v, dout, causal, 0.4, window=window)
    got = bw.attention_backward_from_forward(q, k, v, out, dout, lse, causal, 0.4, window=window)
    for g, w in zip(got, want):
        np.testing.assert_allclose(g, w, rtol=0, atol=1e-12)
    bent = bw.attention_backward_from_forward(q, k, v, out * (1 + 1e-3), dout, lse, causal, 0.4, window=window)
    assert np.array_equal(bent[2], got[2])
    assert not np.allclose(bent[0], got[0], atol=1e-9)


@pytest.mark.parametrize("causal,window", [(True, 0), (False, 0), (True, 29)])
def test_backward_from_forward_sampled_equals_full(causal, window):
    q, k, v, dout = _inputs(2, 4, 2, 150, 230, 8, [48, causal, window])
    out, lse = oracle.attention(q, k, v, causal, 0.3, window=window)
    out = out + 1e-3 * np.sin(np.arange(out.size)).reshape(out.shape)     # any saved out, not the exact one
    full = bw.attention_backward_from_forward(q, k, v, out, dout, lse, causal, 0.3, window=window)
    qr, kr = np.array([0, 7, 100, 149]), np.array([0, 1, 80, 229])
    got = bw.attention_backward_from_forward_sampled(q, k, v, out, dout, lse, causal, 0.3, qr, kr, window=window)
    np.testing.assert_allclose(got[0], full[0][:, :, qr], rtol=0, atol=1e-12)
    np.testing.assert_allclose(got[1], full[1][:, :, kr], rtol=0, atol=1e-12)
    np.testing.assert_allclose(got[2], full[2][:, :, kr], rtol=0, atol=1e-12)
