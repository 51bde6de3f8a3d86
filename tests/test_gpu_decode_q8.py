"""GPU parity of attn_decode_q8 (int8 K/V caches with per-block binary16
scales) against the CPU oracle: the oracle dequantizes each sequence's codes
(oracle.dequantize_q8) and applies the plain attention definition.

Scales of positions past each length hold NaN, and windowed cases poison the
keys before the earliest window start, so any read there shows as NaN.
Covers the ragged 64-sequence workload in full, edge lengths, every head dim,
several group sizes and query rows per sequence, windows, and a caller
workspace.
"""
import numpy as np
import pytest
import torch

import attn_inputs as ai
import oracle

pytestmark = pytest.mark.gpu

from gpu_util import DEV, check_lse, check_out, to_dev, to_np  # noqa: E402


@pytest.fixture(scope="module")
def attn():
    import exact_attention_30_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def q8_cache_on_device(case, lens, per_seq=None):
    """int8 caches and their scales on the device; positions past a length
    hold code 0 and a NaN scale.  per_seq(b, n, k_values, v_values) gets the
    oracle's dequantized rows [Hkv, n, D] of each non-empty sequence."""
    shape = (case.B, case.Hkv, case.Lmax, case.D)
    sshape = (case.B, case.Hkv, case.Lmax, case.D // 32)
    kq = torch.zeros(shape, dtype=torch.int8, device=DEV)
    vq = torch.zeros(shape, dtype=torch.int8, device=DEV)
    ks = torch.full(sshape, float("nan"), dtype=torch.float16, device=DEV)
    vs = torch.full(sshape, float("nan"), dtype=torch.float16, device=DEV)
    for b, n, (kc, ksb), (vc, vsb) in ((b, n, k, v) for b, n, k, v in case.iter_q8_seqs(lens) if n):
        kq[b, :, :n] = torch.from_numpy(kc).to(DEV)
        vq[b, :, :n] = torch.from_numpy(vc).to(DEV)
        ks[b, :, :n] = torch.from_numpy(ksb.view(np.float16)).to(DEV)
        vs[b, :, :n] = torch.from_numpy(vsb.view(np.float16)).to(DEV)
        if per_seq is not None:
            per_seq(b, n, oracle.dequantize_q8(kc, ksb), oracle.dequantize_q8(vc, vsb))
    return kq, ks, vq, vs


def q_bits(case, T):
    return ai.normal_bf16_bits((case.B, case.Hq, T, case.D), [case.wid, 0, case.variant, 2000 + T])


class Reference:
    """Oracle per sequence: the last min(n, T) rows attend [0, n) with the
    bottom-right causal mask (and the window); rows that see no key are
    0 / -inf."""

    def __init__(self, case, T, qb, window=0):
        self.case, self.T, self.window = case, T, window
        self.q = ai.bf16_bits_to_f64(qb)
        self.out = np.zeros((case.B, case.Hq, T, case.D))
        self.lse = np.full((case.B, case.Hq, T), -np.inf)

    def __call__(self, b, n, kv, vv):
        m = min(n, self.T)
        o, l_ = oracle.attention(self.q[b:b + 1, :, self.T - m:], kv[None], vv[None], True, self.case.scale,
                                 window=self.window)
        self.out[b, :, self.T - m:], self.lse[b, :, self.T - m:] = o[0], l_[0]


def run(attn, case, T, window=0, workspace=None):
    lens = case.kv_lens()
    qb = q_bits(case, T)
    ref = Reference(case, T, qb, window)
    kq, ks, vq, vs = q8_cache_on_device(case, lens, per_seq=ref)
    if window:
        # every key before the earliest window start: reading it would give NaN
        for b, n in enumerate(lens):
            start = max(0, int(min(n, case.Lmax)) - T - window + 1)
            if start > 0:
                ks[b, :, :start] = float("nan")
                vs[b, :, :start] = float("nan")
    out, lse = attn.decode_q8(to_dev(qb), kq, ks, vq, vs, torch.from_numpy(lens).to(DEV), scale=case.scale,
                              window=window, workspace=workspace)
    torch.cuda.synchronize()
    check_out(to_np(out), ref.out, f"{case.name} T={T} window={window}")
    check_lse(to_np(lse), ref.lse, f"{case.name} T={T} window={window}")
    return out, lse


RAGGED_Q8 = ai.DecodeCase("q8_ragged_gqa_decode_B64_L1024_32768", 4, B=64, Hq=32, Hkv=8, Lmax=32768, D=128,
                          lens_lo=1024, lens_hi=32768)


def test_q8_decode_ragged_64_sequences(attn):
    run(attn, RAGGED_Q8, 1)


CASES = [
    # (T, case): empty and one-key sequences, block edges, every head dim, group sizes
    # needing one, two and four query-column blocks, two head groups
    (1, ai.DecodeCase("q8_edges_D128_G4", 51, B=10, Hq=8, Hkv=2, Lmax=1100, D=128, lens_lo=0, lens_hi=0,
                      fixed_lens=[0, 1, 31, 32, 33, 64, 95, 1023, 1100, 5000])),
    (1, ai.DecodeCase("q8_D64_G8", 52, B=4, Hq=16, Hkv=2, Lmax=700, D=64, lens_lo=0, lens_hi=0,
                      fixed_lens=[1, 40, 333, 700])),
    (1, ai.DecodeCase("q8_D256_G2", 53, B=3, Hq=4, Hkv=2, Lmax=600, D=256, lens_lo=0, lens_hi=0,
                      fixed_lens=[2, 129, 600])),
    (1, ai.DecodeCase("q8_D128_G32", 54, B=3, Hq=64, Hkv=2, Lmax=900, D=128, lens_lo=0, lens_hi=0,
                      fixed_lens=[17, 500, 900])),
    (4, ai.DecodeCase("q8_T4_G4_D128", 55, B=8, Hq=8, Hkv=2, Lmax=320, D=128, lens_lo=0, lens_hi=0,
                      fixed_lens=[0, 1, 3, 4, 5, 33, 100, 300])),
    (16, ai.DecodeCase("q8_T16_G8_D64_two_groups", 56, B=3, Hq=8, Hkv=1, Lmax=256, D=64, lens_lo=0, lens_hi=0,
                       fixed_lens=[5, 64, 200])),
    (2, ai.DecodeCase("q8_T2_G1_D256", 57, B=3, Hq=2, Hkv=2, Lmax=128, D=256, lens_lo=0, lens_hi=0,
                      fixed_lens=[1, 2, 77])),
    (3, ai.DecodeCase("q8_T3_ragged_B16_G4", 58, B=16, Hq=32, Hkv=8, Lmax=4096, D=128, lens_lo=64, lens_hi=4096)),
]


@pytest.mark.parametrize("T,case", CASES, ids=lambda x: x.name if hasattr(x, "name") else str(x))
def test_q8_decode_parity(attn, T, case):
    run(attn, case, T)


@pytest.mark.parametrize("T,window,idx", [(1, 64, 0), (4, 37, 4), (16, 100, 5), (3, 1000, 7)])
def test_q8_decode_window(attn, T, window, idx):
    run(attn, CASES[idx][1], T, window=window)


def test_q8_decode_caller_workspace_and_determinism(attn):
    T, case = CASES[7]
    nb = attn.decode_multi_workspace_bytes(case.B, case.Hq, case.Hkv, T, case.Lmax, case.D)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    o1, l1 = run(attn, case, T)
    o2, l2 = run(attn, case, T, workspace=ws)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_q8_decode_signed_and_zero_scales(attn):
    """Negative and zero block scales are legal values of the format."""
    case = ai.DecodeCase("q8_signed_scales", 59, B=2, Hq=4, Hkv=1, Lmax=256, D=128, lens_lo=0, lens_hi=0,
                         fixed_lens=[200, 256])
    lens = case.kv_lens()
    qb = q_bits(case, 1)
    kq, ks, vq, vs = q8_cache_on_device(case, lens)
    g = torch.Generator().manual_seed(3)
    flip = (torch.rand(ks.shape, generator=g) < 0.3).to(DEV)
    zero = (torch.rand(ks.shape, generator=g) < 0.1).to(DEV)
    ks = torch.where(flip, -ks, ks).masked_fill(zero, 0.0).contiguous()
    vs = torch.where(flip.flip(-1), -vs, vs).masked_fill(zero.flip(-2), 0.0).contiguous()
    ref = Reference(case, 1, qb)
    ksh, vsh, kqh, vqh = (t.cpu().numpy() for t in (ks, vs, kq, vq))
    for b, n in enumerate(lens):
        ref(b, n, oracle.dequantize_q8(kqh[b, :, :n], ksh[b, :, :n].view(np.uint16)),
            oracle.dequantize_q8(vqh[b, :, :n], vsh[b, :, :n].view(np.uint16)))
    out, lse = attn.decode_q8(to_dev(qb), kq, ks, vq, vs, torch.from_numpy(lens).to(DEV), scale=case.scale)
    torch.cuda.synchronize()
    check_out(to_np(out), ref.out, case.name)
    check_lse(to_np(lse), ref.lse, case.name)
