"""GPU parity of attn_decode / attn_decode_ex against the CPU oracle.

Cache rows past each sequence's length hold NaN, so any read past the end
shows up as a non-finite output.  Covers the ragged 64-sequence workload in
full, the group-size sweep, edge lengths (0, 1, block and chunk boundaries,
beyond Lmax), every head dim, group sizes that need several query-column
blocks or head groups, and independence from the chunk size.
"""
import numpy as np
import pytest
import torch

import attn_inputs as ai
import oracle

pytestmark = pytest.mark.gpu

from gpu_util import DEV, check_lse, check_out, decode_cache_on_device, to_dev, to_np  # noqa: E402


@pytest.fixture(scope="module")
def attn():
    import exact_attention_30_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


class OracleBySeq:
    """The oracle one sequence at a time, fed while the caches are built."""

    def __init__(self, case, qb):
        self.case = case
        self.q = ai.bf16_bits_to_f64(qb)
        self.out = np.zeros((case.B, case.Hq, case.D))
        self.lse = np.full((case.B, case.Hq), -np.inf)

    def __call__(self, b, n, kb, vb):
        o, l_ = oracle.decode(self.q[b:b + 1], ai.bf16_bits_to_f64(kb)[None], ai.bf16_bits_to_f64(vb)[None],
                              np.array([n]), self.case.scale)
        self.out[b], self.lse[b] = o[0], l_[0]


def run_case(attn, case, split_keys=None, lens=None):
    lens = case.kv_lens() if lens is None else np.asarray(lens, dtype=np.int32)
    qb = case.q_bits()
    ref = OracleBySeq(case, qb)
    kc, vc = decode_cache_on_device(case, lens, per_seq=ref)
    q = to_dev(qb)
    lens_d = torch.from_numpy(lens).to(DEV)
    if split_keys is None:
        out = attn.decode(q, kc, vc, lens_d, scale=case.scale)
        out2, lse = attn.decode_ex(q, kc, vc, lens_d, scale=case.scale)
        torch.cuda.synchronize()
        assert torch.equal(out, out2)
    else:
        out, lse = attn.decode_ex(q, kc, vc, lens_d, scale=case.scale, split_keys=split_keys)
        torch.cuda.synchronize()
    check_out(to_np(out), ref.out, case.name)
    check_lse(to_np(lse), ref.lse, case.name)
    del kc, vc
    return out


@pytest.mark.timeout(900)
def test_decode_ragged_64_sequences(attn):
    run_case(attn, ai.RAGGED_DECODE)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("G", ai.G_SWEEP)
def test_decode_gsweep(attn, G):
    run_case(attn, ai.gsweep_decode(G))


EDGE = ai.DecodeCase("edges_D128_G4", 41, B=12, Hq=8, Hkv=2, Lmax=1100, D=128, lens_lo=0, lens_hi=0,
                     fixed_lens=[0, 1, 2, 31, 32, 33, 255, 256, 257, 1099, 1100, 5000])


@pytest.mark.parametrize("split", [128, 256, 384, 1024, 2048])
def test_decode_edge_lengths(attn, split):
    run_case(attn, EDGE, split_keys=split)


MANY = ai.DecodeCase("many_pieces_D128_G4", 46, B=2, Hq=8, Hkv=2, Lmax=11200, D=128, lens_lo=0, lens_hi=0,
                     fixed_lens=[11111, 300])


def test_decode_many_pieces_per_segment(attn):
    """The smallest split spreads the 11,111-key sequence over well over 64
    pieces (a few 32-key blocks each), so the merge of a row's pieces runs
    over several rounds of lanes, with groups of four and a remainder."""
    run_case(attn, MANY, split_keys=128)


def test_decode_negative_length_is_empty(attn):
    c = ai.DecodeCase("neg_len", 42, B=2, Hq=4, Hkv=4, Lmax=300, D=64, lens_lo=0, lens_hi=0, fixed_lens=[-5, 300])
    lens = np.array([-5, 300], dtype=np.int32)
    qb = c.q_bits()
    ref = OracleBySeq(c, qb)
    kc, vc = decode_cache_on_device(c, np.maximum(lens, 0), per_seq=ref)
    out, lse = attn.decode_ex(to_dev(qb), kc, vc, torch.from_numpy(lens).to(DEV), scale=c.scale)
    torch.cuda.synchronize()
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))
    check_out(to_np(out)[1], ref.out[1], "neg_len")


@pytest.mark.parametrize("D,G,Hkv", [(64, 1, 3), (64, 8, 2), (256, 4, 2), (256, 1, 2), (128, 16, 2),
                                     (128, 32, 1), (128, 48, 1), (128, 80, 1), (64, 64, 1), (256, 64, 1)])
def test_decode_head_dims_and_groups(attn, D, G, Hkv):
    c = ai.DecodeCase(f"D{D}_G{G}", 43, B=3, Hq=G * Hkv, Hkv=Hkv, Lmax=900, D=D, lens_lo=1, lens_hi=900,
                      variant=D * 100 + G)
    run_case(attn, c, split_keys=256)


def test_decode_split_size_independence(attn):
    c = ai.DecodeCase("split_indep", 44, B=4, Hq=16, Hkv=4, Lmax=5000, D=128, lens_lo=100, lens_hi=5000)
    lens = c.kv_lens()
    kc, vc = decode_cache_on_device(c, lens)
    q = to_dev(c.q_bits())
    ld = torch.from_numpy(lens).to(DEV)
    res = [attn.decode_ex(q, kc, vc, ld, scale=c.scale, split_keys=s) for s in (128, 512, 1024, 8192)]
    torch.cuda.synchronize()
    for o, l_ in res[1:]:
        np.testing.assert_allclose(to_np(o), to_np(res[0][0]), atol=1e-2, rtol=0)
        np.testing.assert_allclose(to_np(l_), to_np(res[0][1]), atol=1e-5, rtol=0)


def test_decode_equals_last_prefill_row(attn):
    B, Hq, Hkv, L, D = 2, 8, 2, 777, 128
    c = ai.PrefillCase("dec_vs_pre", 45, B=B, Hq=Hq, Hkv=Hkv, Lq=L, Lk=L, D=D)
    q, k, v = to_dev(c.q_bits()), to_dev(c.k_bits()), to_dev(c.v_bits())
    full, lf = attn.prefill(q, k, v, causal=True, scale=c.scale)
    lens = torch.full((B,), L, dtype=torch.int32, device=DEV)
    od, ld = attn.decode_ex(q[:, :, -1].contiguous(), k, v, lens, scale=c.scale, split_keys=256)
    torch.cuda.synchronize()
    np.testing.assert_allclose(to_np(od), to_np(full[:, :, -1]), atol=1e-2, rtol=0)
    np.testing.assert_allclose(to_np(ld), to_np(lf[:, :, -1]), atol=1e-4, rtol=0)


def test_decode_caller_workspace(attn):
    c = ai.DecodeCase("ws", 46, B=3, Hq=8, Hkv=2, Lmax=3000, D=128, lens_lo=500, lens_hi=3000)
    lens = c.kv_lens()
    kc, vc = decode_cache_on_device(c, lens)
    q = to_dev(c.q_bits())
    ld = torch.from_numpy(lens).to(DEV)
    need = attn.decode_multi_workspace_bytes(c.B, c.Hq, c.Hkv, 1, c.Lmax, c.D)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    q4 = q[:, :, None, :].contiguous()
    o1, l1 = attn.decode_multi_ex(q4, kc, vc, ld, scale=c.scale, split_keys=256, workspace=ws)
    o2, l2 = attn.decode_ex(q, kc, vc, ld, scale=c.scale, split_keys=256)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, :, 0], o2) and torch.equal(l1[:, :, 0], l2)
    with pytest.raises(attn.AttnError):
        attn.decode_multi_ex(q4, kc, vc, ld, scale=c.scale, split_keys=256, workspace=ws[:-1])


def test_decode_deterministic(attn):
    c = ai.DecodeCase("det", 47, B=8, Hq=32, Hkv=8, Lmax=4096, D=128, lens_lo=1, lens_hi=4096)
    lens = c.kv_lens()
    kc, vc = decode_cache_on_device(c, lens)
    q = to_dev(c.q_bits())
    ld = torch.from_numpy(lens).to(DEV)
    a = attn.decode(q, kc, vc, ld, scale=c.scale)
    b = attn.decode(q, kc, vc, ld, scale=c.scale)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ---- several new rows per sequence (speculative verification) ---------------

def multi_q_bits(case, T):
    return ai.normal_bf16_bits((case.B, case.Hq, T, case.D), [case.wid, 0, case.variant, 1000 + T])


def multi_reference(case, T, qb, lens, window=0):
    """Oracle per sequence: the last min(n, T) rows attend [0, n) with the
    bottom-right causal mask (and the window, if any); rows that see no key
    are 0 / -inf."""
    q = ai.bf16_bits_to_f64(qb)
    out = np.zeros((case.B, case.Hq, T, case.D))
    lse = np.full((case.B, case.Hq, T), -np.inf)
    for b, n, kb, vb in case.iter_seqs(lens):
        if n == 0:
            continue
        m = min(n, T)
        o, l_ = oracle.attention(q[b:b + 1, :, T - m:], ai.bf16_bits_to_f64(kb)[None], ai.bf16_bits_to_f64(vb)[None],
                                 True, case.scale, window=window)
        out[b, :, T - m:], lse[b, :, T - m:] = o[0], l_[0]
    return out, lse


MULTI = [
    # (T, case, lens): n < T, n = T, block edges, several column blocks and head groups
    (4, ai.DecodeCase("multi_T4_G4_D128", 31, B=8, Hq=8, Hkv=2, Lmax=320, D=128, lens_lo=0, lens_hi=0,
                      fixed_lens=[0, 1, 3, 4, 5, 33, 100, 300]), None),
    (16, ai.DecodeCase("multi_T16_G4_D128", 32, B=3, Hq=8, Hkv=2, Lmax=256, D=128, lens_lo=0, lens_hi=0,
                       fixed_lens=[16, 17, 250]), None),
    (16, ai.DecodeCase("multi_T16_G8_D64_two_groups", 33, B=3, Hq=8, Hkv=1, Lmax=256, D=64, lens_lo=0, lens_hi=0,
                       fixed_lens=[5, 64, 200]), None),
    (2, ai.DecodeCase("multi_T2_G1_D256", 34, B=3, Hq=2, Hkv=2, Lmax=128, D=256, lens_lo=0, lens_hi=0,
                      fixed_lens=[1, 2, 77]), None),
    (7, ai.DecodeCase("multi_T7_G6_D128", 35, B=4, Hq=12, Hkv=2, Lmax=2048, D=128, lens_lo=0, lens_hi=0,
                      fixed_lens=[6, 7, 1000, 2048]), None),
    (4, ai.DecodeCase("multi_T4_ragged_B16_G4", 36, B=16, Hq=32, Hkv=8, Lmax=4096, D=128, lens_lo=64, lens_hi=4096),
     None),
]


@pytest.mark.parametrize("T,case,_", MULTI, ids=lambda x: x.name if hasattr(x, "name") else str(x))
def test_decode_multi_parity(attn, T, case, _):
    lens = case.kv_lens()
    qb = multi_q_bits(case, T)
    kc, vc = decode_cache_on_device(case, lens)
    ro, rl = multi_reference(case, T, qb, lens)
    out, lse = attn.decode_multi(to_dev(qb), kc, vc, torch.from_numpy(lens).to(DEV), scale=case.scale)
    torch.cuda.synchronize()
    check_out(to_np(out), ro, case.name)
    check_lse(to_np(lse), rl, case.name)


# the MULTI cases whose row groups have more than 32 rows (the wide kernel's domain)
WIDE = [m for m in MULTI if m[1].Hq // m[1].Hkv * m[0] > 32]


@pytest.mark.parametrize("mode", ["wide", "main"])
@pytest.mark.parametrize("T,case,_", WIDE, ids=lambda x: x.name if hasattr(x, "name") else str(x))
def test_decode_multi_wide_kernel_parity(attn, mode, T, case, _):
    """Both kernels for wide row groups (each chosen explicitly at small sizes)."""
    lens = case.kv_lens()
    qb = multi_q_bits(case, T)
    kc, vc = decode_cache_on_device(case, lens)
    ro, rl = multi_reference(case, T, qb, lens)
    out, lse = attn.decode_multi_ex(to_dev(qb), kc, vc, torch.from_numpy(lens).to(DEV), scale=case.scale,
                                    kernel=mode)
    torch.cuda.synchronize()
    check_out(to_np(out), ro, f"{case.name} wide={mode}")
    check_lse(to_np(lse), rl, f"{case.name} wide={mode}")


@pytest.mark.parametrize("T,window,idx", [(16, 100, 2), (16, 1, 1), (7, 30, 4)])
def test_decode_multi_wide_kernel_window(attn, T, window, idx):
    """The wide kernel with a window: keys before the earliest window start
    hold NaN and must not be read."""
    case = MULTI[idx][1]
    lens = case.kv_lens()
    qb = multi_q_bits(case, T)
    kc, vc = decode_cache_on_device(case, lens)
    for b, n in enumerate(lens):
        start = max(0, int(min(n, case.Lmax)) - T - window + 1)
        if start > 0:
            kc[b, :, :start] = float("nan")
            vc[b, :, :start] = float("nan")
    ro, rl = multi_reference(case, T, qb, lens, window=window)
    out, lse = attn.decode_multi_ex(to_dev(qb), kc, vc, torch.from_numpy(lens).to(DEV), scale=case.scale,
                                    window=window, kernel="wide")
    torch.cuda.synchronize()
    check_out(to_np(out), ro, f"{case.name} window={window} wide")
    check_lse(to_np(lse), rl, f"{case.name} window={window} wide")


@pytest.mark.timeout(600)
def test_decode_multi_wide_auto_at_scale(attn):
    """T = 16 at Qwen3-8B heads over a 32768-key ragged cache: large enough
    that the library picks the wide kernel by itself (its bits equal the
    forced run's and differ from the other kernel's), and it matches the
    oracle on every sequence."""
    T = 16
    case = ai.DecodeCase("multi_T16_B4_L32768", 38, B=4, Hq=32, Hkv=8, Lmax=32768, D=128, lens_lo=0, lens_hi=0,
                         fixed_lens=[32768, 1, 20000, 31])
    lens = case.kv_lens()
    qb = multi_q_bits(case, T)
    kc, vc = decode_cache_on_device(case, lens)
    q, ld = to_dev(qb), torch.from_numpy(lens).to(DEV)
    o_auto, l_auto = attn.decode_multi(q, kc, vc, ld, scale=case.scale)
    o_on, l_on = attn.decode_multi_ex(q, kc, vc, ld, scale=case.scale, kernel="wide")
    o_off, _ = attn.decode_multi_ex(q, kc, vc, ld, scale=case.scale, kernel="main")
    torch.cuda.synchronize()
    assert torch.equal(o_auto, o_on) and torch.equal(l_auto, l_on)
    assert not torch.equal(o_on, o_off)
    ro, rl = multi_reference(case, T, qb, lens)
    check_out(to_np(o_auto), ro, case.name)
    check_lse(to_np(l_auto), rl, case.name)


@pytest.mark.timeout(600)
def test_decode_multi_d256_wide_group_long_cache(attn):
    """D = 256 with 64 query rows per KV head (G = 4, T = 16) over a cache of
    32,768 keys: served as two groups of 32 rows (the largest group whose
    accumulators fit beside a block of K and V at this head dim), each
    reading the cache; every sequence against the oracle."""
    T = 16
    case = ai.DecodeCase("multi_T16_G4_D256_L32768", 39, B=2, Hq=16, Hkv=4, Lmax=32768, D=256, lens_lo=0,
                         lens_hi=0, fixed_lens=[32768, 20001])
    lens = case.kv_lens()
    qb = multi_q_bits(case, T)
    kc, vc = decode_cache_on_device(case, lens)
    out, lse = attn.decode_multi(to_dev(qb), kc, vc, torch.from_numpy(lens).to(DEV), scale=case.scale)
    torch.cuda.synchronize()
    ro, rl = multi_reference(case, T, qb, lens)
    check_out(to_np(out), ro, case.name)
    check_lse(to_np(lse), rl, case.name)


def test_decode_multi_one_row_is_decode(attn):
    """T = 1 is attn_decode (same kernel path, identical bits)."""
    case = ai.DecodeCase("multi_T1", 37, B=5, Hq=8, Hkv=2, Lmax=700, D=128, lens_lo=0, lens_hi=0,
                         fixed_lens=[0, 1, 31, 300, 700])
    lens = case.kv_lens()
    kc, vc = decode_cache_on_device(case, lens)
    q3 = to_dev(case.q_bits())
    ld = torch.from_numpy(lens).to(DEV)
    o1, l1 = attn.decode_ex(q3, kc, vc, ld, scale=case.scale)
    om, lm = attn.decode_multi(q3[:, :, None, :].contiguous(), kc, vc, ld, scale=case.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, om[:, :, 0]) and torch.equal(l1, lm[:, :, 0])


def test_decode_multi_caller_workspace(attn):
    T, case = MULTI[4][0], MULTI[4][1]
    lens = case.kv_lens()
    kc, vc = decode_cache_on_device(case, lens)
    q = to_dev(multi_q_bits(case, T))
    ld = torch.from_numpy(lens).to(DEV)
    nb = attn.decode_multi_workspace_bytes(case.B, case.Hq, case.Hkv, T, case.Lmax, case.D)
    assert nb > 0
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    o1, l1 = attn.decode_multi(q, kc, vc, ld, scale=case.scale)
    o2, l2 = attn.decode_multi(q, kc, vc, ld, scale=case.scale, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("T,window,idx", [(1, 64, 0), (4, 37, 0), (16, 100, 2), (7, 1, 4), (4, 4000, 5)])
def test_decode_window(attn, T, window, idx):
    """Sliding window over the ragged cache: keys before the earliest window
    start are not read (the cache there could hold anything)."""
    case = MULTI[idx][1]
    lens = case.kv_lens()
    qb = multi_q_bits(case, T)
    kc, vc = decode_cache_on_device(case, lens)
    # poison every key before the earliest window start: reading it would show as NaN
    for b, n in enumerate(lens):
        start = max(0, int(min(n, case.Lmax)) - T - window + 1)
        if start > 0:
            kc[b, :, :start] = float("nan")
            vc[b, :, :start] = float("nan")
    ro, rl = multi_reference(case, T, qb, lens, window=window)
    out, lse = attn.decode_multi(to_dev(qb), kc, vc, torch.from_numpy(lens).to(DEV), scale=case.scale, window=window)
    torch.cuda.synchronize()
    check_out(to_np(out), ro, f"{case.name} window={window}")
    check_lse(to_np(lse), rl, f"{case.name} window={window}")
