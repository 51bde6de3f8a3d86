"""Helpers for the GPU parity tests: seeded inputs onto the device, and the
tolerance checks against the oracle.

Tolerance (stated for this method's bf16 inputs and outputs with fp32
softmax statistics and accumulation, unit-normal inputs):
  * out: max |gpu - oracle| <= 1e-2 and mean |gpu - oracle| <= 1e-3;
    where |oracle| >= 4 the bf16 output grid itself is 2^-5 apart (half a
    step is 0.0156 > 1e-2, so a correctly rounded output may miss 1e-2),
    so there the bound is 1e-2 plus half a bf16 step of |oracle|; such
    elements are counted and reported separately;
  * lse: max |gpu - oracle| <= 1e-3.
"""
from __future__ import annotations

import numpy as np
import torch

import attn_inputs as ai

OUT_MAX_ABS = 1e-2
OUT_MEAN_ABS = 1e-3
LSE_MAX_ABS = 1e-3

DEV = torch.device("cuda:0")


def to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_out(gpu, ref, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    err = np.abs(gpu - ref)
    big = np.abs(ref) >= 4.0
    small_max = float(err[~big].max()) if np.any(~big) else 0.0
    assert small_max <= OUT_MAX_ABS, f"{what}: max|err| {small_max:.3e} > {OUT_MAX_ABS}"
    if np.any(big):
        half_step = np.exp2(np.floor(np.log2(np.abs(ref[big]))) - 8)
        bound = OUT_MAX_ABS + half_step
        worst = float(np.max(err[big] / bound))
        print(f"[{what}] {int(big.sum())} elements with |oracle| >= 4: max|err| {float(err[big].max()):.3e}, "
              f"{worst:.2f} of 1e-2 + half a bf16 step")
        assert worst <= 1.0, f"{what}: error above 1e-2 + half a bf16 step where |out| >= 4"
    mean = float(err.mean())
    assert mean <= OUT_MEAN_ABS, f"{what}: mean|err| {mean:.3e} > {OUT_MEAN_ABS}"
    return small_max, mean


def check_lse(gpu, ref, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(gpu), fin), f"{what}: lse finiteness differs"
    if np.any(fin):
        e = float(np.abs(gpu[fin] - ref[fin]).max())
        assert e <= LSE_MAX_ABS, f"{what}: max|dlse| {e:.3e} > {LSE_MAX_ABS}"
        return e
    return 0.0


class PrefillData:
    """A prefill case's bf16 bits on the host and as device tensors."""

    def __init__(self, case: ai.PrefillCase):
        self.case = case
        self.qb, self.kb, self.vb = case.q_bits(), case.k_bits(), case.v_bits()
        self.q, self.k, self.v = to_dev(self.qb), to_dev(self.kb), to_dev(self.vb)

    def f64(self):
        return ai.bf16_bits_to_f64(self.qb), ai.bf16_bits_to_f64(self.kb), ai.bf16_bits_to_f64(self.vb)


def decode_cache_on_device(case: ai.DecodeCase, lens: np.ndarray, per_seq=None):
    """Caches built on the device sequence by sequence; rows past each length hold NaN.

    per_seq(b, n, k_bits, v_bits), if given, is called for every non-empty
    sequence while its bits are on the host (the oracle uses it).
    """
    shape = (case.B, case.Hkv, case.Lmax, case.D)
    kc = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    vc = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    for b, n, kb, vb in case.iter_seqs(lens):
        if n:
            kc[b, :, :n] = to_dev(kb)
            vc[b, :, :n] = to_dev(vb)
            if per_seq is not None:
                per_seq(b, n, kb, vb)
    return kc, vc
