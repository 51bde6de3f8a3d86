"""Seeded synthetic inputs for the attention workloads.

This module is the only code shared by the CPU oracle (``oracle/``), the GPU
parity tests and the bench.  It holds no attention arithmetic: it draws
standard normals, rounds them to bfloat16 and lays them out; it picks ragged
sequence lengths and sampled query rows.

Recipe (the same for every consumer):
  * every tensor is drawn as float32 ``standard_normal`` from
    ``numpy.random.default_rng([workload_id, tensor_id, variant, ...])`` with
    tensor_id q=0, k=1, v=2, lens=3, rows=7, dout=8 (the upstream gradient
    of the backward pass), and rounded to bfloat16 with
    round-to-nearest-even; the bf16 bit patterns (uint16) are what both the
    oracle (widened to float64) and the GPU (as torch.bfloat16) consume;
  * decode caches are drawn per sequence (seed ``[id, t, variant, b]``) for the
    first ``kv_lens[b]`` rows only; rows past the length hold a NaN fill so
    that a kernel which reads past a sequence's end produces NaN;
  * ragged lengths are integers uniform on [lo, hi], both ends inclusive;
  * sampled query rows are {0, Lq-1} plus distinct uniform rows;
  * int8 caches (tensor ids k=11, v=12): per sequence, codes uniform on
    [-128, 127] and one binary16 scale per 32-element block, uniform on
    [0.5, 1.5) * sqrt(3) / 127 (so the elements have about unit variance),
    from one generator, codes first; positions past the length hold code 0
    and a NaN scale.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
import os

import numpy as np

BF16_NAN_BITS = np.uint16(0x7FC0)
F16_NAN_BITS = np.uint16(0x7E00)

Q_ID, K_ID, V_ID, LENS_ID, ROWS_ID, DOUT_ID = 0, 1, 2, 3, 7, 8
KQ_ID, VQ_ID = 11, 12


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Adds 0x7FFF plus the lowest kept bit to the float32 pattern and keeps the
    upper 16 bits.  Inputs here are finite normals, so no NaN handling.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


def normal_bf16_bits(shape, seed) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def q8_codes_scales(shape, seed):
    """(codes int8 [..., D], scale bits uint16 [..., D/32]) for rows of D elements."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(-128, 127, size=shape, endpoint=True, dtype=np.int16).astype(np.int8)
    sshape = tuple(shape[:-1]) + (shape[-1] // 32,)
    scales = (rng.uniform(0.5, 1.5, size=sshape) * (np.sqrt(3.0) / 127.0)).astype(np.float16)
    return codes, scales.view(np.uint16)


@dataclass
class PrefillCase:
    name: str
    wid: int
    B: int
    Hq: int
    Hkv: int
    Lq: int
    Lk: int
    D: int
    causal: bool = True
    variant: int = 0

    @property
    def scale(self) -> float:
        # the fp32 value 1/sqrt(D), handed unchanged to the GPU and the oracle
        return float(np.float32(1.0 / np.sqrt(self.D)))

    def q_bits(self) -> np.ndarray:
        return normal_bf16_bits((self.B, self.Hq, self.Lq, self.D), [self.wid, Q_ID, self.variant])

    def k_bits(self) -> np.ndarray:
        return normal_bf16_bits((self.B, self.Hkv, self.Lk, self.D), [self.wid, K_ID, self.variant])

    def v_bits(self) -> np.ndarray:
        return normal_bf16_bits((self.B, self.Hkv, self.Lk, self.D), [self.wid, V_ID, self.variant])

    def dout_bits(self) -> np.ndarray:
        return normal_bf16_bits((self.B, self.Hq, self.Lq, self.D), [self.wid, DOUT_ID, self.variant])


@dataclass
class DecodeCase:
    name: str
    wid: int
    B: int
    Hq: int
    Hkv: int
    Lmax: int
    D: int
    lens_lo: int
    lens_hi: int
    variant: int = 0
    fixed_lens: list | None = field(default=None)

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / np.sqrt(self.D)))

    def kv_lens(self) -> np.ndarray:
        if self.fixed_lens is not None:
            return np.asarray(self.fixed_lens, dtype=np.int32)
        if self.lens_lo == self.lens_hi:
            return np.full(self.B, self.lens_lo, dtype=np.int32)
        rng = np.random.default_rng([self.wid, LENS_ID, self.variant])
        return rng.integers(self.lens_lo, self.lens_hi, size=self.B, endpoint=True).astype(np.int32)

    def q_bits(self) -> np.ndarray:
        return normal_bf16_bits((self.B, self.Hq, self.D), [self.wid, Q_ID, self.variant])

    def seq_bits(self, tensor_id: int, b: int, n: int) -> np.ndarray:
        """[Hkv, n, D] rows of sequence b (n = that sequence's length)."""
        return normal_bf16_bits((self.Hkv, n, self.D), [self.wid, tensor_id, self.variant, b])

    def iter_seqs(self, lens: np.ndarray | None = None, workers: int | None = None):
        """Yield (b, n, k_bits [Hkv,n,D], v_bits [Hkv,n,D]) in order of b.

        Sequences are drawn on a thread pool, a few at a time, so that only
        a bounded number of them is held in memory.
        """
        lens = self.kv_lens() if lens is None else lens
        workers = workers or min(16, os.cpu_count() or 1)

        def one(b):
            n = int(min(max(int(lens[b]), 0), self.Lmax))
            if n == 0:
                return b, 0, None, None
            return b, n, self.seq_bits(K_ID, b, n), self.seq_bits(V_ID, b, n)

        with ThreadPoolExecutor(workers) as ex:
            for s0 in range(0, self.B, workers):
                yield from ex.map(one, range(s0, min(self.B, s0 + workers)))

    def q8_seq(self, tensor_id: int, b: int, n: int):
        """int8 rows of sequence b: (codes [Hkv, n, D], scale bits [Hkv, n, D/32])."""
        return q8_codes_scales((self.Hkv, n, self.D), [self.wid, tensor_id, self.variant, b])

    def iter_q8_seqs(self, lens: np.ndarray | None = None):
        """Yield (b, n, (k codes, k scales), (v codes, v scales)) in order of b."""
        lens = self.kv_lens() if lens is None else lens
        for b in range(self.B):
            n = int(min(max(int(lens[b]), 0), self.Lmax))
            if n == 0:
                yield b, 0, None, None
            else:
                yield b, n, self.q8_seq(KQ_ID, b, n), self.q8_seq(VQ_ID, b, n)

    def cache_bits(self, tensor_id: int, lens: np.ndarray | None = None) -> np.ndarray:
        """Full [B, Hkv, Lmax, D] cache; rows past each length are NaN."""
        lens = self.kv_lens() if lens is None else lens
        out = np.full((self.B, self.Hkv, self.Lmax, self.D), BF16_NAN_BITS, dtype=np.uint16)
        for b in range(self.B):
            n = int(min(lens[b], self.Lmax))
            if n > 0:
                out[b, :, :n, :] = self.seq_bits(tensor_id, b, n)
        return out


def sample_rows(Lq: int, n: int, seed) -> np.ndarray:
    """{0, Lq-1} plus n-2 further distinct rows drawn uniformly (sorted)."""
    if Lq <= n:
        return np.arange(Lq, dtype=np.int64)
    rng = np.random.default_rng(seed)
    inner = rng.choice(np.arange(1, Lq - 1), size=n - 2, replace=False)
    return np.sort(np.concatenate([[0, Lq - 1], inner])).astype(np.int64)


def rows_for_head(wid: int, b: int, h: int, Lq: int, n: int = 64) -> np.ndarray:
    return sample_rows(Lq, n, [wid, ROWS_ID, b, h])


# ---------------------------------------------------------------------------
# The workloads.  Shapes follow the Qwen3-8B attention layout (32 query heads,
# 8 KV heads, head dim 128) used throughout the pages, plus a tiny case, a
# group-size sweep and a head-dim-256 case.
# ---------------------------------------------------------------------------
TINY = PrefillCase("tiny_causal_prefill_L256_D64", 1, B=1, Hq=4, Hkv=1, Lq=256, Lk=256, D=64)
QWEN_4K = PrefillCase("qwen3_8b_prefill_L4096", 2, B=1, Hq=32, Hkv=8, Lq=4096, Lk=4096, D=128)
QWEN_16K = PrefillCase("qwen3_8b_prefill_L16384", 3, B=1, Hq=32, Hkv=8, Lq=16384, Lk=16384, D=128, variant=16)
QWEN_32K = PrefillCase("qwen3_8b_prefill_L32768", 3, B=1, Hq=32, Hkv=8, Lq=32768, Lk=32768, D=128, variant=32)
QWEN_CHUNK = PrefillCase("qwen3_8b_chunked_prefill_Lq512_Lk16384", 3, B=1, Hq=32, Hkv=8, Lq=512, Lk=16384,
                         D=128, variant=512)
RAGGED_DECODE = DecodeCase("ragged_gqa_decode_B64_L1024_32768", 4, B=64, Hq=32, Hkv=8, Lmax=32768, D=128,
                           lens_lo=1024, lens_hi=32768)
G_SWEEP = (1, 2, 4, 8, 16, 32, 64)


def gsweep_decode(G: int) -> DecodeCase:
    return DecodeCase(f"gsweep_decode_G{G}_B32_L8192", 5, B=32, Hq=64, Hkv=64 // G, Lmax=8192, D=128,
                      lens_lo=8192, lens_hi=8192, variant=G)


def gsweep_prefill(G: int) -> PrefillCase:
    return PrefillCase(f"gsweep_prefill_G{G}_L8192", 5, B=1, Hq=64, Hkv=64 // G, Lq=8192, Lk=8192, D=128,
                       variant=100 + G)


D256 = PrefillCase("d256_prefill_L4096", 5, B=1, Hq=16, Hkv=8, Lq=4096, Lk=4096, D=256, variant=256)
D256_8K = PrefillCase("d256_prefill_L8192", 5, B=1, Hq=16, Hkv=8, Lq=8192, Lk=8192, D=256, variant=256)
D64_8K = PrefillCase("d64_prefill_L8192", 5, B=1, Hq=32, Hkv=8, Lq=8192, Lk=8192, D=64)
