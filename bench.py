"""Benchmark of the attention hot path on one MI355X.

One step = one causal prefill of a Qwen3-8B-shaped layer at 16,384 tokens
(B=1, Hq=32, Hkv=8, D=128) followed by one ragged GQA decode over 64 cached
sequences (lengths uniform in [1024, 32768], same heads).  Inputs are
synthetic, seeded, and resident in HBM before timing starts.  Before the
warmup steps, untimed steps run for at least --prewarm-ms of wall time: the
device's clock takes about that long to settle, and the timed steps then see
its steady state (the per-configuration records are taken the same way).

Printed: one JSON line.  `value` is the prefill's causal TFLOP/s (FLOPs =
4*B*Hq*D*visible (query, key) pairs of the bottom-right mask, divided by the
prefill kernel's mean duration from HIP events on its stream); the decode's
KV-read GB/s (bytes = sum of lengths * Hkv * D * 2 tensors * 2 B over the
split + combine duration, MALL flushed before each decode) is reported beside
it with its own roofline.  `cpu_baseline` times the CPU oracle on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import attn_inputs as ai  # noqa: E402

METRIC = "prefill causal TFLOP/s + decode KV GB/s (Qwen3-8B heads), % of roofline, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
FLUSH_BYTES = 512 << 20        # > the 256 MB Infinity Cache


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--prewarm-ms", type=float, default=150.0,
                   help="untimed steps for at least this long before the warmup steps (the device's clock "
                        "settles over its first ~100 ms of work)")
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle timing")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU seconds per oracle sample")
    p.add_argument("--all-configs", action="store_true",
                   help="time every prefill and decode configuration (one JSON line each) instead of the step")
    p.add_argument("--only", default="",
                   help="with --all-configs: comma-separated substrings; only configurations whose name contains one")
    p.add_argument("--no-configs", action="store_true",
                   help="skip the per-configuration records the default run adds to its JSON line")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device-to-device copy three times (scale for HBM byte counters)")
    p.add_argument("--gemm-ceiling", action="store_true",
                   help="only time torch.matmul (the vendor bf16 GEMM) on square unit-normal and all-zero operands: "
                        "the matrix rate this GPU sustains under its power limit, next to the attention kernels")
    return p.parse_args()


COPY_BYTES = 1 << 30

# the configurations the default run also times (5 calls each) and reports
# under "configs" in its JSON line: every prefill and decode workload shape,
# the backward at 16K and the int8-cache decode
SUB_CONFIGS = (
    "tiny_causal_prefill_L256_D64", "qwen3_8b_prefill_L4096", "qwen3_8b_prefill_L32768",
    "qwen3_8b_chunked_prefill_Lq512_Lk16384", "d256_prefill_L4096",
    "gsweep_prefill_G1_L8192", "gsweep_prefill_G8_L8192", "gsweep_prefill_G64_L8192",
    "gsweep_decode_G1_B32_L8192", "gsweep_decode_G8_B32_L8192", "gsweep_decode_G64_B32_L8192",
    "qwen3_8b_backward_L16384", "q8_ragged_gqa_decode_B64_L1024_32768_T1",
)


def gemm_ceiling():
    """bf16 GEMM C = A B (torch.matmul, the vendor library) at n = 8192 and
    16384: operands unit-normal (the attention inputs' distribution) and all
    zero (little switching activity, so little power).  One JSON line each:
    median of 10 timed calls after 3 untimed."""
    import torch
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    for n in (8192, 16384):
        a = torch.randn(n, n, device=dev, dtype=torch.bfloat16, generator=g)
        b = torch.randn(n, n, device=dev, dtype=torch.bfloat16, generator=g)
        for data in ("unit_normal", "zeros"):
            if data == "zeros":
                a.zero_()
                b.zero_()
            for _ in range(3):
                torch.matmul(a, b)
            torch.cuda.synchronize()
            ts = []
            for _ in range(10):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                torch.matmul(a, b)
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            ms = sorted(ts)[len(ts) // 2]
            tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
            print(json.dumps({"gemm_ceiling": {"n": n, "dtype": "bf16", "data": data, "ms": round(ms, 4),
                                               "TFLOP/s": round(tf, 1), "frac_bf16_peak": round(tf / 2500.0, 4)}}),
                  flush=True)
        del a, b


def copy_calibration():
    """A copy kernel of known size: reads and writes COPY_BYTES per launch."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(7)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": COPY_BYTES, "launches": 3}), flush=True)


# the sources of the kernels the default bench step launches (and of their launch shapes)
BENCH_SOURCES = ("api.hip", "common.h", "decode.hip", "kernels.h", "prefill.hip")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "exact_attention_30_amd", "csrc")
    for f in BENCH_SOURCES:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def read_traffic(kernel: str, src_hash: str):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        line = line.strip()
        if line.startswith("#") or "=" not in line:
            continue
        k, v = (x.strip() for x in line.split("=", 1))
        vals[k] = v
    if vals.get("source_hash") != src_hash:
        return None
    try:
        return float(vals[f"{kernel}.hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def to_dev(bits, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def build_decode_cache(case: ai.DecodeCase, lens, dev):
    import torch
    shape = (case.B, case.Hkv, case.Lmax, case.D)
    kc = torch.zeros(shape, dtype=torch.bfloat16, device=dev)
    vc = torch.zeros(shape, dtype=torch.bfloat16, device=dev)
    for b, n, kb, vb in case.iter_seqs(lens):
        if n:
            kc[b, :, :n] = to_dev(kb, dev)
            vc[b, :, :n] = to_dev(vb, dev)
    return kc, vc


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return os.cpu_count() or 1


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


def host_info() -> dict:
    """The host the oracle ran on: its logical CPUs (nproc), the CPUs this
    process may use, and the CPU model; `cores` beside it is the BLAS thread
    count the oracle actually used."""
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    return {"nproc": os.cpu_count() or 1, "usable_cpus": usable, "cpu": cpu_model()}


def cpu_prefill_baseline(case: ai.PrefillCase, qb, kb, vb, seconds: float):
    """The oracle's row mode on sampled query rows of the same prefill.

    Rows are drawn per head; the rate is (4*D*visible keys of the rows
    computed) / CPU seconds, in TFLOP/s."""
    import oracle
    q = ai.bf16_bits_to_f64(qb)
    k = ai.bf16_bits_to_f64(kb)
    v = ai.bf16_bits_to_f64(vb)
    off = case.Lk - case.Lq
    R = 2
    spent, flops, rows_done = 0.0, 0.0, 0
    while spent < seconds:
        rows = np.stack([np.stack([ai.sample_rows(case.Lq, R, [case.wid, 99, R, h]) for h in range(case.Hq)])])
        t = time.perf_counter()
        oracle.attention_rows(q, k, v, rows, True, case.scale)
        dt = time.perf_counter() - t
        spent += dt
        flops += 4.0 * case.D * float(np.sum(rows + off + 1))
        rows_done += rows.size
        R = min(case.Lq, R * 2)
    return {"value": flops / spent / 1e12, "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"{rows_done} query rows (sampled per head, all 32 heads) of the L=16384 causal prefill, "
                      f"fp64 numpy row mode, {spent:.1f} s", **host_info()}


def cpu_decode_baseline(case: ai.DecodeCase, lens, seconds: float):
    import oracle
    q = ai.bf16_bits_to_f64(case.q_bits())
    spent, nbytes, seqs = 0.0, 0, 0
    for b, n, kb, vb in case.iter_seqs(lens, workers=4):
        if n == 0:
            continue
        k64, v64 = ai.bf16_bits_to_f64(kb)[None], ai.bf16_bits_to_f64(vb)[None]
        t = time.perf_counter()
        oracle.decode(q[b:b + 1], k64, v64, np.array([n]), case.scale)
        spent += time.perf_counter() - t
        nbytes += n * case.Hkv * case.D * 2 * 2
        seqs += 1
        if spent >= seconds:
            break
    return {"value": nbytes / spent / 1e9, "unit": "GB/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"first {seqs} of the 64 ragged sequences, fp64 numpy, {spent:.1f} s (KV bytes counted as bf16)",
            **host_info()}


def _time_ms(fn, iters: int, stream, between=None) -> float:
    """Median duration of fn() from HIP events recorded on `stream`; `between`
    runs outside the timed window before each call (the MALL flush).  Untimed
    calls first run for at least 100 ms (and at least 3 calls), so that every
    configuration is timed at the clock its own work settles to rather than
    the one the previous configuration or an idle device left behind."""
    import torch
    torch.cuda.synchronize()
    t0, n = time.perf_counter(), 0
    while n < 3 or time.perf_counter() - t0 < 0.1:
        if between is not None:
            between(n)
        fn()
        torch.cuda.synchronize()
        n += 1
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for i, (a, b) in enumerate(evs):
        if between is not None:
            between(i)
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in evs]))


def all_configs(iters: int, only=(), exact=(), emit=None):
    """Every prefill and decode shape of the workload list, timed on the GPU
    (ONLY: name substrings selecting some of them).

    Prefill inputs come from the seeded host generators; the G-sweep decode
    caches (up to 8.6 GB) are filled on the device from a seeded torch
    generator with the same N(0,1)-rounded-to-bf16 distribution, since only
    their timing is taken here (their values are checked in the GPU tests)."""
    import torch
    import exact_attention_30_amd as attn
    from oracle import accounting as acc
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)

    if emit is None:
        def emit(rec):
            print(json.dumps(rec), flush=True)

    def want(name):
        if exact:
            return name in exact
        return not only or any(o in name for o in only)

    prefills = [ai.TINY, ai.QWEN_4K, ai.QWEN_16K, ai.QWEN_32K, ai.QWEN_CHUNK, ai.D256, ai.D256_8K, ai.D64_8K]
    prefills += [ai.gsweep_prefill(G) for G in ai.G_SWEEP]
    for pc in prefills:
        if not want(pc.name):
            continue
        q, k, v = to_dev(pc.q_bits(), dev), to_dev(pc.k_bits(), dev), to_dev(pc.v_bits(), dev)
        out = torch.empty_like(q)
        lse = torch.empty((pc.B, pc.Hq, pc.Lq), dtype=torch.float32, device=dev)
        fn = lambda: attn.prefill(q, k, v, causal=True, scale=pc.scale, out=out, lse=lse)  # noqa: E731
        for _ in range(2):
            fn()
        ms = _time_ms(fn, iters, stream)
        fl = acc.prefill_flops(pc.B, pc.Hq, pc.D, pc.Lq, pc.Lk, True)
        tf = fl / (ms * 1e-3) / 1e12
        emit({"config": pc.name, "kind": "prefill", "B": pc.B, "Hq": pc.Hq, "Hkv": pc.Hkv, "Lq": pc.Lq,
                          "Lk": pc.Lk, "D": pc.D, "ms": round(ms, 4), "flops": fl, "TFLOP/s": round(tf, 1),
                          "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)})
        del q, k, v, out, lse

    # backward (dq, dk, dv from the forward's out and lse) at the Qwen3-8B
    # shapes and the head-dim-256 shape; work counted as 2.5 x the forward's
    # (five matrix products over the visible pairs: QK^T, dO V^T, P^T dO,
    # dS^T Q, dS K)
    for pc in (ai.QWEN_4K, ai.QWEN_16K, ai.D256):
        if not want(pc.name.replace("prefill", "backward")):
            continue
        q, k, v = to_dev(pc.q_bits(), dev), to_dev(pc.k_bits(), dev), to_dev(pc.v_bits(), dev)
        g = to_dev(pc.dout_bits(), dev)
        out, lse = attn.prefill(q, k, v, causal=True, scale=pc.scale)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(attn.backward_workspace_bytes(pc.B, pc.Hq, pc.Lq), dtype=torch.uint8, device=dev)
        fn = lambda: attn.backward(q, k, v, out, g, lse, causal=True, scale=pc.scale, dq=dq, dk=dk, dv=dv,  # noqa: E731
                                   workspace=ws)
        for _ in range(2):
            fn()
        ms = _time_ms(fn, iters, stream)
        fl = 5 * acc.prefill_flops(pc.B, pc.Hq, pc.D, pc.Lq, pc.Lk, True) // 2
        tf = fl / (ms * 1e-3) / 1e12
        emit({"config": pc.name.replace("prefill", "backward"), "kind": "backward", "B": pc.B,
                          "Hq": pc.Hq, "Hkv": pc.Hkv, "Lq": pc.Lq, "Lk": pc.Lk, "D": pc.D, "causal": True,
                          "ms": round(ms, 4), "flops": fl, "TFLOP/s": round(tf, 1),
                          "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)})
        del q, k, v, g, out, lse, dq, dk, dv, ws
    torch.cuda.empty_cache()

    # several new rows per sequence (speculative verification) over the ragged cache
    multi_t = [T for T in (2, 4, 8, 16) if want(f"multi_query_decode_T{T}_ragged_B64")]
    dc = ai.RAGGED_DECODE
    lens = dc.kv_lens()
    kc, vc = build_decode_cache(dc, lens, dev) if multi_t else (None, None)
    dl = torch.from_numpy(lens).to(dev)
    nb = acc.decode_kv_bytes(lens, dc.Hkv, dc.D, dc.Lmax)
    for T in multi_t:
        qm = to_dev(ai.normal_bf16_bits((dc.B, dc.Hq, T, dc.D), [dc.wid, 0, dc.variant, 1000 + T]), dev)
        om = torch.empty_like(qm)
        fn = lambda: attn.decode_multi(qm, kc, vc, dl, scale=dc.scale, out=om, return_lse=False)  # noqa: E731
        for _ in range(2):
            fn()
        ms = _time_ms(fn, iters, stream, between=lambda i: flush.fill_(i & 0xFF))
        gbps = nb / (ms * 1e-3) / 1e9
        emit({"config": f"multi_query_decode_T{T}_ragged_B64", "kind": "decode_multi", "T": T, "B": dc.B,
                          "Hq": dc.Hq, "Hkv": dc.Hkv, "Lmax": dc.Lmax, "D": dc.D, "ms": round(ms, 4), "kv_bytes": nb,
                          "GB/s": round(gbps, 1), "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4),
                          "flops": 4 * dc.D * dc.Hq * T * int(lens.sum())})
    del kc, vc
    torch.cuda.empty_cache()

    # sliding window (4096 keys): prefill at 16K and the ragged decode; work counted on visible keys
    W = 4096
    if want(f"qwen3_8b_prefill_L16384_window{W}"):
        pc = ai.QWEN_16K
        q, k, v = to_dev(pc.q_bits(), dev), to_dev(pc.k_bits(), dev), to_dev(pc.v_bits(), dev)
        out = torch.empty_like(q)
        fn = lambda: attn.prefill_ex(q, k, v, causal=True, scale=pc.scale, window=W, out=out, return_lse=False)  # noqa: E731
        for _ in range(2):
            fn()
        ms = _time_ms(fn, iters, stream)
        i = np.arange(pc.Lq, dtype=np.int64)
        vis = int(np.minimum(W, i + (pc.Lk - pc.Lq) + 1).sum())
        fl = 4 * pc.B * pc.Hq * pc.D * vis
        emit({"config": f"qwen3_8b_prefill_L16384_window{W}", "kind": "prefill", "window": W, "ms": round(ms, 4),
                          "flops": fl, "TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 1),
                          "frac_bf16_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)})
        del q, k, v, out
    if want(f"ragged_gqa_decode_B64_window{W}"):
        dc = ai.RAGGED_DECODE
        lens = dc.kv_lens()
        kc, vc = build_decode_cache(dc, lens, dev)
        dl = torch.from_numpy(lens).to(dev)
        dq = to_dev(dc.q_bits(), dev)[:, :, None, :].contiguous()
        dout = torch.empty_like(dq)
        fn = lambda: attn.decode_multi(dq, kc, vc, dl, scale=dc.scale, window=W, out=dout, return_lse=False)  # noqa: E731
        for _ in range(2):
            fn()
        ms = _time_ms(fn, iters, stream, between=lambda i: flush.fill_(i & 0xFF))
        nb = int(np.minimum(lens, W).sum()) * dc.Hkv * dc.D * 2 * 2
        emit({"config": f"ragged_gqa_decode_B64_window{W}", "kind": "decode", "window": W, "ms": round(ms, 4),
                          "kv_bytes": nb, "GB/s": round(nb / (ms * 1e-3) / 1e9, 1),
                          "frac_hbm_peak": round(nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)})
        del kc, vc
    torch.cuda.empty_cache()

    decodes = [ai.RAGGED_DECODE] + [ai.gsweep_decode(G) for G in ai.G_SWEEP]
    gen = torch.Generator(device=dev)
    bf16_ms = None
    for dc in decodes:
        if not want(dc.name):
            continue
        lens = dc.kv_lens()
        if dc is ai.RAGGED_DECODE:
            kc, vc = build_decode_cache(dc, lens, dev)
        else:
            shape = (dc.B, dc.Hkv, dc.Lmax, dc.D)
            gen.manual_seed(dc.wid * 1000 + dc.Hkv)
            kc = torch.randn(shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
            vc = torch.randn(shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        dq = to_dev(dc.q_bits(), dev)
        dl = torch.from_numpy(lens).to(dev)
        dout = torch.empty_like(dq)
        fn = lambda: attn.decode(dq, kc, vc, dl, scale=dc.scale, out=dout)  # noqa: E731
        for _ in range(2):
            fn()
        ms = _time_ms(fn, iters, stream, between=lambda i: flush.fill_(i & 0xFF))
        nb = acc.decode_kv_bytes(lens, dc.Hkv, dc.D, dc.Lmax)
        gbps = nb / (ms * 1e-3) / 1e9
        emit({"config": dc.name, "kind": "decode", "B": dc.B, "Hq": dc.Hq, "Hkv": dc.Hkv,
                          "Lmax": dc.Lmax, "D": dc.D, "sum_lens": int(lens.sum()), "ms": round(ms, 4),
                          "kv_bytes": nb, "GB/s": round(gbps, 1), "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4),
                          "waves": attn.decode_waves(dc.B, dc.Hq, dc.Hkv, dc.Lmax, dc.D)})
        if dc is ai.RAGGED_DECODE:
            bf16_ms = ms
        del kc, vc
        torch.cuda.empty_cache()

    # int8 (q8_0-style) caches on the ragged workload: codes uniform on
    # [-128, 127], block scales uniform on [0.5, 1.5) * sqrt(3) / 127
    dc = ai.RAGGED_DECODE
    q8_t = [T for T in (1, 4) if want(f"q8_{dc.name}_T{T}")]
    if not q8_t:
        return
    lens = dc.kv_lens()
    shape = (dc.B, dc.Hkv, dc.Lmax, dc.D)
    sshape = (dc.B, dc.Hkv, dc.Lmax, dc.D // 32)
    gen.manual_seed(dc.wid * 1000 + 8)
    kq = torch.randint(-128, 128, shape, generator=gen, device=dev, dtype=torch.int8)
    vq = torch.randint(-128, 128, shape, generator=gen, device=dev, dtype=torch.int8)
    ks = ((torch.rand(sshape, generator=gen, device=dev) + 0.5) * (3 ** 0.5 / 127)).to(torch.float16)
    vs = ((torch.rand(sshape, generator=gen, device=dev) + 0.5) * (3 ** 0.5 / 127)).to(torch.float16)
    dl = torch.from_numpy(lens).to(dev)
    for T in q8_t:
        dq = torch.randn((dc.B, dc.Hq, T, dc.D), generator=gen, device=dev).to(torch.bfloat16)
        dout = torch.empty_like(dq)
        ws = torch.empty(attn.decode_multi_workspace_bytes(dc.B, dc.Hq, dc.Hkv, T, dc.Lmax, dc.D),
                         dtype=torch.uint8, device=dev)
        fn = lambda: attn.decode_q8(dq, kq, ks, vq, vs, dl, scale=dc.scale, out=dout, return_lse=False,  # noqa: E731
                                    workspace=ws)
        for _ in range(2):
            fn()
        ms = _time_ms(fn, iters, stream, between=lambda i: flush.fill_(i & 0xFF))
        nb = acc.decode_q8_kv_bytes(lens, dc.Hkv, dc.D, dc.Lmax)
        gbps = nb / (ms * 1e-3) / 1e9
        rec = {"config": f"q8_{dc.name}_T{T}", "kind": "decode_q8", "B": dc.B, "Hq": dc.Hq, "Hkv": dc.Hkv,
               "T": T, "Lmax": dc.Lmax, "D": dc.D, "sum_lens": int(lens.sum()), "ms": round(ms, 4),
               "kv_bytes": nb, "GB/s": round(gbps, 1), "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4)}
        if T == 1 and bf16_ms is not None:
            rec["bf16_cache_ms"] = round(bf16_ms, 4)
            rec["speedup_vs_bf16_cache"] = round(bf16_ms / ms, 3)
        emit(rec)
    del kq, vq, ks, vs
    torch.cuda.empty_cache()


def main():
    args = parse()
    if args.gemm_ceiling:
        gemm_ceiling()
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only; --gpus {args.gpus} is not supported "
              "(a split of the work across GPUs is not implemented)", file=sys.stderr)
        sys.exit(2)
    if args.all_configs:
        all_configs(max(args.steps, 5), tuple(o for o in args.only.split(",") if o))
        return
    import torch
    import exact_attention_30_amd as attn
    from oracle import accounting as acc

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    # ---- inputs (resident before timing) ------------------------------------
    pc = ai.QWEN_16K
    qb, kb, vb = pc.q_bits(), pc.k_bits(), pc.v_bits()
    q, k, v = to_dev(qb, dev), to_dev(kb, dev), to_dev(vb, dev)
    out = torch.empty_like(q)
    lse = torch.empty((pc.B, pc.Hq, pc.Lq), dtype=torch.float32, device=dev)
    pflops = acc.prefill_flops(pc.B, pc.Hq, pc.D, pc.Lq, pc.Lk, True)

    dc = ai.RAGGED_DECODE
    lens = dc.kv_lens()
    kc, vc = build_decode_cache(dc, lens, dev)
    dq = to_dev(dc.q_bits(), dev)
    dlens = torch.from_numpy(lens).to(dev)
    dout = torch.empty_like(dq)
    dbytes = acc.decode_kv_bytes(lens, dc.Hkv, dc.D, dc.Lmax)
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(i, evs=None):
        if evs:
            evs[0].record(stream)
        attn.prefill(q, k, v, causal=True, scale=pc.scale, out=out, lse=lse)
        if evs:
            evs[1].record(stream)
        flush.fill_(i & 0xFF)
        if evs:
            evs[2].record(stream)
        attn.decode(dq, kc, vc, dlens, scale=dc.scale, out=dout)
        if evs:
            evs[3].record(stream)

    # untimed: steps for at least prewarm_ms of wall time, then the warmup steps
    t_pre = time.perf_counter()
    n_pre = 0
    while (time.perf_counter() - t_pre) * 1e3 < args.prewarm_ms:
        step(n_pre)
        n_pre += 1
        if n_pre % 8 == 0:
            torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    pre_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    dec_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in events]))
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    tflops = pflops / (pre_ms * 1e-3) / 1e12
    gbps = dbytes / (dec_ms * 1e-3) / 1e9

    src = kernel_source_hash()
    ptraffic = read_traffic("prefill", src)
    dtraffic = read_traffic("decode", src)
    rec = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "prewarm_ms": args.prewarm_ms,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "causal prefill L=16384 + ragged GQA decode B=64 (Qwen3-8B heads: Hq=32, Hkv=8, D=128)",
            "prefill": {"B": pc.B, "Hq": pc.Hq, "Hkv": pc.Hkv, "Lq": pc.Lq, "Lk": pc.Lk, "D": pc.D,
                        "causal": True, "flops": pflops, "ms": round(pre_ms, 4)},
            "decode": {"B": dc.B, "Hq": dc.Hq, "Hkv": dc.Hkv, "Lmax": dc.Lmax, "D": dc.D,
                       "lens": "uniform [1024, 32768] seeded", "sum_lens": int(lens.sum()),
                       "kv_bytes": dbytes, "waves": attn.decode_waves(dc.B, dc.Hq, dc.Hkv, dc.Lmax, dc.D),
                       "ms": round(dec_ms, 4), "mall_flushed": True},
            "parallelism": "single GPU",
        },
        "roofline": {"bound": "mfma", "kernel": "prefill_kernel<128,64>", "achieved": round(tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": ptraffic},
        "decode": {"value": round(gbps, 1), "unit": "GB/s",
                   "roofline": {"bound": "hbm", "kernel": "decode_plan_kernel + decode_main_kernel<128,1,false> + decode_combine_kernel<128>",
                                "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": dtraffic}},
        "kernel_source_hash": src,
    }
    if not args.no_configs:
        # the other workloads, timed the same way (fewer calls each), so that
        # one bench line carries every configuration's figure
        del q, k, v, out, lse, kc, vc, dq, dlens, dout, flush
        torch.cuda.empty_cache()
        subs = {}

        def keep(r):
            name = r.pop("config")
            subs[name] = {kk: r[kk] for kk in ("kind", "ms", "TFLOP/s", "frac_bf16_peak", "GB/s", "frac_hbm_peak",
                                               "flops", "kv_bytes") if kk in r}
        all_configs(5, exact=SUB_CONFIGS, emit=keep)
        rec["configs"] = subs
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_prefill_baseline(pc, qb, kb, vb, args.cpu_seconds)
        rec["decode"]["cpu_baseline"] = cpu_decode_baseline(dc, lens, args.cpu_seconds * 0.5)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
