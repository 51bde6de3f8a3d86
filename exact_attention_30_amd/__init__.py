"""Exact GQA attention for MI355X: a thin ctypes binding over libattn.so.

The functions here only check tensors and marshal pointers; every step of the
computation runs in the HIP kernels of libattn.so (see include/attn.h for the
contract).  PyTorch provides device memory and the current stream.  If the
library has not been built, importing this package raises ImportError: there
is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")

ATTN_OK = 0
STATUS_NAMES = {0: "ATTN_OK", -1: "ATTN_ERR_NULL", -2: "ATTN_ERR_SHAPE", -3: "ATTN_ERR_HEADDIM",
                -4: "ATTN_ERR_GQA", -5: "ATTN_ERR_SCALE", -6: "ATTN_ERR_HIP", -7: "ATTN_ERR_SPLIT",
                -8: "ATTN_ERR_WORKSPACE", -9: "ATTN_ERR_KERNEL", -10: "ATTN_ERR_SCRATCH"}


def _load(path: str = LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with __graft_entry__.build() "
                          "(python exact_attention_30_amd/build.py)")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.attn_prefill.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp]
    lib.attn_prefill.restype = i
    lib.attn_prefill_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, i, vp, sz, vp]
    lib.attn_prefill_ex.restype = i
    lib.attn_prefill_splits.argtypes = [i, i, i, i, i, i, i, i, i]
    lib.attn_prefill_splits.restype = i
    lib.attn_prefill_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i, i]
    lib.attn_prefill_workspace_bytes.restype = sz
    lib.attn_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
    lib.attn_decode.restype = i
    lib.attn_decode_ex.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
    lib.attn_decode_noalloc.restype = i
    lib.attn_decode_noalloc_max_bytes.argtypes = []
    lib.attn_decode_noalloc_max_bytes.restype = sz
    lib.attn_decode_ex.restype = i
    lib.attn_decode_multi.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp, sz, vp]
    lib.attn_decode_multi.restype = i
    lib.attn_decode_multi_ex.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, i, vp, sz, vp]
    lib.attn_decode_multi_ex.restype = i
    lib.attn_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, vp, sz, vp]
    lib.attn_backward.restype = i
    lib.attn_backward_workspace_bytes.argtypes = [i, i, i]
    lib.attn_backward_workspace_bytes.restype = sz
    lib.attn_decode_q8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp, sz, vp]
    lib.attn_decode_q8.restype = i
    lib.attn_decode_multi_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.attn_decode_multi_workspace_bytes.restype = sz
    lib.attn_decode_waves.argtypes = [i, i, i, i, i, i]
    lib.attn_decode_waves.restype = i
    lib.attn_status_string.argtypes = [i]
    lib.attn_status_string.restype = ctypes.c_char_p
    return lib


lib = _load()


class AttnError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {lib.attn_status_string(status).decode()}")


def _check(status: int):
    if status != ATTN_OK:
        raise AttnError(status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, dim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dims, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def default_scale(D: int) -> float:
    return float(torch.tensor(1.0 / math.sqrt(D), dtype=torch.float32).item())


def _prefill_args(q, k, v, out, lse, return_lse):
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    if v.shape != k.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", torch.bfloat16, 4)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    if return_lse and lse is None:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, 3)
        if tuple(lse.shape) != (B, Hq, Lq):
            raise ValueError("lse must be [B,Hq,Lq]")
    return B, Hq, Hkv, Lq, Lk, D, out, lse


def prefill(q, k, v, causal: bool = True, scale: float | None = None, out=None, lse=None,
            return_lse: bool = True):
    """attn_prefill: q [B,Hq,Lq,D], k/v [B,Hkv,Lk,D] bf16 -> (out bf16, lse fp32 or None)."""
    B, Hq, Hkv, Lq, Lk, D, out, lse = _prefill_args(q, k, v, out, lse, return_lse)
    scale = default_scale(D) if scale is None else float(scale)
    _check(lib.attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Lq, Lk, D,
                            1 if causal else 0, ctypes.c_float(scale), _stream(q.device)))
    return out, lse


def prefill_ex(q, k, v, causal: bool = True, scale: float | None = None, splits: int = 0, out=None, lse=None,
               return_lse: bool = True, workspace=None, window: int = 0):
    """attn_prefill_ex: prefill with a sliding window (0 = none), a key-split count (0 = automatic) and an
    optional workspace."""
    B, Hq, Hkv, Lq, Lk, D, out, lse = _prefill_args(q, k, v, out, lse, return_lse)
    scale = default_scale(D) if scale is None else float(scale)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.attn_prefill_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Lq, Lk, D,
                               1 if causal else 0, int(window), ctypes.c_float(scale), int(splits), _ptr(workspace),
                               ws_bytes, _stream(q.device)))
    return out, lse


def prefill_splits(B, Hq, Hkv, Lq, Lk, D, causal=True, splits=0, window=0) -> int:
    return int(lib.attn_prefill_splits(B, Hq, Hkv, Lq, Lk, D, 1 if causal else 0, window, splits))


def prefill_workspace_bytes(B, Hq, Hkv, Lq, Lk, D, causal=True, splits=0, window=0) -> int:
    return int(lib.attn_prefill_workspace_bytes(B, Hq, Hkv, Lq, Lk, D, 1 if causal else 0, window, splits))


def decode(q, kcache, vcache, kv_lens, scale: float | None = None, out=None):
    """attn_decode: q [B,Hq,D], caches [B,Hkv,Lmax,D] bf16, kv_lens [B] int32 -> out [B,Hq,D] bf16."""
    B, Hq, Hkv, Lmax, D = _decode_shapes(q, kcache, vcache, kv_lens)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", torch.bfloat16, 3)
    scale = default_scale(D) if scale is None else float(scale)
    _check(lib.attn_decode(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(kv_lens), _ptr(out), B, Hq, Hkv, Lmax, D,
                           ctypes.c_float(scale), _stream(q.device)))
    return out


def decode_noalloc(q, kcache, vcache, kv_lens, scale: float | None = None, out=None):
    """attn_decode_noalloc: attn_decode with its partials in the library's static device scratch (no allocation
    by the library; `out` is allocated here only when not given)."""
    B, Hq, Hkv, Lmax, D = _decode_shapes(q, kcache, vcache, kv_lens)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", torch.bfloat16, 3)
    scale = default_scale(D) if scale is None else float(scale)
    _check(lib.attn_decode_noalloc(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(kv_lens), _ptr(out), B, Hq, Hkv, Lmax,
                                   D, ctypes.c_float(scale), _stream(q.device)))
    return out


def decode_ex(q, kcache, vcache, kv_lens, scale: float | None = None, split_keys: int = 0, out=None,
              return_lse: bool = True):
    """attn_decode_ex: decode plus lse [B,Hq] fp32 and a key-range size override (0 = one range per wave)."""
    B, Hq, Hkv, Lmax, D = _decode_shapes(q, kcache, vcache, kv_lens)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", torch.bfloat16, 3)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if return_lse else None
    scale = default_scale(D) if scale is None else float(scale)
    _check(lib.attn_decode_ex(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(kv_lens), _ptr(out), _ptr(lse), B, Hq,
                              Hkv, Lmax, D, ctypes.c_float(scale), int(split_keys), _stream(q.device)))
    return out, lse


def _multi_args(q, kcache, vcache, kv_lens, out, return_lse):
    _need(q, "q", torch.bfloat16, 4)
    _need(kcache, "kcache", torch.bfloat16, 4)
    _need(vcache, "vcache", torch.bfloat16, 4)
    _need(kv_lens, "kv_lens", torch.int32, 1)
    B, Hq, T, D = q.shape
    Hkv, Lmax = kcache.shape[1], kcache.shape[2]
    if vcache.shape != kcache.shape or kcache.shape[0] != B or kcache.shape[3] != D or kv_lens.shape[0] != B:
        raise ValueError("shape mismatch between q, caches and kv_lens")
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", torch.bfloat16, 4)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device) if return_lse else None
    return B, Hq, Hkv, T, Lmax, D, out, lse


def decode_multi(q, kcache, vcache, kv_lens, scale: float | None = None, out=None, return_lse: bool = True,
                 workspace=None, window: int = 0):
    """attn_decode_multi: q [B,Hq,T,D] (the last T cached tokens of each sequence) -> (out, lse [B,Hq,T]);
    window > 0 limits each row to its window most recent keys."""
    B, Hq, Hkv, T, Lmax, D, out, lse = _multi_args(q, kcache, vcache, kv_lens, out, return_lse)
    scale = default_scale(D) if scale is None else float(scale)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.attn_decode_multi(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(kv_lens), _ptr(out), _ptr(lse), B, Hq,
                                 Hkv, T, int(window), Lmax, D, ctypes.c_float(scale), _ptr(workspace), ws_bytes,
                                 _stream(q.device)))
    return out, lse


DECODE_KERNELS = {"auto": 0, "main": 1, "wide": 2}


def decode_multi_ex(q, kcache, vcache, kv_lens, scale: float | None = None, split_keys: int = 0,
                    kernel: str = "auto", out=None, return_lse: bool = True, workspace=None, window: int = 0):
    """attn_decode_multi_ex: decode_multi with a key-range size (0 = one range per wave) and an explicit main
    kernel ("auto", "main": K/V in registers, "wide": 32-row blocks with K/V staged through LDS)."""
    B, Hq, Hkv, T, Lmax, D, out, lse = _multi_args(q, kcache, vcache, kv_lens, out, return_lse)
    scale = default_scale(D) if scale is None else float(scale)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.attn_decode_multi_ex(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(kv_lens), _ptr(out), _ptr(lse), B,
                                    Hq, Hkv, T, int(window), Lmax, D, ctypes.c_float(scale), int(split_keys),
                                    DECODE_KERNELS[kernel], _ptr(workspace), ws_bytes, _stream(q.device)))
    return out, lse


def decode_q8(q, kq, kscale, vq, vscale, kv_lens, scale: float | None = None, out=None, return_lse: bool = True,
              workspace=None, window: int = 0):
    """attn_decode_q8: decode_multi over int8 caches kq/vq [B,Hkv,Lmax,D] with fp16 block scales
    kscale/vscale [B,Hkv,Lmax,D/32] (element = scale of its 32-element block * code)."""
    _need(q, "q", torch.bfloat16, 4)
    _need(kq, "kq", torch.int8, 4)
    _need(vq, "vq", torch.int8, 4)
    _need(kscale, "kscale", torch.float16, 4)
    _need(vscale, "vscale", torch.float16, 4)
    _need(kv_lens, "kv_lens", torch.int32, 1)
    B, Hq, T, D = q.shape
    Hkv, Lmax = kq.shape[1], kq.shape[2]
    if (vq.shape != kq.shape or kq.shape[0] != B or kq.shape[3] != D or kv_lens.shape[0] != B
            or D % 32 != 0 or kscale.shape != (B, Hkv, Lmax, D // 32) or vscale.shape != kscale.shape):
        raise ValueError("shape mismatch between q, int8 caches, scales and kv_lens")
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", torch.bfloat16, 4)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device) if return_lse else None
    scale = default_scale(D) if scale is None else float(scale)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.attn_decode_q8(_ptr(q), _ptr(kq), _ptr(kscale), _ptr(vq), _ptr(vscale), _ptr(kv_lens), _ptr(out),
                              _ptr(lse), B, Hq, Hkv, T, int(window), Lmax, D, ctypes.c_float(scale),
                              _ptr(workspace), ws_bytes, _stream(q.device)))
    return out, lse


def backward(q, k, v, out, dout, lse, causal: bool = True, scale: float | None = None, window: int = 0,
             dq=None, dk=None, dv=None, workspace=None):
    """attn_backward: (dq, dk, dv) of attention from the forward's out and lse and the gradient dout."""
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    _need(out, "out", torch.bfloat16, 4)
    _need(dout, "dout", torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    if (v.shape != k.shape or k.shape[0] != B or k.shape[3] != D or out.shape != q.shape or dout.shape != q.shape
            or lse.shape != (B, Hq, Lq)):
        raise ValueError("shape mismatch between q, k, v, out, dout and lse")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, n, ref in ((dq, "dq", q), (dk, "dk", k), (dv, "dv", v)):
        _need(t, n, torch.bfloat16, 4)
        if t.shape != ref.shape:
            raise ValueError(f"{n} must have the shape of its input")
    scale = default_scale(D) if scale is None else float(scale)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.attn_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                             _ptr(dv), B, Hq, Hkv, Lq, Lk, D, int(bool(causal)), int(window), ctypes.c_float(scale),
                             _ptr(workspace), ws_bytes, _stream(q.device)))
    return dq, dk, dv


def backward_workspace_bytes(B, Hq, Lq) -> int:
    return int(lib.attn_backward_workspace_bytes(B, Hq, Lq))


def decode_multi_workspace_bytes(B, Hq, Hkv, T, Lmax, D) -> int:
    return int(lib.attn_decode_multi_workspace_bytes(B, Hq, Hkv, T, Lmax, D))


def decode_waves(B, Hq, Hkv, Lmax, D, split_keys=0) -> int:
    return int(lib.attn_decode_waves(B, Hq, Hkv, Lmax, D, split_keys))


def _decode_shapes(q, kcache, vcache, kv_lens):
    _need(q, "q", torch.bfloat16, 3)
    _need(kcache, "kcache", torch.bfloat16, 4)
    _need(vcache, "vcache", torch.bfloat16, 4)
    _need(kv_lens, "kv_lens", torch.int32, 1)
    B, Hq, D = q.shape
    Hkv, Lmax = kcache.shape[1], kcache.shape[2]
    if vcache.shape != kcache.shape or kcache.shape[0] != B or kcache.shape[3] != D or kv_lens.shape[0] != B:
        raise ValueError("shape mismatch between q, caches and kv_lens")
    return B, Hq, Hkv, Lmax, D


__all__ = ["prefill", "prefill_ex", "prefill_splits", "prefill_workspace_bytes", "decode", "decode_noalloc",
           "decode_ex",
           "decode_multi", "decode_multi_ex", "decode_q8", "backward", "backward_workspace_bytes",
           "decode_multi_workspace_bytes", "decode_waves", "AttnError", "lib", "LIB_PATH", "default_scale"]
