"""FlashAttention forward for MI355X (gfx950): exact attention, online softmax.

``forward(q, k, v, causal=False, scale=None)`` returns ``(o, lse)`` computed by
the HIP kernels in libfa.so (C ABI in include/fa.h).  torch supplies device
memory and the stream; every step of the attention runs in the kernels.

The library is loaded on first use, and a missing build raises.
"""
from __future__ import annotations

import math

import torch

from . import _lib
from ._lib import (FA_DTYPE_BF16, FA_DTYPE_F16, FA_DTYPE_F32, FA_ERR_HIP, FA_ERR_INVALID_ARG,
                   FA_ERR_UNSUPPORTED, FA_OK, LibraryNotBuilt, fa_abi_version, fa_error_string,
                   fa_fwd, fa_fwd_tiled, fa_last_error, fa_tile_shapes)

__all__ = ["forward", "fa_fwd", "fa_fwd_tiled", "fa_tile_shapes", "fa_error_string",
           "fa_last_error", "fa_abi_version", "FA_OK", "FA_ERR_INVALID_ARG",
           "FA_ERR_UNSUPPORTED", "FA_ERR_HIP", "FA_DTYPE_F32", "FA_DTYPE_BF16", "FA_DTYPE_F16",
           "LibraryNotBuilt", "load_library"]

_DTYPES = {torch.float32: FA_DTYPE_F32, torch.bfloat16: FA_DTYPE_BF16, torch.float16: FA_DTYPE_F16}


def load_library():
    """Load libfa.so now (raises LibraryNotBuilt when it is missing)."""
    return _lib.load()


def _raise(rc):
    detail = fa_last_error()
    msg = "%s: %s" % (fa_error_string(rc), detail)
    if rc == FA_ERR_INVALID_ARG:
        raise ValueError(msg)
    if rc == FA_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise RuntimeError(msg)


def forward(q, k, v, causal=False, scale=None, block_m=None, block_n=None, out=None, lse=None):
    """Attention forward on the GPU.

    q [B, Hq, N, d]; k, v [B, Hkv, N, d]; float32 or bfloat16 CUDA tensors,
    contiguous, on one device.  Returns (o, lse): o like q, lse [B, Hq, N]
    float32 with lse = m + ln(l) per query row.  ``scale`` defaults to
    1/sqrt(d).  ``block_m``/``block_n`` pick a compiled tile shape (see
    ``fa_tile_shapes``); by default the library chooses.  ``out``/``lse`` may be
    given to write into existing tensors.  Runs on torch's current stream.
    """
    lib = _lib.load()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch.Tensor" % name)
        if t.dim() != 4:
            raise ValueError("%s must be 4-D [B, H, N, d], got %s" % (name, tuple(t.shape)))
        if not t.is_cuda:
            raise ValueError("%s must be a CUDA (HIP) tensor" % name)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k and v must share one dtype")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k and v must be on one device")
    if q.dtype not in _DTYPES:
        raise ValueError("dtype %s is not supported" % q.dtype)
    B, Hq, N, d = q.shape
    if k.shape[0] != B or k.shape[2] != N or k.shape[3] != d or v.shape != k.shape:
        raise ValueError("k and v must be [B, Hkv, N, d] matching q; got %s, %s, %s"
                         % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    Hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or out.device != q.device or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    elif (lse.shape != (B, Hq, N) or lse.dtype != torch.float32 or lse.device != q.device
          or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 tensor [B, Hq, N] on q's device")
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                B, Hq, Hkv, N, d, int(bool(causal)), float(scale), _DTYPES[q.dtype], stream)
        if block_m is None and block_n is None:
            rc = lib.fa_fwd(*args)
        else:
            rc = lib.fa_fwd_tiled(*args, int(block_m or 0), int(block_n or 0))
    if rc != FA_OK:
        _raise(rc)
    return out, lse
