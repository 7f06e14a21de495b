"""FlashAttention forward for MI355X (gfx950): exact attention, online softmax.

``forward(q, k, v, causal=False, scale=None)`` returns ``(o, lse)`` computed by
the HIP kernels in libfa.so (C ABI in include/fa.h).  ``forward_splitkv`` and
``merge`` split the keys into ranges, compute each range's partial state and
combine them; ``attention_kv`` does both for queries that are the last Nq of Nk
positions (e.g. decoding against a cache).  ``softmax`` is the row softmax on
its own.  ``backward`` gives dq, dk, dv from the forward's o and lse, and
``attention`` wraps forward and backward as a torch autograd function.  torch
supplies device memory and the stream; every step runs in the kernels.

The library is loaded on first use, and a missing build raises.
"""
from __future__ import annotations

import math

import torch

from . import _lib
from ._lib import (FA_DTYPE_BF16, FA_DTYPE_F16, FA_DTYPE_F32, FA_ERR_HIP, FA_ERR_INVALID_ARG,
                   FA_ERR_UNSUPPORTED, FA_OK, FA_SOFTMAX_ONLINE, FA_SOFTMAX_SAFE, LibraryNotBuilt,
                   fa_abi_version, fa_bwd, fa_bwd_num_splits, fa_bwd_split, fa_error_string, fa_fwd, fa_fwd_splitkv, fa_fwd_tiled, fa_last_error,
                   fa_merge, fa_softmax, fa_split_chunk, fa_splitkv_num_splits, fa_tile_shapes)

__all__ = ["forward", "forward_splitkv", "merge", "attention_kv", "softmax", "backward", "attention",
           "fa_fwd", "fa_fwd_tiled", "fa_bwd", "fa_bwd_split", "fa_bwd_num_splits",
           "fa_fwd_splitkv", "fa_merge", "fa_split_chunk", "fa_splitkv_num_splits", "fa_softmax",
           "FA_SOFTMAX_ONLINE", "FA_SOFTMAX_SAFE",
           "fa_tile_shapes", "fa_error_string",
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

    q [B, Hq, N, d]; k, v [B, Hkv, N, d]; float32, bfloat16 or float16 CUDA tensors,
    contiguous, on one device.  Returns (o, lse): o like q, lse [B, Hq, N]
    float32 with lse = m + ln(l) per query row.  ``scale`` defaults to
    1/sqrt(d).  ``block_m``/``block_n`` pick a compiled tile shape (see
    ``fa_tile_shapes``); by default the library chooses.  ``out``/``lse`` may be
    given to write into existing tensors.  Runs on torch's current stream.
    """
    lib = _lib.load()
    _check_inputs(q, k, v)
    B, Hq, N, d = q.shape
    if k.shape[2] != N:
        raise ValueError("k and v must be [B, Hkv, N, d] with q's N; got %s, %s, %s"
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


def _check_inputs(q, k, v):
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
    B, Hq, Nq, d = q.shape
    if k.shape[0] != B or k.shape[3] != d or v.shape != k.shape:
        raise ValueError("k and v must be [B, Hkv, Nk, d] matching q; got %s, %s, %s"
                         % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))


def forward_splitkv(q, k, v, num_splits, causal=False, scale=None):
    """Partial states over num_splits key ranges.

    q [B, Hq, Nq, d]; k, v [B, Hkv, Nk, d] bfloat16 or float16 CUDA tensors; the queries are
    the last Nq of the Nk positions (causal: key j visible to query i iff
    j <= i + Nk - Nq).  Returns (o_part [S, B, Hq, Nq, d], lse_part [S, B, Hq, Nq]),
    float32: each range's output over its own visible keys and m + ln l, with
    lse = -inf (o = 0) where a range holds no visible key.  Range s covers keys
    [s*c, (s+1)*c) with c = fa_split_chunk(Nk, num_splits).
    """
    lib = _lib.load()
    _check_inputs(q, k, v)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    S = int(num_splits)
    o_part = torch.empty((max(S, 0), B, Hq, Nq, d), dtype=torch.float32, device=q.device)
    lse_part = torch.empty((max(S, 0), B, Hq, Nq), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = lib.fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_part.data_ptr(),
                                lse_part.data_ptr(), B, Hq, Hkv, Nq, Nk, d, int(bool(causal)),
                                float(scale), _DTYPES[q.dtype], S, stream)
    if rc != FA_OK:
        _raise(rc)
    return o_part, lse_part


def merge(o_part, lse_part, out_dtype=torch.bfloat16, out=None, lse=None):
    """Merge partial states: o_part [S, B, H, N, d], lse_part [S, B, H, N] float32.

    Returns (o [B, H, N, d] in out_dtype, lse [B, H, N] float32).
    """
    lib = _lib.load()
    for name, t in (("o_part", o_part), ("lse_part", lse_part)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
            raise ValueError("%s must be a contiguous CUDA tensor" % name)
        if t.dtype != torch.float32:
            raise ValueError("%s must be float32" % name)
    if o_part.dim() != 5 or lse_part.shape != o_part.shape[:-1]:
        raise ValueError("o_part must be [S, B, H, N, d] and lse_part [S, B, H, N]")
    if out_dtype not in (torch.float32, torch.bfloat16, torch.float16):
        raise ValueError("out_dtype must be float32, bfloat16 or float16")
    S, B, H, N, d = o_part.shape
    if out is None:
        out = torch.empty((B, H, N, d), dtype=out_dtype, device=o_part.device)
    elif (out.shape != (B, H, N, d) or out.dtype != out_dtype or out.device != o_part.device
          or not out.is_contiguous()):
        raise ValueError("out must be a contiguous [B, H, N, d] tensor of out_dtype")
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=o_part.device)
    elif (lse.shape != (B, H, N) or lse.dtype != torch.float32 or lse.device != o_part.device
          or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 tensor [B, H, N]")
    with torch.cuda.device(o_part.device):
        stream = torch.cuda.current_stream(o_part.device).cuda_stream
        rc = lib.fa_merge(o_part.data_ptr(), lse_part.data_ptr(), out.data_ptr(), lse.data_ptr(), S, B, H,
                          N, d, _DTYPES[out_dtype], stream)
    if rc != FA_OK:
        _raise(rc)
    return out, lse


def attention_kv(q, k, v, causal=False, scale=None, num_splits=None):
    """Attention of queries that are the last Nq of Nk positions, by split-KV + merge.

    q [B, Hq, Nq, d]; k, v [B, Hkv, Nk, d] bfloat16 or float16.  num_splits defaults to
    fa_splitkv_num_splits for the shape.  Returns (o like q, lse [B, Hq, Nq]).
    """
    _check_inputs(q, k, v)
    B, Hq, Nq, _ = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if num_splits is None:
        num_splits = max(1, fa_splitkv_num_splits(B, Hq, Hkv, max(Nq, 1), max(Nk, 1)))
    o_part, lse_part = forward_splitkv(q, k, v, num_splits, causal=causal, scale=scale)
    return merge(o_part, lse_part, out_dtype=q.dtype)


_ALGOS = {"online": FA_SOFTMAX_ONLINE, "safe": FA_SOFTMAX_SAFE}


def softmax(x, algo="online", out=None, lse=None):
    """Softmax over the last dimension of a contiguous CUDA tensor (float32, bfloat16 or float16).

    algo "online": the running max and sum in one read of each row, then the
    output (2 reads + 1 write per element); "safe": max, sum, output (3 reads +
    1 write).  Returns (y like x, lse float32 of x's shape without its last
    dimension).  ``out`` may be x itself (in place).
    """
    lib = _lib.load()
    if not isinstance(x, torch.Tensor) or not x.is_cuda or not x.is_contiguous() or x.dim() < 1:
        raise ValueError("x must be a contiguous CUDA tensor with at least one dimension")
    if x.dtype not in _DTYPES:
        raise ValueError("dtype %s is not supported" % x.dtype)
    if algo not in _ALGOS:
        raise ValueError("algo must be 'online' or 'safe'")
    cols = x.shape[-1]
    rows = x.numel() // cols if cols else 0
    if out is None:
        out = torch.empty_like(x)
    elif out.shape != x.shape or out.dtype != x.dtype or out.device != x.device or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like x")
    if lse is None:
        lse = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    elif (lse.shape != x.shape[:-1] or lse.dtype != torch.float32 or lse.device != x.device
          or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 tensor of x's shape without its last dimension")
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        rc = lib.fa_softmax(x.data_ptr(), out.data_ptr(), lse.data_ptr() if rows else None, rows, cols,
                            _DTYPES[x.dtype], _ALGOS[algo], stream)
    if rc != FA_OK:
        _raise(rc)
    return out, lse


def backward(q, k, v, o, lse, do, causal=False, scale=None, dq=None, dk=None, dv=None, delta=None,
             num_splits=None):
    """Gradients of the square attention forward: returns (dq, dk, dv, delta).

    q, o, do [B, Hq, N, d] and k, v [B, Hkv, N, d] bfloat16 or float16 CUDA tensors,
    contiguous; o and lse [B, Hq, N] float32 as ``forward`` returned them for the same
    q, k, v, causal and scale.  delta [B, Hq, N] float32 is rowsum(do * o).  dk and
    dv of a K/V head sum over the query heads that read it.  The gradient buffers
    may be given to write into existing tensors.  ``num_splits`` shares each key
    tile's dK/dV work over that many workgroups through an fp32 workspace this
    function allocates (default: ``fa_bwd_num_splits``; 1 needs no workspace).  Runs
    on torch's current stream.
    """
    lib = _lib.load()
    _check_inputs(q, k, v)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape[2] != N:
        raise ValueError("the backward is for the square problem: k and v need N = %d rows" % N)
    for name, t in (("o", o), ("do", do)):
        if (not isinstance(t, torch.Tensor) or t.shape != q.shape or t.dtype != q.dtype
                or t.device != q.device or not t.is_contiguous()):
            raise ValueError("%s must be a contiguous tensor like q" % name)
    if (not isinstance(lse, torch.Tensor) or lse.shape != (B, Hq, N) or lse.dtype != torch.float32
            or lse.device != q.device or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 tensor [B, Hq, N] on q's device")
    if scale is None:
        scale = 1.0 / math.sqrt(d)

    def _out(t, like, name):
        if t is None:
            return torch.empty_like(like)
        if t.shape != like.shape or t.dtype != like.dtype or t.device != like.device or not t.is_contiguous():
            raise ValueError("%s must be a contiguous tensor like %s" % (name, "q" if like is q else "k"))
        return t

    dq, dk, dv = _out(dq, q, "dq"), _out(dk, k, "dk"), _out(dv, v, "dv")
    if delta is None:
        delta = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    elif (delta.shape != (B, Hq, N) or delta.dtype != torch.float32 or delta.device != q.device
          or not delta.is_contiguous()):
        raise ValueError("delta must be a contiguous float32 tensor [B, Hq, N] on q's device")
    if num_splits is None:
        num_splits = max(1, fa_bwd_num_splits(max(B, 1), Hq, Hkv, max(N, 1)))
    part = None
    if num_splits > 1 and B * N > 0:
        part = torch.empty((2, num_splits) + tuple(k.shape), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = lib.fa_bwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                              do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                              part.data_ptr() if part is not None else None, int(num_splits), B, Hq, Hkv, N, d,
                              int(bool(causal)), float(scale), _DTYPES[q.dtype], stream)
    if rc != FA_OK:
        _raise(rc)
    return dq, dk, dv, delta


class _Attention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, causal, scale):
        o, lse = forward(q, k, v, causal=causal, scale=scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.causal, ctx.scale = causal, scale
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv, _ = backward(q, k, v, o, lse, do.contiguous(), causal=ctx.causal, scale=ctx.scale)
        return dq, dk, dv, None, None


def attention(q, k, v, causal=False, scale=None):
    """softmax(scale q k^T) v with autograd: the forward saves (o, lse), the backward
    recomputes the weights from them (bfloat16 or float16 inputs for the backward)."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    return _Attention.apply(q, k, v, bool(causal), float(scale))
