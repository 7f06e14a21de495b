"""Python handle on the fp64 oracle (``oracle/fa_ref.c``).

TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module; the product path never
does.  It shares nothing with the HIP library.

The oracle is exact scaled-dot-product attention computed the textbook way in
float64 (three passes per row: max, sum, weighted output), see the header of
``fa_ref.c`` for the definition and the page sections it follows.

Only ctypes marshalling lives here: every number comes out of the C code.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fa_ref.c")
_LIB = os.path.join(_HERE, "libfa_ref.so")

_libs = {}


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (-O2, IEEE semantics, OpenMP)."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
               "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
               "-o", tmp, src, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def _load(path: str | None = None):
    path = path or _LIB
    if path not in _libs:
        if path == _LIB and not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.fa_ref_rows.argtypes = [dp, dp, dp, dp, dp,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_double,
                                    ctypes.POINTER(ctypes.c_int64), ctypes.c_int64]
        lib.fa_ref_rows.restype = ctypes.c_int
        lib.fa_ref_rows_kv.argtypes = [dp, dp, dp, dp, dp,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_double, ctypes.c_int, ctypes.c_int,
                                       ctypes.POINTER(ctypes.c_int64), ctypes.c_int64]
        lib.fa_ref_rows_kv.restype = ctypes.c_int
        lib.fa_ref_num_threads.argtypes = []
        lib.fa_ref_num_threads.restype = ctypes.c_int
        _libs[path] = lib
    return _libs[path]


def num_threads() -> int:
    """OpenMP threads the oracle runs on (honours OMP_NUM_THREADS)."""
    return int(_load().fa_ref_num_threads())


def _as_f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor: exact upcast of bf16/fp32 to fp64
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def attention(q, k, v, causal: bool = False, scale: float | None = None, rows=None,
              lib_path: str | None = None):
    """Exact attention in fp64.

    q: [B, Hq, N, d]; k, v: [B, Hkv, N, d] (numpy or torch; upcast exactly).
    rows: optional 1-D array of flat row ids (b*Hq + h)*N + i.

    lib_path: another build of the oracle source (the mutation tests use it).

    Returns (o, lse): o [B, Hq, N, d] and lse [B, Hq, N] for all rows, or
    o [len(rows), d] and lse [len(rows)] for a row list.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be 4-D [B, H, N, d]")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, N, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, Hkv, N, d] matching q")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if rows is None:
        o = np.empty((B, Hq, N, d), dtype=np.float64)
        lse = np.empty((B, Hq, N), dtype=np.float64)
        rows_p = None
        nrows = B * Hq * N
    else:
        rows_a = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1)
        nrows = rows_a.size
        o = np.empty((nrows, d), dtype=np.float64)
        lse = np.empty((nrows,), dtype=np.float64)
        rows_p = rows_a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    rc = _load(lib_path).fa_ref_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                             B, Hq, Hkv, N, d, int(bool(causal)), float(scale),
                             rows_p, nrows)
    if rc != 0:
        raise ValueError("oracle rejected its arguments (code %d)" % rc)
    return o, lse


def attention_kv(q, k, v, causal: bool = False, scale: float | None = None, k_range=None,
                 rows=None, lib_path: str | None = None):
    """Exact attention of Nq queries against Nk keys, over a key range, in fp64.

    q: [B, Hq, Nq, d]; k, v: [B, Hkv, Nk, d].  causal: key j is visible to query i
    iff j <= i + (Nk - Nq).  k_range = (k_lo, k_hi) keeps only keys in [k_lo, k_hi)
    (default: all).  A row with no visible key in the range gets the empty state,
    o = 0 and lse = -inf.  rows: flat ids (b*Hq + h)*Nq + i.

    Returns (o, lse) shaped like ``attention``'s, with Nq in place of N.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be 4-D [B, H, N, d]")
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if k.shape != (B, Hkv, Nk, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, Hkv, Nk, d] matching q")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    k_lo, k_hi = (0, Nk) if k_range is None else (int(k_range[0]), int(k_range[1]))
    if rows is None:
        o = np.empty((B, Hq, Nq, d), dtype=np.float64)
        lse = np.empty((B, Hq, Nq), dtype=np.float64)
        rows_p = None
        nrows = B * Hq * Nq
    else:
        rows_a = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1)
        nrows = rows_a.size
        o = np.empty((nrows, d), dtype=np.float64)
        lse = np.empty((nrows,), dtype=np.float64)
        rows_p = rows_a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    rc = _load(lib_path).fa_ref_rows_kv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                        B, Hq, Hkv, Nq, Nk, d, int(bool(causal)), float(scale),
                                        k_lo, k_hi, rows_p, nrows)
    if rc != 0:
        raise ValueError("oracle rejected its arguments (code %d)" % rc)
    return o, lse


def merge_partials(o_parts, lse_parts):
    """Merge partial attention states of disjoint key sets, in fp64.

    o_parts [S, ..., d] and lse_parts [S, ...]: state s in normalised form
    (o = acc / l, lse = m + ln l; lse = -inf for an empty state).  Each state is
    read as (m, l, acc) = (lse, 1, o), the same state measured against m + ln l,
    and the S states are pooled with the pages' merge (``online_model.merge``:
    take the largest max, rescale each state by exp(its max - that max), add;
    spicyshark.co lesson, "From softmax to attention" and "Check yourself").
    Returns (o, lse) of the union; a row whose states are all empty gives o = 0,
    lse = -inf.
    """
    from oracle import online_model   # the pinned fp64 model of the pages' update

    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    S = o_parts.shape[0]
    d = o_parts.shape[-1]
    if lse_parts.shape != o_parts.shape[:-1]:
        raise ValueError("lse_parts must be o_parts without its last axis")
    flat_o = o_parts.reshape(S, -1, d)
    flat_l = lse_parts.reshape(S, -1)
    R = flat_o.shape[1]
    out_o = np.zeros((R, d), dtype=np.float64)
    out_l = np.full((R,), -np.inf, dtype=np.float64)
    for r in range(R):
        parts = [(flat_l[s, r], 1.0, flat_o[s, r]) for s in range(S)]
        state = online_model.merge(*parts)
        m, l, acc = state
        if l > 0.0:
            out_o[r] = np.asarray(acc) / l
            out_l[r] = m + np.log(l)
    return out_o.reshape(o_parts.shape[1:]), out_l.reshape(lse_parts.shape[1:])


def row_flops(N: int, d: int, causal: bool, rows) -> float:
    """Algorithmic flops of the given rows: 4*d per visible (query, key) pair.

    Used to express the oracle's throughput in the same unit as the kernel's.
    The full-problem convention (4*B*H*N^2*d, halved when causal) is used by the
    benchmark for the kernel; for sampled oracle rows the exact visible-pair
    count is used instead.
    """
    rows = np.asarray(rows, dtype=np.int64)
    i = rows % N
    nvis = (i + 1) if causal else np.full_like(i, N)
    return float(4.0 * d * nvis.sum())
