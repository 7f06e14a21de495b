"""ctypes binding of libfa.so: the C ABI of include/fa.h, name for name.

Argument marshalling only.  ``import torch`` comes first so that libfa binds
to the HIP runtime torch has already loaded (both carry the soname
libamdhip64.so.7): one runtime per process, and torch's stream handles are
valid for libfa.  Loading fails loudly when the library is not built; there is
no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must precede loading libfa; see module docstring)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_OK = 0
FA_ERR_INVALID_ARG = 1
FA_ERR_UNSUPPORTED = 2
FA_ERR_HIP = 3

FA_DTYPE_F32 = 0
FA_DTYPE_BF16 = 1
FA_DTYPE_F16 = 2

FA_SOFTMAX_ONLINE = 0
FA_SOFTMAX_SAFE = 1

# name -> (restype, argtypes), mirroring include/fa.h
_P = ctypes.c_void_p
_I = ctypes.c_int
_FWD_ARGS = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.c_float, _I, _P]
SIGNATURES = {
    "fa_fwd": (_I, _FWD_ARGS),
    "fa_fwd_tiled": (_I, _FWD_ARGS + [_I, _I]),
    "fa_fwd_stamped": (_I, _FWD_ARGS + [_P, ctypes.c_longlong]),
    "fa_fwd_stamp_slots": (ctypes.c_longlong, [_I, _I, _I, _I, _I]),
    "fa_wall_clock_khz": (_I, [_I]),
    "fa_tile_shapes": (_I, [_I, _I, ctypes.POINTER(_I), ctypes.POINTER(_I), _I]),
    "fa_fwd_splitkv": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, ctypes.c_float, _I, _I, _P]),
    "fa_merge": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "fa_split_chunk": (_I, [_I, _I]),
    "fa_splitkv_num_splits": (_I, [_I, _I, _I, _I, _I]),
    "fa_softmax": (_I, [_P, _P, _P, ctypes.c_longlong, _I, _I, _I, _P]),
    "fa_bwd": (_I, [_P] * 10 + [_I] * 6 + [ctypes.c_float, _I, _P]),
    "fa_bwd_split": (_I, [_P] * 11 + [_I] * 7 + [ctypes.c_float, _I, _P]),
    "fa_bwd_num_splits": (_I, [_I, _I, _I, _I]),
    "fa_bwd_split_noalloc": (_I, [_P] * 10 + [_I] * 7 + [ctypes.c_float, _I, _P]),
    "fa_bwd_noalloc_max_bytes": (ctypes.c_longlong, []),
    "fa_error_string": (ctypes.c_char_p, [_I]),
    "fa_last_error": (ctypes.c_char_p, []),
    "fa_abi_version": (_I, []),
}

_lib = None


class LibraryNotBuilt(ImportError):
    pass


class TwoHipRuntimes(RuntimeError):
    pass


def hip_runtimes_mapped():
    """Distinct HIP runtime files (libamdhip64*) mapped into this process (Linux)."""
    try:
        with open("/proc/self/maps") as f:
            return sorted({line.split()[-1] for line in f if "libamdhip64" in line})
    except OSError:
        return []


def check_one_hip_runtime():
    """Raise TwoHipRuntimes when more than one HIP runtime is mapped.

    torch's libraries ask for ``libamdhip64.so`` and find their own copy next to them;
    libfa asks for ``libamdhip64.so.7``, the soname of that copy.  Loaded after torch,
    libfa therefore binds to torch's runtime.  Loaded first, it maps the system
    runtime, and torch then maps its own beside it: torch's stream handles are then
    foreign to the runtime libfa launches on, and the first launch can abort the
    process.  This turns that state into an error before any launch.
    """
    mapped = hip_runtimes_mapped()
    if len(mapped) > 1:
        raise TwoHipRuntimes("two HIP runtimes are mapped into this process (%s): load libfa only after "
                             "torch, through this module" % ", ".join(mapped))


def load():
    """Load libfa.so once; raise LibraryNotBuilt if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LibraryNotBuilt(
                "libfa.so is not built (%s); run `python -c 'import __graft_entry__ as g; g.build()'`"
                % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        check_one_hip_runtime()
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, dtype, stream):
    return load().fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, dtype, stream)


def fa_fwd_tiled(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, dtype, stream, block_m, block_n):
    return load().fa_fwd_tiled(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, dtype, stream,
                               block_m, block_n)


def fa_fwd_stamped(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, dtype, stream, stamps, stamp_slots):
    return load().fa_fwd_stamped(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, dtype, stream, stamps,
                                 stamp_slots)


def fa_fwd_stamp_slots(B, Hq, N, d, dtype):
    return load().fa_fwd_stamp_slots(B, Hq, N, d, dtype)


def fa_wall_clock_khz(device):
    return load().fa_wall_clock_khz(device)


def fa_fwd_splitkv(q, k, v, o_part, lse_part, B, Hq, Hkv, Nq, Nk, d, causal, scale, dtype, num_splits,
                   stream):
    return load().fa_fwd_splitkv(q, k, v, o_part, lse_part, B, Hq, Hkv, Nq, Nk, d, causal, scale, dtype,
                                 num_splits, stream)


def fa_merge(o_part, lse_part, o, lse, num_splits, B, H, N, d, dtype, stream):
    return load().fa_merge(o_part, lse_part, o, lse, num_splits, B, H, N, d, dtype, stream)


def fa_split_chunk(Nk, num_splits):
    return load().fa_split_chunk(Nk, num_splits)


def fa_splitkv_num_splits(B, Hq, Hkv, Nq, Nk):
    return load().fa_splitkv_num_splits(B, Hq, Hkv, Nq, Nk)


def fa_softmax(x, y, lse, rows, cols, dtype, algo, stream):
    return load().fa_softmax(x, y, lse, rows, cols, dtype, algo, stream)


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, Hq, Hkv, N, d, causal, scale, dtype, stream):
    return load().fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, Hq, Hkv, N, d, causal, scale, dtype,
                         stream)


def fa_bwd_split(q, k, v, o, lse, dout, dq, dk, dv, delta, dkv_part, num_splits, B, Hq, Hkv, N, d, causal,
                 scale, dtype, stream):
    return load().fa_bwd_split(q, k, v, o, lse, dout, dq, dk, dv, delta, dkv_part, num_splits, B, Hq, Hkv, N, d,
                               causal, scale, dtype, stream)


def fa_bwd_split_noalloc(q, k, v, o, lse, dout, dq, dk, dv, delta, num_splits, B, Hq, Hkv, N, d, causal, scale,
                         dtype, stream):
    return load().fa_bwd_split_noalloc(q, k, v, o, lse, dout, dq, dk, dv, delta, num_splits, B, Hq, Hkv, N, d,
                                       causal, scale, dtype, stream)


def fa_bwd_noalloc_max_bytes():
    return load().fa_bwd_noalloc_max_bytes()


def fa_bwd_num_splits(B, Hq, Hkv, N):
    return load().fa_bwd_num_splits(B, Hq, Hkv, N)


def fa_tile_shapes(dtype, d):
    """List of (block_m, block_n) compiled for (dtype, d); the first is the default."""
    lib = load()
    n = lib.fa_tile_shapes(dtype, d, None, None, 0)
    if n < 0:
        return []
    bm = (ctypes.c_int * n)()
    bn = (ctypes.c_int * n)()
    lib.fa_tile_shapes(dtype, d, bm, bn, n)
    return list(zip(bm, bn))


def fa_error_string(code):
    return load().fa_error_string(code).decode()


def fa_last_error():
    return load().fa_last_error().decode()


def fa_abi_version():
    return load().fa_abi_version()
