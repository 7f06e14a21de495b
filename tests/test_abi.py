"""The C ABI on the CPU: libfa.so loads, exports what include/fa.h declares, and
rejects bad arguments on the host before any HIP call (so no GPU is needed)."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")
PKG = os.path.join(ROOT, "flashattention_online_softmax_fwd_amd")


@pytest.fixture(scope="module")
def lib():
    from flashattention_online_softmax_fwd_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from flashattention_online_softmax_fwd_amd import build
        build.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_function_is_exported(lib):
    names = declared_functions()
    assert set(names) == {"fa_fwd", "fa_fwd_tiled", "fa_tile_shapes", "fa_error_string",
                          "fa_last_error", "fa_abi_version", "fa_fwd_splitkv", "fa_merge",
                          "fa_split_chunk", "fa_splitkv_num_splits", "fa_softmax", "fa_bwd", "fa_bwd_split",
                          "fa_bwd_num_splits", "fa_fwd_stamped", "fa_fwd_stamp_slots", "fa_wall_clock_khz",
                          "fa_bwd_split_noalloc", "fa_bwd_noalloc_max_bytes"}
    out = subprocess.run(["nm", "-D", "--defined-only", os.path.join(PKG, "libfa.so")],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (fa_\w+)", out))
    assert set(names) <= exported
    for n in names:
        assert hasattr(lib, n)


def test_binding_mirrors_the_header():
    from flashattention_online_softmax_fwd_amd import _lib
    assert sorted(_lib.SIGNATURES) == declared_functions()


def test_library_never_allocates_device_memory():
    out = subprocess.run(["nm", "-D", "--undefined-only", os.path.join(PKG, "libfa.so")],
                         capture_output=True, text=True, check=True).stdout
    for sym in ("hipMalloc", "hipFree", "hipMallocAsync", "hipExtMallocWithFlags", "hipHostMalloc",
                "hipMemcpy", "hipDeviceSynchronize", "hipStreamSynchronize"):
        assert not re.search(r"\b%s\b" % sym, out), sym


def test_product_path_does_not_touch_the_oracle():
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower() or f == "inputs.py", f
    src = open(os.path.join(PKG, "inputs.py")).read()
    assert "import oracle" not in src and "from oracle" not in src


def test_version_and_error_strings(lib):
    assert lib.fa_abi_version() == 7
    assert lib.fa_error_string(0) == b"ok"
    assert lib.fa_error_string(1) == b"invalid argument"
    assert lib.fa_error_string(2) == b"unsupported request"
    assert lib.fa_error_string(3) == b"HIP runtime error"
    assert lib.fa_error_string(99) == b"unknown error code"


def test_tile_shapes(lib):
    from flashattention_online_softmax_fwd_amd import _lib
    for dtype in (0, 1, 2):
        for d in (64, 128):
            shapes = _lib.fa_tile_shapes(dtype, d)
            assert len(shapes) >= 2 and len(set(shapes)) == len(shapes)
    assert lib.fa_tile_shapes(1, 96, None, None, 0) == -1
    assert lib.fa_tile_shapes(7, 64, None, None, 0) == -1


P = 0x10000   # a 16-byte-aligned non-null value; never dereferenced by the checks below


def call(lib, q=P, k=P + 0x100000, v=P + 0x200000, o=P + 0x300000, lse=P + 0x400000, B=1, Hq=2, Hkv=1,
         N=16, d=64, causal=0, scale=0.125, dtype=1, stream=None):
    return lib.fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, dtype, stream)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), 1), (dict(o=0), 1), (dict(lse=0), 1),
    (dict(q=P + 8), 1),                                   # misaligned
    (dict(B=-1), 1), (dict(N=-5), 1), (dict(Hq=0), 1), (dict(Hkv=0), 1),
    (dict(Hq=3, Hkv=2), 1), (dict(d=0), 1), (dict(causal=2), 1),
    (dict(scale=float("inf")), 1), (dict(scale=float("nan")), 1), (dict(scale=3e38), 1),
    (dict(dtype=5), 1), (dict(d=96), 2), (dict(d=256), 2),
    (dict(o=P), 1),                                       # o overlaps q
    (dict(lse=P + 0x300010), 1),                          # lse overlaps o
])
def test_invalid_arguments_are_rejected_before_any_hip_call(lib, kw, code):
    assert call(lib, **kw) == code
    assert lib.fa_last_error() != b""


def test_stamp_slots_count_the_waves_of_the_default_tile(lib):
    for dtype in (1, 2):
        for d in (64, 128):
            # enough rows for 1024 waves of 64 and 512 workgroups of 256: 4 waves of 64 rows
            assert lib.fa_fwd_stamp_slots(2, 32, 4096, d, dtype) == 2 * 32 * (4096 // 256) * 4
            # 1024 waves of 64 but only 256 workgroups of 256: 128-row workgroups, 2 waves of 64
            assert lib.fa_fwd_stamp_slots(1, 8, 8192, d, dtype) == 8 * (8192 // 128) * 2
            # fewer than 1024 waves of 64 (the SIMDs of a 256-CU device): the 32-rows-per-wave
            # kernel, 128-row workgroups of 4 waves
            assert lib.fa_fwd_stamp_slots(1, 3, 200, d, dtype) == 3 * 2 * 4
            assert lib.fa_fwd_stamp_slots(1, 3, 1, d, dtype) == 3 * 1 * 4
            assert lib.fa_fwd_stamp_slots(0, 3, 100, d, dtype) == 0
    assert lib.fa_fwd_stamp_slots(1, 1, 64, 64, 0) == -1      # fp32 kernels carry no stamps
    assert lib.fa_fwd_stamp_slots(1, 1, 64, 96, 1) == -1
    assert lib.fa_fwd_stamp_slots(1, 0, 64, 64, 1) == -1


@pytest.mark.parametrize("stamps,slots,dtype,code", [
    (0, 1 << 20, 1, 1),                 # null stamps
    (P + 0x600010, 1 << 20, 1, 1),      # not 32-byte aligned
    (P + 0x600000, 3, 1, 1),            # fewer slots than waves
    (P + 0x600000, -1, 1, 1),
    (P + 0x300000, 1 << 20, 1, 1),      # overlaps o
    (P + 0x600000, 1 << 20, 0, 2),      # fp32: no stamped kernel
])
def test_stamped_call_checks_its_buffer_before_any_hip_call(lib, stamps, slots, dtype, code):
    args = (P, P + 0x100000, P + 0x200000, P + 0x300000, P + 0x400000, 1, 2, 1, 16, 64, 0, 0.125, dtype, None)
    assert lib.fa_fwd_stamped(*args, stamps, slots) == code
    assert lib.fa_last_error() != b""


def test_empty_problems_return_ok_without_touching_pointers(lib):
    assert call(lib, q=0, k=0, v=0, o=0, lse=0, B=0) == 0
    assert call(lib, q=0, k=0, v=0, o=0, lse=0, N=0) == 0


def test_unknown_tile_is_unsupported(lib):
    args = (P, P + 0x100000, P + 0x200000, P + 0x300000, P + 0x400000, 1, 2, 1, 16, 64, 0, 0.125, 1, None)
    assert lib.fa_fwd_tiled(*args, 96, 64) == 2
    assert lib.fa_fwd_tiled(*args, 0, 64) == 1
    assert lib.fa_fwd_tiled(*args, -128, 64) == 1


def test_python_wrapper_checks_before_the_library():
    import torch

    import flashattention_online_softmax_fwd_amd as fa
    x = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.forward(x, x, x)                     # CPU tensors are refused
    with pytest.raises(ValueError):
        fa.forward(torch.zeros(4, 64), x, x)    # wrong rank
    with pytest.raises(TypeError):
        fa.forward([0.0], x, x)                 # not a tensor
    with pytest.raises(ValueError):
        fa.backward(x, x, x, x, torch.zeros(1, 1, 4), x)   # CPU tensors are refused here too


def call_split(lib, q=P, k=P + 0x100000, v=P + 0x200000, op=P + 0x300000, lp=P + 0x500000, B=1, Hq=2,
               Hkv=1, Nq=4, Nk=300, d=64, causal=1, scale=0.125, dtype=1, splits=3, stream=None):
    return lib.fa_fwd_splitkv(q, k, v, op, lp, B, Hq, Hkv, Nq, Nk, d, causal, scale, dtype, splits, stream)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), 1), (dict(op=0), 1), (dict(lp=P + 4), 1),
    (dict(B=-1), 1), (dict(Nq=-1), 1), (dict(Nk=-1), 1), (dict(Nk=0), 1),
    (dict(Hq=3, Hkv=2), 1), (dict(causal=3), 1), (dict(scale=float("nan")), 1),
    (dict(splits=0), 1), (dict(splits=1025), 1),
    (dict(Nq=301, Nk=300), 1),                            # causal with more queries than keys
    (dict(dtype=0), 2), (dict(dtype=9), 1), (dict(d=96), 2),
    (dict(op=P + 0x100000), 1),                           # o_part overlaps k
    (dict(lp=P + 0x300010), 1),                           # lse_part overlaps o_part
    (dict(Hq=64, Hkv=1, Nq=1 << 25, causal=0, k=P + (1 << 40), v=P + (2 << 40),
          op=P + (4 << 40), lp=P + (8 << 40)), 2),        # G * Nq = 2^31 packed rows per K/V head
])
def test_splitkv_rejects_bad_arguments_before_any_hip_call(lib, kw, code):
    assert call_split(lib, **kw) == code
    assert lib.fa_last_error() != b""


def test_splitkv_and_merge_empty_problems(lib):
    assert call_split(lib, q=0, k=0, v=0, op=0, lp=0, B=0) == 0
    assert call_split(lib, q=0, k=0, v=0, op=0, lp=0, Nq=0) == 0
    assert lib.fa_merge(0, 0, 0, 0, 4, 0, 2, 8, 64, 1, None) == 0
    assert lib.fa_merge(0, 0, 0, 0, 4, 1, 2, 0, 64, 1, None) == 0


@pytest.mark.parametrize("args,code", [
    ((0, P + 0x100000, P + 0x200000, P + 0x300000, 4, 1, 2, 8, 64, 1), 1),       # null o_part
    ((P, P + 0x100000, P + 0x200000, P + 0x300000, 0, 1, 2, 8, 64, 1), 1),       # no splits
    ((P, P + 0x100000, P + 0x200000, P + 0x300000, 4, 1, 0, 8, 64, 1), 1),       # H = 0
    ((P, P + 0x100000, P + 0x200000, P + 0x300000, 4, 1, 2, 8, 96, 1), 2),       # d
    ((P, P + 0x100000, P + 0x200000, P + 0x300000, 4, 1, 2, 8, 64, 7), 1),       # unknown dtype
    ((P, P + 0x100000, P + 8, P + 0x300000, 4, 1, 2, 8, 64, 1), 1),              # o overlaps o_part
])
def test_merge_rejects_bad_arguments(lib, args, code):
    assert lib.fa_merge(*args, None) == code
    assert lib.fa_last_error() != b""


def test_merge_row_limit(lib):
    """One merge launch runs four rows per 256-thread workgroup, and a launch's work-item count
    is 32-bit: more than 4 * (2^24 - 1) rows are refused before any HIP call (only the refused
    side is called here: the accepted side would launch)."""
    rows = 4 * (0xFFFFFFFF // 256) + 1
    # far-apart pointers, so the huge extents do not overlap
    assert lib.fa_merge(1 << 40, 2 << 40, 3 << 40, 4 << 40, 1, 1, 1, rows, 64, 1, None) == 2
    assert b"rows" in lib.fa_last_error()


def test_split_chunk_and_default_splits(lib):
    assert lib.fa_split_chunk(4096, 1) == 4096
    assert lib.fa_split_chunk(4096, 3) == 1408          # ceil(4096/3) = 1366 -> next multiple of 64
    assert lib.fa_split_chunk(100, 8) == 64
    assert lib.fa_split_chunk(-1, 2) == -1 and lib.fa_split_chunk(10, 0) == -1
    for (B, Hq, Hkv, Nq, Nk) in [(8, 32, 8, 1, 32768), (1, 8, 8, 4096, 4096), (1, 1, 1, 1, 100)]:
        s = lib.fa_splitkv_num_splits(B, Hq, Hkv, Nq, Nk)
        assert 1 <= s <= 1024
        assert s <= max(1, (Nk + 255) // 256)
    # one decode row per query head, 4 heads per K/V head: 64 workgroups before splitting
    assert lib.fa_splitkv_num_splits(8, 32, 8, 1, 32768) == 16
    assert lib.fa_splitkv_num_splits(0, 1, 1, 1, 1) == -1
    assert lib.fa_splitkv_num_splits(1, 3, 2, 1, 1) == -1


@pytest.mark.parametrize("args,code", [
    ((0, P + 0x100000, 0, 4, 64, 0, 0), 1),                   # null x
    ((P, P + 0x100000, 0, 4, 64, 5, 0), 1),                   # unknown dtype
    ((P, P + 0x100000, 0, 4, 64, 0, 2), 1),                   # unknown algorithm
    ((P, P + 0x100000, 0, -1, 64, 0, 0), 1),                  # negative rows
    ((P, P + 0x100000, 0, 4, 0, 0, 0), 1),                    # empty rows
    ((P, P + 4, 0, 4, 64, 0, 0), 1),                          # misaligned y
    ((P, P + 0x40, 0, 4, 64, 0, 0), 1),                       # y overlaps x without being x
    ((P, P + 0x100000, P + 0x20, 4, 64, 0, 0), 1),            # lse overlaps x
    ((P, P + 0x100000, 0, 1 << 31, 64, 0, 0), 2),             # too many rows for the grid
    ((P, P, 0, 1, (1 << 31) - 4095, 0, 0), 2),                # one column past the 32-bit index limit
    ((P, P, 0, 1, (1 << 31) - 1, 0, 0), 2),
])
def test_softmax_rejects_bad_arguments(lib, args, code):
    assert lib.fa_softmax(*args, None) == code
    assert lib.fa_last_error() != b""


def test_softmax_empty_matrix_is_ok(lib):
    assert lib.fa_softmax(0, 0, 0, 0, 64, 0, 0, None) == 0
    assert lib.fa_softmax(0, 0, 0, 0, 0, 1, 1, None) == 0


def call_bwd(lib, q=P, k=P + 0x100000, v=P + 0x200000, o=P + 0x300000, lse=P + 0x400000, do=P + 0x500000,
             dq=P + 0x600000, dk=P + 0x700000, dv=P + 0x800000, delta=P + 0x900000, B=1, Hq=2, Hkv=1, N=300,
             d=64, causal=1, scale=0.125, dtype=1, stream=None):
    return lib.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, delta, B, Hq, Hkv, N, d, causal, scale, dtype, stream)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), 1), (dict(lse=0), 1), (dict(do=0), 1), (dict(delta=0), 1), (dict(dv=P + 0x800008), 1),
    (dict(B=-1), 1), (dict(N=-1), 1), (dict(Hq=3, Hkv=2), 1), (dict(Hkv=0), 1), (dict(causal=2), 1),
    (dict(scale=float("inf")), 1), (dict(scale=3e38), 1),
    (dict(dtype=0), 2), (dict(dtype=5), 1), (dict(d=80), 2),
    (dict(dq=P + 0x500000), 1),                           # dq overlaps dO
    (dict(dk=P + 0x600100), 1),                           # dk overlaps dq
    (dict(delta=P + 0x300000), 1),                        # delta overlaps o
    (dict(dv=P + 0x400000), 1),                           # dv overlaps lse
])
def test_bwd_rejects_bad_arguments_before_any_hip_call(lib, kw, code):
    assert call_bwd(lib, **kw) == code
    assert lib.fa_last_error() != b""


def test_bwd_empty_problems(lib):
    z = dict(q=0, k=0, v=0, o=0, lse=0, do=0, dq=0, dk=0, dv=0, delta=0)
    assert call_bwd(lib, B=0, **z) == 0
    assert call_bwd(lib, N=0, **z) == 0


def call_bwd_split(lib, part=P + 0xa00000, splits=2, **kw):
    a = dict(q=P, k=P + 0x100000, v=P + 0x200000, o=P + 0x300000, lse=P + 0x400000, do=P + 0x500000,
             dq=P + 0x600000, dk=P + 0x700000, dv=P + 0x800000, delta=P + 0x900000, B=1, Hq=2, Hkv=1, N=300,
             d=64, causal=1, scale=0.125, dtype=1, stream=None)
    a.update(kw)
    return lib.fa_bwd_split(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"],
                            a["delta"], part, splits, a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], a["causal"],
                            a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(splits=0), 1), (dict(splits=9), 1), (dict(part=0), 1), (dict(part=P + 0xa00008), 1),
    (dict(part=P + 0x700000), 1),                         # workspace overlaps dk
    (dict(part=P + 0x500000), 1),                         # workspace overlaps dO
    (dict(dtype=0), 2), (dict(d=96), 2), (dict(Hq=3, Hkv=2), 1),
])
def test_bwd_split_rejects_bad_arguments(lib, kw, code):
    assert call_bwd_split(lib, **kw) == code
    assert lib.fa_last_error() != b""


def test_bwd_split_needs_no_workspace_for_one_split_and_sizes(lib):
    z = dict(q=0, k=0, v=0, o=0, lse=0, do=0, dq=0, dk=0, dv=0, delta=0)
    assert call_bwd_split(lib, part=0, splits=4, B=0, **z) == 0
    # one split takes no workspace: it reaches the pointer checks, not the workspace check
    assert call_bwd_split(lib, part=0, splits=1, q=0) == 1 and b"null" in lib.fa_last_error()
    # GQA 32/8 at N = 8192, one sequence: 512 key-tile workgroups, so two splits
    assert lib.fa_bwd_num_splits(1, 32, 8, 8192) == 2
    assert lib.fa_bwd_num_splits(2, 32, 32, 4096) == 1
    assert lib.fa_bwd_num_splits(1, 1, 1, 128) == 8
    assert lib.fa_bwd_num_splits(0, 1, 1, 1) == -1 and lib.fa_bwd_num_splits(1, 3, 2, 8) == -1


def test_head_size_limit_leaves_room_for_the_last_tile(lib):
    """Tiles address up to 128 rows past N through 32-bit buffer offsets: a head whose K/V
    with that slack would pass 2^31 - 1 bytes is refused before any HIP call (only the
    refused side is called here: the accepted side would launch)."""
    n_over = (0x7FFFFFFF // 256) - 128 + 1          # d = 128, 2-byte elements: 256 B rows
    assert call(lib, N=n_over, d=128, B=1, Hq=1, Hkv=1) == 2
    assert b"2 GiB" in lib.fa_last_error()
    assert call_split(lib, Nq=1, Nk=n_over, d=128, Hq=1, Hkv=1, causal=0) == 2
    assert call_bwd(lib, N=n_over, d=128, Hq=1, Hkv=1) == 2


def call_bwd_noalloc(lib, splits=2, **kw):
    a = dict(q=P, k=P + 0x100000, v=P + 0x200000, o=P + 0x300000, lse=P + 0x400000, do=P + 0x500000,
             dq=P + 0x600000, dk=P + 0x700000, dv=P + 0x800000, delta=P + 0x900000, B=1, Hq=2, Hkv=1, N=300,
             d=64, causal=1, scale=0.125, dtype=1, stream=None)
    a.update(kw)
    return lib.fa_bwd_split_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"],
                                    a["delta"], splits, a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], a["causal"],
                                    a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(splits=0), 1), (dict(splits=9), 1), (dict(q=0), 1), (dict(dq=P + 0x500000), 1),
    (dict(dtype=0), 2), (dict(d=96), 2), (dict(Hq=3, Hkv=2), 1),
])
def test_bwd_noalloc_rejects_bad_arguments_before_any_hip_call(lib, kw, code):
    assert call_bwd_noalloc(lib, **kw) == code
    assert lib.fa_last_error() != b""


def test_bwd_noalloc_refuses_partials_beyond_its_static_workspace(lib):
    """2 * splits * B * Hkv * N * d * 4 bytes must fit the static array; a larger call is
    refused on the host, before any HIP call, with the sizes in the message."""
    cap = lib.fa_bwd_noalloc_max_bytes()
    assert cap == 128 << 20
    # 2 * 8 * 1 * 8 * 4096 * 128 * 4 = 256 MiB > 128 MiB (pointers spaced so nothing overlaps)
    big = dict(q=P, k=P + (1 << 32), v=P + (2 << 32), o=P + (3 << 32), lse=P + (4 << 32), do=P + (5 << 32),
               dq=P + (6 << 32), dk=P + (7 << 32), dv=P + (8 << 32), delta=P + (9 << 32),
               B=1, Hq=8, Hkv=8, N=4096, d=128)
    assert call_bwd_noalloc(lib, splits=8, **big) == 2
    assert b"static workspace" in lib.fa_last_error()
    z = dict(q=0, k=0, v=0, o=0, lse=0, do=0, dq=0, dk=0, dv=0, delta=0)
    assert call_bwd_noalloc(lib, splits=8, B=0, **z) == 0          # empty: nothing to do


def _fresh(code):
    return subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT)


def test_binding_maps_one_hip_runtime():
    """Through the binding (torch first) libfa binds to torch's HIP runtime: one is mapped."""
    r = _fresh("from flashattention_online_softmax_fwd_amd import _lib\n_lib.load()\n"
               "print(len(_lib.hip_runtimes_mapped()))")
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "1"


def test_loading_libfa_before_torch_is_refused_before_any_launch():
    """libfa loaded ahead of torch maps the system HIP runtime and torch then maps its own:
    the binding refuses to run in that state instead of launching into it."""
    r = _fresh("import ctypes\nctypes.CDLL('flashattention_online_softmax_fwd_amd/libfa.so')\n"
               "from flashattention_online_softmax_fwd_amd import _lib\n"
               "print(len(_lib.hip_runtimes_mapped()))\n"
               "try:\n    _lib.load()\nexcept _lib.TwoHipRuntimes as e:\n    print('refused', e)\n")
    assert r.returncode == 0, r.stderr
    lines = r.stdout.splitlines()
    assert lines[0] == "2" and lines[1].startswith("refused")
