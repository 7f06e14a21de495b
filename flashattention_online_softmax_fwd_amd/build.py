"""Build libfa.so (the gfx950 kernels plus the C ABI) in-tree with hipcc.

Run as ``python -m flashattention_online_softmax_fwd_amd.build`` or through
``__graft_entry__.build()``.  Every call recompiles.  Objects go to
``_build/`` next to this file and the library to ``libfa.so`` beside it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfa.so")

SOURCES = ["fa_host.cpp", "fa_fwd_mfma16.hip", "fa_fwd_w64.hip", "fa_fwd_f32.hip", "fa_merge.hip", "fa_softmax.hip",
           "fa_bwd_mfma16.hip"]
# Sources generated before compiling: the key loop of fa_fwd_w64.hip (gfx950 assembly).
GENERATORS = [os.path.join(CSRC, "gen_fwd_kloop.py")]

ARCH = "gfx950"
# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 anywhere in the device code.
DEVICE_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-Wall", "-Wno-unused-command-line-argument"]


# Per-source additions.  The forward kernel's machine scheduler: the iterative ILP strategy
# measured about 2% faster on the causal d = 128 forwards than the default (same code
# otherwise, bitwise identical results).
SOURCE_FLAGS = {"fa_fwd_mfma16.hip": ["-mllvm", "--amdgpu-sched-strategy=iterative-ilp"]}


def device_flags(src: str) -> list:
    """The hipcc flags a source is compiled with."""
    return DEVICE_FLAGS + SOURCE_FLAGS.get(src, [])


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfa)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc()] + device_flags(src) + ["-I" + INCLUDE, "-I" + CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compiling %s failed:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def generate() -> None:
    """Regenerate the generated sources (fa_fwd_kloop.inc) from their generators."""
    for gen in GENERATORS:
        r = subprocess.run([sys.executable, gen], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("generating from %s failed:\n%s" % (gen, r.stderr))


def build(verbose: bool = False) -> str:
    generate()
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("linking libfa.so failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
