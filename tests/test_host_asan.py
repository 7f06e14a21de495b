"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only, no GPU needed).

Two programs are built with the sanitizers and run here:
- tests/asan/host_abi_checks.cpp against the library's host side (fa_host.cpp compiled with
  the sanitizers on its host pass only, linked with the device objects of the in-tree build):
  every argument check and empty-problem path of the C ABI, none of which reaches HIP;
- tests/asan/oracle_checks.c against the fp64 oracle (oracle/fa_ref.c, built serially):
  odd shapes on exact-size heap buffers, checked against facts that hold for any input.
A sanitizer report ends the program with a nonzero status and its text names the fault.
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "flashattention_online_softmax_fwd_amd")
HERE = os.path.join(ROOT, "tests", "asan")
HIPCC = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")
SAN = ["address", "undefined"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r


def test_oracle_under_sanitizers(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_checks")
    run(["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=" + ",".join(SAN),
         "-fno-sanitize-recover=all", "-fno-fast-math", "-ffp-contract=off",
         os.path.join(HERE, "oracle_checks.c"), os.path.join(ROOT, "oracle", "fa_ref.c"), "-o", exe, "-lm"])
    r = run([exe], env=ENV, timeout=300)
    assert "oracle checks passed" in r.stdout


def test_library_host_checks_under_sanitizers(tmp_path):
    if not HIPCC:
        pytest.skip("hipcc not available")
    from flashattention_online_softmax_fwd_amd import build
    objs = [os.path.join(build.BUILD_DIR, s + ".o") for s in build.SOURCES if s != "fa_host.cpp"]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("the in-tree build has not been run")
    host = []
    for s in SAN:
        host += ["-Xarch_host", "-fsanitize=" + s]
    host += ["-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    inc = ["-I" + os.path.join(ROOT, "include"), "-I" + build.CSRC]
    host_obj = str(tmp_path / "fa_host_san.o")
    run([HIPCC, "-x", "hip", "--offload-arch=" + build.ARCH, "-O1", "-g", "-std=c++17", "-fPIC"] + host + inc +
        ["-c", os.path.join(build.CSRC, "fa_host.cpp"), "-o", host_obj])
    drv_obj = str(tmp_path / "host_abi_checks.o")
    run([HIPCC, "-O1", "-g", "-std=c++17"] + host + inc + ["-c", os.path.join(HERE, "host_abi_checks.cpp"), "-o", drv_obj])
    exe = str(tmp_path / "host_abi_checks")
    run([HIPCC, "--offload-arch=" + build.ARCH] + host + [drv_obj, host_obj] + objs + ["-o", exe])
    r = run([exe], env=ENV, timeout=300)
    assert "host checks passed" in r.stdout
