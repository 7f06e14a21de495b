"""Static checks on the gfx950 code the kernels compile to (CPU only: hipcc here).

The 16-bit (bf16 and fp16) forward and backward kernels stage tiles with loads that
write LDS directly (buffer_load ... lds).  Those loads count in vmcnt, and a workgroup barrier does
not by itself wait for them: every s_barrier must therefore follow an s_waitcnt
that includes vmcnt(0), or a wave could pass the barrier while its part of the
next tile is still landing and other waves would read stale data.
"""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "flashattention_online_softmax_fwd_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")


def compile_asm(tmp_path_factory, source):
    if not HIPCC:
        pytest.skip("hipcc not available")
    from flashattention_online_softmax_fwd_amd import build
    out = str(tmp_path_factory.mktemp("isa") / (source + ".s"))
    flags = [f for f in build.device_flags(source) if f != "-fPIC"]   # the library's own flags
    subprocess.run([HIPCC] + flags + ["-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
                    "--offload-device-only", "-S", os.path.join(CSRC, source), "-o", out],
                   check=True, capture_output=True)
    return open(out).read()


@pytest.fixture(scope="module")
def bf16_asm(tmp_path_factory):
    return compile_asm(tmp_path_factory, "fa_fwd_mfma16.hip")


@pytest.fixture(scope="module")
def bwd_asm(tmp_path_factory):
    return compile_asm(tmp_path_factory, "fa_bwd_mfma16.hip")


def kernels(asm, pattern=r"_ZN2fa12fwd16_kernel"):
    for name in re.findall(r"^(%s\S+):" % pattern, asm, re.M):
        i = asm.index(name + ":")
        j = asm.index(".Lfunc_end", i)
        body = [l.strip() for l in asm[i:j].splitlines()]
        yield name, [l for l in body if l and not l.startswith((";", "."))]


def test_every_barrier_waits_for_lds_dma(bf16_asm):
    found = 0
    for name, ins in kernels(bf16_asm):
        found += 1
        assert any(x.startswith("buffer_load_dwordx4") and x.endswith("lds") for x in ins), name
        for n, x in enumerate(ins):
            if x.startswith("s_barrier"):
                assert ins[n - 1].startswith("s_waitcnt") and "vmcnt(0)" in ins[n - 1], (name, n, ins[n - 1])
    assert found >= 24      # bf16 and fp16: 8 square and 4 split instantiations each


def test_no_packed_fp32_and_no_scratch(bf16_asm):
    for name, ins in kernels(bf16_asm):
        assert not any(x.startswith(("v_pk_add_f32", "v_pk_mul_f32", "v_pk_fma_f32")) for x in ins), name
    # the default tile shapes must not spill
    for name, ins in kernels(bf16_asm):
        if "Li128ELi64E" in name:
            assert not any(x.startswith("scratch_") for x in ins), name


def test_backward_barriers_wait_for_lds_dma_and_nothing_spills(bwd_asm):
    found = 0
    for name, ins in kernels(bwd_asm, r"_ZN2fa1[35]bwd_d\w+_kernel"):
        found += 1
        assert any(x.startswith("buffer_load_dword") and x.endswith("lds") for x in ins), name
        for n, x in enumerate(ins):
            if x.startswith("s_barrier"):
                assert ins[n - 1].startswith("s_waitcnt") and "vmcnt(0)" in ins[n - 1], (name, n, ins[n - 1])
        assert not any(x.startswith(("v_pk_add_f32", "v_pk_mul_f32", "v_pk_fma_f32")) for x in ins), name
        assert not any(x.startswith("scratch_") for x in ins), name
    assert found == 16      # dq and dk/dv, bf16 and fp16, d 64 and 128, causal or not


def test_static_workspace_is_a_device_symbol(bwd_asm):
    """The allocation-free backward looks up its static workspace by name at run time.  The
    device pass must emit the array as a global symbol of its full size: if the device pass
    does not see host code take its address (for instance because that code is compiled
    for the host only), it drops the unused array, and the runtime's lookup of the name the
    host registers then aborts the process."""
    m = re.search(r"^\s*\.globl\s+(\S*scratch\S*)\s*$", bwd_asm, re.M)
    assert m, "no global device symbol for the static workspace"
    size = re.search(r"^\s*\.size\s+%s,\s*(\d+)" % re.escape(m.group(1)), bwd_asm, re.M)
    assert size and int(size.group(1)) == 128 << 20


@pytest.fixture(scope="module")
def w64_asm(tmp_path_factory):
    return compile_asm(tmp_path_factory, "fa_fwd_w64.hip")


def test_w64_kernels_wait_for_lds_dma_before_barriers_and_do_not_spill(w64_asm):
    """The 64-rows-per-wave forward is written as assembly by gen_fwd_kloop.py: every barrier
    must still follow a wait for this wave's LDS DMA loads, and the kernels must fit the
    register file (one wave per SIMD) without scratch.

    Every barrier waits for vmcnt(0) except an item's first one.  There the first item of a
    workgroup has just waited for vmcnt(0) on its own loads (a branch right before), and a
    later item's first tiles were loaded by the item before it ahead of that item's epilogue:
    exactly 2 + 8 d / 32 stores of O and LSE, the only vector memory operations younger than
    those loads, may still be in flight, so the wait is vmcnt(that count)."""
    found = 0
    for name, ins in kernels(w64_asm, r"_ZN2fa14fwd_w64_kernel"):
        found += 1
        nst = 34 if name.endswith("Li128EEEvNS_9FwdParamsE") else 18
        assert any(x.startswith("buffer_load_dwordx4") and x.endswith("lds") for x in ins), name
        barriers = [n for n, x in enumerate(ins) if x.startswith("s_barrier")]
        assert barriers, name
        for k, n in enumerate(barriers):
            w = ins[n - 1]
            assert w.startswith("s_waitcnt"), (name, n, w)
            if k == 0:
                assert "vmcnt(0)" in w or "vmcnt(%d)" % nst in w, (name, n, w)
                assert "s_waitcnt vmcnt(0)" in ins[n - 4:n - 1], (name, n, ins[n - 6:n])
            else:
                assert "vmcnt(0)" in w, (name, n, w)
        assert not any(x.startswith(("v_pk_add_f32", "v_pk_mul_f32", "v_pk_fma_f32")) for x in ins), name
        assert not any(x.startswith("scratch_") for x in ins), name
        assert not any(x.startswith(("s_store", "s_buffer_store", "s_atomic", "s_dcache")) for x in ins), name
    assert found == 16      # bf16 and fp16, causal or not, 2 or 4 waves, d = 64 or 128


def test_generated_key_loop_is_up_to_date():
    """fa_fwd_kloop.inc is what gen_fwd_kloop.py writes (the build regenerates it)."""
    import tempfile
    gen = os.path.join(CSRC, "gen_fwd_kloop.py")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.inc")
        env = dict(os.environ, OUT_INC=out)
        subprocess.run([sys.executable, gen], check=True, env=env)
        assert open(out).read() == open(os.path.join(CSRC, "fa_fwd_kloop.inc")).read()


def test_w64_compiler_code_leaves_m0_to_the_key_loop(w64_asm):
    """The key loop's inline assembly sets m0 (the LDS address of its DMA loads) and lists it
    among its clobbers, which the compiler ignores for this reserved register (it warns so).
    That is safe only while the code the compiler writes around the assembly never reads or
    writes m0: no instruction outside the asm blocks of any instantiation may name it."""
    found = 0
    for name in re.findall(r"^(_ZN2fa14fwd_w64_kernel\S+):", w64_asm, re.M):
        found += 1
        i = w64_asm.index(name + ":")
        j = w64_asm.index(".Lfunc_end", i)
        inside, asm_m0 = False, 0
        for line in w64_asm[i:j].splitlines():
            s = line.strip()
            if s.startswith(";;#ASMSTART"):
                inside = True
                continue
            if s.startswith(";;#ASMEND"):
                inside = False
                continue
            if not s or s.startswith((";", ".")) or not re.search(r"\bm0\b", s):
                continue
            assert inside, (name, s)
            asm_m0 += 1
        assert asm_m0 > 0, name            # the key loop does use m0
    assert found == 16
