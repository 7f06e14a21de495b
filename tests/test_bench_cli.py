"""bench.py's command line on the host: the one-GPU contract and argument checks (no GPU needed)."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from flashattention_online_softmax_fwd_amd import inputs as fin  # noqa: E402


@pytest.mark.parametrize("n", [2, 4, 8])
def test_more_than_one_gpu_is_refused_with_a_message(n, capsys):
    assert bench.main(["--gpus", str(n)]) == 2
    assert "one GPU" in capsys.readouterr().err


@pytest.mark.parametrize("argv", [["--steps", "0"], ["--warmup", "-1"]])
def test_bad_step_counts_are_refused(argv, capsys):
    assert bench.main(argv) == 2
    assert "--steps" in capsys.readouterr().err


def test_kernel_hash_covers_sources_and_flags():
    h = bench.kernel_hash("bf16")
    assert isinstance(h, str) and len(h) == 64
    assert h == bench.kernel_hash("f16")        # one source, one set of flags
    assert h != bench.kernel_hash("bwd")
    assert h != bench.kernel_hash("f32")


def test_committed_shader_counters_are_read_and_go_stale_with_the_kernel(monkeypatch):
    import json
    with open(bench.SQ_FILE) as f:
        stored = json.load(f)["c3_bf16_n4096_d128_causal"]["bf16"]["kernel_source_sha256"]
    monkeypatch.setattr(bench, "kernel_hash", lambda source: stored)     # the kernel the pass measured
    c = bench.counters_for("c3_bf16_n4096_d128_causal", "bf16")
    assert c is not None
    assert 0.0 < c["mfma_busy"] <= 1.0
    assert 0.5 < c["sclk_ghz"] < 2.6
    assert c["lds_bank_conflict_rate"] >= 0.0
    assert bench.counters_for("no_such_workload", "bf16") is None
    monkeypatch.setattr(bench, "kernel_hash", lambda source: "0" * 64)   # the kernel changed since
    assert bench.counters_for("c3_bf16_n4096_d128_causal", "bf16") is None
    assert bench.traffic_for("c3_bf16_n4096_d128_causal", "bf16") is None


def test_backward_counters_are_keyed_per_kernel(monkeypatch):
    import json
    with open(bench.SQ_FILE) as f:
        table = json.load(f)["b1_bf16_bwd_n4096_d128_causal"]
    for part in ("dq", "dkdv"):
        stored = table["bwd/" + part]["kernel_source_sha256"]
        monkeypatch.setattr(bench, "kernel_hash", lambda source: stored)   # the kernel the pass measured
        c = bench.counters_for("b1_bf16_bwd_n4096_d128_causal", "bwd/" + part)
        assert c is not None and 0.0 < c["mfma_busy"] <= 1.0


def test_each_forward_workload_names_its_own_metric():
    from flashattention_online_softmax_fwd_amd import inputs as fin
    with open(os.path.join(ROOT, "BASELINE.json")) as f:
        import json
        headline = json.load(f)["metric"]
    assert bench.metric_for(fin.WORKLOADS[fin.BENCH_WORKLOAD]) == headline
    names = {bench.metric_for(w) for w in fin.WORKLOADS.values()}
    assert len(names) == len(fin.WORKLOADS) - 1      # c3h and c3 differ in dtype; c5s shares c3's shape
    assert "f16 N=2048 d=64 non-causal" in bench.metric_for(fin.WORKLOADS["c2h_f16_n2048_d64"])
    assert "GQA 32/8" in bench.metric_for(fin.WORKLOADS["c4_bf16_gqa_n8192_d128_causal"])


def test_oracle_leg_uses_each_dtypes_parity_bar():
    """The fp16 bar is the bf16 one times 2^-3: an fp16 error the parity tests accept must not
    read as a mismatch, and a bf16-sized error must read as one."""
    import numpy as np

    from oracle import tolerances
    r = np.array([0.5, -1.0, 2.0])
    assert tolerances.within(r + 1.0e-3, r, "f16")
    assert not tolerances.within(r + 1.0e-2, r, "f16")
    assert tolerances.within(r + 1.5e-2, r, "bf16")
    assert not tolerances.within(r + 2e-5, r, "f32")
    assert not tolerances.within(np.array([np.nan, 0, 0]), r, "bf16")
    src = open(os.path.join(ROOT, "bench.py")).read()
    assert "tolerances.within(go, ro, w.dtype)" in src


def test_bench_names_the_kernel_the_library_dispatches():
    """bench.forward_kernel mirrors the library's default choice; the stamp slots the library
    reserves (workgroups x waves, no walk without a GPU) tell the kernels apart."""
    from flashattention_online_softmax_fwd_amd import _lib
    lib = _lib.load()
    for name, w in fin.WORKLOADS.items():
        if w.dtype == "f32":
            continue
        src, kname = bench.forward_kernel(w, 1024)
        code = {"bf16": _lib.FA_DTYPE_BF16, "f16": _lib.FA_DTYPE_F16}[w.dtype]
        units = w.B * w.Hq
        if src == "w64":
            nw = int(kname.split(",")[2])
            rows = 64 * nw
        else:
            nw, rows = 4, 128
        want = units * ((w.N + rows - 1) // rows) * nw
        assert lib.fa_fwd_stamp_slots(w.B, w.Hq, w.N, w.d, code) == want, (name, src, kname)


def test_cpu_baseline_reports_the_whole_workload_time():
    """cpu_baseline's full_problem_seconds: the measured time when every row was done, else the
    sample's time scaled by the workload's flops over the sample's, labelled extrapolated.  Run
    on the CPU with the oracle's own outputs standing in for the GPU's."""
    import torch
    from oracle import fa_oracle
    w = fin.WORKLOADS["c1_f32_n256_d64"]
    q, k, v = fin.workload_inputs(w)
    ro, rl = fa_oracle.attention(q, k, v, causal=w.causal, scale=w.softmax_scale)
    o, lse = torch.from_numpy(ro).float(), torch.from_numpy(rl).float()
    full = bench.cpu_baseline(w, q, k, v, o, lse, 60.0)
    assert full["rows"] == 256 and full["full_problem_seconds_kind"] == "measured"
    assert full["full_problem_seconds"] == pytest.approx(full["seconds"])
    part = bench.cpu_baseline(w, q, k, v, o, lse, 1e-12)      # stops after its first chunk of 64 rows
    assert part["rows"] == 64 and part["full_problem_seconds_kind"] == "extrapolated"
    assert part["gpu_matches_oracle_on_sample"]
    assert part["full_problem_seconds"] > part["seconds"]
