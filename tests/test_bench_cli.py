"""bench.py's command line on the host: the one-GPU contract and argument checks (no GPU needed)."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


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
    c = bench.counters_for("c3_bf16_n4096_d128_causal", "bf16")
    assert c is not None
    assert 0.0 < c["mfma_busy"] <= 1.0
    assert 0.5 < c["sclk_ghz"] < 2.6
    assert c["lds_bank_conflict_rate"] >= 0.0
    assert bench.counters_for("no_such_workload", "bf16") is None
    monkeypatch.setattr(bench, "kernel_hash", lambda source: "0" * 64)
    assert bench.counters_for("c3_bf16_n4096_d128_causal", "bf16") is None
    assert bench.traffic_for("c3_bf16_n4096_d128_causal", "bf16") is None


def test_backward_counters_are_keyed_per_kernel():
    for part in ("dq", "dkdv"):
        c = bench.counters_for("b1_bf16_bwd_n4096_d128_causal", "bwd/" + part)
        assert c is not None and 0.0 < c["mfma_busy"] <= 1.0
