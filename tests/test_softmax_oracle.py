"""Pins for the row-softmax oracle (oracle/softmax_oracle.py).

Pinned against the pages' numbers (the five-score probabilities, the overflow
example), library routines (torch and scipy in float64), and closed forms.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import softmax_oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_five_scores_give_the_pages_probabilities():
    g = _golden("p4_worked_example.json")
    y, lse = softmax_oracle.softmax_rows(np.array([g["scores"]]))
    assert np.allclose(y[0], g["probabilities_4_places"], rtol=0, atol=5e-5)
    assert round(100 * y[0][3]) == g["share_of_top_score_percent"]
    # the normaliser against the max 5 is the table's final l
    assert abs(math.exp(lse[0] - 5.0) - g["table1_by_hand"]["l"][-1]) <= 5e-5


def test_overflow_example_is_finite():
    g = _golden("p4_overflow.json")
    x = np.array([g["naive_softmax_input_float32"]])
    y, lse = softmax_oracle.softmax_rows(x)
    want = np.exp(np.array([-2.0, -1.0, 0.0]))
    assert np.all(np.isfinite(y)) and np.allclose(y[0], want / want.sum(), rtol=0, atol=1e-15)
    assert abs(lse[0] - (1002.0 + math.log(want.sum()))) <= 1e-12


@pytest.mark.parametrize("shape", [(1, 1), (3, 7), (5, 1000), (2, 4097)])
def test_matches_library_softmax(shape):
    rng = np.random.default_rng(shape[1])
    x = rng.standard_normal(shape) * 10.0
    y, lse = softmax_oracle.softmax_rows(x)
    assert np.allclose(y, torch.softmax(torch.from_numpy(x), dim=1).numpy(), rtol=1e-13, atol=0)
    assert np.allclose(y, scipy.special.softmax(x, axis=1), rtol=1e-13, atol=0)
    assert np.allclose(lse, scipy.special.logsumexp(x, axis=1), rtol=0, atol=1e-12)


def test_closed_forms():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 300))
    y, lse = softmax_oracle.softmax_rows(x)
    assert np.allclose(y.sum(axis=1), 1.0, rtol=0, atol=1e-13)            # shares sum to one
    ys, ls = softmax_oracle.softmax_rows(x + 37.5)                          # shift: y unchanged
    assert np.allclose(ys, y, rtol=1e-12, atol=0) and np.allclose(ls, lse + 37.5, rtol=0, atol=1e-12)
    yc, lc = softmax_oracle.softmax_rows(np.full((2, 64), 3.0))            # constant row: uniform
    assert np.allclose(yc, 1 / 64, rtol=1e-15, atol=0) and np.allclose(lc, 3.0 + math.log(64), atol=1e-14)
    xd = np.zeros((1, 10))
    xd[0, 6] = 60.0                                                         # a dominant entry
    yd, _ = softmax_oracle.softmax_rows(xd)
    assert abs(yd[0, 6] - 1.0) < 1e-25 and np.all(yd[0, :6] < 1e-25)
    p = rng.permutation(300)                                                # permutation moves shares
    yp, lp = softmax_oracle.softmax_rows(x[:, p])
    assert np.allclose(yp, y[:, p], rtol=1e-13, atol=0) and np.allclose(lp, lse, rtol=0, atol=1e-13)


def test_masked_entries_and_empty_rows():
    x = np.array([[0.0, -np.inf, math.log(3.0)], [-np.inf, -np.inf, -np.inf]])
    y, lse = softmax_oracle.softmax_rows(x)
    assert np.allclose(y[0], [0.25, 0.0, 0.75], rtol=0, atol=1e-15)
    assert abs(lse[0] - math.log(4.0)) <= 1e-15
    assert np.all(np.isnan(y[1])) and lse[1] == -np.inf


def test_reading_counts_of_the_two_algorithms():
    """The pages' counts: safe softmax reads every score 3 times, online statistics once, online
    softmax with its output twice; with the write that is 4 and 3 accesses per element."""
    g = _golden("p4_reading_once.json")
    n = g["scores"]
    r = g["reads_of_the_scores"]
    assert r["safe softmax (max, sum, output)"] == 3 * n
    assert r["online statistics (m and l only)"] == n
    assert r["online softmax with the output written"] == 2 * n
    acc = g["memory_accesses_per_element_including_the_write"]
    rw = g["reads_and_writes_per_element"]
    assert acc["safe"] == sum(rw["safe"]) and acc["online"] == sum(rw["online"])
    assert abs(acc["safe"] / acc["online"] - 4 / 3) < 1e-12 and g["reported_speedup_up_to"] <= 4 / 3 + 0.01


def test_bench_prices_each_algorithm_with_the_pages_access_counts():
    import bench
    g = _golden("p4_reading_once.json")
    assert {k: list(v) for k, v in bench.SOFTMAX_ACCESSES.items()} == g["reads_and_writes_per_element"]


# Plausible mistakes planted in a copy of the oracle's source; each must fail one of the pins above.
MUTANTS = {
    "no_max_subtraction": ("e = np.exp(x - m)", "e = np.exp(x)"),
    "min_instead_of_max": ("m = x.max(axis=1, keepdims=True)", "m = x.min(axis=1, keepdims=True)"),
    "lse_without_m": ("lse = (m + np.log(l))[:, 0]", "lse = np.log(l)[:, 0]"),
    "lse_log2": ("lse = (m + np.log(l))[:, 0]", "lse = (m + np.log2(l))[:, 0]"),
    "not_normalised": ("y = e / l", "y = e"),
    "sum_over_rows": ("l = e.sum(axis=1, keepdims=True)", "l = e.sum(axis=0, keepdims=True)"),
    "empty_rows_zero": ("y[empty] = np.nan", "y[empty] = 0.0"),
}


def _mutant(name):
    import importlib.util
    import inspect
    src = inspect.getsource(softmax_oracle)
    old, new = MUTANTS[name]
    assert src.count(old) == 1, name
    spec = importlib.util.spec_from_loader("softmax_oracle_" + name, loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(src.replace(old, new), "softmax_oracle_" + name, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_every_planted_mistake_fails_a_pin(name, monkeypatch):
    import warnings
    monkeypatch.setattr(softmax_oracle, "softmax_rows", _mutant(name).softmax_rows)
    pins = [test_five_scores_give_the_pages_probabilities, test_overflow_example_is_finite,
            lambda: test_matches_library_softmax((5, 1000)), test_closed_forms,
            test_masked_entries_and_empty_rows]
    failed = 0
    for pin in pins:
        try:
            with warnings.catch_warnings():
                warnings.simplefilter("ignore")
                pin()
        except (AssertionError, FloatingPointError, ValueError):
            failed += 1
    assert failed >= 1, name
