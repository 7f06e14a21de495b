"""Pins for the fp64 oracle, against facts it does not compute itself.

Each test ties the three-pass oracle (oracle/fa_ref.c) to something outside it:
numbers printed on the pages (tests/golden/*.json, each with its source),
closed forms of attention, invariances of the definition, and two library
routines it never calls (torch's CPU scaled_dot_product_attention in float64
and torch.logsumexp).  The pins are chosen so that a dropped term, a wrong sign
or index, an off-by-one causal mask, a wrong GQA head map, a transposed operand
or a natural/base-2 log mix-up fails at least one of them (see
test_oracle_mutations.py, which plants exactly those mistakes).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import fa_oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def embed(scores, values):
    """Put given scores and values into the 4-D API.

    d = number of value columns; every query is e0, key j is scores[j]*e0, so
    with scale 1 the score of key j is exactly scores[j] for every query.
    """
    s = np.asarray(scores, dtype=np.float64)
    v = np.asarray(values, dtype=np.float64)
    if v.ndim == 1:
        v = v[:, None]
    n, dv = v.shape
    q = np.zeros((1, 1, n, dv))
    q[..., 0] = 1.0
    k = np.zeros((1, 1, n, dv))
    k[0, 0, :, 0] = s
    return q, k, v.reshape(1, 1, n, dv)


def run(scores, values, causal=False):
    q, k, v = embed(scores, values)
    o, lse = fa_oracle.attention(q, k, v, causal=causal, scale=1.0)
    return o[0, 0], lse[0, 0]


# --------------------------------------------------------------- pages' numbers

def test_p1_four_scores_all_at_once():
    g = golden("p1_four_scores.json")
    a = g["all_at_once"]
    o, lse = run(g["scores"], g["values"])
    assert np.all(np.abs(o[:, 0] - a["output_code_printed"]) <= g["rounding_tolerance_8_places"])
    assert abs(o[0, 0] - a["output"]) <= g["rounding_tolerance_4_places"]
    l = math.exp(lse[0] - a["max"])        # normaliser measured against the max
    assert abs(l - a["weights_sum"]) <= g["rounding_tolerance_4_places"]
    assert abs(o[0, 0] * l - a["weighted_sum"]) <= g["rounding_tolerance_4_places"]
    # the weights themselves, through one-hot values
    w, _ = run(g["scores"], np.eye(4))
    assert np.allclose(w[0] * l, a["weights_vs_max"], atol=g["rounding_tolerance_4_places"])


def test_p1_first_block_alone_is_a_causal_prefix():
    """Row 1 under the causal mask sees exactly the first block (scores 1 and 3)."""
    g = golden("p1_four_scores.json")
    b1 = g["two_blocks"]["after_block_1"]
    o, lse = run(g["scores"], g["values"], causal=True)
    assert abs(o[1, 0] - b1["output_2_places"]) <= g["rounding_tolerance_2_places"]
    l1 = math.exp(lse[1] - b1["m"])
    assert abs(l1 - b1["l"]) <= g["rounding_tolerance_4_places"]
    assert abs(l1 * o[1, 0] - b1["acc"]) <= g["rounding_tolerance_4_places"]
    # rescaling that state to the final max 5 gives the page's corrected numbers
    r = g["two_blocks"]["rescaled"]
    assert abs(math.exp(lse[1] - 5.0) - r["l"]) <= g["rounding_tolerance_4_places"]
    assert abs(math.exp(lse[1] - 5.0) * o[1, 0] - r["acc"]) <= g["rounding_tolerance_4_places"]
    # row 0 sees only key 0
    assert o[0, 0] == 10.0 and lse[0] == 1.0


def test_p2_is_not_the_block_mean():
    g = golden("p2_not_block_mean.json")
    x = [0.0, 0.0, math.log(3.0), math.log(3.0)]
    o, _ = run(x, g["values"])
    assert abs(o[0, 0] - g["output"]) <= 1e-12
    halves = [run(x[:2], g["values"][:2])[0][0, 0], run(x[2:], g["values"][2:])[0][0, 0]]
    assert np.allclose(halves, g["block_results"], atol=1e-12)
    assert abs(np.mean(halves) - g["wrong_block_mean"]) <= 1e-12
    assert abs(o[0, 0] - np.mean(halves)) > 0.2
    w, _ = run(x, np.eye(4))
    assert np.allclose(w[0] / w[0, 0], g["unnormalised_weight_proportions"], atol=1e-12)


def test_p4_shares_and_top_score():
    g = golden("p4_worked_example.json")
    w, lse = run(g["scores"], np.eye(5))
    assert np.allclose(w[0], g["probabilities_4_places"], atol=5e-5)
    assert round(100 * w[0, 3]) == g["share_of_top_score_percent"]
    assert abs(w[0].sum() - 1.0) <= 1e-14
    # the denominator check of the page: sum of exp(x - 5) to 5 places
    assert abs(math.exp(lse[0] - 5.0) - g["final_sum_check"]["sum"]) <= 5e-5
    assert np.allclose(w[0] * math.exp(lse[0] - 5.0), g["final_sum_check"]["terms_5_places"],
                       atol=5e-6)


def test_p4_tables_as_causal_prefixes():
    """Row i of a causal run over x = 1,3,2,5,4 is the state after step i+1."""
    g = golden("p4_worked_example.json")
    x = g["scores"]
    o, lse = run(x, g["values"], causal=True)
    prefix_max = np.maximum.accumulate(x)
    l = np.exp(lse - prefix_max)
    assert np.allclose(l, g["table1_by_hand"]["l"], atol=5e-5)
    assert list(prefix_max) == g["table1_by_hand"]["m"] == g["figure4"]["running_max"]
    assert np.allclose(o[:, 0], g["values_table_by_hand"]["output_2_places"], atol=0.005)
    acc = l * o[:, 0]
    assert abs(acc[-1] - g["full_precision_final_acc"]) <= 5e-5
    assert np.max(np.abs(acc - g["values_table_by_hand"]["acc"])) < 2e-3
    assert np.allclose(l, g["figure4"]["running_sum_2_places"], atol=0.005)
    f2 = g["figure2"]
    assert abs(l[2] - f2["tally_before"]) <= 5e-4
    assert abs(l[3] - f2["tally_after"]) <= 5e-4
    assert abs(math.exp(prefix_max[2] - prefix_max[3]) - f2["shrink_factor"]) <= 5e-5
    assert abs(o[-1, 0] - g["textbook_weighted_average_3_places"]) < 2e-3


def test_overflow_inputs_stay_finite():
    """Scores near 1000 overflow a naive exp; the oracle subtracts the max."""
    g = golden("p4_overflow.json")
    x = g["naive_softmax_input_float32"]
    with np.errstate(all="ignore"):
        e = np.exp(np.asarray(x, dtype=np.float32))
        assert np.isnan(e / e.sum()).all()              # the page's failure is real
        assert np.isinf(np.exp(np.float32(88.8))) and np.isfinite(np.exp(np.float32(88.7)))
    w, lse = run(x, np.eye(3))
    want = np.array([math.exp(-2.0), math.exp(-1.0), 1.0])
    want /= want.sum()
    assert np.all(np.isfinite(w)) and np.allclose(w[0], want, atol=1e-15)
    assert abs(lse[0] - (1002.0 + math.log(1 + math.exp(-1.0) + math.exp(-2.0)))) <= 1e-12


# ------------------------------------------------------------- library routines

SDPA_CASES = [
    # B, Hq, Hkv, N, d, causal
    (1, 1, 1, 1, 8, False),
    (1, 1, 1, 1, 8, True),
    (2, 2, 2, 5, 8, True),
    (1, 4, 2, 17, 16, False),
    (1, 4, 1, 17, 16, True),
    (2, 8, 2, 64, 64, True),
    (1, 2, 2, 130, 32, False),
    (1, 6, 3, 65, 128, True),
]


@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal", SDPA_CASES)
def test_matches_torch_sdpa_and_logsumexp(B, Hq, Hkv, N, d, causal):
    rng = np.random.default_rng(B * 1000 + Hq * 100 + N + d)
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    scale = 1.0 / math.sqrt(d)
    o, lse = fa_oracle.attention(q, k, v, causal=causal, scale=scale)
    tq, tk, tv = (torch.from_numpy(a) for a in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=causal, scale=scale, enable_gqa=(Hq != Hkv))
    assert np.max(np.abs(o - ref.numpy())) <= 1e-12
    # LSE: torch.logsumexp over the visible scores, keys of head h // (Hq/Hkv)
    kk = torch.repeat_interleave(tk, Hq // Hkv, dim=1)
    s = torch.matmul(tq, kk.transpose(-1, -2).contiguous()) * scale
    if causal:
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    assert np.max(np.abs(lse - torch.logsumexp(s, dim=-1).numpy())) <= 1e-12


# ----------------------------------------------------------------- closed forms

def rand_qkv(seed, B=1, Hq=2, Hkv=2, N=37, d=16):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, Hq, N, d)), rng.standard_normal((B, Hkv, N, d)),
            rng.standard_normal((B, Hkv, N, d)))


@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_give_the_mean_of_visible_values(causal):
    q, k, v = rand_qkv(1)
    q[:] = 0.0
    o, lse = fa_oracle.attention(q, k, v, causal=causal)
    N = q.shape[2]
    if causal:
        cnt = np.arange(1, N + 1)
        mean = np.cumsum(v, axis=2) / cnt[None, None, :, None]
    else:
        cnt = np.full(N, N)
        mean = np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
    assert np.allclose(o, mean, atol=1e-13)
    assert np.allclose(lse, np.log(cnt)[None, None, :], atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_values_are_returned_exactly(causal):
    q, k, v = rand_qkv(2)
    q *= 12.0
    v[:] = 0.625
    o, _ = fa_oracle.attention(q, k, v, causal=causal)
    assert np.allclose(o, 0.625, atol=1e-14)


def test_single_key():
    q, k, v = rand_qkv(3, N=1)
    o, lse = fa_oracle.attention(q, k, v, causal=False, scale=0.3)
    assert np.allclose(o, v, atol=0)
    assert np.allclose(lse, 0.3 * np.einsum("bhnd,bhnd->bhn", q, k), atol=1e-14)


def test_dominant_key_takes_all_the_weight():
    q, k, v = rand_qkv(4, N=20, d=8)
    q[:] = 0.0
    q[..., 0] = 1.0
    k[..., 0] = 0.0
    k[:, :, 13, 0] = 60.0        # 60 above every other score
    o, _ = fa_oracle.attention(q, k, v, causal=False, scale=1.0)
    assert np.allclose(o, v[:, :, 13:14, :], atol=1e-20 + 19 * math.exp(-60) * 10)


def test_shifting_every_score_moves_only_the_lse():
    q, k, v = rand_qkv(5, d=15)
    scale, c = 0.25, 7.5
    o, lse = fa_oracle.attention(q, k, v, causal=True, scale=scale)
    one = np.ones(q.shape[:3] + (1,))
    q2 = np.concatenate([q, one], axis=-1)
    k2 = np.concatenate([k, np.full(k.shape[:3] + (1,), c / scale)], axis=-1)
    v2 = np.concatenate([v, np.zeros(v.shape[:3] + (1,))], axis=-1)
    o2, lse2 = fa_oracle.attention(q2, k2, v2, causal=True, scale=scale)
    assert np.allclose(o2[..., :-1], o, atol=1e-13)
    assert np.allclose(lse2, lse + c, atol=1e-12)


def test_non_causal_key_permutation_changes_nothing():
    q, k, v = rand_qkv(6)
    perm = np.random.default_rng(0).permutation(q.shape[2])
    o, lse = fa_oracle.attention(q, k, v)
    o2, lse2 = fa_oracle.attention(q, k[:, :, perm], v[:, :, perm])
    assert np.allclose(o, o2, atol=1e-13) and np.allclose(lse, lse2, atol=1e-13)


def test_gqa_equals_repeated_kv_heads():
    q, k, v = rand_qkv(7, B=2, Hq=6, Hkv=2)
    o, lse = fa_oracle.attention(q, k, v, causal=True)
    kr, vr = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)
    o2, lse2 = fa_oracle.attention(q, kr, vr, causal=True)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_scale_is_applied_to_the_dot_product():
    q, k, v = rand_qkv(8)
    o, lse = fa_oracle.attention(q, k, v, scale=0.5)
    o2, lse2 = fa_oracle.attention(q * 4.0, k, v, scale=0.125)
    assert np.allclose(o, o2, atol=1e-13) and np.allclose(lse, lse2, atol=1e-13)


def test_causal_row_sees_exactly_the_keys_up_to_itself():
    q, k, v = rand_qkv(9, N=12)
    o, lse = fa_oracle.attention(q, k, v, causal=True)
    j = 7
    k2, v2 = k.copy(), v.copy()
    k2[:, :, j] += 3.0
    v2[:, :, j] -= 5.0
    o2, lse2 = fa_oracle.attention(q, k2, v2, causal=True)
    assert np.array_equal(o[:, :, :j], o2[:, :, :j]) and np.array_equal(lse[:, :, :j], lse2[:, :, :j])
    assert np.all(np.abs(o[:, :, j:] - o2[:, :, j:]).max(axis=-1) > 0)
    assert np.array_equal(o[:, :, 0], v[:, :, 0])


def test_row_list_matches_full_run():
    q, k, v = rand_qkv(10, B=2, Hq=4, Hkv=2, N=29)
    o, lse = fa_oracle.attention(q, k, v, causal=True)
    rows = np.array([0, 5, 28, 29, 57, 100, 231])
    o2, lse2 = fa_oracle.attention(q, k, v, causal=True, rows=rows)
    assert np.array_equal(o.reshape(-1, 16)[rows], o2)
    assert np.array_equal(lse.reshape(-1)[rows], lse2)


def test_bad_arguments_are_rejected():
    q, k, v = rand_qkv(11, Hq=3, Hkv=2)
    with pytest.raises(ValueError):
        fa_oracle.attention(q, k, v)                    # 3 % 2 != 0
    q, k, v = rand_qkv(11)
    with pytest.raises(ValueError):
        fa_oracle.attention(q, k, v, rows=[10 ** 6])     # row out of range
    with pytest.raises(ValueError):
        fa_oracle.attention(q, k, v, scale=float("nan"))


def test_empty_problem():
    q = np.zeros((0, 2, 5, 8))
    o, lse = fa_oracle.attention(q, np.zeros((0, 2, 5, 8)), np.zeros((0, 2, 5, 8)))
    assert o.shape == (0, 2, 5, 8) and lse.shape == (0, 2, 5)
