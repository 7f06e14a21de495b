"""Pins for the oracle's key-range attention and its merge of partial states.

``fa_oracle.attention_kv`` computes the plain definition over a key range (and
for Nq query rows that are the last Nq positions of Nk keys);
``fa_oracle.merge_partials`` folds partial states with the pages' merge.  Both
are pinned here against things other than themselves:
- the states of the kbwen.com "Two blocks" example, printed on the page;
- the full-row oracle (pinned on its own in test_oracle_pins): merging the
  partials of any partition of the keys must give it back;
- torch's scaled_dot_product_attention with an explicit mask, in fp64;
- the empty state: no weight, the identity of the merge.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import fa_oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _embed(scores, values):
    """A 1-D score row as attention: q = e0, k_j = x_j e0, v_j = val_j e0, scale 1."""
    s = np.asarray(scores, dtype=np.float64)
    n = s.size
    q = np.zeros((1, 1, n, 1))
    q[..., 0] = 1.0
    k = s.reshape(1, 1, n, 1)
    v = np.asarray(values, dtype=np.float64).reshape(1, 1, n, 1)
    return q, k, v


def test_two_blocks_states_match_the_page():
    g = _golden("p1_four_scores.json")
    tb = g["two_blocks"]
    tol4 = g["rounding_tolerance_4_places"]
    q, k, v = _embed(g["scores"], g["values"])
    qlast = q[:, :, -1:]                       # one query, non-causal: sees every key
    o1, l1 = fa_oracle.attention_kv(qlast, k, v, scale=1.0, k_range=(0, 2))
    o2, l2 = fa_oracle.attention_kv(qlast, k, v, scale=1.0, k_range=(2, 4))
    b1, b2 = tb["after_block_1"], tb["block_2_own"]
    # block 1 against its own max 3: l, acc, and the output "for a query with only these keys"
    assert abs(math.exp(l1[0, 0, 0] - b1["m"]) - b1["l"]) <= tol4
    assert abs(o1[0, 0, 0, 0] * b1["l"] - b1["acc"]) <= 4 * tol4 * b1["acc"]
    assert abs(o1[0, 0, 0, 0] - b1["output_2_places"]) <= g["rounding_tolerance_2_places"]
    # block 2 against the new max 5
    l2_own = math.exp(l2[0, 0, 0] - 5.0)
    assert abs(l2_own - b2["l"]) <= tol4
    assert abs(o2[0, 0, 0, 0] * l2_own - b2["acc"]) <= 4 * tol4 * b2["acc"]
    # the merge of the two gives the totals and the output
    o, lse = fa_oracle.merge_partials(np.stack([o1, o2]), np.stack([l1, l2]))
    fin = tb["final"]
    assert abs(math.exp(lse[0, 0, 0] - 5.0) - fin["l"]) <= tol4
    assert abs(o[0, 0, 0, 0] - g["all_at_once"]["output_code_printed"]) <= g["rounding_tolerance_8_places"]


CASES = [  # B, Hq, Hkv, Nq, Nk, d, causal
    (1, 2, 1, 37, 37, 8, True),
    (2, 4, 2, 29, 29, 5, False),
    (1, 2, 2, 5, 41, 6, True),     # trailing queries against a longer key sequence
    (1, 3, 1, 1, 50, 4, True),     # one query: the decode shape
    (1, 1, 1, 7, 33, 3, False),
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("splits", [1, 2, 3, 7])
def test_merging_partitions_gives_the_full_row(case, splits):
    B, Hq, Hkv, Nq, Nk, d, causal = case
    rng = np.random.default_rng(100 * Nq + Nk + splits)
    q = rng.standard_normal((B, Hq, Nq, d))
    k = rng.standard_normal((B, Hkv, Nk, d))
    v = rng.standard_normal((B, Hkv, Nk, d))
    full_o, full_l = fa_oracle.attention_kv(q, k, v, causal=causal, scale=0.7)
    cuts = np.linspace(0, Nk, splits + 1).round().astype(int)
    parts = [fa_oracle.attention_kv(q, k, v, causal=causal, scale=0.7, k_range=(lo, hi))
             for lo, hi in zip(cuts[:-1], cuts[1:])]
    o, lse = fa_oracle.merge_partials(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    assert np.all(np.abs(o - full_o) <= 1e-12)
    assert np.all(np.abs(lse - full_l) <= 1e-12)
    if Nq == Nk:   # the square case is the forward oracle itself
        sq_o, sq_l = fa_oracle.attention(q, k, v, causal=causal, scale=0.7)
        assert np.array_equal(sq_o, full_o) and np.array_equal(sq_l, full_l)


@pytest.mark.parametrize("case", CASES)
def test_key_range_matches_masked_sdpa(case):
    """The definition with an explicit mask: visible iff lo <= j < hi and (causal) j <= i + Nk - Nq."""
    B, Hq, Hkv, Nq, Nk, d, causal = case
    rng = np.random.default_rng(7 * Nq + Nk)
    q = rng.standard_normal((B, Hq, Nq, d))
    k = rng.standard_normal((B, Hkv, Nk, d))
    v = rng.standard_normal((B, Hkv, Nk, d))
    lo, hi = Nk // 4, Nk - Nk // 5
    o, lse = fa_oracle.attention_kv(q, k, v, causal=causal, scale=0.5, k_range=(lo, hi))
    i = np.arange(Nq)[:, None]
    j = np.arange(Nk)[None, :]
    vis = np.broadcast_to((j >= lo) & (j < hi), (Nq, Nk)).copy()
    if causal:
        vis &= j <= i + (Nk - Nq)
    tq, tk, tv = (torch.from_numpy(a) for a in (q, k, v))
    tk = torch.repeat_interleave(tk, Hq // Hkv, dim=1)
    tv = torch.repeat_interleave(tv, Hq // Hkv, dim=1)
    s = torch.matmul(tq, tk.transpose(-1, -2).contiguous()) * 0.5
    s = s.masked_fill(~torch.from_numpy(vis), float("-inf"))
    rows_with_keys = vis.any(axis=1)
    lref = torch.logsumexp(s, dim=-1).numpy()
    w = torch.softmax(s, dim=-1)
    oref = torch.matmul(w, tv).numpy()
    assert np.all(np.abs(o[:, :, rows_with_keys] - oref[:, :, rows_with_keys]) <= 1e-12)
    assert np.all(np.abs(lse[:, :, rows_with_keys] - lref[:, :, rows_with_keys]) <= 1e-12)
    # rows with no visible key: the empty state
    assert np.all(o[:, :, ~rows_with_keys] == 0.0)
    assert np.all(lse[:, :, ~rows_with_keys] == -np.inf)


def test_empty_state_is_the_identity_of_the_merge():
    rng = np.random.default_rng(5)
    o = rng.standard_normal((3, 4))
    lse = rng.standard_normal(3)
    empty_o, empty_l = np.zeros((3, 4)), np.full(3, -np.inf)
    for stack in ([empty_o, o], [o, empty_o], [empty_o, o, empty_o]):
        ls = [empty_l if x is empty_o else lse for x in stack]
        mo, ml = fa_oracle.merge_partials(np.stack(stack), np.stack(ls))
        assert np.allclose(mo, o, rtol=0, atol=1e-15) and np.allclose(ml, lse, rtol=0, atol=1e-15)
    mo, ml = fa_oracle.merge_partials(np.stack([empty_o, empty_o]), np.stack([empty_l, empty_l]))
    assert np.all(mo == 0.0) and np.all(ml == -np.inf)


def test_merge_does_not_depend_on_the_order():
    rng = np.random.default_rng(11)
    S, R, d = 5, 6, 3
    o = rng.standard_normal((S, R, d))
    lse = rng.standard_normal((S, R)) * 30.0     # spread maxima: every rescale path is taken
    ref_o, ref_l = fa_oracle.merge_partials(o, lse)
    for perm in ([4, 3, 2, 1, 0], [2, 0, 4, 1, 3]):
        po, pl = fa_oracle.merge_partials(o[perm], lse[perm])
        assert np.allclose(po, ref_o, rtol=1e-13, atol=1e-13) and np.allclose(pl, ref_l, rtol=0, atol=1e-12)
    # weights exp(lse_s - lse) sum to one: a closed form of the merged lse
    assert np.allclose(ref_l, np.log(np.exp(lse - lse.max(0)).sum(0)) + lse.max(0), rtol=0, atol=1e-12)
