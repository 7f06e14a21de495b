"""Plant plausible mistakes in the oracle's C source and show the pins catch each.

Every mutant is a copy of oracle/fa_ref.c with one textual change, built with
gcc into a temporary directory and driven through the same Python handle.  All
mutants stay inside the arrays they are given, so a wrong build cannot crash
the test process.  The unmutated source must pass every check, and every
mutant must fail at least one.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import fa_oracle

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "fa_ref.c")

MUTANTS = {
    "pass2_without_max": [("l += exp(s[j] - m);", "l += exp(s[j]);")],
    "no_max_anywhere": [("l += exp(s[j] - m);", "l += exp(s[j]);"),
                        ("const double w = exp(s[j] - m) / l;", "const double w = exp(s[j]) / l;")],
    "min_as_reference": [("if (s[j] > m) m = s[j];", "if (s[j] < m || m == -INFINITY) m = s[j];")],
    "causal_excludes_diagonal": [("causal ? i + (Nk - Nq) : Nk - 1", "causal ? i + (Nk - Nq) - 1 : Nk - 1")],
    "causal_one_key_too_many": [("causal ? i + (Nk - Nq) : Nk - 1", "causal ? i + (Nk - Nq) + 1 : Nk - 1")],
    "causal_ignored": [("causal ? i + (Nk - Nq) : Nk - 1", "Nk - 1")],
    "causal_offset_dropped": [("causal ? i + (Nk - Nq) : Nk - 1", "causal ? i : Nk - 1")],
    "range_start_ignored": [("const int j_lo = k_lo;", "const int j_lo = 0;")],
    "range_end_ignored": [("const int j_hi = last + 1 < k_hi ? last + 1 : k_hi;", "const int j_hi = last + 1;")],
    "empty_range_lse_zero": [("*lse_out = -INFINITY;\n        return;", "*lse_out = 0.0;\n        return;")],
    "gqa_modulo_map": [("const int hk = h / group;", "const int hk = h % Hkv;")],
    "lse_in_log2": [("*lse_out = m + log(l);", "*lse_out = m + log2(l);")],
    "lse_drops_max": [("*lse_out = m + log(l);", "*lse_out = log(l);")],
    "scale_dropped": [("s[j] = scale * dot;", "s[j] = dot;")],
    "scores_transposed": [("const double* qi = q + row * d;",
                           "const double* qi = k + ((int64_t)b * Hkv + hk) * Nk * d + (int64_t)i * d;"),
                          ("const double* kh = k + ((int64_t)b * Hkv + hk) * Nk * d;",
                           "const double* kh = q + ((int64_t)b * Hq + h) * Nq * d;")],
    "key_index_reversed": [("const double* kj = kh + (int64_t)j * d;",
                            "const double* kj = kh + (int64_t)(j_hi - 1 - (j - j_lo)) * d;")],
    "values_reversed": [("const double* vj = vh + (int64_t)j * d;",
                         "const double* vj = vh + (int64_t)(j_hi - 1 - (j - j_lo)) * d;")],
    "weights_not_normalised": [("const double w = exp(s[j] - m) / l;", "const double w = exp(s[j] - m);")],
    "weight_sign_flipped": [("const double w = exp(s[j] - m) / l;", "const double w = exp(m - s[j]) / l;")],
    "dot_drops_last_term": [("for (t = 0; t < d; ++t) dot += qi[t] * kj[t];",
                             "for (t = 0; t < d - 1; ++t) dot += qi[t] * kj[t];")],
}


def _embed(scores, values):
    s = np.asarray(scores, dtype=np.float64)
    v = np.asarray(values, dtype=np.float64)
    v = v[:, None] if v.ndim == 1 else v
    n, dv = v.shape
    q = np.zeros((1, 1, n, dv))
    q[..., 0] = 1.0
    k = np.zeros((1, 1, n, dv))
    k[0, 0, :, 0] = s
    return q, k, v.reshape(1, 1, n, dv)


def _run(lib, scores, values, causal=False):
    q, k, v = _embed(scores, values)
    o, lse = fa_oracle.attention(q, k, v, causal=causal, scale=1.0, lib_path=lib)
    return o[0, 0], lse[0, 0]


def check_p1(lib):
    o, lse = _run(lib, [1.0, 3.0, 5.0, 2.0], [10.0, 20.0, 30.0, 40.0])
    return (abs(o[0, 0] - 28.98474626) <= 5e-9 and abs(math.exp(lse[0] - 5.0) - 1.2034) <= 5e-5)


def check_p4_prefixes(lib):
    x = [1.0, 3.0, 2.0, 5.0, 4.0]
    o, lse = _run(lib, x, [10.0, 20.0, 30.0, 40.0, 50.0], causal=True)
    l = np.exp(lse - np.maximum.accumulate(x))
    return (np.allclose(o[:, 0], [10.0, 18.81, 21.55, 36.88, 39.95], atol=0.005)
            and np.allclose(l, [1.0, 1.1353, 1.5032, 1.2034, 1.5713], atol=5e-5))


def check_p2(lib):
    o, _ = _run(lib, [0.0, 0.0, math.log(3.0), math.log(3.0)], [0.0, 0.0, 1.0, 1.0])
    return abs(o[0, 0] - 0.75) <= 1e-12


def check_overflow(lib):
    with np.errstate(all="ignore"):
        w, lse = _run(lib, [1000.0, 1001.0, 1002.0], np.eye(3))
        want = np.array([math.exp(-2.0), math.exp(-1.0), 1.0])
        want /= want.sum()
        ok = np.all(np.isfinite(w)) and np.allclose(w[0], want, atol=1e-15)
        w2, _ = _run(lib, [-1000.0, 0.0, 1000.0], np.eye(3))
        ok = ok and np.all(np.isfinite(w2)) and np.allclose(w2[0], [0.0, 0.0, 1.0], atol=1e-15)
    return bool(ok)


def check_sdpa(lib):
    ok = True
    for (B, Hq, Hkv, N, d, causal) in [(2, 4, 2, 19, 16, True), (1, 2, 2, 23, 8, False)]:
        rng = np.random.default_rng(N)
        q = rng.standard_normal((B, Hq, N, d))
        k = rng.standard_normal((B, Hkv, N, d))
        v = rng.standard_normal((B, Hkv, N, d))
        scale = 0.3
        with np.errstate(all="ignore"):
            o, lse = fa_oracle.attention(q, k, v, causal=causal, scale=scale, lib_path=lib)
        tq, tk, tv = (torch.from_numpy(a) for a in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, is_causal=causal, scale=scale, enable_gqa=(Hq != Hkv)).numpy()
        kk = torch.repeat_interleave(tk, Hq // Hkv, dim=1)
        s = torch.matmul(tq, kk.transpose(-1, -2).contiguous()) * scale
        if causal:
            s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
        lref = torch.logsumexp(s, dim=-1).numpy()
        ok = ok and bool(np.all(np.abs(o - ref) <= 1e-12)) and bool(np.all(np.abs(lse - lref) <= 1e-12))
    return ok


def _run_kv(lib, scores, values, n_query, k_range, causal=False):
    """The embedded example with only the last n_query rows as queries, keys cut to k_range."""
    q, k, v = _embed(scores, values)
    o, lse = fa_oracle.attention_kv(q[:, :, -n_query:], k, v, causal=causal, scale=1.0,
                                    k_range=k_range, lib_path=lib)
    return o[0, 0], lse[0, 0]


def check_two_blocks(lib):
    """kbwen.com 'Two blocks': each block's own state, and the output of the first alone."""
    o1, l1 = _run_kv(lib, [1.0, 3.0, 5.0, 2.0], [10.0, 20.0, 30.0, 40.0], 1, (0, 2))
    o2, l2 = _run_kv(lib, [1.0, 3.0, 5.0, 2.0], [10.0, 20.0, 30.0, 40.0], 1, (2, 4))
    return (abs(o1[0, 0] - 18.81) <= 0.005 and abs(math.exp(l1[0] - 3.0) - 1.1353) <= 5e-5
            and abs(math.exp(l2[0] - 5.0) - 1.0498) <= 5e-5
            and abs(o2[0, 0] * math.exp(l2[0] - 5.0) - 31.9915) <= 5e-4)


def check_trailing_queries(lib):
    """The last two positions of the five-score example as queries: the causal prefixes 4 and 5."""
    o, _ = _run_kv(lib, [1.0, 3.0, 2.0, 5.0, 4.0], [10.0, 20.0, 30.0, 40.0, 50.0], 2, (0, 5), causal=True)
    return bool(np.allclose(o[:, 0], [36.88, 39.95], atol=0.005))


def check_empty_range(lib):
    """Row 0 of a causal square problem sees no key in [3, 5): the empty state."""
    o, lse = _run_kv(lib, [1.0, 3.0, 2.0, 5.0, 4.0], [10.0, 20.0, 30.0, 40.0, 50.0], 5, (3, 5), causal=True)
    return bool(o[0, 0] == 0.0 and lse[0] == -math.inf and np.isfinite(lse[4]))


CHECKS = [check_p1, check_p4_prefixes, check_p2, check_overflow, check_sdpa, check_two_blocks,
          check_trailing_queries, check_empty_range]


def _build(tmpdir, name, edits):
    text = open(SRC).read()
    for old, new in edits:
        assert text.count(old) == 1, (name, old)
        text = text.replace(old, new)
    src = os.path.join(tmpdir, name + ".c")
    with open(src, "w") as f:
        f.write(text)
    return fa_oracle.build(force=True, src=src, out=os.path.join(tmpdir, "lib_%s.so" % name))


@pytest.fixture(scope="module")
def builds(tmp_path_factory):
    d = str(tmp_path_factory.mktemp("oracle_mutants"))
    out = {"original": _build(d, "original", [])}
    for name, edits in MUTANTS.items():
        out[name] = _build(d, name, edits)
    return out


def test_original_source_passes_every_check(builds):
    assert [c.__name__ for c in CHECKS if not c(builds["original"])] == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_each_mutant_fails_a_check(builds, name):
    failed = [c.__name__ for c in CHECKS if not c(builds[name])]
    assert failed, "mutant %s passed every pin" % name
