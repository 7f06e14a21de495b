"""Split-KV partial states and their merge on the GPU, against the fp64 oracle.

fa_fwd_splitkv writes, per key range, the state of the pages' two-block example
in normalised form (o = acc / l, lse = m + ln l); fa_merge folds the ranges with
the pages' merge.  The oracle side is ``attention_kv`` (the plain definition
over a key range) and ``merge_partials`` (the pages' merge in fp64), both pinned
on the CPU in test_oracle_splitkv.

Tolerance: the forward's bar for the input dtype, |x - r| <= 1e-2 + 2e-2 |r| for
bf16 and 1.25e-3 + 2.5e-3 |r| for fp16, on partial o and lse (P is rounded to the
input dtype before the PV product, as in the forward) and on the merged result;
the merge kernel alone, on float32 states, is held to |x - r| <= 2e-6 + 2e-6 |r|
for a float32 output and the 16-bit bar for a 16-bit one.
Empty states must be exactly o = 0, lse = -inf.
"""
import math

import numpy as np
import pytest
import torch

from flashattention_online_softmax_fwd_amd import inputs as fin

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    import flashattention_online_softmax_fwd_amd as fa_mod
    fa_mod.load_library()
    return fa_mod


@pytest.fixture(scope="module")
def oracle():
    from oracle import fa_oracle
    return fa_oracle


def check(x, r, atol, rtol, what):
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    assert x.shape == r.shape, (what, x.shape, r.shape)
    fin_r = np.isfinite(r)
    assert np.array_equal(np.isfinite(x), fin_r), "%s: non-finite pattern differs" % what
    assert np.array_equal(x[~fin_r], r[~fin_r]), "%s: infinite values differ" % what
    err = np.abs(x[fin_r] - r[fin_r])
    bad = err > atol + rtol * np.abs(r[fin_r])
    if bad.any():
        k = int(np.argmax(err - (atol + rtol * np.abs(r[fin_r]))))
        raise AssertionError("%s: %d of %d outside tolerance; worst got %r want %r (max abs err %.3e)"
                             % (what, int(bad.sum()), bad.size, x[fin_r][k], r[fin_r][k], err.max()))
    return float(err.max()) if err.size else 0.0


from oracle import tolerances  # noqa: E402

BF16 = tolerances.forward_bar("bf16")
F16 = tolerances.forward_bar("f16")
TOL = {"bf16": BF16, "f16": F16}

# B, Hq, Hkv, Nq, Nk, d, causal, splits
SPLIT_CASES = [
    (1, 2, 1, 419, 419, 128, True, 3),     # square, ragged, several tiles per range
    (1, 2, 2, 419, 419, 64, False, 4),
    (2, 4, 2, 1, 1000, 128, True, 4),      # one query (decode), GQA
    (1, 2, 1, 5, 700, 128, True, 5),       # offset 695: the diagonal straddles key tiles
    (1, 2, 1, 37, 300, 64, True, 2),       # offset 263
    (1, 3, 3, 130, 300, 128, False, 3),    # more query rows than one tile, non-causal
    (1, 1, 1, 64, 200, 128, True, 16),     # more ranges than tiles: empty ranges
    (1, 2, 1, 200, 200, 128, True, 7),     # square causal: later ranges empty for early rows
    (1, 8, 2, 40, 500, 128, True, 3),      # 4 query heads per K/V head: a row tile spans heads
    (2, 4, 1, 100, 333, 64, True, 2),      # 400 packed rows per K/V head, ragged
]


def _case_inputs(B, Hq, Hkv, Nq, Nk, d, seed, dtype):
    return fin.make_qkv(B, Hq, Hkv, Nq, d, dtype, seed, 1.0, Nk=Nk)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("case", SPLIT_CASES)
def test_partial_states_match_the_oracle_range_by_range(fa, oracle, case, dtype):
    B, Hq, Hkv, Nq, Nk, d, causal, S = case
    q, k, v = _case_inputs(B, Hq, Hkv, Nq, Nk, d, 2000 + Nq + Nk + S, dtype)
    sc = 1.0 / math.sqrt(d)
    print("splitkv partial states", case, dtype, flush=True)
    op, lp = fa.forward_splitkv(q.cuda(), k.cuda(), v.cuda(), S, causal=causal, scale=sc)
    torch.cuda.synchronize()
    op, lp = op.cpu().numpy(), lp.cpu().numpy()
    c = fa.fa_split_chunk(Nk, S)
    for s in range(S):
        lo, hi = min(Nk, s * c), min(Nk, (s + 1) * c)
        ro, rl = oracle.attention_kv(q, k, v, causal=causal, scale=sc, k_range=(lo, hi))
        tag = "%s range %d [%d, %d)" % (case, s, lo, hi)
        check(lp[s], rl, *TOL[dtype], "lse_part " + tag)
        empty = ~np.isfinite(rl)
        assert np.all(op[s][empty] == 0.0), "o_part of empty states must be 0: " + tag
        check(op[s][~empty], ro[~empty], *TOL[dtype], "o_part " + tag)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("case", SPLIT_CASES)
def test_split_and_merge_match_the_full_oracle(fa, oracle, case, dtype):
    B, Hq, Hkv, Nq, Nk, d, causal, S = case
    q, k, v = _case_inputs(B, Hq, Hkv, Nq, Nk, d, 3000 + Nq + Nk + S, dtype)
    sc = 1.0 / math.sqrt(d)
    print("splitkv + merge", case, dtype, flush=True)
    o, lse = fa.attention_kv(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=sc, num_splits=S)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_kv(q, k, v, causal=causal, scale=sc)
    assert o.dtype == q.dtype
    check(o.float().cpu().numpy(), ro, *TOL[dtype], "O %s %s" % (case, dtype))
    check(lse.cpu().numpy(), rl, *TOL[dtype], "LSE %s %s" % (case, dtype))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_one_range_matches_the_forward(fa, oracle, d, causal, dtype):
    """S = 1 over a square problem: one range, normalised once and merged with weight 1, is the
    whole attention.  The split kernel and the square forward are different kernels (the
    square forward lets its reference lag further and sums in another order), so each meets
    the bar against the oracle and they agree to within the sum of their bars."""
    q, k, v = fin.make_qkv(2, 4, 2, 333, d, dtype, 4000 + d)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    print("split S=1 vs forward d=%d causal=%d" % (d, causal), flush=True)
    o_ref, l_ref = fa.forward(qd, kd, vd, causal=causal)
    o, lse = fa.attention_kv(qd, kd, vd, causal=causal, num_splits=1)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(q, k, v, causal=causal, scale=1.0 / math.sqrt(d))
    atol, rtol = TOL[dtype]
    check(o.float().cpu().numpy(), ro, atol, rtol, "split S=1 o")
    check(lse.cpu().numpy(), rl, atol, rtol, "split S=1 lse")
    check(o_ref.float().cpu().numpy(), ro, atol, rtol, "forward o")
    check(o.float().cpu().numpy(), o_ref.float().cpu().numpy(), 2 * atol, 2 * rtol, "split S=1 o vs forward o")
    check(lse.cpu().numpy(), l_ref.cpu().numpy(), 2 * atol, 2 * rtol, "split S=1 lse vs forward lse")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_merge_kernel_matches_the_pages_merge(fa, oracle, d, out_dtype):
    S, B, H, N = 6, 2, 3, 50
    rng = np.random.default_rng(5000 + d)
    o_part = rng.standard_normal((S, B, H, N, d)).astype(np.float32)
    lse_part = (rng.standard_normal((S, B, H, N)) * 20.0).astype(np.float32)
    empty = rng.random((S, B, H, N)) < 0.3
    empty[:, 0, 0, 0] = True                          # one row with no key at all
    lse_part[empty] = -np.inf
    o_part[empty] = 0.0
    print("merge kernel d=%d %s" % (d, out_dtype), flush=True)
    o, lse = fa.merge(torch.from_numpy(o_part).cuda(), torch.from_numpy(lse_part).cuda(), out_dtype=out_dtype)
    torch.cuda.synchronize()
    ro, rl = oracle.merge_partials(o_part, lse_part)
    tol_o = {torch.float32: (2e-6, 2e-6), torch.bfloat16: BF16, torch.float16: F16}[out_dtype]
    check(o.float().cpu().numpy(), ro, *tol_o, "merged o")
    check(lse.cpu().numpy(), rl, 2e-6, 2e-6, "merged lse")
    assert lse[0, 0, 0].item() == -math.inf and torch.all(o[0, 0, 0] == 0)


def test_results_are_deterministic(fa):
    q, k, v = fin.make_qkv(1, 4, 1, 7, 128, "bf16", 6000, 1.0, Nk=3000)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    a = fa.attention_kv(qd, kd, vd, causal=True, num_splits=5)
    b = fa.attention_kv(qd, kd, vd, causal=True, num_splits=5)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("name", sorted(fin.KV_WORKLOADS))
def test_measured_workloads_at_full_size(fa, oracle, name):
    """The decode workloads at their real size, in the launch configuration the bench times."""
    w = fin.KV_WORKLOADS[name]
    q, k, v = fin.kv_workload_inputs(w)
    S = fa.fa_splitkv_num_splits(w.B, w.Hq, w.Hkv, w.Nq, w.Nk)
    print("full-size split-KV workload", name, "splits", S, flush=True)
    o, lse = fa.attention_kv(q.cuda(), k.cuda(), v.cuda(), causal=w.causal, num_splits=S)
    torch.cuda.synchronize()
    o, lse = o.float().cpu(), lse.cpu()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    total = w.B * w.Hq * w.Nq
    rows = np.unique(np.concatenate([[0, total - 1], np.random.default_rng(w.seed).choice(total, 96, replace=False)]))
    ro, rl = oracle.attention_kv(q, k, v, causal=w.causal, scale=w.softmax_scale, rows=rows)
    check(o.reshape(-1, w.d).numpy()[rows], ro, *BF16, "O " + name)
    check(lse.reshape(-1).numpy()[rows], rl, *BF16, "LSE " + name)


def test_longest_key_head_the_abi_accepts(fa, oracle):
    """One decode row against the longest K/V head the ABI takes at d = 128: (Nk + 128) d 2 bytes
    just below 2^31.  With one key range a single workgroup walks the whole head, so its buffer
    range and the last tile's offsets are the largest any launch can use; the default split count
    is checked too.  Four keys score far above the 8.4M others (16 to 17.5 against about N(0, 1))
    and carry distinct value rows: the first key, the middle one, one in the last tile and the very
    last, so a range cut short or mis-addressed near its end moves O far past the bar.  One key
    more is refused before anything is launched."""
    d = 128
    nk = 0x7FFFFFFF // (2 * d) - 128
    print("longest accepted head: Nk", nk, flush=True)
    q, k, v = fin.make_qkv_device(1, 1, 1, 1, nk, d, "bf16", seed=1201)
    scale = 1.0 / math.sqrt(d)
    qf = q.float().reshape(d)
    spikes = [(0, 16.0), (nk // 2, 16.5), (nk - 65, 17.0), (nk - 1, 17.5)]
    for n, (pos, target) in enumerate(spikes):
        k[0, 0, pos] = (qf * (target / (scale * float(qf @ qf)))).to(torch.bfloat16)
        row = torch.zeros(d, device=v.device)
        row[8 * n + 3] = 8.0
        v[0, 0, pos] = row.to(torch.bfloat16)
    results = {}
    for S in (1, fa.fa_splitkv_num_splits(1, 1, 1, 1, nk)):
        results[S] = fa.attention_kv(q, k, v, causal=True, num_splits=S)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_kv(q.cpu(), k.cpu(), v.cpu(), causal=True, scale=scale)
    for n in range(len(spikes)):   # every planted key carries a visible share of O
        assert ro[0, 0, 0, 8 * n + 3] > 0.4, (n, ro[0, 0, 0, 8 * n + 3])
    for S, (o, lse) in results.items():
        check(o.float().cpu().numpy(), ro, *BF16, "O at the longest head, %d ranges" % S)
        check(lse.cpu().numpy(), rl, *BF16, "LSE at the longest head, %d ranges" % S)
    op = torch.empty((1, 1, 1, 1, d), dtype=torch.float32, device=q.device)
    lp = torch.empty((1, 1, 1, 1), dtype=torch.float32, device=q.device)
    rc = fa.fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), op.data_ptr(), lp.data_ptr(),
                           1, 1, 1, 1, nk + 1, d, 1, scale, fa.FA_DTYPE_BF16, 1, None)
    assert rc == fa.FA_ERR_UNSUPPORTED and "2 GiB" in fa.fa_last_error()
