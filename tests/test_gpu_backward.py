"""The backward kernels (fa_bwd) on the GPU, against the fp64 backward oracle.

Both sides get the same rounded q, k, v and dO.  The GPU side also takes o and
lse from the GPU forward, as a training step would; the oracle recomputes
everything in fp64 from q, k, v and dO.

Tolerance, from the arithmetic of the kernels.  Products run on 16-bit operands
with fp32 accumulation; besides the inputs, the operands rounded to the 16-bit
type (unit roundoff u: 2^-8 for bf16, 2^-11 for fp16, counting the full spacing)
are P (for dV) and dS = P (dP - D) (for dQ and dK), and D = rowsum(dO o) uses the
forward's rounded o, whose own error is at most about u times (P |V|).  So each
gradient element errs by at most a few u times the sum of the absolute values of
the terms it adds, plus its own final rounding:
    |g - r| <= 4u * M + u * |r| + a * (1 + 4 * C) + 1e-30
with M = |P|^T |dO| for dV, scale * A^T |Q| for dK, scale * A |K| for dQ, and
A = P * (|dP| + (|dO| (P |V|)) summed over d), all in fp64 from the P of the
same inputs.  The factor 4 covers the three roundings that reach one term and
fp32 sums.  a is the absolute error of rounding a value below the type's smallest
normal: 2^-25 for fp16 (its subnormal spacing is 2^-24; P and dS of a few times
1e-6 lose most of their relative precision there), 0 for bf16 (whose smallest
normal is fp32's).  C is the same sum as M with every visible P replaced by 1
(|dO| summed over the visible queries for dV, scale times |Q| or |K| summed over
the visible partners for dK and dQ).  A wrong index, a dropped tile or a
transposed operand costs errors of order M.
delta, in fp32 from the rounded o: |D - r| <= 2u * sum_e |dO| (P |V|) + 1e-6.
"""
import numpy as np
import pytest
import torch

from flashattention_online_softmax_fwd_amd import inputs as fin

pytestmark = pytest.mark.gpu

UNIT = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}
SUBNORMAL = {"bf16": 0.0, "f16": 2.0 ** -25}


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    import flashattention_online_softmax_fwd_amd as fa_mod
    fa_mod.load_library()
    return fa_mod


@pytest.fixture(scope="module")
def oracle():
    from oracle import backward_oracle
    return backward_oracle


def _f64(t):
    return t.detach().to("cpu").double().numpy()


def magnitudes(q, k, v, do, causal, scale):
    """Per element, the sums M and C of the module docstring: ((M, C) for dq, dk, dv, and
    the bound term of delta)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, Hq, N, d = q.shape
    G = Hq // k.shape[1]
    mq = np.zeros_like(q)
    mk = np.zeros_like(k)
    mv = np.zeros_like(v)
    cq = np.zeros_like(q)
    ck = np.zeros_like(k)
    cv = np.zeros_like(v)
    md = np.zeros(q.shape[:3])
    masked = np.triu(np.ones((N, N), dtype=bool), 1) if causal else np.zeros((N, N), dtype=bool)
    for b in range(B):
        for h in range(Hq):
            kh, vh = k[b, h // G], v[b, h // G]
            s = scale * (q[b, h] @ kh.T)
            s[masked] = -np.inf
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            dabs = (np.abs(do[b, h]) * (p @ np.abs(vh))).sum(axis=1)
            a = p * (np.abs(do[b, h] @ vh.T) + dabs[:, None])
            mq[b, h] = abs(scale) * (a @ np.abs(kh))
            mk[b, h // G] += abs(scale) * (a.T @ np.abs(q[b, h]))
            mv[b, h // G] += p.T @ np.abs(do[b, h])
            md[b, h] = dabs
            vis = (~masked).astype(np.float64)
            cq[b, h] = abs(scale) * (vis @ np.abs(kh))
            ck[b, h // G] += abs(scale) * (vis.T @ np.abs(q[b, h]))
            cv[b, h // G] += vis.T @ np.abs(do[b, h])
    return (mq, cq), (mk, ck), (mv, cv), md


def check(g, r, mc, dtype, what):
    g = np.asarray(g, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.all(np.isfinite(g)), "%s: non-finite values" % what
    m, c = mc
    u, a = UNIT[dtype], SUBNORMAL[dtype]
    err = np.abs(g - r)
    bound = 4 * u * m + u * np.abs(r) + a * (1 + 4 * c) + 1e-30
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err / bound), err.shape)
        raise AssertionError("%s: %d of %d outside tolerance; worst at %s: got %r want %r bound %.3e"
                             % (what, int(bad.sum()), bad.size, i, g[i], r[i], bound[i]))


def run_gpu(fa, q, k, v, do, causal, scale, num_splits=None):
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = fa.forward(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv, delta = fa.backward(qd, kd, vd, o, lse, dod, causal=causal, scale=scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu(), delta.cpu()


def compare(fa, oracle, q, k, v, do, causal, scale, dtype, what, num_splits=None):
    print("backward", what, flush=True)
    dq, dk, dv, delta = run_gpu(fa, q, k, v, do, causal, scale, num_splits)
    rq, rk, rv, rd = oracle.attention_backward(q, k, v, do, causal=causal, scale=scale)
    mq, mk, mv, md = magnitudes(q, k, v, do, causal, scale)
    check(dq.double().numpy(), rq, mq, dtype, what + " dq")
    check(dk.double().numpy(), rk, mk, dtype, what + " dk")
    check(dv.double().numpy(), rv, mv, dtype, what + " dv")
    assert np.all(np.abs(delta.double().numpy() - rd) <= 2 * UNIT[dtype] * md + 1e-6), what + " delta"
    return dq, dk, dv, delta


# (B, Hq, Hkv, N): one row, ragged tails of both the 128-row tiles and the 32-query
# tiles, several tiles, GQA groups of 2 and 4.
SHAPES = [(1, 1, 1, 1), (1, 2, 1, 17), (2, 2, 2, 64), (1, 4, 2, 130), (2, 2, 1, 257), (1, 8, 2, 384),
          (1, 2, 2, 1000)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("shape", SHAPES)
def test_matches_the_oracle(fa, oracle, shape, d, causal, dtype):
    B, Hq, Hkv, N = shape
    seed = 7 * N + d + causal
    q, k, v = fin.make_qkv(B, Hq, Hkv, N, d, dtype, seed)
    do = fin.make_dout(B, Hq, N, d, dtype, seed + 50000)
    compare(fa, oracle, q, k, v, do, causal, 1.0 / np.sqrt(d), dtype, "%s d%d causal%d %s" % (shape, d, causal, dtype))


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("splits", [1, 2, 3, 8])
@pytest.mark.parametrize("shape", [(1, 2, 1, 17), (1, 4, 2, 130), (2, 8, 2, 384), (1, 4, 1, 1000)])
def test_split_dkdv_matches_the_oracle(fa, oracle, shape, splits, causal):
    """Each key tile's query tiles shared over 1-8 workgroups (some get none when a key
    tile has fewer tiles than splits) with fp32 partials summed in split order."""
    B, Hq, Hkv, N = shape
    q, k, v = fin.make_qkv(B, Hq, Hkv, N, 128, "bf16", 900 + N)
    do = fin.make_dout(B, Hq, N, 128, "bf16", 901 + N)
    compare(fa, oracle, q, k, v, do, causal, 1.0 / np.sqrt(128), "bf16",
            "%s split%d causal%d" % (shape, splits, causal), splits)


def test_split_dkdv_is_deterministic_and_matches_one_split(fa):
    q, k, v = (t.cuda() for t in fin.make_qkv(1, 8, 2, 700, 64, "f16", 71))
    do = fin.make_dout(1, 8, 700, 64, "f16", 72).cuda()
    o, lse = fa.forward(q, k, v, causal=True)
    one = fa.backward(q, k, v, o, lse, do, causal=True, num_splits=1)
    a = fa.backward(q, k, v, o, lse, do, causal=True, num_splits=4)
    b = fa.backward(q, k, v, o, lse, do, causal=True, num_splits=4)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    assert torch.equal(a[0], one[0]) and torch.equal(a[3], one[3])      # dq and D do not depend on the split
    for x, y in zip(a[1:3], one[1:3]):                                    # dk, dv: fp32 sums regrouped
        assert torch.allclose(x.float(), y.float(), rtol=2 ** -9, atol=1e-6)


@pytest.mark.parametrize("scale", [1.0, -0.3, 0.0])
def test_other_scales(fa, oracle, scale):
    """scale 1 with large scores (peaked P), a negative scale and the uniform P of scale 0."""
    q, k, v = fin.make_qkv(1, 2, 1, 200, 128, "bf16", 31, q_mult=3.0)
    do = fin.make_dout(1, 2, 200, 128, "bf16", 32)
    compare(fa, oracle, q, k, v, do, True, scale, "bf16", "scale %g" % scale)


def test_single_key_closed_form(fa):
    """N = 1: P = 1, so dv is dO summed over the group and dq = dk = 0 (up to the
    fp32 rounding of dP - D, two sums of the same products in different orders)."""
    q, k, v = fin.make_qkv(2, 4, 2, 1, 128, "bf16", 41)
    do = fin.make_dout(2, 4, 1, 128, "bf16", 42)
    dq, dk, dv, _ = run_gpu(fa, q, k, v, do, True, 0.1)
    want = do.double().reshape(2, 2, 2, 1, 128).sum(2)
    assert dq.abs().max().item() < 1e-4 and dk.abs().max().item() < 1e-4
    assert torch.allclose(dv.double(), want, rtol=2 ** -8, atol=0)


def test_deterministic_and_autograd(fa):
    q, k, v = (t.cuda() for t in fin.make_qkv(1, 4, 2, 300, 64, "bf16", 51))
    do = fin.make_dout(1, 4, 300, 64, "bf16", 52).cuda()
    o, lse = fa.forward(q, k, v, causal=True)
    a = fa.backward(q, k, v, o, lse, do, causal=True)
    b = fa.backward(q, k, v, o, lse, do, causal=True)
    qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
    out = fa.attention(qa, ka, va, causal=True)
    out.backward(do)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    assert torch.equal(out.detach(), o)
    assert torch.equal(qa.grad, a[0]) and torch.equal(ka.grad, a[1]) and torch.equal(va.grad, a[2])


def test_zero_upstream_gradient(fa):
    q, k, v = (t.cuda() for t in fin.make_qkv(1, 2, 2, 100, 128, "f16", 61))
    o, lse = fa.forward(q, k, v)
    dq, dk, dv, delta = fa.backward(q, k, v, o, lse, torch.zeros_like(q))
    torch.cuda.synchronize()
    assert all(torch.all(t == 0) for t in (dq, dk, dv, delta))


def test_rejects_f32_and_bad_shapes(fa):
    q, k, v = (t.cuda() for t in fin.make_qkv(1, 1, 1, 8, 64, "f32", 1))
    o, lse = fa.forward(q, k, v)
    with pytest.raises(NotImplementedError):
        fa.backward(q, k, v, o, lse, q.clone())
    qb, kb, vb = (t.to(torch.bfloat16) for t in (q, k, v))
    with pytest.raises(ValueError):
        fa.backward(qb, kb, vb, o.to(torch.bfloat16), lse[..., :4].contiguous(), qb.clone())


@pytest.mark.parametrize("name", sorted(fin.BWD_WORKLOADS))
def test_measured_workloads_at_full_size(fa, oracle, name):
    """The benchmarked launch at full size; the oracle on the first and the last K/V head
    (each with every query head that reads it), which are independent of the others."""
    w = fin.BWD_WORKLOADS[name]
    q, k, v, do = fin.bwd_workload_inputs(w)
    print("full-size backward", name, flush=True)
    dq, dk, dv, delta = run_gpu(fa, q, k, v, do, w.causal, w.softmax_scale)
    G = w.Hq // w.Hkv
    picks = [(0, 0), (w.B - 1, w.Hkv - 1)]
    for b, hk in picks:
        hs = slice(hk * G, (hk + 1) * G)
        sq, sk, sv, sdo = q[b:b + 1, hs], k[b:b + 1, hk:hk + 1], v[b:b + 1, hk:hk + 1], do[b:b + 1, hs]
        rq, rk, rv, rd = oracle.attention_backward(sq, sk, sv, sdo, causal=w.causal, scale=w.softmax_scale)
        mq, mk, mv, md = magnitudes(sq, sk, sv, sdo, w.causal, w.softmax_scale)
        what = "%s b%d hkv%d" % (name, b, hk)
        check(dq[b:b + 1, hs].double().numpy(), rq, mq, w.dtype, what + " dq")
        check(dk[b:b + 1, hk:hk + 1].double().numpy(), rk, mk, w.dtype, what + " dk")
        check(dv[b:b + 1, hk:hk + 1].double().numpy(), rv, mv, w.dtype, what + " dv")
        assert np.all(np.abs(delta[b:b + 1, hs].double().numpy() - rd) <= 2 * UNIT[w.dtype] * md + 1e-6), \
            what + " delta"
    for t in (dq, dk, dv, delta):
        assert torch.all(torch.isfinite(t.float())).item()


@pytest.mark.parametrize("B,Hq,Hkv,splits", [(1, 8, 8, 1), (3, 8, 8, 2), (3, 24, 8, 3), (1, 16, 16, 1)])
def test_every_gradient_under_each_block_order(fa, oracle, B, Hq, Hkv, splits):
    """B*Hq and B*Hkv with one, an odd and an even number of heads per XCD, with and without
    split dK/dV: every dq, dk and dv row is compared."""
    q, k, v = fin.make_qkv(B, Hq, Hkv, 260, 64, "bf16", 500 + B + Hq)
    do = fin.make_dout(B, Hq, 260, 64, "bf16", 501 + B + Hq)
    compare(fa, oracle, q, k, v, do, True, 0.125, "bf16", "order B%d Hq%d Hkv%d" % (B, Hq, Hkv), splits)


def _random_cases(count, seed):
    """Seeded random shapes within a size budget (B*Hq*N^2 <= 6e6), both dtypes and masks."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        B = int(rng.integers(1, 4))
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 4, 8]))
        N = int(rng.integers(1, 1200))
        if B * Hkv * G * N * N > 6e6:
            continue
        out.append((B, G * Hkv, Hkv, N, int(rng.choice([64, 128])), str(rng.choice(["bf16", "f16"])),
                    bool(rng.integers(0, 2)), int(rng.integers(1, 9))))
    return out


@pytest.mark.parametrize("case", _random_cases(24, 2024))
def test_random_shapes(fa, oracle, case):
    """Forward output, LSE and all three gradients on seeded random shapes, split counts and masks."""
    B, Hq, Hkv, N, d, dtype, causal, splits = case
    seed = (B * 131 + Hq * 17 + N * 7 + d) % 100000
    q, k, v = fin.make_qkv(B, Hq, Hkv, N, d, dtype, seed)
    do = fin.make_dout(B, Hq, N, d, dtype, seed + 1)
    compare(fa, oracle, q, k, v, do, causal, 1.0 / np.sqrt(d), dtype, "random %s" % (case,), splits)
