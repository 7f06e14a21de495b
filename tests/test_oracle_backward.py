"""Pins for the backward oracle (oracle/backward_oracle.py).

The pages give no backward numbers, so the gradients are pinned against two
independent routes and against identities the mathematics fixes:
- torch autograd through a float64 attention written with torch ops;
- central finite differences of the forward oracle (the C three-pass oracle),
  entry by entry, on tiny shapes;
- sum over keys of dK is 0 (every row of dS sums to 0, a softmax identity);
  delta = rowsum(dO * O) = rowsum(P * dP); dO = 0 gives zero gradients;
  GQA gradients equal those of the repeated-K/V problem summed over each group.
"""
import numpy as np
import pytest
import torch

from oracle import backward_oracle, fa_oracle


def _inputs(B, Hq, Hkv, N, d, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    do = rng.standard_normal((B, Hq, N, d))
    return q, k, v, do


def _autograd(q, k, v, do, causal, scale, G):
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    kk = torch.repeat_interleave(tk, G, dim=1)
    vv = torch.repeat_interleave(tv, G, dim=1)
    s = torch.matmul(tq, kk.transpose(-1, -2).contiguous()) * scale
    if causal:
        N = q.shape[2]
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), vv)
    o.backward(torch.from_numpy(do))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy(), o.detach().numpy()


@pytest.mark.parametrize("case", [(1, 2, 1, 17, 8, True), (2, 4, 2, 23, 5, False), (1, 4, 1, 40, 16, True),
                                  (1, 1, 1, 1, 4, True)])
def test_matches_autograd(case):
    B, Hq, Hkv, N, d, causal = case
    q, k, v, do = _inputs(B, Hq, Hkv, N, d, N * 10 + d)
    dq, dk, dv, delta = backward_oracle.attention_backward(q, k, v, do, causal=causal, scale=0.4)
    gq, gk, gv, o = _autograd(q, k, v, do, causal, 0.4, Hq // Hkv)
    assert np.allclose(dq, gq, rtol=1e-11, atol=1e-12)
    assert np.allclose(dk, gk, rtol=1e-11, atol=1e-12)
    assert np.allclose(dv, gv, rtol=1e-11, atol=1e-12)
    assert np.allclose(delta, (do * o).sum(-1), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_matches_finite_differences_of_the_forward_oracle(causal):
    B, Hq, Hkv, N, d = 1, 2, 1, 5, 3
    q, k, v, do = _inputs(B, Hq, Hkv, N, d, 7 + causal)
    scale = 0.8
    dq, dk, dv, _ = backward_oracle.attention_backward(q, k, v, do, causal=causal, scale=scale)

    def loss(qq, kk, vv):
        o, _ = fa_oracle.attention(qq, kk, vv, causal=causal, scale=scale)
        return float((o * do).sum())

    h = 1e-6
    rng = np.random.default_rng(11)
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(8):
            idx = tuple(int(rng.integers(0, n)) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            fd = (loss(args_p["q"], args_p["k"], args_p["v"]) - loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
            assert abs(fd - g[idx]) <= 1e-7 * max(1.0, abs(g[idx])), (name, idx, fd, g[idx])


@pytest.mark.parametrize("causal", [False, True])
def test_identities(causal):
    q, k, v, do = _inputs(2, 4, 2, 31, 8, 3)
    dq, dk, dv, delta = backward_oracle.attention_backward(q, k, v, do, causal=causal, scale=0.3)
    # each row of dS sums to zero, so dK summed over the keys vanishes
    assert np.allclose(dk.sum(axis=2), 0.0, atol=1e-11)
    # zero upstream gradient: zero gradients, zero delta
    z = backward_oracle.attention_backward(q, k, v, np.zeros_like(do), causal=causal, scale=0.3)
    assert all(np.all(t == 0.0) for t in z)
    # GQA: the grouped problem equals the repeated-K/V one, summed over each group
    rq, rk, rv, rd = backward_oracle.attention_backward(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1), do,
                                                        causal=causal, scale=0.3)
    assert np.allclose(dq, rq, rtol=1e-13, atol=1e-13) and np.allclose(delta, rd, rtol=1e-13, atol=1e-13)
    assert np.allclose(dk, rk.reshape(2, 2, 2, 31, 8).sum(2), rtol=1e-12, atol=1e-12)
    assert np.allclose(dv, rv.reshape(2, 2, 2, 31, 8).sum(2), rtol=1e-12, atol=1e-12)


def test_single_key_closed_form():
    """N = 1: P = 1, O = v, so dv = sum of dO over the group's heads and dq = dk = 0."""
    q, k, v, do = _inputs(1, 2, 1, 1, 6, 5)
    dq, dk, dv, delta = backward_oracle.attention_backward(q, k, v, do, causal=True, scale=0.5)
    assert np.allclose(dv[0, 0], do[0].sum(0), atol=1e-15)
    assert np.all(np.abs(dq) < 1e-15) and np.all(np.abs(dk) < 1e-15)
    assert np.allclose(delta[0, :, 0], (do[0, :, 0] * v[0, 0, 0]).sum(-1), atol=1e-15)


# Plausible mistakes planted in a copy of the backward oracle's source; each must fail a pin.
MUTANTS = {
    "no_delta": ("ds = p * (dp - dd[:, None])", "ds = p * dp"),
    "delta_sign": ("ds = p * (dp - dd[:, None])", "ds = p * (dp + dd[:, None])"),
    "ds_without_p": ("ds = p * (dp - dd[:, None])", "ds = (dp - dd[:, None])"),
    "dq_unscaled": ("dq[b, h] = scale * (ds @ kh)", "dq[b, h] = ds @ kh"),
    "dk_transposed_ds": ("dk[b, hk] += scale * (ds.T @ q[b, h])", "dk[b, hk] += scale * (ds @ q[b, h])"),
    "dv_not_transposed": ("dv[b, hk] += p.T @ do[b, h]", "dv[b, hk] += p @ do[b, h]"),
    "gqa_overwrite": ("dv[b, hk] += p.T @ do[b, h]", "dv[b, hk] = p.T @ do[b, h]"),
    "dp_wrong_operand": ("dp = do[b, h] @ vh.T", "dp = do[b, h] @ kh.T"),
    "mask_ignored": ("s[masked] = -np.inf", "pass"),
    "delta_from_v": ("dd = (do[b, h] * o).sum(axis=1)", "dd = (do[b, h] * vh).sum(axis=1)"),
}


def _mutant(name):
    import importlib.util
    import inspect
    src = inspect.getsource(backward_oracle)
    old, new = MUTANTS[name]
    assert src.count(old) == 1, name
    spec = importlib.util.spec_from_loader("backward_oracle_" + name, loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(src.replace(old, new), "backward_oracle_" + name, "exec"), mod.__dict__)
    return mod


def _pins_pass(mod):
    """The pins above, as booleans: autograd on causal GQA and full shapes, and the identities."""
    for case in [(1, 4, 2, 19, 8, True), (2, 2, 1, 13, 5, False)]:
        B, Hq, Hkv, N, d, causal = case
        q, k, v, do = _inputs(B, Hq, Hkv, N, d, 40 + N)
        try:
            dq, dk, dv, delta = mod.attention_backward(q, k, v, do, causal=causal, scale=0.4)
        except Exception:
            return False
        gq, gk, gv, o = _autograd(q, k, v, do, causal, 0.4, Hq // Hkv)
        if not (np.allclose(dq, gq, rtol=1e-9, atol=1e-10) and np.allclose(dk, gk, rtol=1e-9, atol=1e-10)
                and np.allclose(dv, gv, rtol=1e-9, atol=1e-10)
                and np.allclose(delta, (do * o).sum(-1), rtol=1e-10, atol=1e-10)):
            return False
    return True


def test_the_pins_pass_the_oracle_itself():
    assert _pins_pass(backward_oracle)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_every_planted_mistake_fails_a_pin(name):
    assert not _pins_pass(_mutant(name)), name
