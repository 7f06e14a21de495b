"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on the GPU.

Inputs come from the seeded generators in flashattention_online_softmax_fwd_amd.inputs;
the oracle reads the very tensors the GPU reads, upcast exactly to float64.

Tolerance (the method's bar, read elementwise in allclose form because values
near zero make a pure relative bound meaningless and rounding O to bf16 alone
can cost up to 1/64 where |O| is in [4, 8)):
    bf16 inputs:  |x - r| <= 1e-2 + 2e-2 * |r|       on O and on LSE
    fp16 inputs:  |x - r| <= 1.25e-3 + 2.5e-3 * |r|  (the bf16 bar times 2^-3, the
                  ratio of the two formats' unit roundoffs)
    fp32 inputs:  |x - r| <= 1e-5 + 2^-22 * |r|      on O and on LSE (the relative term is
                  two float32 roundings: 1e-5 alone is finer than float32's spacing
                  for |x| >= 128)
Every O and LSE value must also be finite.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from flashattention_online_softmax_fwd_amd import inputs as fin

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


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


def tol(dtype):
    """bf16: the method's bar; fp16: that bar scaled by 2^-3, the ratio of fp16's unit
    roundoff (2^-11) to bf16's (2^-8); fp32: 1e-5."""
    from oracle import tolerances
    return tolerances.forward_bar(dtype)


def check(x, r, dtype, what):
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    assert x.shape == r.shape, (what, x.shape, r.shape)
    assert np.all(np.isfinite(x)), "%s: non-finite values" % what
    atol, rtol = tol(dtype)
    err = np.abs(x - r)
    bad = err > atol + rtol * np.abs(r)
    if bad.any():
        i = np.unravel_index(np.argmax(err - (atol + rtol * np.abs(r))), err.shape)
        raise AssertionError("%s: %d of %d outside tolerance; worst at %s: got %r want %r (max abs err %.3e)"
                             % (what, int(bad.sum()), bad.size, i, x[i], r[i], err.max()))
    return float(err.max())


def run_gpu(fa, q, k, v, causal, scale, tile=None):
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    if tile is None:
        o, lse = fa.forward(qd, kd, vd, causal=causal, scale=scale)
    else:
        o, lse = fa.forward(qd, kd, vd, causal=causal, scale=scale, block_m=tile[0], block_n=tile[1])
    torch.cuda.synchronize()
    return o.float().cpu(), lse.cpu()


def parity(fa, oracle, B, Hq, Hkv, N, d, dtype, causal, seed, scale=None, q_mult=1.0, tile=None, rows=None):
    q, k, v = fin.make_qkv(B, Hq, Hkv, N, d, dtype, seed, q_mult)
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    o, lse = run_gpu(fa, q, k, v, causal, sc, tile)
    tag = "B%d Hq%d Hkv%d N%d d%d %s causal=%d seed=%d tile=%s" % (B, Hq, Hkv, N, d, dtype, causal, seed, tile)
    if rows is None:
        ro, rl = oracle.attention(q, k, v, causal=causal, scale=sc)
        e1 = check(o.numpy(), ro, dtype, "O " + tag)
        e2 = check(lse.numpy(), rl, dtype, "LSE " + tag)
    else:
        ro, rl = oracle.attention(q, k, v, causal=causal, scale=sc, rows=rows)
        assert np.all(np.isfinite(o.numpy())) and np.all(np.isfinite(lse.numpy())), tag
        e1 = check(o.reshape(-1, d).numpy()[rows], ro, dtype, "O " + tag)
        e2 = check(lse.reshape(-1).numpy()[rows], rl, dtype, "LSE " + tag)
    return e1, e2


# ------------------------------------------------------------ worked examples

def embed(scores, values, d, dtype, value_scale):
    """q_i = e0, k_j = x_j e0, v_j = (val_j * value_scale) e0; with scale 1 every
    query sees exactly the page's scores."""
    n = len(scores)
    q = torch.zeros(1, 1, n, d)
    q[..., 0] = 1.0
    k = torch.zeros(1, 1, n, d)
    k[0, 0, :, 0] = torch.tensor(scores, dtype=torch.float64).float()
    v = torch.zeros(1, 1, n, d)
    v[0, 0, :, 0] = torch.tensor(values, dtype=torch.float64).float() * value_scale
    td = fin.torch_dtype(dtype)
    return q.to(td), k.to(td), v.to(td)


def page_bar(dtype, want, printed_places):
    """The method's bar on an embedded value, widened by the page's rounding."""
    atol, rtol = tol(dtype)
    return atol + rtol * abs(want) + 0.5 * 10.0 ** (-printed_places) / 64


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
def test_p1_worked_example(fa, dtype, d):
    g = golden("p1_four_scores.json")
    q, k, v = embed(g["scores"], g["values"], d, dtype, 1 / 64)
    o, lse = run_gpu(fa, q, k, v, False, 1.0)
    want = g["all_at_once"]["output_code_printed"] / 64
    assert np.all(np.abs(o[0, 0, :, 0].numpy() - want) <= page_bar(dtype, want, 8))
    assert np.all(o[0, 0, :, 1:].numpy() == 0.0)
    l = np.exp(lse[0, 0].numpy().astype(np.float64) - 5.0)
    assert np.allclose(l, g["all_at_once"]["weights_sum"], atol=5e-5 if dtype == "f32" else 1e-3)
    # causal: row 1 is the first block alone, row 0 sees key 0 only
    o, lse = run_gpu(fa, q, k, v, True, 1.0)
    b1 = g["two_blocks"]["after_block_1"]["output_2_places"] / 64
    assert abs(o[0, 0, 1, 0].item() - b1) <= page_bar(dtype, b1, 2)
    assert abs(o[0, 0, 0, 0].item() - 10.0 / 64) <= page_bar(dtype, 10.0 / 64, 8)


def test_p2_not_the_block_mean(fa):
    g = golden("p2_not_block_mean.json")
    x = [0.0, 0.0, math.log(3.0), math.log(3.0)]
    q, k, v = embed(x, g["values"], 64, "f32", 1.0)
    o, _ = run_gpu(fa, q, k, v, False, 1.0)
    assert np.allclose(o[0, 0, :, 0].numpy(), g["output"], atol=1e-5)
    assert abs(o[0, 0, 0, 0].item() - g["wrong_block_mean"]) > 0.2


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_p4_tables_as_causal_prefixes(fa, dtype):
    g = golden("p4_worked_example.json")
    q, k, v = embed(g["scores"], g["values"], 64, dtype, 1 / 64)
    o, lse = run_gpu(fa, q, k, v, True, 1.0)
    out = o[0, 0, :, 0].numpy()
    for got, page in zip(out, g["values_table_by_hand"]["output_2_places"]):
        assert abs(got - page / 64) <= page_bar(dtype, page / 64, 2)
    l = np.exp(lse[0, 0].numpy().astype(np.float64) - np.maximum.accumulate(g["scores"]))
    assert np.allclose(l, g["table1_by_hand"]["l"], atol=5e-5 if dtype == "f32" else 1e-3)
    # shares through one-hot values
    q, k, _ = embed(g["scores"], g["values"], 64, dtype, 1.0)
    v = torch.zeros(1, 1, 5, 64)
    v[0, 0, :, :5] = torch.eye(5)
    o, _ = run_gpu(fa, q, k, v.to(fin.torch_dtype(dtype)), False, 1.0)
    w = o[0, 0, 0, :5].numpy()
    for got, page in zip(w, g["probabilities_4_places"]):
        atol, rtol = tol(dtype)
        assert abs(got - page) <= atol + rtol * page + 5e-5
    assert round(100 * w[3]) == g["share_of_top_score_percent"]


# ------------------------------------------------------------- brute force grid

TINY_N = [1, 2, 3, 5, 17, 63, 64, 65, 127, 128, 129, 255, 257]
# every (Hq, Hkv) with Hq, Hkv in {1, 2, 4, 8} and Hkv dividing Hq
TINY_HEADS = [(hq, hkv) for hq in (1, 2, 4, 8) for hkv in (1, 2, 4, 8) if hq % hkv == 0]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", TINY_N)
def test_tiny_shapes(fa, oracle, N, d, causal, dtype):
    """The brute-force grid: every tiny N against every head layout."""
    for Hq, Hkv in TINY_HEADS:
        parity(fa, oracle, 1, Hq, Hkv, N, d, dtype, causal, seed=N * 10 + d + Hq * 1000 + Hkv * 100)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (2, 2), (4, 2), (8, 1), (8, 8)])
def test_head_layouts(fa, oracle, Hq, Hkv, dtype):
    parity(fa, oracle, 2, Hq, Hkv, 193, 128, dtype, True, seed=Hq * 10 + Hkv)
    parity(fa, oracle, 2, Hq, Hkv, 150, 64, dtype, False, seed=Hq * 10 + Hkv + 1)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f16", 128), ("f16", 64), ("f32", 128),
                                     ("f32", 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_every_tile_shape(fa, oracle, dtype, d, causal):
    code = {"bf16": fa.FA_DTYPE_BF16, "f16": fa.FA_DTYPE_F16, "f32": fa.FA_DTYPE_F32}[dtype]
    shapes = fa.fa_tile_shapes(code, d)
    assert len(shapes) >= 2
    for tile in shapes:
        parity(fa, oracle, 1, 4, 2, 419, d, dtype, causal, seed=7, tile=tile)
        # many key tiles per query tile: every tile barrier must see the whole tile
        parity(fa, oracle, 1, 2, 1, 1531, d, dtype, causal, seed=8, tile=tile)


# ------------------------------------------------------------- closed forms

@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_constant_values(fa, dtype, causal):
    q, k, v = fin.make_qkv(1, 4, 4, 300, 128, dtype, 3, q_mult=12.0)
    v = torch.full_like(v, 0.625)
    o, lse = run_gpu(fa, q, k, v, causal, 1 / math.sqrt(128))
    check(o.numpy(), np.full(o.shape, 0.625), dtype, "O constant values")
    assert torch.all(torch.isfinite(lse))


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_average_the_visible_values(fa, dtype, causal):
    q, k, v = fin.make_qkv(1, 2, 2, 200, 64, dtype, 4)
    q = torch.zeros_like(q)
    o, lse = run_gpu(fa, q, k, v, causal, 0.125)
    vv = v.double()
    if causal:
        cnt = torch.arange(1, 201, dtype=torch.float64)
        want = vv.cumsum(2) / cnt[None, None, :, None]
    else:
        cnt = torch.full((200,), 200.0, dtype=torch.float64)
        want = vv.mean(2, keepdim=True).expand_as(vv)
    check(o.numpy(), want.numpy(), dtype, "O zero queries")
    check(lse.numpy(), np.broadcast_to(np.log(cnt.numpy()), (1, 2, 200)), dtype, "LSE zero queries")


def test_single_key_gives_its_value(fa):
    for dtype in ("f32", "bf16", "f16"):
        q, k, v = fin.make_qkv(2, 2, 1, 1, 128, dtype, 5)
        o, lse = run_gpu(fa, q, k, v, True, 0.3)
        assert torch.equal(o, v.float().repeat_interleave(2, dim=1))
        s = 0.3 * (q.double() * k.double().repeat_interleave(2, dim=1)).sum(-1)
        assert np.allclose(lse.numpy(), s.numpy(), atol=1e-5 + 1e-6 * float(s.abs().max()))


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale", [-0.3, -1.0 / math.sqrt(128), 0.0])
def test_nonpositive_scales(fa, oracle, dtype, causal, scale):
    """A negative scale flips every score (the kernel folds the sign into Q); a zero scale
    gives every visible key the same weight (O = the mean of the visible values,
    LSE = ln of their count)."""
    e = parity(fa, oracle, 2, 4, 2, 321, 128, dtype, causal, seed=11, scale=scale)
    assert max(e) < 1.0
    parity(fa, oracle, 1, 2, 2, 200, 64, dtype, causal, seed=12, scale=scale)


@pytest.mark.parametrize("dtype,scale,k_unit", [
    ("f32", 1e5, 1.0), ("bf16", 1e5, 1.0), ("f16", 1e5, 1.0),
    ("f32", -1e5, 1.0), ("bf16", -1e5, 1.0), ("f16", -1e5, 1.0),
    ("f32", 1e30, 2.0 ** -80), ("bf16", 1e30, 2.0 ** -80),
    ("f32", -1e30, 2.0 ** -80), ("bf16", -1e30, 2.0 ** -80),
])
@pytest.mark.parametrize("causal", [False, True])
def test_huge_scales_pick_the_best_keys(fa, oracle, dtype, scale, k_unit, causal):
    """|scale| up to 1e30, within the ABI's limit (scale * log2(e) finite in float32), with
    the scaled scores inside the documented range (below 2^29).  The softmax is then a hard
    maximum.  q holds integers in [-2, 2] and k those integers times a power of two, so every
    dot product is exact on both sides: the kernel and the oracle see the same maxima and the
    same ties, O is the mean of the tied keys' values and LSE = scale * max + ln(ties)."""
    g = torch.Generator().manual_seed(13)
    B, Hq, Hkv, N, d = 1, 4, 2, 300, 64
    q = torch.randint(-2, 3, (B, Hq, N, d), generator=g).float()
    k = torch.randint(-2, 3, (B, Hkv, N, d), generator=g).float() * k_unit
    v = torch.randn((B, Hkv, N, d), generator=g)
    td = fin.torch_dtype(dtype)
    q, k, v = q.to(td), k.to(td), v.to(td)
    o, lse = run_gpu(fa, q, k, v, causal, scale)
    ro, rl = oracle.attention(q, k, v, causal=causal, scale=scale)
    assert float(np.abs(rl).max()) * math.log2(math.e) < 2.0 ** 29
    tag = "scale %g %s causal=%d" % (scale, dtype, causal)
    check(o.numpy(), ro, dtype, "O " + tag)
    check(lse.numpy(), rl, dtype, "LSE " + tag)


def test_max_in_the_last_key_tile(fa, oracle):
    """Every row's largest score is in the last key tile: all earlier sums must shrink."""
    for dtype in ("f32", "bf16", "f16"):
        q, k, v = fin.make_qkv(1, 2, 2, 517, 128, dtype, 6)
        u = q[:, :, :1].float()
        q = u.expand_as(q).to(q.dtype).contiguous()            # one query vector for every row
        k = k.clone()
        k[:, :, 514:515] = (0.5 * u).to(k.dtype)                # its score ~ |u|^2 / (2 sqrt d)
        scale = 1 / math.sqrt(128)
        s = q.double()[0, 0, 0] @ k.double()[0, 0].T
        assert int(torch.argmax(s)) == 514
        o, lse = run_gpu(fa, q, k, v, False, scale)
        ro, rl = oracle.attention(q, k, v, causal=False, scale=scale)
        check(o.numpy(), ro, dtype, "O last tile max")
        check(lse.numpy(), rl, dtype, "LSE last tile max")


# climb of the scores from one block of 32 keys to the next, and the scale: each climb
# (times scale * log2 e) passes the slack the dtype's kernels leave their running reference
# (fp32: none, the reference follows every tile; fp16: 8 or 15; bf16: 8 or 48), while the
# fp32 scaled scores stay below 128, where their rounding (2^-18) is within that bar.
CLIMB = {"f32": (16.0, 0.5), "f16": (16.0, 1.0), "bf16": (40.0, 1.0)}


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_reference_moves_every_half_tile(fa, oracle, dtype, causal, d):
    """Every block of 32 keys holds each offset 0..31 once, on top of a base that climbs by
    CLIMB[dtype] from block to block: every row's maximum outruns its reference in every
    block it reads, so the kernel rescales O and l each time.  q is a unit vector, so a score
    is the first component of its key (bf16 rounds some above 256 to even values; both sides
    read the rounded inputs)."""
    B, Hq, Hkv, N = 1, 2, 2, 300
    climb, scale = CLIMB[dtype]
    g = torch.Generator().manual_seed(21)
    q = torch.zeros(B, Hq, N, d)
    q[..., 0] = 1.0
    j = torch.arange(N, dtype=torch.float32)
    k = torch.zeros(B, Hkv, N, d)
    k[..., 0] = climb * torch.div(j, 32, rounding_mode="floor") + torch.remainder(j * 7, 32)
    v = torch.randn((B, Hkv, N, d), generator=g)
    td = fin.torch_dtype(dtype)
    q, k, v = q.to(td), k.to(td), v.to(td)
    o, lse = run_gpu(fa, q, k, v, causal, scale)
    ro, rl = oracle.attention(q, k, v, causal=causal, scale=scale)
    tag = "%s causal=%d d=%d" % (dtype, causal, d)
    check(o.numpy(), ro, dtype, "O climbing scores " + tag)
    check(lse.numpy(), rl, dtype, "LSE climbing scores " + tag)


def test_gqa_equals_repeated_kv_bitwise(fa):
    q, k, v = fin.make_qkv(2, 8, 2, 333, 128, "bf16", 8)
    o1, l1 = run_gpu(fa, q, k, v, True, 0.1)
    o2, l2 = run_gpu(fa, q, k.repeat_interleave(4, dim=1), v.repeat_interleave(4, dim=1), True, 0.1)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_runs_are_bitwise_deterministic(fa):
    q, k, v = fin.make_qkv(1, 8, 8, 1024, 128, "bf16", 9)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o1, l1 = fa.forward(qd, kd, vd, causal=True)
    o2, l2 = fa.forward(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_scale_one_overflow_stress(fa, oracle):
    """Scaled scores in the hundreds: exp of them would overflow float32."""
    w = fin.WORKLOADS["c5s_bf16_n4096_d128_causal_q12_scale1"]
    q, k, v = fin.workload_inputs(w)
    o, lse = run_gpu(fa, q, k, v, w.causal, w.softmax_scale)
    ro, rl = oracle.attention(q, k, v, causal=True, scale=w.softmax_scale)      # every row
    assert np.all(np.isfinite(o.numpy())) and np.all(np.isfinite(lse.numpy()))
    assert float(rl.max()) > 89.0
    check(o.numpy(), ro, "bf16", "O scale-1 stress")
    check(lse.numpy(), rl, "bf16", "LSE scale-1 stress")


def test_longest_head_the_abi_accepts(fa, oracle):
    """The square causal forward on the longest head the ABI takes at d = 128 in bf16: (N + 128)
    d 2 bytes just below 2^31, one head, the default kernel and grid walk.  Buffer ranges and
    offsets are then the largest a launch can use; the last query tile holds 127 rows and the
    last key tile 63 keys.  Twelve rows are compared with the oracle: both ends, the middle, and
    rows of the last two query tiles (the diagonal key tile among them).  Those rows share one
    query vector u, and four keys score 16 to 17.5 against it (about N(0, 1) for the 8.4M others)
    with distinct value rows: the first key, the middle one, one in the second-to-last key tile
    and the very last, so a tile mis-addressed near the end of the head moves O far past the bar.
    One row more is refused before anything is launched.  (At d = 64 the longest head is twice as
    long and four times the work, so d = 128 stands for both.)"""
    d = 128
    n = 0x7FFFFFFF // (2 * d) - 128
    print("longest accepted head: N", n, flush=True)
    q, k, v = fin.make_qkv_device(1, 1, 1, n, n, d, "bf16", seed=1401)
    scale = 1.0 / math.sqrt(d)
    rows = np.array([0, 1, 4096, n // 2, n // 2 + 1, n - 300, n - 128, n - 127, n - 66, n - 65, n - 2, n - 1])
    u = q[0, 0, 0].clone()
    q[0, 0, torch.from_numpy(rows).to(q.device)] = u
    uf = u.float()
    spikes = [(0, 16.0), (n // 2, 16.5), (n - 65, 17.0), (n - 1, 17.5)]
    for i, (pos, target) in enumerate(spikes):
        k[0, 0, pos] = (uf * (target / (scale * float(uf @ uf)))).to(torch.bfloat16)
        row = torch.zeros(d, device=v.device)
        row[8 * i + 3] = 8.0
        v[0, 0, pos] = row.to(torch.bfloat16)
    o, lse = fa.forward(q, k, v, causal=True, scale=scale)
    torch.cuda.synchronize()
    idx = torch.from_numpy(rows).to(q.device)
    o_rows = o[0, 0, idx].float().cpu().numpy()
    lse_rows = lse[0, 0, idx].cpu().numpy()
    ro, rl = oracle.attention(q.cpu(), k.cpu(), v.cpu(), causal=True, scale=scale, rows=rows)
    for i, (pos, _) in enumerate(spikes):      # every planted key a row sees carries a visible share
        seen = rows >= pos
        assert np.all(ro[seen, 8 * i + 3] > 0.2), (i, ro[seen, 8 * i + 3])
    check(o_rows, ro, "bf16", "O at the longest head")
    check(lse_rows, rl, "bf16", "LSE at the longest head")
    rc = fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                   1, 1, 1, n + 1, d, 1, scale, fa.FA_DTYPE_BF16, None)
    assert rc == fa.FA_ERR_UNSUPPORTED and "2 GiB" in fa.fa_last_error()


def test_no_device_memory_beyond_the_outputs(fa):
    """The method never holds a row of scores (spicyshark.co lesson: its opening prices the score
    table of 32,768 tokens at 4 GiB per head, and the last check of "Proof it works" catches a
    streaming version that quietly builds every score).  A causal forward over 8 heads of 32768
    keys, whose fp32 score table would take 34 GB, with O and LSE given: after one warm-up call
    (which loads the code objects), three more calls leave torch's allocator untouched and the
    device's free memory (hipMemGetInfo) unchanged within 64 MiB."""
    n = 32768
    q, k, v = fin.make_qkv_device(1, 8, 8, n, n, 128, "bf16", seed=1701)
    o = torch.empty_like(q)
    lse = torch.empty((1, 8, n), dtype=torch.float32, device=q.device)
    fa.forward(q, k, v, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    alloc0, reserved0 = torch.cuda.memory_allocated(), torch.cuda.memory_reserved()
    for _ in range(3):
        fa.forward(q, k, v, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert torch.cuda.memory_allocated() == alloc0 and torch.cuda.memory_reserved() == reserved0
    assert abs(free0 - free1) < 64 << 20, (free0, free1)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


def test_empty_problem_enqueues_nothing(fa):
    q = torch.zeros(0, 2, 16, 64, device="cuda", dtype=torch.bfloat16)
    o, lse = fa.forward(q, q, q)
    assert o.shape == q.shape and lse.shape == (0, 2, 16)


def test_invalid_arguments_raise(fa):
    q = torch.zeros(1, 3, 16, 64, device="cuda", dtype=torch.bfloat16)
    k = torch.zeros(1, 2, 16, 64, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.forward(q, k, k)
    with pytest.raises(NotImplementedError):
        x = torch.zeros(1, 1, 16, 96, device="cuda", dtype=torch.bfloat16)
        fa.forward(x, x, x)
    with pytest.raises(ValueError):
        x = torch.zeros(1, 1, 16, 64, device="cuda", dtype=torch.float64)
        fa.forward(x, x, x)
    with pytest.raises(ValueError):
        x = torch.zeros(1, 1, 16, 64, device="cuda", dtype=torch.bfloat16)
        fa.forward(x, x, x, out=x)


# ------------------------------------------------------------ the five workloads

@pytest.mark.parametrize("name", list(fin.WORKLOADS))
def test_workload(fa, oracle, name):
    w = fin.WORKLOADS[name]
    q, k, v = fin.workload_inputs(w)
    o, lse = run_gpu(fa, q, k, v, w.causal, w.softmax_scale)
    assert np.all(np.isfinite(o.numpy())) and np.all(np.isfinite(lse.numpy()))
    if w.oracle_rows is None:      # every row of every head
        ro, rl = oracle.attention(q, k, v, causal=w.causal, scale=w.softmax_scale)
        check(o.numpy(), ro, w.dtype, "O " + name)
        check(lse.numpy(), rl, w.dtype, "LSE " + name)
    else:
        rows = fin.sample_rows(w, w.oracle_rows)
        ro, rl = oracle.attention(q, k, v, causal=w.causal, scale=w.softmax_scale, rows=rows)
        check(o.reshape(-1, w.d).numpy()[rows], ro, w.dtype, "O " + name)
        check(lse.reshape(-1).numpy()[rows], rl, w.dtype, "LSE " + name)
    if name.startswith("c5_"):
        qf, kf = q.double()[0], k.double()[0]
        raw = (qf[:, :256] @ kf[:, :256].transpose(-1, -2)).abs().max()
        assert float(raw) > 89.0          # the unscaled q.k is beyond float32 exp's range


@pytest.mark.parametrize("B,Hq,Hkv", [(1, 8, 8), (3, 8, 8), (1, 16, 4), (5, 8, 2), (2, 24, 8)])
def test_every_row_under_each_block_order(fa, oracle, B, Hq, Hkv):
    """Head counts that make the XCD block order walk one head per XCD, an odd number of
    heads per XCD (one at a time) and even numbers (in pairs): every row of every head
    must be written once, at every query tile, causal and not."""
    for causal in (True, False):
        parity(fa, oracle, B, Hq, Hkv, 384, 64, "bf16", causal, seed=B * 100 + Hq + Hkv)


@pytest.mark.parametrize("B,Hq,Hkv,N", [(256, 64, 8, 1), (128, 64, 64, 3), (97, 8, 8, 1)])
def test_many_heads_of_few_keys(fa, oracle, B, Hq, Hkv, N):
    """Thousands of (batch, head) units of one to three keys: the block order must reach every
    unit exactly once (16384, 8192 and 776 units: paired, paired and one-at-a-time XCD walks).
    With one key, O is that key's value exactly."""
    q, k, v = fin.make_qkv(B, Hq, Hkv, N, 128, "bf16", seed=B + Hq + N)
    scale = 1.0 / math.sqrt(128)
    o, lse = run_gpu(fa, q, k, v, True, scale)
    if N == 1:
        assert torch.equal(o, v.float().repeat_interleave(Hq // Hkv, dim=1))
    ro, rl = oracle.attention(q, k, v, causal=True, scale=scale)
    check(o.numpy(), ro, "bf16", "O many heads")
    check(lse.numpy(), rl, "bf16", "LSE many heads")


def walks(units, N, causal):
    """Whether the library walks pairs of 256-row query tiles for this grid: the rule of
    w64_walk_blocks (fa_fwd_w64.hip), written out here with this device's CU count."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nt = (N + 255) // 256
    if units * nt <= cus:
        return False
    rounds = -(-(units * ((nt + 1) // 2)) // cus)
    if causal:
        walk, tiles = rounds * (nt + 1), max(units * nt * (nt + 1) / 2 / cus, nt)
    else:
        walk, tiles = 2 * rounds, -(-(units * nt) // cus)
    return walk <= 1.03 * tiles


@pytest.mark.parametrize("B,Hq,Hkv,N,d,dtype,causal", [
    (2, 32, 32, 4000, 128, "bf16", True),      # last query tile 160 rows, its last key tile 32 keys
    (1, 32, 8, 4050, 128, "f16", True),        # grouped K/V, 210-row last tile
    (2, 32, 32, 3900, 64, "f16", True),
    (4, 16, 16, 2000, 64, "bf16", False),      # every item the same length, 208-row last tile
])
def test_walked_grids_with_a_ragged_last_tile(fa, oracle, B, Hq, Hkv, N, d, dtype, causal):
    """Grids large enough for the 256-row walk, where each item loads the next item's first
    tiles and Q rows during its last steps, with N not a multiple of the tile: the items
    differ in key-tile count, the last one holds rows past N.  Every row against the oracle."""
    assert walks(B * Hq, N, causal)
    parity(fa, oracle, B, Hq, Hkv, N, d, dtype, causal, seed=N + d)
