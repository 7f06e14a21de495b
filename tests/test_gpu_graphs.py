"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

A caller that runs the same shapes over and over can capture the calls once and replay them:
every entry point only enqueues kernels on the stream it is given (no allocation, no memset, no
host synchronisation), so the graph holds the launches alone.  Each test warms the call up on a
side stream, captures it, then replays it several times; between replays it copies new values
into the captured inputs, runs the same call eagerly and synchronises the device, and every
replay must equal the eager result bit for bit (the kernels are deterministic).
"""
import math

import pytest
import torch

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    import flashattention_online_softmax_fwd_amd as fa_mod
    fa_mod.load_library()
    return fa_mod


def fill(tensors, seed):
    """New standard normal values (times 3) in place, drawn on the device."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    for t in tensors:
        t.copy_(torch.randn(t.shape, generator=g, device=t.device, dtype=torch.float32) * 3.0)


def replays_match_eager(fn, inputs, seed):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = fn()
    for i in range(REPLAYS):
        fill(inputs, seed + i)
        eager = [t.clone() for t in fn()]
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n, (a, b) in enumerate(zip(captured, eager)):
            assert torch.equal(a, b), "replay %d, output %d differs from the eager call" % (i, n)
    return captured


@pytest.mark.parametrize("B,Hq,Hkv,N,d,dtype,causal", [
    (2, 16, 16, 2048, 128, torch.bfloat16, True),    # 1024 waves of 64 rows: the walked 64-row kernel
    (1, 4, 2, 300, 64, torch.float16, False),        # a small grid: the 32-rows-per-wave kernel
    (1, 2, 1, 200, 64, torch.float32, True),         # fp32
])
def test_forward(fa, B, Hq, Hkv, N, d, dtype, causal):
    print("graph forward", B, Hq, Hkv, N, d, dtype, causal, flush=True)
    q = torch.empty((B, Hq, N, d), dtype=dtype, device="cuda")
    k = torch.empty((B, Hkv, N, d), dtype=dtype, device="cuda")
    v = torch.empty_like(k)
    fill((q, k, v), 1600)
    replays_match_eager(lambda: fa.forward(q, k, v, causal=causal), (q, k, v), 1610)


def test_split_kv_and_merge(fa):
    """A decode step: one query row per head against 5000 cached keys, split and merged."""
    q = torch.empty((2, 8, 1, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((2, 2, 5000, 128), dtype=torch.bfloat16, device="cuda")
    v = torch.empty_like(k)
    fill((q, k, v), 1620)
    replays_match_eager(lambda: fa.attention_kv(q, k, v, causal=True, num_splits=6), (q, k, v), 1630)


@pytest.mark.parametrize("algo", ["online", "safe"])
def test_softmax(fa, algo):
    x = torch.empty((100, 3000), dtype=torch.float32, device="cuda")
    fill((x,), 1640)
    replays_match_eager(lambda: fa.softmax(x, algo=algo), (x,), 1650)


def test_backward_with_split_dkdv(fa):
    """The forward and the backward (dK/dV shared over three workgroups per key tile through the
    fp32 workspace, which the capture allocates from the graph's memory pool) in one graph."""
    B, Hq, Hkv, N, d = 1, 8, 2, 1000, 64
    q = torch.empty((B, Hq, N, d), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((B, Hkv, N, d), dtype=torch.bfloat16, device="cuda")
    v = torch.empty_like(k)
    do = torch.empty_like(q)
    fill((q, k, v, do), 1660)
    scale = 1.0 / math.sqrt(d)

    def step():
        o, lse = fa.forward(q, k, v, causal=True, scale=scale)
        dq, dk, dv, _ = fa.backward(q, k, v, o, lse, do, causal=True, scale=scale, num_splits=3)
        return o, lse, dq, dk, dv

    replays_match_eager(step, (q, k, v, do), 1670)
