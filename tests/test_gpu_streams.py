"""The library keeps no state between calls: calls on different streams and from different
host threads give the same bits as serial calls, and each host thread sees its own error
message.  All streams keep the default priority."""
import threading

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


def problems():
    """Two different problems (shapes, masks, dtypes), seeded."""
    a = fin.make_qkv(1, 4, 2, 1000, 128, "bf16", seed=811)
    b = fin.make_qkv(2, 8, 8, 777, 64, "f16", seed=812)
    return [(tuple(t.cuda() for t in a), True), (tuple(t.cuda() for t in b), False)]


def serial(fa, probs):
    out = []
    for (q, k, v), causal in probs:
        o, lse = fa.forward(q, k, v, causal=causal)
        torch.cuda.synchronize()
        out.append((o.clone(), lse.clone()))
    return out


def test_interleaved_calls_on_two_streams_match_serial_calls(fa):
    probs = problems()
    ref = serial(fa, probs)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[None, None] for _ in probs]
    for _ in range(3):                       # several rounds, launches interleaved across streams
        for i, ((q, k, v), causal) in enumerate(probs):
            with torch.cuda.stream(streams[i]):
                outs[i] = list(fa.forward(q, k, v, causal=causal))
    torch.cuda.synchronize()
    for (o, lse), (ro, rl) in zip(outs, ref):
        assert torch.equal(o, ro)
        assert torch.equal(lse, rl)


def test_calls_from_two_host_threads_match_serial_calls(fa):
    probs = problems()
    ref = serial(fa, probs)
    results = [None, None]
    errors = []

    def work(i):
        try:
            (q, k, v), causal = probs[i]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(4):
                    o, lse = fa.forward(q, k, v, causal=causal)
            s.synchronize()
            results[i] = (o, lse)
        except Exception as e:               # reported below, on the test's own thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not errors, errors
    for (o, lse), (ro, rl) in zip(results, ref):
        assert torch.equal(o, ro)
        assert torch.equal(lse, rl)


def test_error_messages_are_per_thread(fa):
    """A refused call on one thread leaves its message there; a good call elsewhere clears its own."""
    (q, k, v), _ = problems()[0]
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    seen = {}
    bad_done = threading.Event()

    def bad():
        rc = fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                       B, Hq, Hkv, N, d, 3, 0.125, fa.FA_DTYPE_BF16, None)   # causal = 3: refused
        seen["bad"] = (rc, fa.fa_last_error())
        bad_done.set()

    def good():
        bad_done.wait(timeout=30)
        rc = fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                       B, Hq, Hkv, N, d, 1, 0.125, fa.FA_DTYPE_BF16, None)
        torch.cuda.synchronize()
        seen["good"] = (rc, fa.fa_last_error())

    threads = [threading.Thread(target=bad), threading.Thread(target=good)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert seen["bad"][0] == fa.FA_ERR_INVALID_ARG and "causal" in seen["bad"][1]
    assert seen["good"] == (fa.FA_OK, "")


@pytest.mark.parametrize("bad", [dict(causal=2), dict(Hkv=3), dict(d=96), dict(scale=float("inf")), dict(dtype=7)])
def test_refused_calls_leave_the_outputs_untouched(fa, bad):
    (q, k, v), _ = problems()[0]
    o = torch.full_like(q, 7.0)
    lse = torch.full(q.shape[:3], -3.0, dtype=torch.float32, device=q.device)
    B, Hq, N, d = q.shape
    args = dict(B=B, Hq=Hq, Hkv=k.shape[1], N=N, d=d, causal=1, scale=0.125, dtype=fa.FA_DTYPE_BF16)
    args.update(bad)
    rc = fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), args["B"], args["Hq"],
                   args["Hkv"], args["N"], args["d"], args["causal"], args["scale"], args["dtype"], None)
    torch.cuda.synchronize()
    assert rc in (fa.FA_ERR_INVALID_ARG, fa.FA_ERR_UNSUPPORTED)
    assert fa.fa_last_error() != ""
    assert bool((o == 7.0).all()) and bool((lse == -3.0).all())
