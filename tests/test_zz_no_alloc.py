"""The allocation-free split backward (fa_bwd_split_noalloc) against fa_bwd_split.

fa_bwd_split_noalloc runs the same kernels as fa_bwd_split with the dK/dV partials in
the library's static workspace instead of a caller-provided one, so every output must
be bitwise fa_bwd_split's for the same arguments (which the backward parity tests hold
to the fp64 oracle).  Two calls in a row, the second smaller, show that the workspace
keeps no state a call depends on.
"""
import math

import pytest
import torch

from flashattention_online_softmax_fwd_amd import _lib
from flashattention_online_softmax_fwd_amd import inputs as fin

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    import flashattention_online_softmax_fwd_amd as fa_mod
    fa_mod.load_library()
    return fa_mod


def run_pair(fa, B, Hq, Hkv, N, d, causal, dtype, splits, seed):
    q, k, v = (t.cuda() for t in fin.make_qkv(B, Hq, Hkv, N, d, dtype, seed))
    do = fin.make_dout(B, Hq, N, d, dtype, seed + 1).cuda()
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale)
    code = {"bf16": _lib.FA_DTYPE_BF16, "f16": _lib.FA_DTYPE_F16}[dtype]
    stream = torch.cuda.current_stream().cuda_stream
    outs = []
    for noalloc in (False, True):
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        delta = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
        args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr())
        sizes = (B, Hq, Hkv, N, d, int(causal), scale, code, stream)
        if noalloc:
            rc = _lib.fa_bwd_split_noalloc(*args, splits, *sizes)
        else:
            part = torch.empty((2, splits) + tuple(k.shape), dtype=torch.float32, device=q.device)
            rc = _lib.fa_bwd_split(*args, part.data_ptr(), splits, *sizes)
        assert rc == 0, _lib.fa_last_error()
        torch.cuda.synchronize()
        outs.append((dq, dk, dv, delta))
    for name, a, b in zip(("dq", "dk", "dv", "delta"), *outs):
        assert torch.isfinite(a.float()).all(), name
        assert torch.equal(a, b), "%s differs between fa_bwd_split and fa_bwd_split_noalloc" % name


def test_noalloc_backward_matches_the_workspace_entry_point_twice(fa):
    # the first call fills most of the static workspace: 2 * 4 * 2 * 4 * 1024 * 128 * 4 = 32 MiB
    run_pair(fa, 2, 8, 4, 1024, 128, True, "bf16", 4, seed=21)
    # the second, smaller call reads only what it wrote itself
    run_pair(fa, 1, 4, 2, 333, 64, False, "f16", 3, seed=22)
    # one split takes no workspace at all
    run_pair(fa, 1, 2, 1, 200, 128, True, "bf16", 1, seed=23)


def test_noalloc_refuses_what_its_workspace_cannot_hold(fa):
    B, Hq, Hkv, N, d = 1, 8, 8, 4096, 128            # 8 splits: 2*8*8*4096*128*4 = 256 MiB
    assert 2 * 8 * B * Hkv * N * d * 4 > _lib.fa_bwd_noalloc_max_bytes()
    q = torch.zeros((B, Hq, N, d), dtype=torch.bfloat16, device="cuda")
    t = [torch.zeros_like(q) for _ in range(7)]
    lse = torch.zeros((B, Hq, N), dtype=torch.float32, device="cuda")
    delta = torch.zeros_like(lse)
    rc = _lib.fa_bwd_split_noalloc(q.data_ptr(), t[0].data_ptr(), t[1].data_ptr(), t[2].data_ptr(), lse.data_ptr(),
                                   t[3].data_ptr(), t[4].data_ptr(), t[5].data_ptr(), t[6].data_ptr(),
                                   delta.data_ptr(), 8, B, Hq, Hkv, N, d, 1, 0.1, _lib.FA_DTYPE_BF16,
                                   torch.cuda.current_stream().cuda_stream)
    assert rc == _lib.FA_ERR_UNSUPPORTED and "static workspace" in _lib.fa_last_error()
