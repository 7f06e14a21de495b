"""Seeded synthetic inputs and the named workloads.

This module holds no attention arithmetic: it only draws random numbers and
rounds them to the input dtype.  The tests hand the very same tensors to the
HIP library and to the fp64 oracle, which is the only thing the two sides
share.

Recipe: ``numpy.random.default_rng(seed)`` draws Q, K and V (in that order) as
float32 standard normals of shape [B, Hq, N, d], [B, Hkv, N, d], [B, Hkv, N, d];
Q is then multiplied by ``q_mult``; bf16 workloads round to bfloat16 with
round-to-nearest-even (``torch.Tensor.to``), fp16 ones likewise.  The oracle reads the rounded
values upcast exactly to float64.  The backward's upstream gradient dO is drawn the same
way, from its own generator seeded with the workload's seed + 50000.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    dtype: str            # "f32", "bf16" or "f16"
    causal: bool
    q_mult: float = 1.0
    scale: float | None = None   # None: 1/sqrt(d)
    seed: int = 0
    oracle_rows: int | None = None   # rows the parity test samples for the oracle (None: every row)

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.d)

    @property
    def flops(self) -> float:
        """4*B*Hq*N^2*d, halved when causal (the metric's convention)."""
        f = 4.0 * self.B * self.Hq * self.N * self.N * self.d
        return f / 2 if self.causal else f

    @property
    def esize(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def algorithmic_bytes(self) -> int:
        """Q, K, V read once, O and LSE written once; no N x N term."""
        return (self.B * self.N * self.d * self.esize * (2 * self.Hq + 2 * self.Hkv)
                + 4 * self.B * self.Hq * self.N)


# The five workloads of the method's contract, plus the scale-1 overflow stress.
WORKLOADS = {
    "c1_f32_n256_d64": Workload("c1_f32_n256_d64", 1, 1, 1, 256, 64, "f32", False, seed=1001),
    "c2_bf16_n2048_d64": Workload("c2_bf16_n2048_d64", 4, 16, 16, 2048, 64, "bf16", False, seed=1002),
    "c3_bf16_n4096_d128_causal": Workload("c3_bf16_n4096_d128_causal", 2, 32, 32, 4096, 128, "bf16",
                                          True, seed=1003),
    "c4_bf16_gqa_n8192_d128_causal": Workload("c4_bf16_gqa_n8192_d128_causal", 1, 32, 8, 8192, 128,
                                              "bf16", True, seed=1004),
    "c5_bf16_n32768_d128_causal_q12": Workload("c5_bf16_n32768_d128_causal_q12", 1, 8, 8, 32768, 128,
                                               "bf16", True, q_mult=12.0, seed=1005, oracle_rows=32768),
    "c5s_bf16_n4096_d128_causal_q12_scale1": Workload("c5s_bf16_n4096_d128_causal_q12_scale1", 1, 8, 8,
                                                      4096, 128, "bf16", True, q_mult=12.0, scale=1.0,
                                                      seed=1006),
    # fp16 inputs at the shapes of the d = 64 and the bench workload
    "c2h_f16_n2048_d64": Workload("c2h_f16_n2048_d64", 4, 16, 16, 2048, 64, "f16", False, seed=1007),
    "c3h_f16_n4096_d128_causal": Workload("c3h_f16_n4096_d128_causal", 2, 32, 32, 4096, 128, "f16", True,
                                          seed=1008),
    # fp32 inputs at the bench workload's shape (the fp32 contract config is too small to time)
    "c3f_f32_n4096_d128_causal": Workload("c3f_f32_n4096_d128_causal", 2, 32, 32, 4096, 128, "f32", True,
                                          seed=1009),
}

BENCH_WORKLOAD = "c3_bf16_n4096_d128_causal"

# Backward workloads: the shapes of the bench forward (bf16 and fp16), of the GQA forward
# and of the d = 64 forward, with their own seeds (dO drawn like Q, K and V).
BWD_WORKLOADS = {
    "b1_bf16_bwd_n4096_d128_causal": Workload("b1_bf16_bwd_n4096_d128_causal", 2, 32, 32, 4096, 128, "bf16",
                                              True, seed=1301),
    "b2_bf16_bwd_gqa_n8192_d128_causal": Workload("b2_bf16_bwd_gqa_n8192_d128_causal", 1, 32, 8, 8192, 128,
                                                  "bf16", True, seed=1302),
    "b3_bf16_bwd_n2048_d64": Workload("b3_bf16_bwd_n2048_d64", 4, 16, 16, 2048, 64, "bf16", False, seed=1303),
    "b4_f16_bwd_n4096_d128_causal": Workload("b4_f16_bwd_n4096_d128_causal", 2, 32, 32, 4096, 128, "f16", True,
                                             seed=1304),
}


@dataclasses.dataclass(frozen=True)
class KVWorkload:
    """Queries that are the last Nq of Nk positions (split-KV + merge)."""
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    causal: bool
    seed: int = 0
    dtype: str = "bf16"

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def visible_pairs(self) -> int:
        """(query, key) pairs the mask keeps, per head."""
        if not self.causal:
            return self.Nq * self.Nk
        off = self.Nk - self.Nq
        return sum(i + off + 1 for i in range(self.Nq))

    @property
    def flops(self) -> float:
        """4*d flops per visible (query, key) pair."""
        return 4.0 * self.B * self.Hq * self.visible_pairs * self.d

    @property
    def algorithmic_bytes(self) -> int:
        """Q, K, V read once, O (bf16) and LSE written once."""
        return (2 * self.B * self.d * (2 * self.Hq * self.Nq + 2 * self.Hkv * self.Nk)
                + 4 * self.B * self.Hq * self.Nq)


# Decoding against a long cache (one new query, or a block of 16 draft queries), GQA 32/8.
KV_WORKLOADS = {
    "d1_bf16_decode_b8_hq32_hkv8_nk32768_d128": KVWorkload(
        "d1_bf16_decode_b8_hq32_hkv8_nk32768_d128", 8, 32, 8, 1, 32768, 128, True, seed=1101),
    "d2_bf16_nq16_b8_hq32_hkv8_nk32768_d128": KVWorkload(
        "d2_bf16_nq16_b8_hq32_hkv8_nk32768_d128", 8, 32, 8, 16, 32768, 128, True, seed=1102),
}


@dataclasses.dataclass(frozen=True)
class SoftmaxWorkload:
    """A [rows, cols] matrix of scores drawn N(0, sigma^2), softmaxed row by row."""
    name: str
    rows: int
    cols: int
    dtype: str
    seed: int = 0
    sigma: float = 4.0

    @property
    def esize(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def io_bytes(self) -> int:
        """x read once and y written once: the least any softmax must move."""
        return 2 * self.rows * self.cols * self.esize


# Scores N(0, 4^2) like the pages' random test of the online update.  Long rows (each
# pass over a row goes to HBM: 1 MiB or 256 KiB per row, far more rows in flight than
# the caches hold) and short rows (a 16 KiB row stays in L2 between its passes).
SOFTMAX_WORKLOADS = {
    "s1_f32_softmax_r1024_c262144": SoftmaxWorkload("s1_f32_softmax_r1024_c262144", 1024, 262144, "f32",
                                                    seed=1201),
    "s2_f32_softmax_r65536_c4096": SoftmaxWorkload("s2_f32_softmax_r65536_c4096", 65536, 4096, "f32",
                                                   seed=1202),
    "s3_bf16_softmax_r4096_c131072": SoftmaxWorkload("s3_bf16_softmax_r4096_c131072", 4096, 131072, "bf16",
                                                     seed=1203),
}


def make_scores(rows, cols, dtype="f32", seed=0, sigma=4.0):
    """Seeded [rows, cols] scores N(0, sigma^2) as a CPU torch tensor in the dtype."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return torch.from_numpy(x).to(torch_dtype(dtype))


def softmax_workload_inputs(w: SoftmaxWorkload):
    return make_scores(w.rows, w.cols, w.dtype, w.seed, w.sigma)


def kv_workload_inputs(w: KVWorkload):
    return make_qkv(w.B, w.Hq, w.Hkv, w.Nq, w.d, w.dtype, w.seed, 1.0, Nk=w.Nk)


def torch_dtype(dtype: str):
    if dtype == "f32":
        return torch.float32
    if dtype == "bf16":
        return torch.bfloat16
    if dtype == "f16":
        return torch.float16
    raise ValueError("unknown dtype %r" % (dtype,))


def make_qkv(B, Hq, Hkv, N, d, dtype="bf16", seed=0, q_mult=1.0, Nk=None):
    """Seeded Q, K, V as CPU torch tensors in the input dtype.

    Q has N rows per head; K and V have Nk rows per head (default N).
    """
    nk = N if Nk is None else Nk
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, N, d), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, nk, d), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, nk, d), dtype=np.float32)
    if q_mult != 1.0:
        q *= np.float32(q_mult)
    td = torch_dtype(dtype)
    return (torch.from_numpy(q).to(td), torch.from_numpy(k).to(td), torch.from_numpy(v).to(td))


def make_qkv_device(B, Hq, Hkv, Nq, Nk, d, dtype="bf16", seed=0, device="cuda"):
    """Seeded Q, K, V drawn on a device (torch's Philox generator there), for problems whose
    K/V are too large to draw on the host in reasonable time.  Standard normals rounded to the
    input dtype; deterministic for a given seed and device type."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    td = torch_dtype(dtype)
    q = torch.randn((B, Hq, Nq, d), generator=g, device=device, dtype=torch.float32).to(td)
    k = torch.randn((B, Hkv, Nk, d), generator=g, device=device, dtype=torch.float32).to(td)
    v = torch.randn((B, Hkv, Nk, d), generator=g, device=device, dtype=torch.float32).to(td)
    return q, k, v


def workload_inputs(w: Workload):
    return make_qkv(w.B, w.Hq, w.Hkv, w.N, w.d, w.dtype, w.seed, w.q_mult)


def make_dout(B, Hq, N, d, dtype="bf16", seed=0):
    """Seeded upstream gradient dO [B, Hq, N, d]: float32 standard normals rounded to the dtype."""
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((B, Hq, N, d), dtype=np.float32)
    return torch.from_numpy(g).to(torch_dtype(dtype))


def bwd_workload_inputs(w: Workload):
    """(q, k, v, dO) of a backward workload; dO is drawn with seed + 50000."""
    q, k, v = workload_inputs(w)
    return q, k, v, make_dout(w.B, w.Hq, w.N, w.d, w.dtype, w.seed + 50000)


def bwd_flops(w: Workload) -> float:
    """The five products of the backward (S, dP, dV, dK, dQ), 2*N^2*d flops each per
    head, halved when causal: 2.5 times the forward's count."""
    return 2.5 * w.flops


def sample_rows(w: Workload, count: int, seed: int | None = None):
    """Sorted flat row ids (b*Hq + h)*N + i drawn without replacement.

    The first row of the first head and the last row of the last head always
    replace the first two draws, so both ends of the causal triangle are covered.
    """
    total = w.B * w.Hq * w.N
    count = min(count, total)
    rng = np.random.default_rng((w.seed + 1) if seed is None else seed)
    rows = rng.choice(total, size=count, replace=False)
    if count >= 2:
        first = 0
        last = total - 1
        rows = rows[~np.isin(rows, [first, last])]
        rows = np.concatenate([[first, last], rows[: count - 2]])
    return np.sort(rows.astype(np.int64))
