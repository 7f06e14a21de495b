"""Parity bars between the HIP forward and the fp64 oracle.

TEST INFRASTRUCTURE ONLY, like everything under ``oracle/``: the tests, the
smoke check and the benchmark's oracle leg read these; the product path never
does.

The method's bar for 16-bit inputs with fp32 accumulation is an absolute error
of 1e-2 with a relative error of 2e-2, against the oracle run on the same
rounded inputs; for fp32 inputs 1e-5.  It is read elementwise in allclose form,
|x - r| <= atol + rtol * |r|, because values near zero make a pure relative bound
meaningless and rounding O to bf16 alone costs up to 1/64 where |O| is in
[4, 8).  The pages name no fp16 bar: fp16 takes the bf16 bar times 2^-3, the
ratio of fp16's unit roundoff (2^-11) to bf16's (2^-8).  fp32 adds a relative
2^-22, two float32 roundings of the result: the absolute 1e-5 alone is finer
than float32's own spacing for |x| >= 128 (an LSE of 6e6 is stored to 0.5).
Every value must also be finite.
"""
from __future__ import annotations

import numpy as np

FORWARD = {"bf16": (1e-2, 2e-2), "f16": (1.25e-3, 2.5e-3), "f32": (1e-5, 2.0 ** -22)}


def forward_bar(dtype: str):
    """(atol, rtol) of the forward's bar for inputs of this dtype."""
    return FORWARD[dtype]


def within(x, r, dtype: str) -> bool:
    """True when every x is finite and |x - r| <= atol + rtol * |r| elementwise."""
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    atol, rtol = FORWARD[dtype]
    return bool(np.all(np.isfinite(x)) and np.all(np.abs(x - r) <= atol + rtol * np.abs(r)))
