"""Softmax of every row of a matrix in fp64: the oracle for the row-softmax kernel.

TEST INFRASTRUCTURE ONLY: the tests and the benchmark's CPU-baseline leg may
import this module; the product path never does.  It shares nothing with the
HIP library.

What it computes, for each row x of x[R][C] (the pages' safe softmax):
    m   = max_j x_j                       subtract the largest score first
    l   = sum_j exp(x_j - m)              the normaliser, measured against m
    y_j = exp(x_j - m) / l
    lse = m + ln l                        the log of the normaliser
Sources: spicyshark.co online-softmax lesson, "Scores become shares" (softmax
turns scores into shares that sum to one), "The naive approach, and why it
fails" (exp overflows without the subtraction), "The fix: subtract the maximum"
(the common factor cancels) and "The cost: three passes" (max, sum, output).

A row whose entries are all -inf has no softmax: m = -inf, every term is
exp(nan) and the definition gives nan for y and -inf for lse, as written out
below (the reading used for the kernel too).  numpy in float64 with its own
exp and log; no blocking and no streaming.
"""
from __future__ import annotations

import numpy as np


def softmax_rows(x):
    """x [R, C] (any real dtype, upcast exactly) -> (y [R, C], lse [R]) in float64."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2 or x.shape[1] < 1:
        raise ValueError("x must be [rows, cols] with cols >= 1")
    m = x.max(axis=1, keepdims=True)
    with np.errstate(invalid="ignore"):
        e = np.exp(x - m)                      # pass 2 and 3 of the three-pass method
        l = e.sum(axis=1, keepdims=True)
        y = e / l
        lse = (m + np.log(l))[:, 0]
    empty = np.isneginf(m[:, 0])               # all -inf: no softmax
    y[empty] = np.nan
    lse[empty] = -np.inf
    return y, lse
