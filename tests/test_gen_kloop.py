"""Static checks of the generated key loop (gen_fwd_kloop.py), on the CPU.

The generator reuses four K and four V staging slots for the operands it reads from LDS
ahead of the matrix products.  Along every path of every variant, each read into a slot
must be consumed by a product before the slot is written again, and no read may be left
unconsumed: a read that runs too far ahead would overwrite an operand before its product
issues (the hardware does not interlock that), and the product would take the wrong tile.
"""
import importlib.util
import os

import pytest

GEN = os.path.join(os.path.dirname(__file__), "..", "flashattention_online_softmax_fwd_amd", "csrc",
                   "gen_fwd_kloop.py")


@pytest.fixture(scope="module")
def gen():
    spec = importlib.util.spec_from_file_location("gen_fwd_kloop", GEN)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def flatten(gen, items, out):
    for it in items:
        if isinstance(it, gen.Ins):
            out.append(it)
        else:
            flatten(gen, it.body, out)
    return out


def staging_events(gen, seq):
    lo, hi = gen.KST(0), gen.VST(3) + 4
    ev = {}
    for ins in seq:
        if ins.kind == "lds":
            for r in ins.defs:
                ev.setdefault(r, []).append("W")
        elif ins.kind == "mfma":
            for r in ins.uses:
                if r.startswith("v") and lo <= int(r[1:]) < hi:
                    ev.setdefault(r, []).append("U")
    return ev


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("nw", [2, 4])
@pytest.mark.parametrize("causal", [False, True])
def test_staging_slots_are_consumed_before_reuse(gen, d, nw, causal):
    gen.D = d
    g, prog, path_a, path_b, tail = gen.build("bf16", causal, nw)
    setup = flatten(gen, prog, [])
    for name, body in (("L >= 1", path_a), ("L == 0", path_b)):
        seq = setup + flatten(gen, body, []) + flatten(gen, tail, [])
        for reg, e in staging_events(gen, seq).items():
            assert e[0] == "W", (name, reg, "used before any read")
            for a, b in zip(e, e[1:]):
                assert not (a == "W" and b == "W"), (name, reg, "overwritten before use")
            assert e[-1] == "U", (name, reg, "read but never used")


def test_the_checker_sees_a_read_that_runs_too_far_ahead(gen):
    """With the reads four product groups ahead, the score-only half after the prologue reads
    K rows into slot 0 again before its first product has used them: the check must fail."""
    gen.D = 128
    lead = gen.LEAD
    try:
        gen.LEAD = 4
        g, prog, path_a, path_b, tail = gen.build("bf16", True, 4)
    finally:
        gen.LEAD = lead
    seq = flatten(gen, prog, []) + flatten(gen, path_a, []) + flatten(gen, tail, [])
    doubled = [reg for reg, e in staging_events(gen, seq).items()
               if any(a == "W" and b == "W" for a, b in zip(e, e[1:]))]
    assert doubled
