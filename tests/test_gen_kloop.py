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
                if lo <= int(r[1:]) < hi:        # Q read back from its LDS staging is no operand slot
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


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_next_item_loads_are_older_than_the_stores_its_first_barrier_may_leave(gen, d, causal):
    """An item's first barrier waits for vmcnt(n) with n = the epilogue's store count: the
    item before loaded this item's Q (staged in LDS) and first tiles ahead of its epilogue, so
    with vector memory completing in issue order those loads are done once at most n younger
    operations remain.  That holds when the Q staging in the tail is followed by exactly the
    epilogue's stores, and when a wave that stages Q later (in its duty steps, after its
    stores) waits for everything before the item ends."""
    gen.D = d
    g, prog, path_a, path_b, tail = gen.build("bf16", causal, 4)
    n = gen.nstores()
    assert n == 2 + 8 * (d // 32)
    conds = [k for k, it in enumerate(tail) if isinstance(it, gen.Cond) and any("%[pq]" in x for x in it.test)]
    assert len(conds) == 1
    rest = tail[conds[0] + 1:]
    duty = [it for it in rest if isinstance(it, gen.Cond) and any(isinstance(b, gen.Loop) for b in it.body)]
    assert len(duty) == 1
    # the tail's own tile loads run only while %[kit] < %[nt], never in the step (%[kit] == %[nt])
    # that stages Q
    def at_last_step(items, out):
        for it in items:
            if isinstance(it, gen.Ins):
                out.append(it)
            elif not (isinstance(it, gen.Cond) and any(x.startswith("s_cmp_lt_u32") and "%[nt]" in x for x in it.test)):
                at_last_step(it.body, out)
        return out
    straight = at_last_step([it for it in rest if it is not duty[0]], [])
    assert sum(1 for ins in straight if ins.kind == "vstore") == n
    assert not any(ins.kind in ("dma", "vload") for ins in straight)
    assert duty[0].body[-1].text == "s_waitcnt vmcnt(0)"
    loop = [b for b in duty[0].body if isinstance(b, gen.Loop)][0]
    assert any(isinstance(it, gen.Cond) and any("%[pq]" in x for x in it.test) for it in loop.body)
    # the first barrier: the item's own loads (first item) are waited for in full just before
    seq = flatten(gen, prog, [])
    k = next(i for i, ins in enumerate(seq) if ins.kind == "barrier")
    assert seq[k - 1].text == "s_waitcnt vmcnt(%d) lgkmcnt(0)" % n
    own = [it for it in prog if isinstance(it, gen.Cond) and it.test == ["s_cmp_eq_u32 %[pf], 0"]]
    assert [b.text for b in own[-1].body] == ["s_waitcnt vmcnt(0)"]
