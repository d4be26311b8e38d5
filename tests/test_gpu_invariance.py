"""GPU batch invariance: an input's attention rows and scores are bit-identical
whether it is scored alone or packed with others, in any order, at any token
budget (PyPI page "spinf-serve 0.1.1", "What it does": batch invariance)."""
import numpy as np
import pytest

import synth
from tests.gpu_helpers import Case, lm_head, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _by_input(case: Case):
    """{original input id: (attention rows bytes keyed by logical row offset, scores)}"""
    from oracle import tree as OT  # only for the logical row numbering of the check
    out = {}
    res = case.branch_results()
    lay = OT.build_layout(case.prob, floors=case.floors)
    for n, i in enumerate(case.inputs):
        li = lay.inputs[n]
        nrows = int((lay.row_input == n).sum())
        rows = list(range(li.first_row, li.first_row + nrows))
        got = case.job.attention_by_logical_row(rows)
        att = [got[r][0].view(np.uint32).copy() for r in rows]
        sc = {q: tuple(np.asarray(x).view(np.uint32).copy() if isinstance(x, np.ndarray)
                       else np.float32(x).view(np.uint32) for x in res[(n, q)])
              for q in case.prob.questions_of(n)}
        out[i] = (att, sc)
    return out


def _same(a, b, what):
    att_a, sc_a = a
    att_b, sc_b = b
    assert len(att_a) == len(att_b)
    for r, (x, y) in enumerate(zip(att_a, att_b)):
        assert np.array_equal(x, y), f"{what}: attention row {r} differs"
    assert sc_a.keys() == sc_b.keys()
    for q in sc_a:
        for f, (x, y) in enumerate(zip(sc_a[q], sc_b[q])):
            assert np.array_equal(x, y), f"{what}: question {q} field {f} differs"


def _random_wl(dtype="bf16"):
    wl = synth.make_workload("news", hq=8, hkv=4, head_dim=128, hidden=128, vocab=1000, dtype=dtype)
    wl.problem = synth.make_problem("random", 91, vocab=1000, n_inputs=6, n_questions=6, min_content=10,
                                    max_content=260, max_len=30, max_options=5, max_option_tokens=4)
    wl.inputs = synth.logical_inputs(wl.problem, True)
    return wl


SHARP = pytest.mark.parametrize("sharp", [False, True], ids=["metric", "sharp"])


@SHARP
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_packed_equals_alone_random_multitoken(dtype, sharp):
    # sharp: planted keys whose scores rise far above their chunk's running
    # maximum, so rows rescale mid-way; the bits must still not depend on the
    # packing
    wl = _random_wl(dtype)
    W, _ = lm_head(wl)
    say(f"case: random multi-token problem, packed vs alone, dtype={dtype} sharp={sharp}")
    packed = Case(wl, 16384, peaked=True, sharp=sharp)
    packed.run(W)
    P = _by_input(packed)
    for i in range(wl.problem.n_inputs):
        alone = Case(wl, 16384, inputs=[i], peaked=True, sharp=sharp)
        alone.run(W)
        _same(P[i], _by_input(alone)[i], f"input {i} alone")


@SHARP
def test_orders_and_budgets_bit_identical_fp8(sharp):
    wl = synth.make_workload("fp8", n_inputs=24)
    W, _ = lm_head(wl)
    cache = {}
    say(f"case: fp8, 3 orders x 3 budgets + alone; the third order's passes share lm-head launches "
        f"(head groups); sharp={sharp}")
    ref = None
    for seed in (101, 102, 103):
        order = np.random.default_rng(seed).permutation(wl.problem.n_inputs).tolist()
        for budget in (8192, 16384, 32768):
            c = Case(wl, budget, inputs=order, head_rows=768 if seed == 103 else 0, peaked=sharp, sharp=sharp,
                     cache=cache)
            c.run(W)
            got = _by_input(c)
            say(f"  order seed {seed} budget {budget}: {c.plan.n_passes} passes, "
                f"{len(c.job.head_groups)} lm-head launches")
            if ref is None:
                ref = got
            else:
                for i in ref:
                    _same(ref[i], got[i], f"input {i} order {seed} budget {budget}")
    for i in (0, 5, 17):
        c = Case(wl, 16384, inputs=[i], peaked=sharp, sharp=sharp, cache=cache)
        c.run(W)
        _same(ref[i], _by_input(c)[i], f"input {i} alone")


@SHARP
def test_spilled_input_matches_alone_extreme_shape(sharp):
    # inputs larger than a pass: content re-staged per pass, same bits as alone
    wl = synth.make_workload("extreme", n_inputs=3, n_questions=300, content=700, hidden=128, vocab=4096)
    W, _ = lm_head(wl)
    say(f"case: extreme shape (scaled), spill at budget 2048, sharp={sharp}")
    packed = Case(wl, 2048, peaked=sharp, sharp=sharp)
    packed.run(W)
    assert packed.plan.n_passes > 3
    P = _by_input(packed)
    alone = Case(wl, 16384, inputs=[1], peaked=sharp, sharp=sharp)
    alone.run(W)
    _same(P[1], _by_input(alone)[1], "input 1 unspilled alone")


def test_run_to_run_deterministic():
    wl = _random_wl()
    W, _ = lm_head(wl)
    a = Case(wl, 700, peaked=True)
    a.run(W)
    A = _by_input(a)
    a.job.run(W)
    import torch
    torch.cuda.synchronize()
    a.res = a.job.finalize()
    B = _by_input(a)
    for i in A:
        _same(A[i], B[i], f"input {i} second run")


@SHARP
def test_fp8_async_copy_kernel_equals_register_staged(sharp):
    # e4m3 attention two ways: V widened to bf16 in a workspace with K/V
    # copied asynchronously into LDS, or K/V staged through registers.  Same
    # MFMAs in the same order per row, so the same bits, across spilling
    # passes of 8,192 tokens; scores follow.
    wl = synth.make_workload("fp8", n_inputs=30)
    W, _ = lm_head(wl)
    cache = {}
    say(f"case: fp8 attention, async-copy kernel vs register-staged kernel, sharp={sharp}")
    a = Case(wl, 8192, peaked=sharp, sharp=sharp, cache=cache, fp8_dma=True)
    a.run(W)
    assert a.job.att_ws is not None
    A = _by_input(a)
    a.job = None
    b = Case(wl, 8192, peaked=sharp, sharp=sharp, cache=cache, fp8_dma=False)
    b.run(W)
    assert b.job.att_ws is None
    B = _by_input(b)
    for i in A:
        _same(A[i], B[i], f"input {i}: async-copy vs staged")
