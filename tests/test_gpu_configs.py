"""GPU parity and batch invariance at the full sizes of the moderation,
many-questions and fp8 configurations, in the launch configuration the
benchmark uses.  The oracle checks a seeded sample of branches (attention rows
and full-vocabulary scores); invariance compares whole packings.

Each test runs twice: on the metric draws (Q, K ~ N(0,1)/sqrt(d), hidden
N(0,1)/sqrt(H)), whose softmax is almost a plain average and whose logits are
almost flat, and on "sharp" draws (scores of std about 1 with planted keys
far above their chunk's reference, hidden N(0,1)), where guards require that a
plain V average, constant logits and a neighbouring token's logit would each
fail the comparison by a wide margin."""
import gc

import numpy as np
import pytest

import synth
from tests.gpu_helpers import Case, check_attention, check_scores, lm_head, oracle_scores, say

SHARP = pytest.mark.parametrize("sharp", [False, True], ids=["metric", "sharp"])

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _free(*cases, keep_cache=False):
    import torch
    for c in cases:
        if not keep_cache:
            c._blocks.clear()
        c.job = None
    gc.collect()
    torch.cuda.empty_cache()


def _scores_bits(case, inputs):
    """{original input id: [per question: uint32 bit patterns of lp, p, residual, floor_p, lift]}"""
    res = case.branch_results()
    out = {}
    for n, i in enumerate(case.inputs):
        if i not in inputs:
            continue
        out[i] = [tuple(np.asarray(x, np.float32).view(np.uint32).copy() for x in res[(n, q)])
                  for q in case.prob.questions_of(n)]
    return out


def _att_bits(case, inputs):
    from oracle import tree as OT
    lay = OT.build_layout(case.prob, floors=case.floors)
    out = {}
    for n, i in enumerate(case.inputs):
        if i not in inputs:
            continue
        li = lay.inputs[n]
        nrows = int((lay.row_input == n).sum())
        got = case.job.attention_by_logical_row(range(li.first_row, li.first_row + nrows))
        out[i] = np.stack([got[r][0] for r in range(li.first_row, li.first_row + nrows)]).view(np.uint32)
    return out


def _same(a, b, what):
    assert a.keys() == b.keys()
    for i in a:
        if isinstance(a[i], np.ndarray):
            assert np.array_equal(a[i], b[i]), f"{what}: attention rows of input {i} differ"
        else:
            for q, (x, y) in enumerate(zip(a[i], b[i])):
                for f, (u, v) in enumerate(zip(x, y)):
                    assert np.array_equal(u, v), f"{what}: input {i} branch {q} field {f} differs"


def _guards(case, Wh, keys, sharp):
    return [oracle_scores(case, Wh, keys, wrong=w) for w in ("flat", "neighbour")] if sharp else ()


@SHARP
def test_moderation_full_size(sharp):
    wl = synth.make_workload("moderation")
    W, Wh = lm_head(wl)
    say(f"case: moderation, 300 contents x 106 questions, multi-token options, sharp={sharp}")
    case = Case(wl, 16384, peaked=sharp, sharp=sharp)
    case.run(W)
    say(f"  {case.plan.n_passes} passes, {case.plan.info()['n_tokens']} tokens")
    rng = np.random.default_rng(3)
    n_in = wl.problem.n_inputs
    sample = sorted(rng.choice(n_in, size=3, replace=False).tolist())
    ea = check_attention(case, inputs=sample + [n_in + 5], branches_per_input=3, rng=rng, guard=sharp)
    keys = [(n, q) for n in sample for q in rng.choice(106, size=3, replace=False).tolist()]
    es = check_scores(case, oracle_scores(case, Wh, keys), _guards(case, Wh, keys, sharp))
    say(f"  attention rel err {ea:.2e}; scores {es}")
    packed_s, packed_a = _scores_bits(case, sample[:2]), _att_bits(case, sample[:2])
    _free(case)
    for i in sample[:2]:
        alone = Case(wl, 16384, inputs=[i], peaked=sharp, sharp=sharp)
        alone.run(W)
        _same({i: packed_s[i]}, _scores_bits(alone, [i]), f"moderation input {i} alone")
        _same({i: packed_a[i]}, _att_bits(alone, [i]), f"moderation input {i} alone")
        _free(alone)


@SHARP
def test_many_questions_full_size(sharp):
    wl = synth.make_workload("extreme")
    W, Wh = lm_head(wl)
    say(f"case: many questions, 8 contents x 1000 questions, spilling passes, sharp={sharp}")
    case = Case(wl, 16384, peaked=sharp, sharp=sharp)
    case.run(W)
    say(f"  {case.plan.n_passes} passes, {case.plan.info()['n_tokens']} tokens")
    rng = np.random.default_rng(4)
    ea = check_attention(case, inputs=[2, 8 + 17], branches_per_input=4, rng=rng, guard=sharp)
    keys = [(2, q) for q in rng.choice(1000, size=4, replace=False).tolist()] + [(6, 999), (6, 0)]
    es = check_scores(case, oracle_scores(case, Wh, keys), _guards(case, Wh, keys, sharp))
    say(f"  attention rel err {ea:.2e}; scores {es}")
    packed_s, packed_a = _scores_bits(case, [5]), _att_bits(case, [5])
    _free(case)
    alone = Case(wl, 16384, inputs=[5], peaked=sharp, sharp=sharp)
    alone.run(W)
    _same(packed_s, _scores_bits(alone, [5]), "extreme input 5 alone")
    _same(packed_a, _att_bits(alone, [5]), "extreme input 5 alone")
    _free(alone)


@SHARP
def test_fp8_full_size_orders_budgets_and_alone(sharp):
    # sharp: the e4m3 scales are calibrated on the sharp draws
    wl = synth.make_workload("fp8")
    W, Wh = lm_head(wl)
    n_in = wl.problem.n_inputs
    rng = np.random.default_rng(5)
    watch = sorted(rng.choice(n_in, size=4, replace=False).tolist())
    say(f"case: fp8, 500 contents, 3 orders x 3 budgets, watching inputs {watch}, sharp={sharp}")
    ref_s = ref_a = None
    cache = {}
    for seed in (101, 102, 103):
        order = np.random.default_rng(seed).permutation(n_in).tolist()
        for budget in (8192, 16384, 32768):
            c = Case(wl, budget, inputs=order, cache=cache, peaked=sharp, sharp=sharp)
            c.run(W)
            s_bits = _scores_bits(c, set(range(n_in)))
            a_bits = _att_bits(c, watch)
            say(f"  order {seed} budget {budget}: {c.plan.n_passes} passes")
            if ref_s is None:
                ref_s, ref_a = s_bits, a_bits
                ea = check_attention(c, inputs=[order.index(watch[0])], branches_per_input=3, rng=rng,
                                     guard=sharp)
                keys = [(order.index(watch[1]), q) for q in c.prob.questions_of(order.index(watch[1]))[:3]]
                es = check_scores(c, oracle_scores(c, Wh, keys), _guards(c, Wh, keys, sharp))
                say(f"  attention rel err {ea:.2e}; scores {es}")
            else:
                _same(ref_s, s_bits, f"order {seed} budget {budget}")
                _same(ref_a, a_bits, f"order {seed} budget {budget}")
            _free(c, keep_cache=True)
    for i in watch:
        alone = Case(wl, 16384, inputs=[i], cache=cache, peaked=sharp, sharp=sharp)
        alone.run(W)
        _same({i: ref_s[i]}, _scores_bits(alone, [i]), f"fp8 input {i} alone")
        _same({i: ref_a[i]}, _att_bits(alone, [i]), f"fp8 input {i} alone")
        _free(alone, keep_cache=True)
    cache.clear()
