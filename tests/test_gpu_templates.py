"""GPU parity and invariance on template token tries: an input's questions
whose templates share prefixes read those tokens once (spinf-serve pages,
"Template tries").  The HIP path against the float64 oracle on the same seeded
inputs, and an input's bits packed with others, spilled or alone."""
import numpy as np
import pytest

import synth
from tests.gpu_helpers import Case, check_attention, check_scores, lm_head, oracle_scores, say
from tests.test_gpu_invariance import _by_input, _same

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import shared_prefix_branch_amd as spb
    spb.lib()


def _grid_wl(dtype="bf16", hq=8, hkv=4, d=128, n_inputs=3):
    wl = synth.make_workload("grid", hq=hq, hkv=hkv, head_dim=d, hidden=256, vocab=2000, dtype=dtype,
                             n_inputs=n_inputs, n_templates=2, min_content=100, max_content=300)
    return wl


def _shared_wl(dtype, hq, hkv, d):
    wl = synth.make_workload("grid", hq=hq, hkv=hkv, head_dim=d, hidden=128, vocab=1000, dtype=dtype)
    wl.problem = synth.make_problem("random_shared", 41, vocab=1000, n_inputs=5, n_questions=8, min_content=0,
                                    max_content=150, max_lead=40, tail_vocab=3, max_options=4,
                                    max_option_tokens=3)
    wl.inputs = synth.logical_inputs(wl.problem, True)
    return wl


def test_grid_templates_parity():
    wl = _grid_wl()
    W, Wh = lm_head(wl)
    for budget in (16384, 400):
        say(f"case: grid templates bf16 budget {budget}")
        case = Case(wl, budget, peaked=True)
        case.run(W)
        ea = check_attention(case)
        es = check_scores(case, oracle_scores(case, Wh))
        say(f"  passes {case.plan.n_passes} tokens {case.plan.info()['n_tokens']} "
            f"attention rel err {ea:.2e}; scores {es}")


@pytest.mark.parametrize("sharp", [False, True], ids=["metric", "sharp"])
@pytest.mark.parametrize("dtype,hq,hkv,d", [("bf16", 8, 2, 64), ("bf16", 4, 4, 128), ("f32", 4, 2, 128),
                                             ("fp8", 8, 2, 128)])
def test_random_shared_templates_parity(dtype, hq, hkv, d, sharp):
    # long shared lead-ins (stems over several 32-key chunks), empty contents,
    # inputs whose questions share nothing, spills at a small budget; sharp:
    # planted keys in the stems and branch chunks, with the comparison's guard
    wl = _shared_wl(dtype, hq, hkv, d)
    W, Wh = lm_head(wl)
    for budget in (16384, 180):
        say(f"case: random shared templates dtype={dtype} hq={hq} hkv={hkv} d={d} budget {budget} sharp={sharp}")
        case = Case(wl, budget, peaked=True, sharp=sharp)
        case.run(W)
        ea = check_attention(case, guard=sharp)
        es = check_scores(case, oracle_scores(case, Wh))
        say(f"  passes {case.plan.n_passes} attention rel err {ea:.2e}; scores {es}")


def test_shared_templates_packed_spilled_and_alone_bit_identical():
    wl = _grid_wl(n_inputs=4)
    W, _ = lm_head(wl)
    say("case: grid templates, packed vs spilled vs alone")
    packed = Case(wl, 16384)
    packed.run(W)
    P = _by_input(packed)
    spilled = Case(wl, 360, inputs=[2, 0, 3, 1])
    spilled.run(W)
    assert spilled.plan.n_passes > 4
    S = _by_input(spilled)
    for i in range(wl.problem.n_inputs):
        _same(P[i], S[i], f"input {i} spilled")
    for i in (0, 3):
        alone = Case(wl, 16384, inputs=[i])
        alone.run(W)
        _same(P[i], _by_input(alone)[i], f"input {i} alone")
