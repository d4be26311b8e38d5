"""GPU parity: libspb's HIP path against the float64 oracle on the same seeded
inputs, through the C ABI.  Run on an MI355X."""
import numpy as np
import pytest

import synth
from tests.gpu_helpers import Case, check_attention, check_scores, lm_head, oracle_scores, say, SCORE_TOL, TOL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import shared_prefix_branch_amd as spb
    spb.lib()


def test_tiny_config_full_oracle():
    wl = synth.make_workload("tiny")
    say("case: tiny config, f32 inputs, full oracle")
    case = Case(wl, 16384)
    W, Wh = lm_head(wl)
    case.run(W)
    ea = check_attention(case)
    es = check_scores(case, oracle_scores(case, Wh))
    say(f"tiny: attention rel err {ea:.2e}; score errors {es}")


def test_tiny_config_chained_hidden_is_attention_output():
    # hidden = the row's attention output, heads concatenated (Hq * d = 256 = H)
    import torch
    import shared_prefix_branch_amd as spb
    from oracle import attention as OA, scoring as OS, tree as OT
    wl = synth.make_workload("tiny")
    say("case: tiny config chained")
    case = Case(wl, 16384)
    W, Wh = lm_head(wl)
    case.run(W)
    job = case.job
    buf = job.passes[0]
    hid = buf.o.reshape(buf.o.shape[0], -1).contiguous()
    spb.score_options(case.plan, 0, buf.meta, hid, W, buf.workspace, buf.lp, buf.p, buf.residual)
    torch.cuda.synchronize()
    res = job.finalize(copy=True)
    lay = OT.build_layout(case.prob, floors=True)
    att = {}
    for n, li in enumerate(lay.inputs):
        q, k, v, _ = case.oracle_inputs(n)
        a = OA.attention_input(lay, li, q, k, v)
        for r in range(a.shape[0]):
            att[li.first_row + r] = a[r].reshape(-1)
    sc = OS.score_branches(lay, lambda rows: np.stack([att[r] for r in rows]), Wh)
    OS.join_floors(lay, sc)
    pos = 0
    for b in lay.branches():
        if b.is_floor:
            continue
        s = sc[(b.input_no, b.question)]
        k = len(s.lp)
        assert np.max(np.abs(res["lp"][pos:pos + k] - s.lp) / np.abs(s.lp)) <= SCORE_TOL
        assert np.max(np.abs(res["p"][pos:pos + k] - s.p)) <= SCORE_TOL
        assert np.max(np.abs(res["floor_p"][pos:pos + k] - s.floor_p)) <= SCORE_TOL
        pos += k


@pytest.mark.parametrize("sharp", [False, True], ids=["metric", "sharp"])
@pytest.mark.parametrize("dtype,hq,hkv,d", [("bf16", 8, 4, 128), ("bf16", 4, 4, 64), ("bf16", 8, 2, 64),
                                             ("f32", 4, 2, 128), ("fp8", 8, 2, 128)])
def test_random_problem_several_tiles_ragged(dtype, hq, hkv, d, sharp):
    # several 128-row tiles per segment, ragged tile and vocabulary tails,
    # multi-token options sharing trie prefixes, spills at a small budget;
    # "sharp": scores of std about 1 with planted keys far above their
    # chunk's reference (the f32 and e4m3 inputs run the register-staged
    # kernel), and hidden rows of 512 so that the logits spread (std about 0.45)
    wl = synth.make_workload("news", hq=hq, hkv=hkv, head_dim=d, hidden=512 if sharp else 128, vocab=1000,
                             dtype=dtype)
    wl.problem = synth.make_problem("random", 77, vocab=1000, n_inputs=5, n_questions=6, min_content=40,
                                    max_content=300, max_len=30, max_options=5, max_option_tokens=5)
    wl.inputs = synth.logical_inputs(wl.problem, True)
    say(f"case: random problem dtype={dtype} hq={hq} hkv={hkv} d={d} sharp={sharp}")
    for budget in (16384, 700):
        case = Case(wl, budget, peaked=True, sharp=sharp)
        W, Wh = lm_head(wl)
        case.run(W)
        ea = check_attention(case, guard=sharp)
        guards = [oracle_scores(case, Wh, wrong=w) for w in ("flat", "neighbour")] if sharp else ()
        es = check_scores(case, oracle_scores(case, Wh), guards)
        say(f"  budget {budget}: passes {case.plan.n_passes} attention rel err {ea:.2e}; scores {es}")


@pytest.mark.parametrize("sharp", [False, True], ids=["metric", "sharp"])
def test_news_full_size_sampled(sharp):
    # the news configuration at full size and launch shape; the oracle checks a
    # seeded sample of branches (attention rows and full-vocabulary scores),
    # and two inputs scored alone must give the packed run's bits.  "sharp":
    # scores of std about 1 with planted keys, hidden rows N(0, 1) (logits of
    # std about 1.2), and guards that a plain V average, constant logits and a
    # neighbouring token's logit would all fail the comparison
    from tests.test_gpu_configs import _att_bits, _free, _same, _scores_bits
    wl = synth.make_workload("news")
    say(f"case: news full size, sampled, sharp={sharp}")
    case = Case(wl, 16384, peaked=sharp, sharp=sharp)
    W, Wh = lm_head(wl)
    case.run(W)
    assert case.plan.n_passes == 3
    rng = np.random.default_rng(0)
    n_in = wl.problem.n_inputs
    inputs = sorted(rng.choice(n_in, size=2, replace=False).tolist()) + [n_in + 3]  # two inputs and a floor
    ea = check_attention(case, inputs=inputs, branches_per_input=3, rng=rng, guard=sharp)
    keys = [(n, q) for n in inputs[:2] for q in rng.choice(56, size=4, replace=False).tolist()]
    guards = [oracle_scores(case, Wh, keys, wrong=w) for w in ("flat", "neighbour")] if sharp else ()
    es = check_scores(case, oracle_scores(case, Wh, keys), guards)
    say(f"news: attention rel err {ea:.2e}; scores {es}")
    alone_in = inputs[:2]
    packed_s, packed_a = _scores_bits(case, alone_in), _att_bits(case, alone_in)
    _free(case)
    for i in alone_in:
        alone = Case(wl, 16384, inputs=[i], peaked=sharp, sharp=sharp)
        alone.run(W)
        _same({i: packed_s[i]}, _scores_bits(alone, [i]), f"news input {i} alone")
        _same({i: packed_a[i]}, _att_bits(alone, [i]), f"news input {i} alone")
        _free(alone)
