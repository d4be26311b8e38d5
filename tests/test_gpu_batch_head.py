"""GPU: the one-stream lm head over several passes (spb_score_options_batch)
gives, bit for bit, the scores of the per-pass head, and matches the oracle;
so do head groups (consecutive passes sharing one launch up to a row cap)."""
import numpy as np
import pytest

import synth
from tests.gpu_helpers import Case, check_scores, lm_head, oracle_scores, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bits(case):
    return {k: tuple(np.asarray(x, np.float32).view(np.uint32).copy() for x in v[:2]) +
            (np.float32(v[2]).view(np.uint32),) + tuple(np.asarray(x, np.float32).view(np.uint32).copy() for x in v[3:])
            for k, v in case.branch_results().items()}


def _compare(wl, budget, inputs=None, peaked=False, n_check=4, seed=0, head_rows=0):
    W, Wh = lm_head(wl)
    cache = {}
    per = Case(wl, budget, inputs=inputs, peaked=peaked, cache=cache)
    per.run(W)
    bat = Case(wl, budget, inputs=inputs, peaked=peaked, cache=cache, batch_head=head_rows == 0,
               head_rows=head_rows)
    bat.run(W)
    groups = bat.job.head_groups
    rows = [sum(per.plan.info(k)["n_scored_rows"] for k in g) for g in groups]
    say(f"  {per.plan.n_passes} passes in {len(groups)} head launches of {rows} scored rows")
    if head_rows:
        assert len(groups) > 1 and max(len(g) for g in groups) > 1, "the case must group some passes"
        assert all(r <= head_rows for r, g in zip(rows, groups) if len(g) > 1)
        assert [k for g in groups for k in g] == list(range(per.plan.n_passes))
    a, b = _bits(per), _bits(bat)
    assert a.keys() == b.keys()
    for key in a:
        for f, (u, v) in enumerate(zip(a[key], b[key])):
            assert np.array_equal(u, v), f"branch {key} field {f}: batched head differs from per-pass head"
    rng = np.random.default_rng(seed)
    keys = list(a.keys())
    pick = [keys[i] for i in sorted(rng.choice(len(keys), size=min(n_check, len(keys)), replace=False))]
    err = check_scores(bat, oracle_scores(bat, Wh, pick))
    say(f"  bit-identical; oracle errors {err}")


def test_batch_head_news_full_size():
    say("case: news, 3 passes, batched vs per-pass head")
    _compare(synth.make_workload("news"), 16384, n_check=3)


def test_batch_head_multitoken_many_passes():
    wl = synth.make_workload("news", hq=8, hkv=4, head_dim=128, hidden=256, vocab=4096)
    wl.problem = synth.make_problem("random", 31, vocab=4096, n_inputs=12, n_questions=5, min_content=5,
                                    max_content=60, max_len=8, max_options=4, max_option_tokens=3)
    wl.inputs = synth.logical_inputs(wl.problem, True)
    say("case: random multi-token options, small budget (many passes)")
    _compare(wl, 110, peaked=True, n_check=6, seed=1)


def test_head_groups_news_small_budget():
    wl = synth.make_workload("news")
    say("case: news, 6 contents at budget 4096, head groups of at most 250 scored rows vs per-pass head")
    _compare(wl, 4096, inputs=list(range(6)), n_check=3, seed=2, head_rows=250)


def test_head_groups_multitoken_many_passes():
    wl = synth.make_workload("news", hq=8, hkv=4, head_dim=128, hidden=256, vocab=4096)
    wl.problem = synth.make_problem("random", 31, vocab=4096, n_inputs=12, n_questions=5, min_content=5,
                                    max_content=60, max_len=8, max_options=4, max_option_tokens=3)
    wl.inputs = synth.logical_inputs(wl.problem, True)
    say("case: random multi-token options, small budget, head groups of at most 40 scored rows")
    _compare(wl, 110, peaked=True, n_check=6, seed=3, head_rows=40)
