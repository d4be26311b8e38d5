"""GPU: the lm head's output kinds (f32out, bf16, fp32) against the oracle;
for bf16 hidden rows the fp32 head equals f32out bit for bit, and the batched
head equals the per-pass head for every kind."""
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
            (np.float32(v[2]).view(np.uint32),)
            for k, v in case.branch_results().items()}


def _multitoken_wl():
    wl = synth.make_workload("news", hq=8, hkv=4, head_dim=128, hidden=256, vocab=4096)
    wl.problem = synth.make_problem("random", 37, vocab=4096, n_inputs=6, n_questions=4, min_content=5,
                                    max_content=60, max_len=8, max_options=4, max_option_tokens=3)
    wl.inputs = synth.logical_inputs(wl.problem, True)
    return wl


@pytest.mark.parametrize("kind", [0, 1, 2])
def test_tiny_f32_hidden_each_kind(kind):
    # the tiny workload has f32 hidden rows: fp32 differs from f32out, bf16 too
    wl = synth.make_workload("tiny")
    W, Wh = lm_head(wl)
    say(f"case: tiny, lm-head kind {kind}")
    c = Case(wl, 16384, peaked=True, lm_head_kind=kind)
    c.run(W)
    err = check_scores(c, oracle_scores(c, Wh))
    say(f"  oracle errors {err}")


def test_kinds_differ_and_fp32_equals_f32out_for_bf16_hidden():
    wl = _multitoken_wl()
    W, Wh = lm_head(wl)
    cache = {}
    runs = {}
    for kind in (0, 1, 2):
        c = Case(wl, 200, peaked=True, cache=cache, lm_head_kind=kind)
        c.run(W)
        runs[kind] = c
        err = check_scores(c, oracle_scores(c, Wh))
        say(f"  kind {kind}: {c.plan.n_passes} passes, oracle errors {err}")
    a, b, f = _bits(runs[0]), _bits(runs[1]), _bits(runs[2])
    # bf16 hidden rows: the fp32 head's extra planes are zero
    for key in a:
        for u, v in zip(a[key], f[key]):
            assert np.array_equal(u, v), f"branch {key}: fp32 head differs from f32out on bf16 hidden rows"
    assert any(not np.array_equal(u, v) for key in a for u, v in zip(a[key], b[key])), \
        "bf16 logits changed no score"


@pytest.mark.parametrize("kind", [1, 2])
def test_batched_head_equals_per_pass_for_kind(kind):
    wl = synth.make_workload("tiny")
    wl.problem = synth.make_problem("random", 41, vocab=1024, n_inputs=8, n_questions=4, min_content=5,
                                    max_content=40, max_len=8, max_options=4, max_option_tokens=3)
    wl.inputs = synth.logical_inputs(wl.problem, True)
    W, Wh = lm_head(wl)
    cache = {}
    per = Case(wl, 120, peaked=True, cache=cache, lm_head_kind=kind)
    per.run(W)
    bat = Case(wl, 120, peaked=True, cache=cache, lm_head_kind=kind, batch_head=True)
    bat.run(W)
    say(f"case: random f32 hidden, {per.plan.n_passes} passes, kind {kind}, batched vs per-pass")
    a, b = _bits(per), _bits(bat)
    for key in a:
        for u, v in zip(a[key], b[key]):
            assert np.array_equal(u, v), f"branch {key}: batched head differs from per-pass (kind {kind})"
    err = check_scores(bat, oracle_scores(bat, Wh))
    say(f"  bit-identical; oracle errors {err}")
