"""GPU: the persistent lm head, whose resident work groups each walk several
tiles as one stream of K stages, at shapes that put tile boundaries where the
stream's bookkeeping is hardest: a vocabulary that is not a multiple of the
2,048 rows one round of slices covers (so XCDs hold different tile counts) and
ends in a partial slice; hidden sizes of one and three 64-element stages (the
W copies of a stage two ahead then belong to the tile after next); the fp32
kind, whose K stream sweeps W once per plane of the hidden rows.  Scores
against the float64 oracle with the comparison's guards, and an input's bits
scored in the full pass (several tiles per work group) against the same input
scored alone (one tile per work group)."""
import numpy as np
import pytest

import synth
from tests.gpu_helpers import Case, check_scores, lm_head, oracle_scores, say
from tests.test_gpu_invariance import _by_input, _same

pytestmark = pytest.mark.gpu

VOCAB = 70001  # 274 slices of 256 (274 = 34 x 8 + 2), the last one of 113 rows


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import shared_prefix_branch_amd as spb
    spb.lib()


def _wl(hidden):
    wl = synth.make_workload("news", hq=8, hkv=4, head_dim=64, hidden=hidden, vocab=VOCAB)
    wl.problem = synth.make_problem("random", 17, vocab=VOCAB, n_inputs=6, n_questions=40, min_content=10,
                                    max_content=60, max_len=8, max_options=3, max_option_tokens=2)
    wl.inputs = synth.logical_inputs(wl.problem, True)
    return wl


@pytest.mark.parametrize("hidden,kind", [(64, 0), (192, 0), (192, 1), (64, 2)],
                         ids=["h64-f32out", "h192-f32out", "h192-bf16", "h64-fp32"])
def test_head_stream_parity_and_alone(hidden, kind):
    wl = _wl(hidden)
    W, _ = lm_head(wl)
    # W ~ N(0, 0.02^2) gives logits of spread 0.02 sqrt(H) on the peaked hidden
    # rows; a power-of-two scale (exact in bf16) brings it to about 1.2, where
    # the comparison's guards (constant logits, the neighbouring token) fail
    W = W * (8 if hidden < 128 else 4)
    Wh = W.cpu()
    case = Case(wl, 16384, peaked=True, lm_head_kind=kind)
    m = case.plan.info(0)["n_scored_rows"]
    say(f"case: head stream H={hidden} V={VOCAB} kind={kind}: {case.plan.n_passes} pass(es), {m} scored rows")
    # the full pass has more tiles than 32 work groups per XCD, so groups walk several
    assert case.plan.n_passes == 1 and m > 256
    case.run(W)
    rng = np.random.default_rng(hidden + kind)
    keys = sorted(case.branch_results().keys())
    pick = [keys[i] for i in sorted(rng.choice(len(keys), size=12, replace=False))]
    guards = [oracle_scores(case, Wh, pick, wrong=w) for w in ("flat", "neighbour")]
    es = check_scores(case, oracle_scores(case, Wh, pick), guards=guards)
    say(f"  scores vs oracle {es}")
    full = _by_input(case)
    for i in (0, 5):
        alone = Case(wl, 16384, inputs=[i], peaked=True, lm_head_kind=kind)
        alone.run(W)
        _same(full[i], _by_input(alone)[i], f"input {i} alone")
