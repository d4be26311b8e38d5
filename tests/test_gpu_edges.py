"""GPU parity and invariance at the request limits, and the device path of the
metadata upload.

The man page's request limits ("spinf-serve", PARAMETERS: --max-content-tokens
4,096, --max-query-tokens 256) bound what one input may hold; an input's scores
must not depend on how it was packed (PyPI "spinf-serve 0.1.1", "What it
does": batch invariance).  Here: a content of 4,096 tokens (64 content chunks
per row), templates of 100-256 tokens (up to eight 32-key branch chunks), sharp
scores with planted keys, checked against the oracle, then packed vs spilled vs
alone bit for bit; and spb_plan_upload's own device copy against the staged
copy the engine loop uses."""
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


def _long_wl(dtype, hq=8, hkv=2):
    wl = synth.make_workload("news", hq=hq, hkv=hkv, head_dim=128, hidden=512, vocab=1000, dtype=dtype)
    wl.problem = synth.make_problem("long", 8, vocab=1000)
    wl.inputs = synth.logical_inputs(wl.problem, True)
    assert int(wl.problem.content_len.max()) == 4096 and int(wl.problem.q_len.max()) == 256
    return wl


@pytest.mark.parametrize("dtype,hq,hkv", [("bf16", 8, 2), ("bf16", 8, 8), ("fp8", 8, 2), ("f32", 4, 2)])
def test_limits_parity_and_invariance(dtype, hq, hkv):
    wl = _long_wl(dtype, hq, hkv)
    W, Wh = lm_head(wl)
    cache = {}
    say(f"case: 4096-token content, 100-256-token templates, dtype={dtype} hq={hq} hkv={hkv}, sharp")
    packed = Case(wl, 16384, peaked=True, sharp=True, cache=cache)
    packed.run(W)
    assert packed.plan.n_passes == 1
    rng = np.random.default_rng(8)
    n_in = wl.problem.n_inputs
    ea = check_attention(packed, inputs=[0, 1, 2, n_in + 2], branches_per_input=3, rng=rng, guard=True)
    keys = [(n, q) for n in range(n_in) for q in packed.prob.questions_of(n)]
    guards = [oracle_scores(packed, Wh, keys, wrong=w) for w in ("flat", "neighbour")]
    es = check_scores(packed, oracle_scores(packed, Wh, keys), guards)
    say(f"  attention rel err {ea:.2e}; scores {es}")
    P = _by_input(packed)
    packed.job = None
    # content + the longest branch fits 4,608 tokens: the 4,096-token input
    # spills over several passes, its content re-staged in each
    spilled = Case(wl, 4608, inputs=[2, 0, 1], peaked=True, sharp=True, cache=cache)
    spilled.run(W)
    assert spilled.plan.n_passes >= 4
    S = _by_input(spilled)
    for i in range(n_in):
        _same(P[i], S[i], f"input {i} spilled at 4608")
    spilled.job = None
    for i in range(n_in):
        alone = Case(wl, 16384, inputs=[i], peaked=True, sharp=True, cache=cache)
        alone.run(W)
        _same(P[i], _by_input(alone)[i], f"input {i} alone")
        alone.job = None


def test_plan_upload_device_path():
    # spb_plan_upload copies a pass's metadata into a device buffer on the
    # caller's stream: the bytes equal the staged copy, and attention and
    # scoring run from it give the engine loop's bits
    import torch
    import shared_prefix_branch_amd as spb
    wl = _long_wl("bf16")
    W, _ = lm_head(wl)
    case = Case(wl, 4608, peaked=True, sharp=True)
    case.run(W)
    job = case.job
    stream = torch.cuda.Stream()
    for k, buf in enumerate(job.passes):
        say(f"case: plan upload, pass {k} of {case.plan.n_passes}")
        d_meta = torch.full_like(buf.meta, 0x5A)
        case.plan.upload(k, d_meta, stream=stream)
        stream.synchronize()
        assert torch.equal(d_meta.cpu(), buf.meta.cpu()), f"pass {k}: uploaded metadata differs"
        o = torch.empty_like(buf.o)
        lp, p, res = torch.empty_like(buf.lp), torch.empty_like(buf.p), torch.empty_like(buf.residual)
        ws = torch.empty_like(buf.workspace)
        with torch.cuda.stream(stream):
            spb.branch_attention(case.plan, k, d_meta, buf.q, buf.k, buf.v, o, stream=stream)
            spb.score_options(case.plan, k, d_meta, buf.hidden, W, ws, lp, p, res, stream=stream)
        stream.synchronize()
        assert torch.equal(o.view(torch.int16), buf.o.view(torch.int16)), f"pass {k}: attention differs"
        for a, b, f in ((lp, buf.lp, "lp"), (p, buf.p, "p"), (res, buf.residual, "residual")):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"pass {k}: {f} differs"
    # a buffer smaller than the pass's metadata is refused before any copy
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(spb.SpbError):
        case.plan.upload(0, small, stream=stream)


def test_attention_q_rows_past_4gib():
    # one pass of 625,505 rows at 32 query heads x 128 (bf16): Q rows from
    # 524,288 on start more than 2^32 bytes into Q, K and V stay under 4 GiB.
    # Inputs at the start, across that row and at the end (the floors are
    # packed last) against the oracle, sharp scores with the guard.
    wl = synth.make_workload("news", hq=32, hkv=8, head_dim=128, hidden=128, vocab=1000)
    wl.problem = synth.make_problem("random", 41, vocab=1000, n_inputs=1100, n_questions=6, min_content=420,
                                    max_content=560, max_len=30, max_options=4, max_option_tokens=3)
    wl.inputs = synth.logical_inputs(wl.problem, True)
    say("case: one pass of 625,505 rows, Q over 4 GiB, bf16 hq=32 hkv=8, sharp")
    case = Case(wl, 800000, peaked=True, sharp=True)
    assert case.plan.n_passes == 1
    n_tok = case.plan.info(0)["n_tokens"]
    assert n_tok * 32 * 128 * 2 > 2 ** 32 + 2 ** 28
    lr, _ = case.plan.rows(0)
    off, _ = case.plan.inputs()

    def pass_rows(n):
        return np.nonzero((lr >= off[n]) & (lr < off[n + 1]))[0]

    n_in = wl.problem.n_inputs
    across = next(n for n in range(n_in) if pass_rows(n).min() <= 524288 <= pass_rows(n).max())
    inputs = [0, across, n_in - 2, n_in - 1, n_in + 1]
    assert all(pass_rows(n).min() > 524288 for n in inputs[2:])
    W, _ = lm_head(wl)
    case.run(W)
    ea = check_attention(case, inputs=inputs, branches_per_input=2, rng=np.random.default_rng(41), guard=True)
    say(f"  inputs {inputs}: attention rel err {ea:.2e}")
