"""The allocation-free head (spb_score_options_noalloc) against spb_score_options
through the C ABI: same plan, hidden rows and lm head, outputs equal bit for
bit, on two calls in a row, the second with a smaller pass (the shared scratch
then holds the first call's contents), and for every lm-head output kind."""
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import shared_prefix_branch_amd as spb
    spb.lib()


def _pass_inputs(prob, H, seed):
    import torch
    import shared_prefix_branch_amd as spb
    plan = spb.pack_pass(prob, token_budget=16384)
    assert plan.n_passes == 1
    inf = plan.info(0)
    meta = torch.empty(inf["meta_bytes"], dtype=torch.uint8, device="cuda")
    plan.upload(0, meta)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    hid = torch.randn((inf["n_tokens"], H), generator=g, device="cuda").to(torch.bfloat16)
    return plan, inf, meta, hid


def _outputs(inf):
    import torch
    return (torch.full((inf["n_options"],), float("nan"), device="cuda"),
            torch.full((inf["n_options"],), float("nan"), device="cuda"),
            torch.full((inf["n_branches"],), float("nan"), device="cuda"))


@pytest.mark.parametrize("kind", [0, 1, 2])
def test_noalloc_equals_workspace_head_two_calls(kind):
    import torch
    import shared_prefix_branch_amd as spb
    H, V = 512, 5000  # a vocabulary that ends in a partial 256-row slice
    big = synth.make_problem("random", 13, vocab=V, n_inputs=6, n_questions=8, min_content=20, max_content=200,
                             max_len=20, max_options=5, max_option_tokens=4)
    small = big.subset([1, 4])
    W = (torch.randn((V, H), generator=torch.Generator(device="cuda").manual_seed(7), device="cuda") * 0.05
         ).to(torch.bfloat16)
    sizes = []
    for n, (prob, seed) in enumerate(((big, 1), (small, 2))):
        plan, inf, meta, hid = _pass_inputs(prob, H, seed)
        sizes.append(inf["n_scored_rows"])
        print(f"case: no-alloc head, kind {kind}, call {n + 1}: {inf['n_scored_rows']} scored rows", flush=True)
        ws = torch.empty(spb.score_workspace_bytes(plan, 0, V, H, kind), dtype=torch.uint8, device="cuda")
        ref = _outputs(inf)
        spb.score_options(plan, 0, meta, hid, W, ws, *ref, lm_head_kind=kind)
        got = _outputs(inf)
        spb.score_options_noalloc(plan, 0, meta, hid, W, *got, lm_head_kind=kind)
        torch.cuda.synchronize()
        for a, b, f in zip(got, ref, ("lp", "p", "residual")):
            assert not torch.isnan(b).any(), f"reference {f} incomplete"
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"call {n + 1}: {f} differs"
    assert sizes[1] < sizes[0]
