"""CPU tests of the packer on template token tries: questions of one input
whose templates share prefixes hold those tokens once (spinf-serve pages,
"Template tries" and "Packed forward").  The plan's placement, the keys each
row attends to, and the attention work items are checked against the oracle's
layout; no kernel runs here."""
import numpy as np
import pytest

import shared_prefix_branch_amd as spb
import synth
from oracle import tree as OT
from test_host_plan import _check_plan, _meta_arrays

STEM_CHUNK = 1 << 30


def _shared(seed, **over):
    kw = dict(vocab=64, n_inputs=3, n_questions=6, max_content=12, tail_vocab=3, max_options=3,
              max_option_tokens=3)
    kw.update(over)
    return synth.make_problem("random_shared", seed, **kw)


def _check_visibility(prob, plan, lay):
    for k in range(plan.n_passes):
        lr, _ = plan.rows(k)
        for x in range(len(lr)):
            keys = plan.visible(k, x)
            assert len(set(keys)) == len(keys)
            assert sorted(lr[keys].tolist()) == sorted(OT.root_path(lay, int(lr[x])))


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("budget", [24, 40, 200, 16384])
def test_shared_plan_places_rows_and_visibility_equals_root_paths(seed, budget):
    prob = _shared(400 + seed)
    try:
        plan = spb.pack_pass(prob, token_budget=budget)
    except spb.SpbError as e:
        assert e.code == -2  # content + one branch larger than the budget
        return
    lay = _check_plan(prob, plan, budget)
    _check_visibility(prob, plan, lay)


def test_shared_tokens_are_packed_once_and_pairs_follow_the_tree():
    n_shared = 0
    for seed in range(6):
        prob = _shared(500 + seed)
        plan = spb.pack_pass(prob, token_budget=16384)
        lay = OT.build_layout(prob, floors=True)
        inf = plan.info()
        assert inf["n_passes"] == 1
        assert inf["n_tokens"] == lay.n_rows
        assert inf["unmasked_pairs"] == sum(len(OT.root_path(lay, x)) for x in range(lay.n_rows))
        unshared = spb.pack_pass(synth.Problem(**{**prob.__dict__, "tmpl_tok": None}), token_budget=16384)
        n_shared += unshared.info()["n_tokens"] - inf["n_tokens"]
    assert n_shared > 0


def test_distinct_templates_give_the_unshared_plan_byte_for_byte():
    # template ids whose first tokens all differ share nothing: the metadata
    # equals that of a plan packed without template ids
    prob = synth.make_problem("random", 31, vocab=64, n_inputs=4, n_questions=5, max_content=20,
                              max_len=6, max_options=3, max_option_tokens=3)
    tmpl = np.concatenate([np.full(int(L), q, np.int32) for q, L in enumerate(prob.q_len)])
    with_ids = spb.pack_pass(synth.Problem(**{**prob.__dict__, "tmpl_tok": tmpl}), token_budget=64)
    without = spb.pack_pass(prob, token_budget=64)
    assert with_ids.n_passes == without.n_passes
    for k in range(without.n_passes):
        a = np.zeros(without.info(k)["meta_bytes"], np.uint8)
        b = np.zeros(with_ids.info(k)["meta_bytes"], np.uint8)
        without.meta_copy(k, a)
        with_ids.meta_copy(k, b)
        assert a.tobytes() == b.tobytes()


def test_grid_templates_share_lead_ins_and_fillings():
    prob = synth.make_problem("grid", 6, vocab=4096, n_inputs=2, n_templates=2, min_content=30, max_content=50)
    plan = spb.pack_pass(prob, token_budget=16384)
    lay = _check_plan(prob, plan, 16384)
    _check_visibility(prob, plan, lay)
    unshared = spb.pack_pass(synth.Problem(**{**prob.__dict__, "tmpl_tok": None}), token_budget=16384)
    assert plan.info()["n_tokens"] < 0.7 * unshared.info()["n_tokens"]


def test_spill_restages_the_stems_a_pass_needs():
    prob = synth.make_problem("grid", 6, vocab=4096, n_inputs=1, n_templates=2, min_content=30, max_content=50)
    budget = 160
    plan = spb.pack_pass(prob, token_budget=budget)
    assert plan.n_passes > 1
    lay = _check_plan(prob, plan, budget)
    _check_visibility(prob, plan, lay)


def _branch_keys(r, ep):
    # template rows see the template causally; trie nodes the whole template
    # and their own trie ancestors
    e, L, depth = int(r[3]), int(r[4]), int(r[5])
    if e < L:
        return ep <= e
    if ep < L:
        return True
    a = [int(r[6]) & 0xFFFF, (int(r[6]) >> 16) & 0xFFFF, int(r[7]) & 0xFFFF, (int(r[7]) >> 16) & 0xFFFF]
    return ep in a[:depth]


def _item_keys(r, seg, ncc, chunks):
    """Keys a row reaches by walking an item's chunk list the way the bf16
    attention kernel does: content chunks, then stem and branch chunks."""
    keys = [seg + j for j in range(min(int(r[0]), 64 * ncc))]
    for key0, info, pre, post_nvis in chunks:
        c = info & 1023
        lo = key0 - 32 * c
        if info & STEM_CHUNK:
            post, nvis = post_nvis & 0xFFFFFF, post_nvis >> 24
            own = int(r[2]) == lo
            anc = pre <= int(r[8]) < post and not own
            thr = min(max(int(r[3]) + 1 - 32 * c, 0), nvis) if own else (nvis if anc else 0)
            keys += [key0 + j for j in range(thr)]
        elif int(r[2]) == lo:
            keys += [key0 + j for j in range(32) if _branch_keys(r, 32 * c + j)]
    return keys


@pytest.mark.parametrize("budget", [40, 16384])
def test_work_item_chunk_lists_reach_exactly_the_visible_keys(budget):
    for prob in [_shared(600), _shared(601, n_inputs=2, max_content=80),
                 synth.make_problem("grid", 6, vocab=4096, n_inputs=1, n_templates=1, min_content=60,
                                    max_content=80)]:
        try:
            plan = spb.pack_pass(prob, token_budget=budget)
        except spb.SpbError as e:
            assert e.code == -2
            continue
        for k in range(plan.n_passes):
            buf = np.zeros(plan.info(k)["meta_bytes"], np.uint8)
            plan.meta_copy(k, buf)
            n, rows, br, items, bchunks = _meta_arrays(buf)
            for g in range(3):
                seen = np.zeros(n, np.int32)
                for it in items[g]:
                    row0, nrows, seg, ncc, boff, bn, cost = (int(v) for v in it[:7])
                    seen[row0:row0 + nrows] += 1
                    chunks = [tuple(int(v) for v in c) for c in bchunks[boff:boff + bn]]
                    pres = [c[2] for c in chunks if c[1] & STEM_CHUNK]
                    assert pres == sorted(pres)  # stems root first
                    for x in range(row0, row0 + nrows):
                        got = _item_keys(rows[x], seg, ncc, chunks)
                        assert len(got) == len(set(got))
                        assert sorted(got) == sorted(plan.visible(k, x)), (k, g, x)
                assert (seen == 1).all()
