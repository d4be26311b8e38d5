"""Pins of the float64 oracle against what the pages and the mathematics fix.

Each check here would fail under a plausible mistake in the oracle (dropped
term, wrong sign, wrong index, transposed operand, wrong head mapping); the
planted-mistake tests at the bottom show that for several of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import numerics as ON
from oracle import scoring as OS
from oracle import tree as OT
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- worked example

def test_worked_example_p_residual():
    g = json.load(open(os.path.join(GOLDEN, "worked_example_refund.json")))
    lp = np.asarray(g["logprob"])
    p = OS.renormalise(lp)
    r = OS.residual(lp)
    nd = g["printed_decimals"]
    assert np.allclose(np.round(p, nd), g["p"], atol=1e-12)
    assert round(r, nd) == pytest.approx(g["residual"], abs=1e-12)
    # p_total + residual = 1 (the options' vocab-wide mass plus the rest)
    assert np.exp(lp).sum() + r == pytest.approx(1.0, abs=1e-15)
    # the printed floor is itself a distribution over the two options
    assert sum(g["floor_p"]) == pytest.approx(1.0, abs=1e-12)


def test_worked_example_rounding_box():
    # every logprob pair that prints as (-0.90, -1.86) gives p and residual
    # within about one printed unit of the printed (0.72, 0.28) and 0.44
    g = json.load(open(os.path.join(GOLDEN, "worked_example_refund.json")))
    for a in np.linspace(-0.905, -0.895, 5):
        for b in np.linspace(-1.865, -1.855, 5):
            lp = np.array([a, b])
            assert np.all(np.abs(OS.renormalise(lp) - g["p"]) <= 0.0055)
            assert abs(OS.residual(lp) - g["residual"]) <= 0.0055


def test_worked_example_lift():
    g = json.load(open(os.path.join(GOLDEN, "worked_example_refund.json")))
    # lift through join_floors on a one-question problem and its floor
    prob = synth.Problem(np.array([3], np.int32), np.array([0, 1], np.int32), np.array([0], np.int32),
                         np.array([2], np.int32), np.array([0, 2], np.int32), np.array([0, 1, 2], np.int32),
                         np.array([5, 6], np.int32), 8)
    lay = OT.build_layout(prob, floors=True)
    sc = {(0, 0): OS.BranchScores(np.log(g["p"]), np.array(g["p"]), 0.0),
          (1, 0): OS.BranchScores(np.log(g["floor_p"]), np.array(g["floor_p"]), 0.0)}
    OS.join_floors(lay, sc)
    assert np.allclose(sc[(0, 0)].floor_p, g["floor_p"])
    assert np.allclose(sc[(0, 0)].lift, np.array(g["p"]) - np.array(g["floor_p"]))
    assert sc[(0, 0)].lift.sum() == pytest.approx(0.0, abs=1e-12)
    # the " billing" example: floor 0.47 -> 0.91 is a lift of 0.44
    assert g["topic_billing_p"] - g["topic_billing_floor_p"] == pytest.approx(0.44)


# ----------------------------------------------------------------------------- numerics

def test_e4m3_table_against_definition_points_and_torch():
    T = ON.E4M3_TABLE
    assert T[0x7E] == 448.0 and T[0xFE] == -448.0          # largest finite
    assert T[0x38] == 1.0                                   # exponent field 7 = 2^0
    assert T[0x08] == 2.0 ** -6                             # smallest normal
    assert T[0x01] == 2.0 ** -9                             # smallest subnormal
    assert T[0x07] == 7 * 2.0 ** -9                         # largest subnormal
    assert math.isnan(T[0x7F]) and math.isnan(T[0xFF])
    assert T[0x80] == 0.0 and math.copysign(1, T[0x80]) == -1
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    both_nan = np.isnan(ref) & np.isnan(T)
    assert np.array_equal(ref[~both_nan], T[~both_nan])
    assert np.array_equal(np.isnan(ref), np.isnan(T))


def test_bf16_decode_exact():
    x = torch.randn(4096, dtype=torch.float32).to(torch.bfloat16)
    assert np.array_equal(ON.to_f64(x), x.double().numpy())


def test_round_to_bf16_matches_torch_with_ties():
    # random f32 values plus exact midpoints between neighbouring bf16 values
    # (representable in f32), which must go to the even significand
    rng = np.random.default_rng(5)
    x = rng.normal(size=4096).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 4096).astype(np.float32)
    b = torch.from_numpy(rng.normal(size=2048).astype(np.float32)).to(torch.bfloat16).float().numpy()
    ulp = np.ldexp(1.0, np.frexp(b.astype(np.float64))[1] - 8)
    mid = (b.astype(np.float64) + ulp / 2).astype(np.float32)  # exact in f32
    x = np.concatenate([x, mid, np.float32([0.0, -0.0, 2.0 ** -130, -(2.0 ** -140)])])
    want = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(ON.round_to_bf16(x.astype(np.float64)), want)
    # by hand: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> 1 (even);
    # 1 + 3 2^-8 halfway between 1 + 2^-7 and 1 + 2^-6 -> 1 + 2^-6 (even)
    assert ON.round_to_bf16(1 + 2.0 ** -8) == 1.0
    assert ON.round_to_bf16(1 + 3 * 2.0 ** -8) == 1 + 2.0 ** -6


# ----------------------------------------------------------------------------- scoring closed forms

def test_bf16_lm_head_rounds_the_logits():
    # vocabulary of 3, hidden size 1, h = 1: the logits are W itself.
    # z0 = 1 + 2^-9 is not a bf16 value and rounds to 1.
    prob, lay = _layout_one_branch(0, 1, [(0,), (1,)], 3)
    W = np.array([[1 + 2.0 ** -9], [0.5], [-1.0]])
    hid = np.ones((lay.n_rows, 1))
    def by_hand(z):
        lse = math.log(sum(math.exp(v) for v in z))
        return [z[0] - lse, z[1] - lse]
    for kind, z in (("f32out", [1 + 2.0 ** -9, 0.5, -1.0]), ("fp32", [1 + 2.0 ** -9, 0.5, -1.0]),
                    ("bf16", [1.0, 0.5, -1.0])):
        sc = OS.score_branches(lay, lambda rows: hid[rows], W, lm_head=kind)[(0, 0)]
        assert np.allclose(sc.lp, by_hand(z), rtol=0, atol=1e-15), kind
        e = np.exp(by_hand(z))
        assert np.allclose(sc.p, e / e.sum(), rtol=0, atol=1e-15)
        assert sc.residual == pytest.approx(1 - e.sum(), abs=1e-15)
    with pytest.raises(ValueError):
        OS.score_branches(lay, lambda rows: hid[rows], W, lm_head="f16")


def _layout_one_branch(C, L, options, vocab, floors=False):
    opts_flat = [t for o in options for t in o]
    tok_off = np.concatenate([[0], np.cumsum([len(o) for o in options])]).astype(np.int32)
    prob = synth.Problem(np.array([C], np.int32), np.array([0, 1], np.int32), np.array([0], np.int32),
                         np.array([L], np.int32), np.array([0, len(options)], np.int32), tok_off,
                         np.array(opts_flat, np.int32), vocab)
    return prob, OT.build_layout(prob, floors=floors)


def test_whole_vocab_options_is_softmax():
    V, H = 16, 8
    rng = np.random.default_rng(0)
    prob, lay = _layout_one_branch(3, 4, [(t,) for t in range(V)], V)
    W = rng.normal(size=(V, H))
    hid = rng.normal(size=(lay.n_rows, H))
    sc = OS.score_branches(lay, lambda rows: hid[rows], W)[(0, 0)]
    b = lay.inputs[0].branches[0]
    z = torch.from_numpy(W @ hid[b.last_row])
    assert abs(sc.residual) < 1e-13
    assert np.allclose(sc.p, torch.softmax(z, 0).numpy(), atol=1e-14)
    assert np.allclose(sc.lp, torch.log_softmax(z, 0).numpy(), atol=1e-13)


def test_single_option_has_p_one():
    V, H = 32, 8
    rng = np.random.default_rng(1)
    prob, lay = _layout_one_branch(2, 3, [(7, 3)], V)
    W = rng.normal(size=(V, H))
    hid = rng.normal(size=(lay.n_rows, H))
    sc = OS.score_branches(lay, lambda rows: hid[rows], W)[(0, 0)]
    assert sc.p[0] == 1.0
    assert sc.residual == pytest.approx(1 - math.exp(sc.lp[0]), abs=1e-15)


def test_chain_rule_complete_two_token_set():
    # all 64 two-token sequences over an 8-token vocabulary: prefix-free and
    # complete, so their probabilities sum to one and p(a,b) = P(a) P(b|a)
    V, H = 8, 5
    rng = np.random.default_rng(2)
    opts = [(a, b) for a in range(V) for b in range(V)]
    prob, lay = _layout_one_branch(4, 3, opts, V)
    W = rng.normal(size=(V, H))
    hid = rng.normal(size=(lay.n_rows, H))
    sc = OS.score_branches(lay, lambda rows: hid[rows], W)[(0, 0)]
    b = lay.inputs[0].branches[0]
    assert len(b.trie.prefixes) == V
    assert abs(sc.residual) < 1e-13
    P0 = torch.softmax(torch.from_numpy(W @ hid[b.last_row]), 0).numpy()
    for i, (a, c) in enumerate(opts):
        node_row = b.node_row0 + b.trie.index[(a,)]
        Pa = torch.softmax(torch.from_numpy(W @ hid[node_row]), 0).numpy()
        assert sc.p[i] == pytest.approx(P0[a] * Pa[c], rel=1e-12)
        assert sc.lp[i] == pytest.approx(math.log(P0[a] * Pa[c]), abs=1e-12)


def test_trie_sharing_and_order():
    opts = [(5, 1, 2), (5, 1, 3), (5, 4), (9,)]
    # proper prefixes only: (5, 4) and (9,) are leaves, so the nodes are (5,), (5, 1)
    tr = OT.build_trie(opts)
    assert tr.prefixes == [(5,), (5, 1)]
    assert tr.chains[0] == [(-1, 5), (0, 1), (1, 2)]
    assert tr.chains[2] == [(-1, 5), (0, 4)]
    assert tr.chains[3] == [(-1, 9)]


# ----------------------------------------------------------------------------- attention special cases

def _sdpa_causal(q, k, v):
    """torch's CPU scaled_dot_product_attention, causal, float64, GQA by repeat."""
    g = q.shape[1] // k.shape[1]
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(k).repeat_interleave(g, dim=1).permute(1, 0, 2)
    vt = torch.from_numpy(v).repeat_interleave(g, dim=1).permute(1, 0, 2)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True).permute(1, 0, 2).numpy()


@pytest.mark.parametrize("C", [0, 9])
def test_one_branch_is_causal_sdpa(C):
    rng = np.random.default_rng(3 + C)
    prob, lay = _layout_one_branch(C, 7, [(1,), (2,)], 16)
    n = lay.n_rows
    q = rng.normal(size=(n, 4, 8)); k = rng.normal(size=(n, 2, 8)); v = rng.normal(size=(n, 2, 8))
    out = OA.attention_input(lay, lay.inputs[0], q, k, v)
    ref = _sdpa_causal(q, k, v)
    assert np.allclose(out, ref, atol=1e-12)


def test_option_chain_is_causal_sdpa():
    # a branch with one 4-token option: its 3 trie nodes continue the sequence
    rng = np.random.default_rng(5)
    prob, lay = _layout_one_branch(6, 5, [(3, 4, 5, 6)], 16)
    n = lay.n_rows
    assert n == 6 + 5 + 3
    q = rng.normal(size=(n, 4, 8)); k = rng.normal(size=(n, 2, 8)); v = rng.normal(size=(n, 2, 8))
    out = OA.attention_input(lay, lay.inputs[0], q, k, v)
    assert np.allclose(out, _sdpa_causal(q, k, v), atol=1e-12)


def test_branches_do_not_see_each_other_and_match_separate_prompts():
    # "the same answers" as separate prompts: branch b of a packed input equals
    # causal attention over content + template b run on its own
    prob = synth.make_problem("random", 5, vocab=32)
    lay = OT.build_layout(prob, floors=True)
    rng = np.random.default_rng(7)
    n = lay.n_rows
    q = rng.normal(size=(n, 4, 8)); k = rng.normal(size=(n, 2, 8)); v = rng.normal(size=(n, 2, 8))
    for li in lay.inputs:
        lo = li.first_row
        hi = lo + int((lay.row_input == lay.row_input[lo]).sum())
        out = OA.attention_input(lay, li, q[lo:hi], k[lo:hi], v[lo:hi])
        for b in li.branches:
            seq = np.r_[lo:lo + li.C, b.first_row:b.first_row + b.L]
            ref = _sdpa_causal(q[seq], k[seq], v[seq])[li.C:]
            assert np.allclose(out[b.first_row - lo:b.first_row - lo + b.L], ref, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_per_sequence_equals_dense_mask(seed):
    prob = synth.make_problem("random", 100 + seed, vocab=16, n_inputs=3, n_questions=4,
                              max_content=10, max_len=5, max_options=4, max_option_tokens=4)
    lay = OT.build_layout(prob, floors=True)
    rng = np.random.default_rng(seed)
    n = lay.n_rows
    q = rng.normal(size=(n, 4, 8)); k = rng.normal(size=(n, 2, 8)); v = rng.normal(size=(n, 2, 8))
    dense = OA.attention_dense(lay, q, k, v)
    for li in lay.inputs:
        lo = li.first_row
        hi = lo + int((lay.row_input == lay.row_input[lo]).sum())
        per = OA.attention_input(lay, li, q[lo:hi], k[lo:hi], v[lo:hi])
        assert np.allclose(per, dense[lo:hi], atol=1e-12)


def _shared_problem(seed, **kw):
    args = dict(vocab=16, n_inputs=3, n_questions=6, max_content=8, max_lead=4, tail_vocab=4,
                max_options=3, max_option_tokens=3)
    args.update(kw)
    return synth.make_problem("random_shared", seed, **args)


def test_shared_template_layout_by_hand():
    # one input (C = 2) asking (1,2,3), (1,2,4), (1,5), (6,): the proper prefixes
    # (1) [3 questions] and (1,2) [2 questions] are shared; last tokens never
    prob = synth.Problem(np.array([2], np.int32), np.array([0, 4], np.int32), np.array([0, 1, 2, 3], np.int32),
                         np.array([3, 3, 2, 1], np.int32), np.arange(5, dtype=np.int32),
                         np.arange(5, dtype=np.int32), np.array([7, 8, 9, 10], np.int32), 16,
                         np.array([1, 2, 3, 1, 2, 4, 1, 5, 6], np.int32))
    lay = OT.build_layout(prob, floors=False)
    # rows: content 0,1 | (1) 2, (1,2) 3, q0 own "3" 4 | q1 own "4" 5 | q2 own "5" 6 | q3 own "6" 7
    assert lay.n_rows == 8
    assert lay.parent.tolist() == [-1, 0, 1, 2, 3, 3, 2, 1]
    b = lay.inputs[0].branches
    assert [x.template_rows for x in b] == [[2, 3, 4], [2, 3, 5], [2, 6], [7]]
    assert [x.last_row for x in b] == [4, 5, 6, 7]
    assert lay.row_branch.tolist() == [-1, -1, -1, -1, 0, 1, 2, 3]
    M = OA.dense_mask(lay)
    assert np.nonzero(M[4])[0].tolist() == [0, 1, 2, 3, 4]
    assert np.nonzero(M[6])[0].tolist() == [0, 1, 2, 6]
    assert np.nonzero(M[7])[0].tolist() == [0, 1, 7]
    # a template that is a proper prefix of two others keeps its last token:
    # (1,2) alone; (1,2,3) and (1,2,4) share (1) and (1,2)
    prob2 = synth.Problem(np.array([0], np.int32), np.array([0, 3], np.int32), np.array([0, 1, 2], np.int32),
                          np.array([2, 3, 3], np.int32), np.arange(4, dtype=np.int32),
                          np.arange(4, dtype=np.int32), np.array([7, 8, 9], np.int32), 16,
                          np.array([1, 2, 1, 2, 3, 1, 2, 4], np.int32))
    lay2 = OT.build_layout(prob2, floors=False)
    b2 = lay2.inputs[0].branches
    assert [x.template_rows for x in b2] == [[0, 1], [0, 2, 3], [0, 2, 4]]
    M2 = OA.dense_mask(lay2)
    assert np.nonzero(M2[1])[0].tolist() == [0, 1]        # q0's last token does not see (1,2)
    for x in range(lay2.n_rows):
        assert set(np.nonzero(M2[x])[0].tolist()) == set(OT.root_path(lay2, x))


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_shared_templates_per_sequence_equals_dense_mask(seed):
    prob = _shared_problem(200 + seed)
    lay = OT.build_layout(prob, floors=True)
    assert any(b.stem_rows for b in lay.branches())
    M = OA.dense_mask(lay)
    for x in range(lay.n_rows):
        assert set(np.nonzero(M[x])[0].tolist()) == set(OT.root_path(lay, x))
    rng = np.random.default_rng(seed)
    n = lay.n_rows
    q = rng.normal(size=(n, 4, 8)); k = rng.normal(size=(n, 2, 8)); v = rng.normal(size=(n, 2, 8))
    dense = OA.attention_dense(lay, q, k, v, mask=M)
    for li in lay.inputs:
        lo = li.first_row
        hi = lo + int((lay.row_input == lay.row_input[lo]).sum())
        per = OA.attention_input(lay, li, q[lo:hi], k[lo:hi], v[lo:hi])
        assert np.allclose(per, dense[lo:hi], atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_sharing_template_tokens_only_packs_them_once(seed):
    # the same problem without template token ids gives every question its own
    # copy of its template; copies that carry the shared tokens' activations give
    # the same attention rows and the same scores
    prob = _shared_problem(300 + seed)
    unshared = synth.Problem(prob.content_len, prob.branch_off, prob.branch_q, prob.q_len, prob.opt_off,
                             prob.tok_off, prob.tok, prob.vocab)
    S = OT.build_layout(prob, floors=True)
    U = OT.build_layout(unshared, floors=True)
    assert S.n_rows < U.n_rows
    # U row -> S row carrying the same token
    to_s = np.empty(U.n_rows, np.int64)
    for ls, lu in zip(S.inputs, U.inputs):
        for t in range(lu.C):
            to_s[lu.first_row + t] = ls.first_row + t
        for bs, bu in zip(ls.branches, lu.branches):
            assert bu.L == len(bs.template_rows)
            to_s[bu.first_row:bu.first_row + bu.L] = bs.template_rows
            nn = len(bu.trie.prefixes)
            to_s[bu.node_row0:bu.node_row0 + nn] = np.arange(bs.node_row0, bs.node_row0 + nn)
    rng = np.random.default_rng(seed)
    n, H = S.n_rows, 6
    q = rng.normal(size=(n, 4, 8)); k = rng.normal(size=(n, 2, 8)); v = rng.normal(size=(n, 2, 8))
    hid = rng.normal(size=(n, H)); W = rng.normal(size=(prob.vocab, H))

    def att(lay, q, k, v):
        out = []
        for li in lay.inputs:
            lo = li.first_row
            hi = lo + int((lay.row_input == lay.row_input[lo]).sum())
            out.append(OA.attention_input(lay, li, q[lo:hi], k[lo:hi], v[lo:hi]))
        return np.concatenate(out)

    a_s = att(S, q, k, v)
    a_u = att(U, q[to_s], k[to_s], v[to_s])
    assert np.allclose(a_u, a_s[to_s], atol=1e-12)
    sc_s = OS.score_branches(S, lambda rows: hid[rows], W)
    sc_u = OS.score_branches(U, lambda rows: hid[to_s[rows]], W)
    for key in sc_u:
        assert np.allclose(sc_u[key].lp, sc_s[key].lp, atol=1e-12)
        assert np.allclose(sc_u[key].p, sc_s[key].p, atol=1e-12)


def test_dense_mask_matches_root_paths():
    prob = synth.make_problem("random", 7, vocab=8, n_inputs=2, n_questions=3, max_content=6,
                              max_len=4, max_options=4, max_option_tokens=4)
    lay = OT.build_layout(prob, floors=True)
    M = OA.dense_mask(lay)
    for x in range(lay.n_rows):
        assert set(np.nonzero(M[x])[0].tolist()) == set(OT.root_path(lay, x))


# ----------------------------------------------------------------------------- brute force

def _brute(prob, floors, q, k, v, hid, W, scale):
    """Pure-Python loops: every prompt materialised as an explicit token list."""
    # rebuild the logical rows from the problem without the tree module
    rows = []      # (input_no, kind, payload)
    prompts = {}   # row -> list of rows it attends to (its own prompt)
    n_in = len(prob.content_len)
    plan = [(int(prob.content_len[i]), [int(x) for x in prob.branch_q[prob.branch_off[i]:prob.branch_off[i + 1]]])
            for i in range(n_in)]
    if floors:
        plan += [(0, [qq]) for qq in sorted(set(int(x) for x in prob.branch_q))]
    scored = {}    # (input_no, question) -> (template_last_row, {prefix: row}, options)
    r = 0
    for n, (C, qs) in enumerate(plan):
        content = list(range(r, r + C))
        for t in range(C):
            prompts[r + t] = content[:t + 1]
        r += C
        for qq in qs:
            L = int(prob.q_len[qq])
            tmpl = list(range(r, r + L))
            for j in range(L):
                prompts[r + j] = content + tmpl[:j + 1]
            r += L
            opts = []
            for o in range(int(prob.opt_off[qq]), int(prob.opt_off[qq + 1])):
                opts.append(tuple(int(t) for t in prob.tok[prob.tok_off[o]:prob.tok_off[o + 1]]))
            node_row = {}
            for o in opts:
                for kk in range(1, len(o)):
                    pre = o[:kk]
                    if pre not in node_row:
                        node_row[pre] = r
                        r += 1
            for pre, row in node_row.items():
                prompts[row] = content + tmpl + [node_row[pre[:j]] for j in range(1, len(pre) + 1)]
            scored[(n, qq)] = (tmpl[-1], node_row, opts)
    N = r
    hq, d = q.shape[1], q.shape[2]
    g = hq // k.shape[1]
    att = np.zeros((N, hq, d))
    for x in range(N):
        keys = prompts[x]
        for h in range(hq):
            s = [sum(q[x, h, e] * k[y, h // g, e] for e in range(d)) * scale for y in keys]
            mx = max(s)
            w = [math.exp(si - mx) for si in s]
            tot = sum(w)
            for e in range(d):
                att[x, h, e] = sum(w[i] * v[keys[i], h // g, e] for i in range(len(keys))) / tot
    Vv = W.shape[0]

    def logsm(row, tok):
        z = [sum(W[t, e] * hid[row, e] for e in range(W.shape[1])) for t in range(Vv)]
        mx = max(z)
        return z[tok] - (mx + math.log(sum(math.exp(zz - mx) for zz in z)))

    res = {}
    for key, (last, node_row, opts) in scored.items():
        lps = []
        for o in opts:
            acc = 0.0
            for kk, tok in enumerate(o):
                src = last if kk == 0 else node_row[o[:kk]]
                acc += logsm(src, tok)
            lps.append(acc)
        tot = sum(math.exp(a) for a in lps)
        res[key] = (lps, [math.exp(a) / tot for a in lps], 1.0 - tot)
    return att, res


@pytest.mark.parametrize("seed", [11, 12])
def test_brute_force_tiny(seed):
    prob = synth.make_problem("random", seed, vocab=12, n_inputs=2, n_questions=3, max_content=5,
                              max_len=3, max_options=3, max_option_tokens=3)
    lay = OT.build_layout(prob, floors=True)
    assert lay.n_rows <= 48
    rng = np.random.default_rng(seed)
    n, H = lay.n_rows, 6
    q = rng.normal(size=(n, 2, 4)); k = rng.normal(size=(n, 1, 4)); v = rng.normal(size=(n, 1, 4))
    hid = rng.normal(size=(n, H)); W = rng.normal(size=(prob.vocab, H))
    scale = 0.5
    att_b, sc_b = _brute(prob, True, q, k, v, hid, W, scale)
    att = np.concatenate([
        OA.attention_input(lay, li, q[li.first_row:li.first_row + cnt], k[li.first_row:li.first_row + cnt],
                           v[li.first_row:li.first_row + cnt], scale=scale)
        for li, cnt in ((li, int((lay.row_input == lay.row_input[li.first_row]).sum()) if lay.n_rows else 0)
                        for li in lay.inputs)])
    assert np.allclose(att, att_b, atol=1e-12)
    sc = OS.score_branches(lay, lambda rows: hid[rows], W)
    assert set(sc) == set(sc_b)
    for key, (lps, ps, r) in sc_b.items():
        assert np.allclose(sc[key].lp, lps, atol=1e-12)
        assert np.allclose(sc[key].p, ps, atol=1e-12)
        assert sc[key].residual == pytest.approx(r, abs=1e-12)


def test_floor_equals_question_alone_on_empty_content():
    prob = synth.make_problem("random", 21, vocab=16, n_inputs=2, n_questions=3, max_content=6,
                              max_len=4, max_options=3, max_option_tokens=3)
    lay = OT.build_layout(prob, floors=True)
    rng = np.random.default_rng(21)
    H = 5
    hid = rng.normal(size=(lay.n_rows, H)); W = rng.normal(size=(16, H))
    sc = OS.score_branches(lay, lambda rows: hid[rows], W)
    OS.join_floors(lay, sc)
    for li in lay.inputs:
        if li.kind != "floor":
            continue
        qq = li.ident
        alone = synth.Problem(np.array([0], np.int32), np.array([0, 1], np.int32), np.array([qq], np.int32),
                              prob.q_len, prob.opt_off, prob.tok_off, prob.tok, prob.vocab)
        la = OT.build_layout(alone, floors=False)
        nrow = la.n_rows
        h_alone = hid[li.first_row:li.first_row + nrow]
        sa = OS.score_branches(la, lambda rows: h_alone[rows], W)[(0, qq)]
        for (n, q2), s in sc.items():
            if q2 == qq and lay.inputs[n].kind == "input":
                assert np.array_equal(s.floor_p, sa.p)
                assert np.allclose(s.lift, s.p - sa.p)


def test_invariants_on_random_problem():
    prob = synth.make_problem("random", 31, vocab=64, n_inputs=4, n_questions=5, max_content=8,
                              max_len=5, max_options=5, max_option_tokens=3)
    lay = OT.build_layout(prob, floors=True)
    rng = np.random.default_rng(31)
    H = 7
    hid = rng.normal(size=(lay.n_rows, H)); W = rng.normal(size=(64, H))
    sc = OS.score_branches(lay, lambda rows: hid[rows], W)
    for s in sc.values():
        assert s.p.sum() == pytest.approx(1.0, abs=1e-14)
        assert np.exp(s.lp).sum() + s.residual == pytest.approx(1.0, abs=1e-14)
        assert s.residual >= 0  # prefix-free options


# ----------------------------------------------------------------------------- planted mistakes

def test_planted_mistake_gqa_mapping_is_caught(monkeypatch):
    rng = np.random.default_rng(3)
    prob, lay = _layout_one_branch(5, 4, [(1,)], 8)
    n = lay.n_rows
    q = rng.normal(size=(n, 4, 8)); k = rng.normal(size=(n, 2, 8)); v = rng.normal(size=(n, 2, 8))
    ref = _sdpa_causal(q, k, v)
    orig = OA.causal_attention_tail

    def wrong(q_, k_, v_, scale):  # head h reads kv head h % Hkv instead of h // (Hq/Hkv)
        hkv = k_.shape[1]
        return np.concatenate([orig(q_[:, h:h + 1], k_[:, [h % hkv]], v_[:, [h % hkv]], scale)
                               for h in range(q_.shape[1])], axis=1)

    monkeypatch.setattr(OA, "causal_attention_tail", wrong)
    out = OA.attention_input(lay, lay.inputs[0], q, k, v)
    assert not np.allclose(out, ref, atol=1e-6)


def test_planted_mistake_residual_sign_is_caught(monkeypatch):
    g = json.load(open(os.path.join(GOLDEN, "worked_example_refund.json")))
    monkeypatch.setattr(OS, "residual", lambda lp: float(np.expm1(np.log(np.exp(lp).sum()))))
    assert round(OS.residual(np.asarray(g["logprob"])), 2) != g["residual"]


def test_planted_mistake_wrong_scoring_row_is_caught(monkeypatch):
    # scoring an option's first token from the first template row instead of the last
    V, H = 8, 5
    rng = np.random.default_rng(2)
    opts = [(a, b) for a in range(V) for b in range(V)]
    prob, lay = _layout_one_branch(4, 3, opts, V)
    W = rng.normal(size=(V, H)); hid = rng.normal(size=(lay.n_rows, H))
    monkeypatch.setattr(OT.LBranch, "last_row", property(lambda self: self.first_row))
    sc = OS.score_branches(lay, lambda rows: hid[rows], W)[(0, 0)]
    b = lay.inputs[0].branches[0]
    P0 = torch.softmax(torch.from_numpy(W @ hid[b.first_row + b.L - 1]), 0).numpy()
    Pa = torch.softmax(torch.from_numpy(W @ hid[b.node_row0 + b.trie.index[(0,)]]), 0).numpy()
    assert sc.p[0] != pytest.approx(P0[0] * Pa[0], rel=1e-6)
