"""CPU tests of libspb's host side: exports, the packer's plan, error paths,
the floor join.  No kernel runs here."""
import collections
import ctypes
import os
import re

import numpy as np
import pytest

import shared_prefix_branch_amd as spb
import synth
from oracle import tree as OT

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "spb.h")).read()
    declared = set(re.findall(r"\b(spb_[a-z_0-9]+)\s*\(", hdr))
    assert declared == set(spb.EXPORTED_SYMBOLS)
    L = spb.lib()
    for name in sorted(declared):
        assert hasattr(L, name), name
    assert spb.fingerprint().startswith("spb-")


def _placements(plan):
    out = []
    for k in range(plan.n_passes):
        lr, sr = plan.rows(k)
        out.append((lr, sr))
    return out


def _check_plan(prob, plan, budget, floors=True):
    lay = OT.build_layout(prob, floors=floors)
    seen = collections.Counter()
    # content and shared template rows may be re-staged in several passes
    restaged = set(np.nonzero((lay.row_kind == 0) | ((lay.row_kind == 1) & (lay.row_branch < 0)))[0].tolist())
    scored = set(OT.scored_rows(lay))
    for k in range(plan.n_passes):
        lr, sr = plan.rows(k)
        assert len(lr) <= budget
        assert len(set(lr.tolist())) == len(lr)          # no row twice in one pass
        seen.update(lr.tolist())
        # scored rows: the template's last row and every trie node
        want = sorted(x for x in range(len(lr)) if int(lr[x]) in scored)
        assert sorted(sr.tolist()) == want
    # every branch row exactly once; content rows at least once, and in every
    # pass that holds one of the input's branches
    for r in range(lay.n_rows):
        if r in restaged:
            assert seen[r] >= 1
        else:
            assert seen[r] == 1, r
    return lay


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("budget", [40, 64, 200, 16384])
def test_plan_places_every_row_and_visibility_equals_root_paths(seed, budget):
    prob = synth.make_problem("random", 200 + seed, vocab=32, n_inputs=4, n_questions=5, max_content=24,
                              max_len=6, max_options=4, max_option_tokens=5)
    try:
        plan = spb.pack_pass(prob, token_budget=budget)
    except spb.SpbError as e:
        assert e.code == -2  # content + one branch larger than the budget
        return
    lay = _check_plan(prob, plan, budget)
    for k in range(plan.n_passes):
        lr, _ = plan.rows(k)
        for x in range(len(lr)):
            keys = plan.visible(k, x)
            assert len(set(keys)) == len(keys)
            assert sorted(lr[keys].tolist()) == sorted(OT.root_path(lay, int(lr[x])))


def test_plan_counts_and_pairs():
    prob = synth.make_problem("random", 9, vocab=16, n_inputs=3, n_questions=4, max_content=12,
                              max_len=5, max_options=3, max_option_tokens=4)
    plan = spb.pack_pass(prob, token_budget=16384)
    lay = OT.build_layout(prob, floors=True)
    inf = plan.info()
    assert inf["n_tokens"] == lay.n_rows
    assert inf["unmasked_pairs"] == sum(len(OT.root_path(lay, x)) for x in range(lay.n_rows))
    assert inf["n_branches"] == sum(len(li.branches) for li in lay.inputs)
    assert inf["n_content_branches"] == len(prob.branch_q)
    assert inf["n_scored_rows"] == len(OT.scored_rows(lay))


def test_spill_restages_content():
    # extreme shape, scaled down: inputs larger than a pass spill at branch
    # boundaries with the content re-staged
    wl = synth.make_workload("extreme", n_questions=60, content=100)
    prob = wl.problem
    budget = 512
    plan = spb.pack_pass(prob, token_budget=budget)
    lay = _check_plan(prob, plan, budget)
    for k in range(plan.n_passes):
        lr, _ = plan.rows(k)
        ins = set(int(lay.row_input[r]) for r in lr if lay.row_kind[r] != 0)
        for i in ins:
            li = lay.inputs[i]
            c = set(range(li.first_row, li.first_row + li.C))
            assert c <= set(lr.tolist())      # the content is in every pass of the input
    assert plan.n_passes > 1


def test_news_two_pass_and_21x_token_saving():
    # the pages: 24 articles of ~470 tokens x 56 two-option questions pack into
    # two 16k passes, and the shared read saves ~21x the tokens of asking each
    # question with its own copy of the article
    wl = synth.make_workload("news2")
    prob = wl.problem
    plan = spb.pack_pass(prob, token_budget=16384)
    assert plan.n_passes == 2
    lay = OT.build_layout(prob, floors=False)
    shared = lay.n_rows
    separate = sum(int(prob.content_len[i]) + int(prob.q_len[q])
                   for i in range(prob.n_inputs) for q in prob.questions_of(i))
    assert 19.0 < separate / shared < 23.0
    # the configured news shape (templates 14-26 tokens) needs a third pass
    assert spb.pack_pass(synth.make_workload("news").problem).n_passes == 3


def test_floors_deduplicated_per_question():
    wl = synth.make_workload("fp8", n_inputs=30)
    plan = spb.pack_pass(wl.problem, token_budget=8192)
    asked = set(int(q) for q in wl.problem.branch_q)
    inf = plan.info()
    assert inf["n_branches"] == len(wl.problem.branch_q) + len(asked)


def _prob(**kw):
    base = dict(content_len=[3], branch_off=[0, 1], branch_q=[0], q_len=[2], opt_off=[0, 2],
                tok_off=[0, 1, 2], tok=[1, 2], vocab=8)
    base.update(kw)
    return synth.Problem(*(np.asarray(base[f], np.int32) for f in
                           ("content_len", "branch_off", "branch_q", "q_len", "opt_off", "tok_off", "tok")),
                         base["vocab"])


@pytest.mark.parametrize("kw,code", [
    (dict(tok=[1, 1]), -1),                                   # duplicate option
    (dict(tok=[1, 9]), -1),                                   # token id >= vocab
    (dict(branch_q=[3]), -1),                                 # question out of range
    (dict(branch_off=[0, 2]), -1),                            # CSR past the end of branch_q
    (dict(q_len=[0]), -1),                                    # empty template
    (dict(content_len=[-1]), -1),
    (dict(content_len=[5000]), -2),                           # max_content_tokens 4096
    (dict(q_len=[300]), -2),                                  # max_query_tokens 256
    (dict(tok_off=[0, 1, 8], tok=[1, 2, 3, 4, 5, 6, 7, 0]), -2),  # 6-token option > 5
])
def test_error_paths(kw, code):
    p = _prob(**kw)
    if kw.get("branch_off") == [0, 2]:
        p.branch_q = np.asarray([0, 7], np.int32)
    with pytest.raises(spb.SpbError) as e:
        spb.pack_pass(p)
    assert e.value.code == code
    assert spb.lib().spb_last_error().decode() != ""


def test_budget_too_small_and_processed_limit():
    with pytest.raises(spb.SpbError) as e:
        spb.pack_pass(_prob(), token_budget=4)   # content 3 + branch 2 > 4
    assert e.value.code == -2
    with pytest.raises(spb.SpbError) as e:
        spb.pack_pass(_prob(), max_processed_tokens=4)
    assert e.value.code == -2
    with pytest.raises(spb.SpbError) as e:
        spb.pack_pass(_prob(), max_options=1)
    assert e.value.code == -2


def test_unrunnable_attention_item_rejected_when_packed():
    # a raised content limit can make one attention work item's key-chunk list
    # longer than the kernel runs (320 chunks: 64-key content chunks plus
    # branch chunks); the packer refuses such a plan instead of handing out one
    # that fails after staging
    ok = spb.pack_pass(_prob(content_len=[20000]), token_budget=32768, max_content_tokens=30000)
    assert ok.n_passes == 1
    with pytest.raises(spb.SpbError) as e:
        spb.pack_pass(_prob(content_len=[20500]), token_budget=32768, max_content_tokens=30000)
    assert e.value.code == -2
    assert "key chunks" in spb.lib().spb_last_error().decode()


def test_kernel_entry_points_validate_before_any_hip_call():
    plan = spb.pack_pass(_prob())
    L = spb.lib()
    A = spb._AttnArgs()
    A.q = A.k = A.v = A.o = 256
    A.in_dtype, A.out_dtype, A.hq, A.hkv, A.head_dim, A.rows = spb.BF16, spb.BF16, 4, 2, 96, 1 << 20
    meta = ctypes.c_void_p(4096)
    assert L.spb_branch_attention(plan.handle, 0, meta, ctypes.byref(A), None) == -3   # head_dim
    A.head_dim = 128
    A.hq = 24; A.hkv = 3
    assert L.spb_branch_attention(plan.handle, 0, meta, ctypes.byref(A), None) == -3   # GQA 8
    A.hq, A.hkv = 4, 2
    A.rows = 2
    assert L.spb_branch_attention(plan.handle, 0, meta, ctypes.byref(A), None) == -4   # rows < n_tokens
    assert L.spb_branch_attention(plan.handle, 5, meta, ctypes.byref(A), None) == -1   # no such pass
    S = spb._ScoreArgs()
    S.hidden = S.lm_head = S.workspace = 256
    S.h_dtype, S.hidden_dim, S.rows, S.vocab, S.workspace_bytes = spb.BF16, 100, 1 << 20, 8, 1 << 20
    assert L.spb_score_options(plan.handle, 0, meta, ctypes.byref(S), None) == -3      # hidden % 64
    S.hidden_dim = 128
    S.vocab = 2
    assert L.spb_score_options(plan.handle, 0, meta, ctypes.byref(S), None) == -1      # token >= vocab
    S.vocab = 8
    S.workspace_bytes = 16
    assert L.spb_score_options(plan.handle, 0, meta, ctypes.byref(S), None) == -4      # workspace
    S.workspace_bytes = 1 << 30
    S.lm_head_kind = 3
    assert L.spb_score_options(plan.handle, 0, meta, ctypes.byref(S), None) == -1      # lm-head kind
    S.lm_head_kind = spb.HEAD_FP32
    need = spb.score_workspace_bytes(plan, 0, 8, 128, spb.HEAD_FP32)
    S.workspace_bytes = need - 1
    assert L.spb_score_options(plan.handle, 0, meta, ctypes.byref(S), None) == -4      # fp32 workspace


def test_lm_head_kind_workspace():
    # the fp32 head keeps three bf16 planes of every gathered row; the other
    # kinds one; kinds outside 0..2 are rejected
    plan = spb.pack_pass(_prob())
    f32out = spb.score_workspace_bytes(plan, 0, 1000, 256, spb.HEAD_F32OUT)
    assert spb.score_workspace_bytes(plan, 0, 1000, 256, spb.HEAD_BF16) == f32out
    fp32 = spb.score_workspace_bytes(plan, 0, 1000, 256, spb.HEAD_FP32)
    m = plan.info(0)["n_scored_rows"]
    assert fp32 - f32out >= 2 * m * 256 * 2
    with pytest.raises(spb.SpbError):
        spb.score_workspace_bytes(plan, 0, 1000, 256, 3)
    with pytest.raises(spb.SpbError):
        spb.score_batch_workspace_bytes(plan, [0], 1000, 256, -1)


def test_attention_workspace_size_and_checks():
    # e4m3 attention may take a workspace of n_tokens * hkv * d * 2 bytes
    # (V widened to bf16); other dtypes need none.  A short or misaligned one
    # is refused on the host before any HIP call.
    plan = spb.pack_pass(_prob())
    n = plan.info(0)["n_tokens"]
    assert spb.attention_workspace_bytes(plan, 0, spb.FP8_E4M3, 2, 128) == n * 2 * 128 * 2
    assert spb.attention_workspace_bytes(plan, 0, spb.BF16, 2, 128) == 0
    with pytest.raises(spb.SpbError):
        spb.attention_workspace_bytes(plan, 3, spb.FP8_E4M3, 2, 128)
    L = spb.lib()
    A = spb._AttnArgs()
    A.q = A.k = A.v = A.o = 256
    A.in_dtype, A.out_dtype, A.hq, A.hkv, A.head_dim, A.rows = spb.FP8_E4M3, spb.BF16, 4, 2, 128, 1 << 20
    A.s_q = A.s_k = A.s_v = 1.0
    A.workspace = 4096
    A.workspace_bytes = n * 2 * 128 * 2 - 1
    meta = ctypes.c_void_p(4096)
    assert L.spb_branch_attention(plan.handle, 0, meta, ctypes.byref(A), None) == -4
    A.workspace_bytes += 1
    A.workspace = 4096 + 64
    assert L.spb_branch_attention(plan.handle, 0, meta, ctypes.byref(A), None) == -1


def test_upload_rejects_small_or_misaligned_buffers():
    plan = spb.pack_pass(_prob())
    L = spb.lib()
    need = plan.info(0)["meta_bytes"]
    assert L.spb_plan_upload(plan.handle, 0, ctypes.c_void_p(4096), need - 1, None) == -4
    assert L.spb_plan_upload(plan.handle, 0, ctypes.c_void_p(4097), need, None) == -1


def test_batched_score_validation():
    # host-side checks of the one-stream head for several passes; no GPU work
    prob = synth.make_problem("random", 23, vocab=64, n_inputs=6, n_questions=3, max_content=20,
                              max_len=5, max_options=3, max_option_tokens=2)
    plan = spb.pack_pass(prob, token_budget=40)
    assert plan.n_passes >= 3
    L = spb.lib()
    ps = np.arange(plan.n_passes, dtype=np.int32)
    n = ctypes.c_size_t()
    i32 = ctypes.POINTER(ctypes.c_int32)
    assert L.spb_score_batch_workspace_bytes(plan.handle, len(ps), ps.ctypes.data_as(i32), 64, 128, 0,
                                             ctypes.byref(n)) == 0
    tot_m = sum(plan.info(k)["n_scored_rows"] for k in range(plan.n_passes))
    tot_t = sum(plan.info(k)["n_targets"] for k in range(plan.n_passes))
    assert n.value >= tot_m * 4 * 2 + tot_t * 4 + tot_m * 4 + tot_m * 128 * 2 + (tot_m + 1) * 4 + tot_t * 4
    # same answer through the binding
    assert spb.score_batch_workspace_bytes(plan, list(range(plan.n_passes)), 64, 128) == n.value
    dup = np.array([0, 0], np.int32)
    assert L.spb_score_batch_workspace_bytes(plan.handle, 2, dup.ctypes.data_as(i32), 64, 128, 0, ctypes.byref(n)) == -1
    bad = np.array([plan.n_passes], np.int32)
    assert L.spb_score_batch_workspace_bytes(plan.handle, 1, bad.ctypes.data_as(i32), 64, 128, 0, ctypes.byref(n)) == -1
    assert L.spb_score_batch_workspace_bytes(plan.handle, 0, ps.ctypes.data_as(i32), 64, 128, 0, ctypes.byref(n)) == -2
    big = np.zeros(65, np.int32)
    assert L.spb_score_batch_workspace_bytes(plan.handle, 65, big.ctypes.data_as(i32), 64, 128, 0, ctypes.byref(n)) == -2
    # argument checks before any launch (fake device pointers are never touched)
    k = len(ps)
    metas = (ctypes.c_void_p * k)(*[4096 * (i + 1) for i in range(k)])
    A = (spb._ScoreArgs * k)()
    for i in range(k):
        A[i].hidden, A[i].h_dtype, A[i].hidden_dim, A[i].rows = 1 << 20, spb.BF16, 128, 1 << 20
        A[i].lm_head, A[i].vocab = 1 << 21, 64
        A[i].lp = A[i].p = A[i].residual = ctypes.cast(ctypes.c_void_p(1 << 22), ctypes.POINTER(ctypes.c_float))
    ws_ok = n.value
    call = lambda ws, nbytes: L.spb_score_options_batch(plan.handle, k, ps.ctypes.data_as(i32), metas, A,
                                                        ctypes.c_void_p(ws), nbytes, None)
    L.spb_score_batch_workspace_bytes(plan.handle, k, ps.ctypes.data_as(i32), 64, 128, 0, ctypes.byref(n))
    assert call(1 << 23, n.value - 1) == -4                 # workspace too small
    assert call((1 << 23) + 4, n.value) == -1               # workspace misaligned
    A[1].hidden_dim = 192
    assert call(1 << 23, n.value) == -1                     # entries disagree
    A[1].hidden_dim = 128
    A[1].lm_head_kind = spb.HEAD_BF16
    assert call(1 << 23, n.value) == -1                     # entries disagree on the lm-head kind
    A[1].lm_head_kind = 0
    for i in range(k):
        A[i].vocab = 8
    assert call(1 << 23, 1 << 30) == -1                     # a token >= vocab
    for i in range(k):
        A[i].vocab = 64
    A[2].rows = 1
    assert call(1 << 23, ws_ok) == -4                       # hidden too short
    A[2].rows = 1 << 20
    metas[1] = 4096 + 8
    assert call(1 << 23, ws_ok) == -1                       # metadata misaligned


def test_meta_copy_matches_the_pass_layout():
    # the host copy carries the same metadata blob spb_plan_upload sends: header
    # magic "SPB1", the pass index and its counts, and the plan's row placement
    prob = synth.make_problem("random", 17, vocab=32, n_inputs=4, n_questions=3, max_content=20,
                              max_len=5, max_options=3, max_option_tokens=2)
    plan = spb.pack_pass(prob, token_budget=60)
    for k in range(plan.n_passes):
        inf = plan.info(k)
        buf = np.zeros(inf["meta_bytes"] + 64, np.uint8)
        plan.meta_copy(k, buf)
        head = buf[:48].view(np.int32)
        assert head[0] == 0x53504231 and head[2] == k
        assert head[3] == inf["n_tokens"] and head[4] == inf["n_tiles"]
        assert head[5] == inf["n_branches"] and head[6] == inf["n_options"] and head[7] == inf["n_scored_rows"]
        assert not buf[inf["meta_bytes"]:].any()  # nothing written past meta_bytes
    L = spb.lib()
    small = np.zeros(plan.info(0)["meta_bytes"] - 1, np.uint8)
    assert L.spb_plan_meta_copy(plan.handle, 0, ctypes.c_void_p(small.ctypes.data), small.nbytes) == -4
    assert L.spb_plan_meta_copy(plan.handle, 0, None, 1 << 20) == -1
    assert L.spb_plan_meta_copy(plan.handle, plan.n_passes, ctypes.c_void_p(small.ctypes.data), small.nbytes) == -1


def test_score_finalize_joins_floors_in_logical_order():
    prob = synth.make_problem("random", 41, vocab=16, n_inputs=5, n_questions=3, max_content=10,
                              max_len=4, max_options=3, max_option_tokens=2)
    plan = spb.pack_pass(prob, token_budget=30)
    lay = OT.build_layout(prob, floors=True)
    # per-pass outputs encode (logical branch, option) so the join can be read back
    lps, ps, rs = [], [], []
    for k in range(plan.n_passes):
        lb, of = plan.branches(k)
        inf = plan.info(k)
        lp = np.zeros(inf["n_options"], np.float32)
        p = np.zeros(inf["n_options"], np.float32)
        r = np.zeros(inf["n_branches"], np.float32)
        for b in range(len(lb)):
            r[b] = lb[b]
            q = list(lay.branches())[lb[b]].question
            n_opt = prob.opt_off[q + 1] - prob.opt_off[q]
            for o in range(n_opt):
                lp[of[b] + o] = -(lb[b] * 10 + o)
                p[of[b] + o] = lb[b] * 10 + o
        lps.append(lp); ps.append(p); rs.append(r)
    out = spb.score_finalize(plan, lps, ps, rs)
    branches = list(lay.branches())
    nb = len(prob.branch_q)
    floor_of = {b.question: i for i, b in enumerate(branches) if b.is_floor}
    pos = 0
    for b in range(nb):
        q = branches[b].question
        assert out["residual"][b] == b
        n_opt = prob.opt_off[q + 1] - prob.opt_off[q]
        for o in range(n_opt):
            assert out["p"][pos] == b * 10 + o
            assert out["lp"][pos] == -(b * 10 + o)
            assert out["floor_p"][pos] == floor_of[q] * 10 + o
            assert out["lift"][pos] == np.float32(b * 10 + o) - np.float32(floor_of[q] * 10 + o)
            pos += 1
    assert pos == len(out["p"])


def test_score_workspace_covers_gathered_hidden_rows():
    # the lm head packs the scored rows' hidden states into the workspace, so
    # its size must grow with the hidden size by at least M rows of bf16
    prob = synth.make_problem("random", 5, vocab=1000, n_inputs=4, n_questions=5, max_content=40,
                              max_len=8, max_options=4, max_option_tokens=3)
    plan = spb.pack_pass(prob)
    M = plan.info(0)["n_scored_rows"]
    small = spb.score_workspace_bytes(plan, 0, 1000, 64)
    big = spb.score_workspace_bytes(plan, 0, 1000, 3840)
    assert big - small >= M * (3840 - 64) * 2
    assert small >= M * 64 * 2 + M * 4 * 2 * 4  # hidden rows + (max, sum) per 256-row vocabulary slice
    with pytest.raises(spb.SpbError):
        spb.score_workspace_bytes(plan, 0, 1000, 0)


def _meta_arrays(buf):
    """Header fields and arrays of a pass metadata blob (layout of spb_meta.h)."""
    i32 = buf[:48].view(np.int32)
    i64 = buf[48:48 + 16 * 8].view(np.int64)
    tail = buf[48 + 16 * 8:48 + 16 * 8 + 16].view(np.int32)
    n_tokens, n_branches = int(i32[3]), int(i32[5])
    off_rows, off_branches = int(i64[0]), int(i64[2])
    rows = buf[off_rows:off_rows + 48 * n_tokens].view(np.int32).reshape(-1, 12)
    br = buf[off_branches:off_branches + 32 * n_branches].view(np.int32).reshape(-1, 8)
    items = []
    for g in range(3):
        off, n = int(i64[12 + g]), int(tail[g])
        items.append(buf[off:off + 32 * n].view(np.int32).reshape(-1, 8))
    off_bc, n_bc = int(i64[15]), int(tail[3])
    bchunks = buf[off_bc:off_bc + 16 * n_bc].view(np.int32).reshape(-1, 4)
    return n_tokens, rows, br, items, bchunks


@pytest.mark.parametrize("budget", [120, 200, 600])
def test_attention_work_items_cover_rows_and_visible_chunks(budget):
    # the bf16 attention kernel walks, per work item, the content chunks its
    # rows see and the chunks of every branch meeting its rows; derive both
    # from the rows' own visibility fields and compare
    prob = synth.make_problem("random", 23, vocab=64, n_inputs=6, n_questions=5, max_content=70,
                              max_len=40, max_options=3, max_option_tokens=3)
    plan = spb.pack_pass(prob, token_budget=budget)
    for k in range(plan.n_passes):
        buf = np.zeros(plan.info(k)["meta_bytes"], np.uint8)
        plan.meta_copy(k, buf)
        n, rows, br, items, bchunks = _meta_arrays(buf)
        start_of = {int(s): b for b, s in enumerate(br[:, 0])}
        for g in range(3):
            per = 32 << g
            seen = np.zeros(n, np.int32)
            costs = []
            for it in items[g]:
                row0, nrows, seg, ncc, boff, bn, cost = (int(v) for v in it[:7])
                assert 1 <= nrows <= per and cost == ncc + bn
                costs.append(cost)
                seen[row0:row0 + nrows] += 1
                r = rows[row0:row0 + nrows]
                # rows that see content see the item's segment (floor rows see none)
                assert (r[r[:, 0] > 0, 1] == seg).all()
                assert ncc == -(-int(r[:, 0].max()) // 64)
                want = []
                for b0 in sorted(set(int(v) for v in r[:, 2] if v >= 0)):
                    emax = int(r[r[:, 2] == b0, 3].max())
                    want += [(b0 + 32 * c, (start_of[b0] << 10) | c) for c in range(emax // 32 + 1)]
                got = [tuple(int(v) for v in e[:2]) for e in bchunks[boff:boff + bn]]
                assert got == want
            assert (seen == 1).all()  # every row in exactly one item
            assert costs == sorted(costs, reverse=True)


def test_repacking_gives_identical_metadata():
    # plans reuse freed host blocks; every byte of a pass's metadata is
    # written on each pack, so a block that held another plan leaves no trace
    news = synth.make_workload("news").problem
    other = synth.make_problem("random_shared", 5, vocab=1000, n_inputs=40, n_questions=30, max_content=400,
                               max_lead=30)

    def blobs(prob):
        plan = spb.pack_pass(prob, token_budget=16384)
        out = []
        for k in range(plan.n_passes):
            b = np.zeros(plan.info(k)["meta_bytes"], np.uint8)
            plan.meta_copy(k, b)
            out.append(b.tobytes())
        del plan
        return out

    first = blobs(news)
    blobs(other)
    assert blobs(news) == first
    assert blobs(other) == blobs(other)


def test_head_groups_rule():
    """Head groups (driver): consecutive passes while their scored rows total
    at most the cap, at most 64 per launch; a pass above the cap alone; no cap
    means one launch per pass; batch_head one launch for all."""
    from shared_prefix_branch_amd.driver import Job
    pr = synth.make_problem("random", 31, vocab=4096, n_inputs=12, n_questions=5, min_content=5,
                            max_content=60, max_len=8, max_options=4, max_option_tokens=3)
    plan = spb.pack_pass(pr, token_budget=110)
    m = [plan.info(k)["n_scored_rows"] for k in range(plan.n_passes)]
    assert m == [21, 16, 13, 21, 6, 23, 25, 11, 26, 14]

    def groups(**kw):
        return Job(plan, 8, 4, 128, 256, 4096, None, None, None, device="cpu", **kw).head_groups

    assert groups() == [[k] for k in range(10)]
    assert groups(batch_head=True) == [list(range(10))]
    assert groups(head_rows=40) == [[0, 1], [2, 3, 4], [5], [6, 7], [8, 9]]  # 37, 40, 23, 36, 40
    assert groups(head_rows=30) == [[0], [1, 2], [3, 4], [5], [6], [7], [8], [9]]  # 29 and 27 fit
    assert groups(head_rows=20) == [[k] for k in range(10)]  # no two neighbours fit
    assert groups(head_rows=10 ** 6) == [list(range(10))]
    # the 64-pass limit of one batched launch
    pr = synth.make_problem("random", 5, vocab=4096, n_inputs=70, n_questions=1, min_content=5,
                            max_content=8, max_len=4, max_options=2, max_option_tokens=1)
    plan = spb.pack_pass(pr, token_budget=12, floors=False)
    assert plan.n_passes == 70
    g = groups(head_rows=10 ** 6)
    assert [len(x) for x in g] == [64, plan.n_passes - 64]


def test_job_and_scoring_refuse_plans_of_other_shapes():
    # buffers are sized from the plan a job was made for: a re-packed plan
    # with more rows, options or branches in a pass is refused on the host
    # instead of writing past the device buffers
    import torch
    from shared_prefix_branch_amd.driver import Job
    wl = synth.make_workload("fp8", n_inputs=6, hidden=128, vocab=1000)
    plan = spb.pack_pass(wl.problem, token_budget=8192)
    same = spb.pack_pass(wl.problem, token_budget=8192)
    other = spb.pack_pass(wl.problem.subset([0, 1, 2, 3, 4]), token_budget=8192)
    job = Job(plan, 8, 2, 128, 128, 1000, torch.uint8, torch.bfloat16, torch.bfloat16, device="cpu")
    job.check_shapes(same)
    with pytest.raises(spb.SpbError) as e:
        job.check_shapes(other)
    assert e.value.code == -4
    inf = plan.info(0)
    meta = torch.empty(inf["meta_bytes"], dtype=torch.uint8)
    hid = torch.empty((inf["n_tokens"], 128), dtype=torch.bfloat16)
    W = torch.empty((1000, 128), dtype=torch.bfloat16)
    ws = torch.empty(256, dtype=torch.uint8)
    lp, p = torch.empty(inf["n_options"]), torch.empty(inf["n_options"])
    res = torch.empty(inf["n_branches"])
    sc = spb.PreparedScore(0, meta, hid, W, ws, lp, p, res)
    sc.check_plan(same)
    small = spb.PreparedScore(0, meta, hid, W, ws, lp[:-1], p, res)
    with pytest.raises(spb.SpbError) as e:
        small.check_plan(plan)
    assert e.value.code == -4


def test_noalloc_head_refuses_a_pass_beyond_its_scratch():
    # the allocation-free head has 64 MiB of scratch per GPU: a pass whose
    # head workspace is larger is refused on the host, before any HIP call,
    # with SPB_ERR_SIZE (host tensors stand in for the device buffers: the
    # call returns before it reads them)
    import torch
    H, V, M = 4096, 262144, 2200
    prob = synth.Problem(np.array([0], np.int32), np.array([0, M], np.int32), np.arange(M, dtype=np.int32),
                         np.ones(M, np.int32), np.arange(0, 2 * M + 1, 2, dtype=np.int32),
                         np.arange(2 * M + 1, dtype=np.int32), (np.arange(2 * M) * 97 % V).astype(np.int32), V)
    plan = spb.pack_pass(prob, floors=False)
    assert spb.score_workspace_bytes(plan, 0, V, H, spb.HEAD_FP32) > 64 << 20
    assert spb.score_workspace_bytes(plan, 0, V, H, spb.HEAD_F32OUT) < 64 << 20
    inf = plan.info(0)
    meta = torch.empty(inf["meta_bytes"] + 256, dtype=torch.uint8)
    meta = meta[(-meta.data_ptr()) % 256:][:inf["meta_bytes"]]
    hid = torch.empty((inf["n_tokens"], H), dtype=torch.bfloat16)
    W = torch.empty((1, H), dtype=torch.bfloat16).expand(V, H)
    outs = (torch.empty(inf["n_options"]), torch.empty(inf["n_options"]), torch.empty(inf["n_branches"]))
    with pytest.raises(spb.SpbError) as e:
        spb.score_options_noalloc(plan, 0, meta, hid, W, *outs, stream=0, lm_head_kind=spb.HEAD_FP32)
    assert e.value.code == -4
    assert "allocation-free scratch" in spb.lib().spb_last_error().decode()


def test_mfma_calibration_validates_before_any_hip_call():
    # the roofline calibration entry refuses bad sizes on the host
    L = spb.lib()
    assert L.spb_mfma_calibration(None, 1, 1, 1, None) == -1
    assert L.spb_mfma_calibration(ctypes.c_void_p(4096), 0, 1, 1, None) == -1
    assert L.spb_mfma_calibration(ctypes.c_void_p(4096), 1, 0, 1, None) == -1
    assert L.spb_mfma_calibration(ctypes.c_void_p(4096), (1 << 20) + 1, 1, 1, None) == -2
