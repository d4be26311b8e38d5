"""CPU tests of the decoder-stack host side: each pass row's position against
the oracle's root-path positions, the rotary table against its closed form,
and argument checks of spb_rmsnorm / spb_linear that fail before any HIP call."""
import ctypes
import math

import numpy as np
import pytest

import shared_prefix_branch_amd as spb
import synth
from oracle import forward as OF
from oracle import tree as OT


@pytest.mark.parametrize("kind,budget", [("random", 16384), ("random", 60), ("shared", 16384), ("shared", 40),
                                         ("grid", 400)])
def test_positions_equal_root_path_positions(kind, budget):
    if kind == "random":
        prob = synth.make_problem("random", 8, vocab=64, n_inputs=4, n_questions=5, max_content=30, max_len=6,
                                  max_options=4, max_option_tokens=4)
    elif kind == "shared":
        prob = synth.make_problem("random_shared", 15, vocab=16, n_inputs=3, n_questions=6, max_content=10,
                                  max_lead=5, tail_vocab=3, max_options=3, max_option_tokens=3)
    else:
        prob = synth.make_problem("grid", 6, vocab=4096, n_inputs=2, n_templates=2, min_content=30, max_content=60)
    plan = spb.pack_pass(prob, token_budget=budget)
    lay = OT.build_layout(prob, floors=True)
    want = OF.positions(lay)
    for k in range(plan.n_passes):
        lr, _ = plan.rows(k)
        assert plan.positions(k).tolist() == want[lr].tolist()


def test_rope_table_closed_form():
    t = spb.rope_table(50, 8, 10000.0)
    assert t.shape == (50, 4, 2)
    p = np.arange(50)[:, None]
    ang = p * 10000.0 ** (-np.arange(4) * 2.0 / 8)[None, :]
    assert np.array_equal(t[..., 0], np.cos(ang).astype(np.float32))
    assert np.array_equal(t[..., 1], np.sin(ang).astype(np.float32))
    assert t[3, 0, 0] == np.float32(math.cos(3.0)) and t[1, 1, 1] == np.float32(math.sin(0.1))
    with pytest.raises(spb.SpbError):
        spb.rope_table(10, 7)


def test_layer_entry_points_validate_before_any_hip_call():
    L = spb.lib()
    N = spb._NormArgs()
    N.x = N.gain = N.out = 256
    N.rows, N.dim, N.eps = 10, 6, 1e-6
    assert L.spb_rmsnorm(ctypes.byref(N), None) == -1          # dim % 4
    N.dim = 8
    N.x = 258
    assert L.spb_rmsnorm(ctypes.byref(N), None) == -1          # alignment
    N.x, N.rows = 256, 0
    assert L.spb_rmsnorm(ctypes.byref(N), None) == 0           # nothing to do
    A = spb._LinearArgs()
    A.x = A.w = A.y = A.resid = 256
    A.m, A.n, A.k, A.mode = 100, 256, 96, spb.LINEAR_BF16
    assert L.spb_linear(ctypes.byref(A), None) == -1           # k % 64
    A.k, A.n = 128, 100
    assert L.spb_linear(ctypes.byref(A), None) == -1           # n % 8
    A.n, A.mode = 96, spb.LINEAR_SILU_GATE
    assert L.spb_linear(ctypes.byref(A), None) == -1           # gate blocks of 64 rows
    A.mode = 7
    assert L.spb_linear(ctypes.byref(A), None) == -1           # mode
    A.mode, A.n = spb.LINEAR_QKV_ROPE, 512
    A.hq, A.hkv, A.head_dim = 2, 1, 96
    assert L.spb_linear(ctypes.byref(A), None) == -3           # head_dim
    A.head_dim = 128
    assert L.spb_linear(ctypes.byref(A), None) == -1           # n != (hq + 2 hkv) d
    A.hq, A.hkv = 2, 1
    A.n = 512
    assert L.spb_linear(ctypes.byref(A), None) == -1           # q/k/v/pos/table missing
    A.mode, A.m, A.k, A.n = spb.LINEAR_BF16, 1 << 20, 4096, 256
    assert L.spb_linear(ctypes.byref(A), None) == -2           # x over 4 GiB
    A.m = 0
    assert L.spb_linear(ctypes.byref(A), None) == 0            # nothing to do


@pytest.mark.parametrize("budget", [16384, 150])
def test_slot_prefix_runs_equal_the_root_path(budget):
    prob = synth.make_problem("random_shared", 71, vocab=1000, n_inputs=3, n_questions=6, min_content=0,
                              max_content=120, max_lead=40, tail_vocab=3, max_options=3, max_option_tokens=3)
    plan = spb.pack_pass(prob, token_budget=budget)
    lay = OT.build_layout(prob, floors=True)
    lbs = [b for li in lay.inputs for b in li.branches]
    pos = OF.positions(lay)
    for lb, b in enumerate(lbs):
        s = plan.slot(lb)
        lr, _ = plan.rows(s["pass"])
        assert lr[s["row"]] == b.last_row
        assert s["position"] == pos[b.last_row]
        keys = [y for first, n in s["ranges"] for y in range(first, first + n)]
        assert keys == plan.visible(s["pass"], s["row"])
        assert sorted(lr[keys].tolist()) == sorted(OT.root_path(lay, b.last_row))
    with pytest.raises(spb.SpbError):
        plan.slot(len(lbs))


def test_decode_entry_points_validate_before_any_hip_call():
    L = spb.lib()
    T = spb._TopkArgs()
    T.logits = T.ids = T.lp = T.lse = 256
    T.rows, T.vocab, T.k = 4, 100, 17
    assert L.spb_topk_lse(ctypes.byref(T), None) == -1         # k > 16
    T.k, T.mask_of_row = 4, 256
    assert L.spb_topk_lse(ctypes.byref(T), None) == -1         # mask_of_row without masks
    T.mask_of_row = None
    T.workspace, T.workspace_bytes = 256, 8
    assert L.spb_topk_lse(ctypes.byref(T), None) == -4         # workspace too small
    assert spb.topk_workspace_bytes(4, 100) > 0
    D = spb._DecodeAttnArgs()
    D.q = D.k_pass = D.v_pass = D.k_dec = D.v_dec = D.o = D.ranges = D.n_ranges = D.path = 256
    D.rows, D.beams, D.hq, D.hkv, D.head_dim, D.t_cap, D.n_path, D.n_pass_rows = 8, 4, 4, 2, 128, 5, 5, 10
    assert L.spb_decode_attention(ctypes.byref(D), None) == -1  # n_path >= t_cap
    D.n_path, D.rows = 2, 6
    assert L.spb_decode_attention(ctypes.byref(D), None) == -1  # rows % beams
    D.rows, D.hq = 8, 24
    assert L.spb_decode_attention(ctypes.byref(D), None) == -3  # hq / hkv = 12
    Bm = spb._BeamArgs()
    Bm.n_slots, Bm.beams, Bm.k, Bm.t_cap, Bm.step = 2, 17, 4, 5, 0
    assert L.spb_beam_step(ctypes.byref(Bm), None) == -1        # beams > 16
    Bm.beams, Bm.step = 4, 5
    assert L.spb_beam_step(ctypes.byref(Bm), None) == -1        # step >= t_cap
    Bm.step = 1
    Bm.stop = Bm.ids = Bm.lp = Bm.tok_out = Bm.len_out = Bm.fin_out = Bm.path_out = Bm.nb_out = 256
    Bm.score_out = Bm.feed = 256
    assert L.spb_beam_step(ctypes.byref(Bm), None) == -1        # later steps need the previous state
    G = spb._GatherArgs()
    G.src = G.idx = G.dst_f32 = G.dst_bf16 = 256
    G.rows, G.dim, G.n_src = 4, 8, 10
    assert L.spb_gather_rows(ctypes.byref(G), None) == -1       # two destinations
