"""Pins of the oracle's decoder stack (oracle/forward.py), on the CPU: closed
forms of rmsnorm, RoPE and SiLU, torch's CPU routines for the special cases
they cover, the stack with its branches switched off, form (i) against form
(ii) on tree layouts (template sharing included), and positions from the
layout's own fields."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle import forward as OF
from oracle import tree as OT


def _model(seed=0, H=32, hq=4, hkv=2, d=8, ffn=48, layers=2, base=10000.0):
    rng = np.random.default_rng(seed)

    def mat(r, c):
        return rng.normal(size=(r, c)) / math.sqrt(c)

    Ls = []
    for _ in range(layers):
        Ls.append(dict(wq=mat(hq * d, H), wk=mat(hkv * d, H), wv=mat(hkv * d, H), wo=mat(H, hq * d),
                       wg=mat(ffn, H), wu=mat(ffn, H), wd=mat(H, ffn),
                       g_attn=rng.uniform(0.5, 1.5, H), g_mlp=rng.uniform(0.5, 1.5, H)))
    return OF.Model(H, hq, hkv, d, base, 1e-6, Ls, rng.uniform(0.5, 1.5, H))


def test_rms_norm_closed_forms_and_torch():
    g = np.array([0.5, 2.0, -1.0, 3.0])
    # a constant vector c: rms = |c|, so the output is sign(c) * g
    for c in (3.0, -0.25):
        out = OF.rms_norm(np.full(4, c), g, 0.0)
        assert np.allclose(out, np.sign(c) * g, atol=1e-15)
    x = np.random.default_rng(1).normal(size=(5, 16)) * 7
    y = OF.rms_norm(x, np.ones(16), 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, atol=1e-14)
    gg = np.random.default_rng(2).uniform(0.5, 1.5, 16)
    ref = F.rms_norm(torch.from_numpy(x), (16,), torch.from_numpy(gg), eps=1e-6).numpy()
    assert np.allclose(OF.rms_norm(x, gg, 1e-6), ref, atol=1e-13)


def test_rope_closed_forms():
    # d = 2: one pair at frequency 1, rotated counter-clockwise by pos radians
    e1 = np.array([[[1.0, 0.0]]])
    e2 = np.array([[[0.0, 1.0]]])
    assert np.allclose(OF.rope(e1, np.array([1]), 10000.0), [[[math.cos(1), math.sin(1)]]], atol=1e-15)
    assert np.allclose(OF.rope(e2, np.array([1]), 10000.0), [[[-math.sin(1), math.cos(1)]]], atol=1e-15)
    # d = 4: the second pair turns at base^(-2/4) = 0.01 rad per position
    x = np.array([[[0.0, 0.0, 1.0, 0.0]]])
    assert np.allclose(OF.rope(x, np.array([3]), 10000.0), [[[0, 0, math.cos(0.03), math.sin(0.03)]]], atol=1e-15)
    # position 0 is the identity; rotations keep each pair's norm
    y = np.random.default_rng(0).normal(size=(6, 3, 16))
    assert np.array_equal(OF.rope(y, np.zeros(6), 10000.0), y)
    r = OF.rope(y, np.arange(6) * 37, 10000.0)
    assert np.allclose(r[..., 0::2] ** 2 + r[..., 1::2] ** 2, y[..., 0::2] ** 2 + y[..., 1::2] ** 2, atol=1e-12)


def test_rope_equals_complex_multiplication_and_is_relative():
    # the textbook complex form: each pair (a, b) is a + ib times exp(i pos theta_j)
    rng = np.random.default_rng(3)
    x = rng.normal(size=(5, 2, 8))
    pos = np.array([0, 1, 7, 100, 4095])
    theta = 500.0 ** (-np.arange(4) * 2.0 / 8)
    z = torch.view_as_complex(torch.from_numpy(x).reshape(5, 2, 4, 2).contiguous())
    rot = torch.polar(torch.ones(5, 1, 4, dtype=torch.float64),
                      torch.from_numpy(pos[:, None, None] * theta[None, None, :]))
    ref = torch.view_as_real(z * rot).reshape(5, 2, 8).numpy()
    assert np.allclose(OF.rope(x, pos, 500.0), ref, atol=1e-12)
    # q(m) . k(n) depends on m - n only
    q, k = rng.normal(size=(1, 1, 8)), rng.normal(size=(1, 1, 8))
    a = np.sum(OF.rope(q, np.array([9]), 500.0) * OF.rope(k, np.array([4]), 500.0))
    b = np.sum(OF.rope(q, np.array([1009]), 500.0) * OF.rope(k, np.array([1004]), 500.0))
    assert abs(a - b) < 1e-10


def test_silu_closed_forms_and_torch():
    assert OF.silu(np.array([0.0]))[0] == 0.0
    assert abs(OF.silu(np.array([40.0]))[0] - 40.0) < 1e-12
    assert abs(OF.silu(np.array([-40.0]))[0]) < 1e-15
    z = np.linspace(-8, 8, 101)
    assert np.allclose(OF.silu(z), F.silu(torch.from_numpy(z)).numpy(), atol=1e-15)


def _torch_stack(m, x0):
    """The same reading built from torch's CPU routines: rms_norm, complex-form
    RoPE, scaled_dot_product_attention (causal, key/value heads repeated for
    the grouped query heads) and silu."""
    x = torch.from_numpy(np.array(x0))
    n = x.shape[0]
    d, hq, hkv = m.head_dim, m.hq, m.hkv
    theta = m.rope_base ** (-torch.arange(d // 2, dtype=torch.float64) * 2.0 / d)
    rot = torch.polar(torch.ones(n, 1, d // 2, dtype=torch.float64),
                      torch.arange(n, dtype=torch.float64)[:, None, None] * theta[None, None, :])

    def rope(t):
        z = torch.view_as_complex(t.reshape(n, t.shape[1], d // 2, 2).contiguous())
        return torch.view_as_real(z * rot).reshape(n, t.shape[1], d)

    T = lambda a: torch.from_numpy(a)  # noqa: E731
    for L in m.layers:
        h = F.rms_norm(x, (m.hidden,), T(L["g_attn"]), eps=m.eps)
        q = rope((h @ T(L["wq"]).T).reshape(n, hq, d))
        k = rope((h @ T(L["wk"]).T).reshape(n, hkv, d))
        v = (h @ T(L["wv"]).T).reshape(n, hkv, d)
        rep = hq // hkv
        k, v = k.repeat_interleave(rep, dim=1), v.repeat_interleave(rep, dim=1)
        o = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1), is_causal=True)
        x = x + o.transpose(0, 1).reshape(n, hq * d) @ T(L["wo"]).T
        h = F.rms_norm(x, (m.hidden,), T(L["g_mlp"]), eps=m.eps)
        x = x + (F.silu(h @ T(L["wg"]).T) * (h @ T(L["wu"]).T)) @ T(L["wd"]).T
    return F.rms_norm(x, (m.hidden,), T(m.g_final), eps=m.eps).numpy()


@pytest.mark.parametrize("hkv", [4, 2, 1])
def test_decoder_sequence_matches_torch_routines(hkv):
    m = _model(seed=hkv, hkv=hkv)
    x0 = np.random.default_rng(10 + hkv).normal(size=(9, 32))
    assert np.allclose(OF.decoder_sequence(m, x0), _torch_stack(m, x0), atol=1e-10)


def test_planted_mistakes_are_caught():
    m = _model(seed=5)
    x0 = np.random.default_rng(6).normal(size=(7, 32))
    ref = _torch_stack(m, x0)
    # a rotation in the wrong direction
    orig = OF.rope
    try:
        OF.rope = lambda x, pos, base: orig(x, -np.asarray(pos), base)
        assert not np.allclose(OF.decoder_sequence(m, x0), ref, atol=1e-6)
    finally:
        OF.rope = orig
    # rotate-half pairing (i, i + d/2) instead of adjacent pairs
    try:
        def half(x, pos, base):
            d = x.shape[-1]
            perm = np.r_[0:d:2, 1:d:2]
            inv = np.argsort(perm)
            return orig(x[..., inv], pos, base)[..., perm]
        OF.rope = half
        assert not np.allclose(OF.decoder_sequence(m, x0), ref, atol=1e-6)
    finally:
        OF.rope = orig
    # a missing residual around the MLP
    mm = _model(seed=5)
    for L in mm.layers:
        L["wd"] = np.zeros_like(L["wd"])
    assert not np.allclose(OF.decoder_sequence(mm, x0), ref, atol=1e-6)


def test_switched_off_branches_leave_the_embedding():
    # Wo = 0 and Wd = 0: every layer adds zero, the head reads rmsnorm(x0) * g_final
    m = _model(seed=7)
    for L in m.layers:
        L["wo"] = np.zeros_like(L["wo"])
        L["wd"] = np.zeros_like(L["wd"])
    x0 = np.random.default_rng(8).normal(size=(6, 32))
    assert np.allclose(OF.decoder_sequence(m, x0), OF.rms_norm(x0, m.g_final, m.eps), atol=1e-14)


def _layout_and_x0(prob, seed, H=32):
    lay = OT.build_layout(prob, floors=True)
    return lay, np.random.default_rng(seed).normal(size=(lay.n_rows, H))


def test_positions_from_layout_fields():
    prob = synth.make_problem("random", 4, vocab=32, n_inputs=3, n_questions=4, max_content=9,
                              max_len=5, max_options=4, max_option_tokens=4)
    lay = OT.build_layout(prob, floors=True)
    pos = OF.positions(lay)
    for li in lay.inputs:
        assert pos[li.first_row:li.first_row + li.C].tolist() == list(range(li.C))
        for b in li.branches:
            assert pos[b.template_rows].tolist() == list(range(li.C, li.C + len(b.template_rows)))
            for ni, p in enumerate(b.trie.prefixes):
                assert pos[b.node_row0 + ni] == li.C + len(b.template_rows) - 1 + len(p)


@pytest.mark.parametrize("kind,seed", [("random", 11), ("random", 12), ("shared", 13), ("shared", 15)])
def test_per_sequence_equals_dense_tree_mask(kind, seed):
    if kind == "random":
        prob = synth.make_problem("random", seed, vocab=32, n_inputs=3, n_questions=4, max_content=8,
                                  max_len=4, max_options=3, max_option_tokens=3)
    else:
        prob = synth.make_problem("random_shared", seed, vocab=16, n_inputs=2, n_questions=5, max_content=6,
                                  max_lead=4, tail_vocab=3, max_options=3, max_option_tokens=3)
    m = _model(seed=seed)
    lay, x0 = _layout_and_x0(prob, seed)
    if kind == "shared":
        assert any(b.stem_rows for b in lay.branches())
    dense = OF.forward_dense(m, lay, x0)
    for li in lay.inputs:
        lo = li.first_row
        hi = lo + int((lay.row_input == lay.row_input[lo]).sum())
        per = OF.forward_input(m, lay, li, x0[lo:hi])
        assert np.allclose(per, dense[lo:hi], atol=1e-10)


def test_question_rows_equal_the_question_asked_alone():
    # a branch's rows are those of the question asked on its own content
    prob = synth.make_problem("random", 21, vocab=32, n_inputs=2, n_questions=4, max_content=8,
                              max_len=4, max_options=3, max_option_tokens=3)
    m = _model(seed=21)
    lay, x0 = _layout_and_x0(prob, 21)
    li = lay.inputs[1]
    lo = li.first_row
    hi = lo + int((lay.row_input == 1).sum())
    full = OF.forward_input(m, lay, li, x0[lo:hi])
    q = int(prob.branch_q[prob.branch_off[1]])
    alone = synth.Problem(prob.content_len[1:2], np.array([0, 1], np.int32), np.array([q], np.int32), prob.q_len,
                          prob.opt_off, prob.tok_off, prob.tok, prob.vocab)
    la = OT.build_layout(alone, floors=False)
    b = li.branches[0]
    rows = list(range(li.C)) + [r - lo for r in b.template_rows] + \
        list(range(b.node_row0 - lo, b.node_row0 - lo + len(b.trie.prefixes)))
    got = OF.forward_input(m, la, la.inputs[0], x0[lo:hi][rows])
    assert np.allclose(got, full[rows], atol=1e-12)


def test_round_to_e4m3_against_the_table_and_torch():
    from oracle import numerics as ON
    grid = np.unique(ON.E4M3_TABLE[~np.isnan(ON.E4M3_TABLE)])
    # every representable value maps to itself
    assert np.array_equal(ON.round_to_e4m3(grid), grid)
    # midpoints between neighbours go to the neighbour with the even code
    pos = grid[grid >= 0]
    mids = (pos[:-1] + pos[1:]) / 2
    codes = {float(v): b for b, v in enumerate(ON.E4M3_TABLE) if b < 128 and not np.isnan(v)}
    for lo, hi, mid in zip(pos[:-1], pos[1:], mids):
        want = lo if codes[float(lo)] % 2 == 0 else hi
        assert ON.round_to_e4m3(mid) == want
    assert ON.round_to_e4m3(1000.0) == 448.0 and ON.round_to_e4m3(-470.0) == -448.0
    # torch's cast (saturated first) on random values across the range
    x = np.random.default_rng(0).normal(size=20000) * np.exp2(np.random.default_rng(1).uniform(-12, 10, 20000))
    ref = torch.from_numpy(np.clip(x, -448, 448)).float().to(torch.float8_e4m3fn).double().numpy()
    xf = x.astype(np.float32).astype(np.float64)  # torch rounds the f32 value
    assert np.array_equal(ON.round_to_e4m3(np.clip(xf, -448, 448)), ref)


def test_fp8_linears_quantize_weights_and_inputs_per_tensor():
    # q8 by hand: 1.0625 / 1 is the midpoint of 1 and 1.125 -> 1 (even code);
    # with scale 2, 3.3 -> 1.65 -> 1.625 -> 3.25
    assert OF.q8(np.array([1.0625]), 1.0)[0] == 1.0
    assert OF.q8(np.array([3.3]), 2.0)[0] == 3.25
    assert OF.q8(np.array([5000.0]), 1.0)[0] == 448.0
    # a linear whose weight and input already sit on the scaled e4m3 grid is exact
    m = _model(seed=3)
    rng = np.random.default_rng(4)
    sx, sw = 0.5, 0.01
    x = OF.q8(rng.normal(size=(5, 32)), sx)
    w = OF.q8(rng.normal(size=(16, 32)) * 0.1, sw)
    m.fp8 = [dict(x_o=sx, s_o=sw)] * 2
    assert np.array_equal(OF._lin(m, 0, x, w, "o"), x @ w.T)
    # off the grid, both operands are rounded: the product moves
    x2, w2 = rng.normal(size=(5, 32)), rng.normal(size=(16, 32)) * 0.1
    y = OF._lin(m, 0, x2, w2, "o")
    assert not np.allclose(y, x2 @ w2.T, atol=1e-6)
    assert np.allclose(y, OF.q8(x2, sx) @ OF.q8(w2, sw).T, atol=1e-12)


def _fp8_scales(m, sx=(8 / 448, 4 / 448, 8 / 448, 16 / 448)):
    out = []
    for L in m.layers:
        out.append(dict(s_qkv=np.abs(np.concatenate([L["wq"], L["wk"], L["wv"]])).max() / 448,
                        s_o=np.abs(L["wo"]).max() / 448, s_gu=np.abs(np.concatenate([L["wg"], L["wu"]])).max() / 448,
                        s_d=np.abs(L["wd"]).max() / 448, x_qkv=sx[0], x_o=sx[1], x_gu=sx[2], x_d=sx[3]))
    return out


def test_fp8_stack_per_sequence_equals_dense_and_stays_near_exact():
    prob = synth.make_problem("random_shared", 13, vocab=16, n_inputs=2, n_questions=5, max_content=6,
                              max_lead=4, tail_vocab=3, max_options=3, max_option_tokens=3)
    m = _model(seed=13)
    lay, x0 = _layout_and_x0(prob, 13)
    exact = OF.forward_dense(m, lay, x0)
    m.fp8 = _fp8_scales(m)
    dense = OF.forward_dense(m, lay, x0)
    for li in lay.inputs:
        lo = li.first_row
        hi = lo + int((lay.row_input == lay.row_input[lo]).sum())
        assert np.allclose(OF.forward_input(m, lay, li, x0[lo:hi]), dense[lo:hi], atol=1e-10)
    rel = np.linalg.norm(dense - exact, axis=1) / np.linalg.norm(exact, axis=1)
    assert 0 < rel.max() < 0.2   # e4m3 keeps 4 significant bits
