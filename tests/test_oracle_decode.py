"""Pins of the oracle's searched decoding (oracle/decode.py), on the CPU:
brute-force enumeration when the beam holds every candidate, greedy decoding
at width 1, exact tie-breaks worked by hand, the allowed-token set, and the
model's next-token distribution against the forward and scoring oracles."""
import itertools
import math

import numpy as np
import pytest

import synth
from oracle import decode as OD
from oracle import forward as OF
from oracle import tree as OT


def _table_lp(V, seed):
    """A fixed next-token log-probability for every prefix (hashed)."""
    def f(tokens):
        rng = np.random.default_rng([seed] + [t + 1 for t in tokens])
        return OD.log_softmax(rng.normal(size=V) * 2)
    return f


def test_full_width_equals_brute_force():
    V, T, stop = 3, 3, 2
    f = _table_lp(V, 5)
    beams = OD.beam_search(f, 1000, T, stop)
    want = []
    for n in range(1, T + 1):
        for seq in itertools.product(range(V), repeat=n):
            if stop in seq[:-1]:
                continue
            if seq[-1] != stop and n < T:
                continue  # unfinished sequences only end at the length limit
            lp = sum(f(seq[:i])[seq[i]] for i in range(n))
            want.append((seq, lp, seq[-1] == stop))
    want.sort(key=lambda w: -w[1])
    assert [(b.tokens, b.finished) for b in beams] == [(w[0], w[2]) for w in want]
    assert np.allclose([b.lp for b in beams], [w[1] for w in want], atol=1e-12)


def test_width_one_is_greedy():
    V, T, stop = 7, 6, 3
    f = _table_lp(V, 9)
    seq = ()
    while len(seq) < T:
        lp = f(seq)
        x = int(np.argmax(lp))
        seq += (x,)
        if x == stop:
            break
    (b,) = OD.beam_search(f, 1, T, stop)
    assert b.tokens == seq and b.finished == (seq[-1] == stop)


def test_exact_ties_by_hand():
    # lp: token 0 -> -1, token 1 -> -2, stop (2) -> -3 after every prefix, so
    # scores are exact integers and ties are broken by beam, then token:
    # step 1 keeps (0,0) -2, (0,1) -3, (1,0) -3 and drops (2,) -3 (a later beam);
    # step 2 keeps (0,0,0) -3, (0,0,1) -4, (0,1,0) -4
    f = lambda tokens: np.array([-1.0, -2.0, -3.0])  # noqa: E731
    beams = OD.beam_search(f, 3, 3, 2)
    assert [b.tokens for b in beams] == [(0, 0, 0), (0, 0, 1), (0, 1, 0)]
    assert [b.lp for b in beams] == [-3.0, -4.0, -4.0]
    assert not any(b.finished for b in beams)
    # with width 4 the finished (2,) -3 is kept, after the -3 candidates of earlier beams
    beams = OD.beam_search(f, 4, 2, 2)
    assert [(b.tokens, b.finished) for b in beams] == [((0, 0), False), ((0, 1), False), ((1, 0), False),
                                                       ((2,), True)]


def test_allowed_tokens_and_stop():
    f = _table_lp(6, 3)
    beams = OD.beam_search(f, 5, 4, 5, allowed=[1, 3])
    assert beams and all(set(b.tokens) <= {1, 3, 5} for b in beams)
    assert all(b.finished == (b.tokens[-1] == 5) for b in beams)
    assert all((5 not in b.tokens[:-1]) for b in beams)


def test_model_next_lp_matches_forward_and_head():
    prob = synth.make_problem("random", 2, vocab=40, n_inputs=1, n_questions=2, max_content=6, max_len=4,
                              max_options=2, max_option_tokens=1)
    lay = OT.build_layout(prob, floors=False)
    rng = np.random.default_rng(0)
    H = 16
    m = OF.Model(H, 2, 1, 8, 10000.0, 1e-6,
                 [dict(wq=rng.normal(size=(16, H)) / 4, wk=rng.normal(size=(8, H)) / 4,
                       wv=rng.normal(size=(8, H)) / 4, wo=rng.normal(size=(H, 16)) / 4,
                       wg=rng.normal(size=(24, H)) / 4, wu=rng.normal(size=(24, H)) / 4,
                       wd=rng.normal(size=(H, 24)) / 5, g_attn=np.ones(H), g_mlp=np.ones(H))], np.ones(H))
    x0 = rng.normal(size=(lay.n_rows, H))
    E = rng.normal(size=(40, H))
    W = rng.normal(size=(40, H))
    li = lay.inputs[0]
    b = li.branches[1]
    path = OT.root_path(lay, b.last_row)
    f = OD.model_next_lp(m, x0[path], E, W)
    hid = OF.forward_input(m, lay, li, x0)[b.last_row]
    z = W @ hid
    assert np.allclose(f(()), z - (z.max() + math.log(np.exp(z - z.max()).sum())), atol=1e-12)
    # one decoded token is one more position on the same sequence
    seq = np.concatenate([x0[path], E[[7]]])
    z2 = W @ OF.decoder_sequence(m, seq)[-1]
    assert np.allclose(f((7,)), OD.log_softmax(z2), atol=1e-12)
    assert abs(np.exp(f(())).sum() - 1) < 1e-12
