"""Searched decoding of extraction slots, in float64 (oracle).

TEST INFRASTRUCTURE ONLY -- see the package header.

What the pages fix.  Besides scoring, a template can hold a slot -- {*}
text, {n} a number, {$} an amount -- whose contents are decoded from the same
read, with their probabilities; the response lists the most likely answers
with their probabilities [PyPI "spinf-serve 0.1.1", "What it does":
Extraction and generation; article, after the response example].  A
searched slot costs about as much as a few hundred scoring tokens, and the
slots of many inputs are decoded together [PyPI "Speed and scale"].

Reading taken (the search itself is not described): beam search of width B.
  * lp(x | s) is the model's next-token log-probability after the sequence s:
    the log-softmax over the whole vocabulary of z = W h, h the head's input
    at s's last position (the same vocab-wide log-probability as option
    scoring);
  * step 0 extends the template itself; every later step extends each
    unfinished beam by one token; a candidate's score is the sum of its
    tokens' lps;
  * only the slot kind's tokens are proposed (the whole vocabulary for {*});
    the stop token is always proposed and finishes a candidate;
  * finished beams stay candidates with their scores; the B best candidates
    are kept, ordered by score (descending), then by the earlier beam, then
    by the smaller token id;
  * after T tokens, or once every beam is finished, the B beams are the
    answers (tokens, lp, p = exp(lp), finished or cut at T).
"""
from __future__ import annotations

import dataclasses
from typing import Callable, List, Optional, Sequence

import numpy as np

from .forward import Model, decoder_sequence


@dataclasses.dataclass
class Beam:
    tokens: tuple
    lp: float
    finished: bool


def beam_search(next_lp: Callable[[tuple], np.ndarray], B: int, T: int, stop: int,
                allowed: Optional[Sequence[int]] = None, margins: Optional[list] = None) -> List[Beam]:
    """next_lp(tokens) -> float64 [V] log-probabilities of the next token after
    the slot's prefix followed by ``tokens``.  ``margins``, if given, receives
    per step the score gap between the last kept and the first dropped
    candidate (how close the step was to a different choice)."""
    first = next_lp(())
    V = first.shape[0]
    cand_ids = np.arange(V) if allowed is None else np.unique(np.r_[np.asarray(allowed, np.int64), stop])
    # step 0: the template's own next-token distribution
    ranked = sorted(cand_ids.tolist(), key=lambda x: (-first[x], x))
    order = ranked[:B]
    if margins is not None and len(ranked) > B:
        margins.append(float(first[ranked[B - 1]] - first[ranked[B]]))
    beams = [Beam((x,), float(first[x]), x == stop) for x in order]
    for _ in range(1, T):
        if all(b.finished for b in beams):
            break
        cands = []  # (score, parent, token, beam)
        for bi, b in enumerate(beams):
            if b.finished:
                cands.append((b.lp, bi, -1, b))
                continue
            lp = next_lp(b.tokens)
            for x in cand_ids.tolist():
                cands.append((b.lp + float(lp[x]), bi, x, None))
        cands.sort(key=lambda c: (-c[0], c[1], c[2]))
        if margins is not None and len(cands) > B:
            margins.append(cands[B - 1][0] - cands[B][0])
        nxt = []
        for score, bi, x, kept in cands[:B]:
            if kept is not None:
                nxt.append(kept)
            else:
                nxt.append(Beam(beams[bi].tokens + (x,), score, x == stop))
        beams = nxt
    return beams


def log_softmax(z: np.ndarray) -> np.ndarray:
    m = np.max(z)
    return z - (m + np.log(np.sum(np.exp(z - m))))


def model_next_lp(m: Model, x0_prefix: np.ndarray, embed: np.ndarray, W: np.ndarray):
    """next_lp for a slot whose prefix (content + template, in path order) has
    input embeddings x0_prefix: a decoded token x enters the stack as
    embed[x]; W is the lm head [V, H]."""
    cache = {}

    def f(tokens: tuple) -> np.ndarray:
        if tokens not in cache:
            seq = x0_prefix if not tokens else np.concatenate([x0_prefix, embed[list(tokens)]], axis=0)
            h = decoder_sequence(m, seq)[-1]
            cache[tokens] = log_softmax(W @ h)
        return cache[tokens]

    return f
