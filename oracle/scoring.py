"""Option scores from the scored rows, in float64 (oracle).

TEST INFRASTRUCTURE ONLY -- see the package header.

What the pages fix [article "Bulk classification and decision inference on one
GPU", the response example and the paragraph after it; PyPI "spinf-serve
0.1.1", "What it does": Scoring]:
  * each option has a log-probability under the model's full next-token
    distribution (``logprob``);
  * ``p`` is the probability among the given options: the options'
    probabilities renormalised to sum to one;
  * ``residual`` is the probability mass left to tokens other than the options:
    one minus the options' total probability;
  * ``floor_p`` is ``p`` for the same question on empty content; the lift,
    ``p - floor_p``, measures the content's own contribution.
The lm head's output precision [man page "spinf-serve", PARAMETERS: --lm-head]
is one of f32out (the default: f32 logits), bf16 or fp32.  The oracle keeps
float64 throughout and models the kinds as: f32out and fp32, the exact
product of the hidden rows it is given with W (the caller passes bf16-rounded
rows for f32out, unrounded f32 rows for fp32); bf16, that product rounded to
the nearest bf16 before the log-sum-exp and the option gather (reading: the
logits themselves are bf16).

Readings (pages silent): a multi-token option's log-probability is the chain
rule along its trie path, sum over k of log softmax(z_{k-1})[t_k], where
z_0 is the logit row of the template's last token and z_k that of the trie
node of the first k tokens; the lift is a difference, per option.
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Dict, List, Sequence, Tuple

import numpy as np

from .numerics import round_to_bf16, to_f64
from .tree import Layout, LBranch


def logits(W, h_rows: np.ndarray, rows_per_block: int = 8192) -> np.ndarray:
    """z = h W^T in float64 for every vocabulary entry.

    W: [V, H] (torch bf16/f32 tensor or numpy); h_rows: [M, H] float64.
    Vocabulary rows are converted to float64 a block at a time; each z entry is
    one dot product, so the blocking only bounds memory.
    """
    V = W.shape[0]
    h = np.asarray(h_rows, dtype=np.float64)
    z = np.empty((h.shape[0], V), dtype=np.float64)
    for r0 in range(0, V, rows_per_block):
        r1 = min(V, r0 + rows_per_block)
        z[:, r0:r1] = h @ to_f64(W[r0:r1]).T
    return z


def logsumexp(z: np.ndarray) -> np.ndarray:
    """log sum exp over the last axis, the textbook max-shifted form."""
    m = np.max(z, axis=-1, keepdims=True)
    return (m + np.log(np.sum(np.exp(z - m), axis=-1, keepdims=True)))[..., 0]


@dataclasses.dataclass
class BranchScores:
    lp: np.ndarray        # [n_options] vocab-wide log-probability
    p: np.ndarray         # [n_options] renormalised over the options
    residual: float       # 1 - sum(exp(lp))
    floor_p: np.ndarray = None
    lift: np.ndarray = None


def option_logprobs(b: LBranch, lse: Dict[int, float], z_at: Callable[[int, int], float]) -> np.ndarray:
    """Chain rule over the option trie: lp_o = sum_k z_{src_k}[t_k] - LSE(src_k)."""
    lp = np.empty(len(b.trie.chains))
    for o, steps in enumerate(b.trie.chains):
        acc = 0.0
        for src, tok in steps:
            r = b.row_of(src)
            acc += z_at(r, tok) - lse[r]
        lp[o] = acc
    return lp


def renormalise(lp: np.ndarray) -> np.ndarray:
    """p over the given options: softmax of the log-probabilities."""
    m = np.max(lp)
    e = np.exp(lp - m)
    return e / np.sum(e)


def residual(lp: np.ndarray) -> float:
    """Probability outside the options, 1 - sum(exp(lp)), as -expm1(logsumexp)."""
    m = np.max(lp)
    return float(-np.expm1(m + np.log(np.sum(np.exp(lp - m)))))


LM_HEAD_KINDS = ("f32out", "bf16", "fp32")


def score_branches(layout: Layout, hidden: Callable[[Sequence[int]], np.ndarray], W,
                   branches: Sequence[LBranch] = None, lm_head: str = "f32out") -> Dict[Tuple[int, int], BranchScores]:
    """Scores of the listed branches (default: all), keyed (input number, question).

    ``hidden(rows)`` returns the float64 hidden states [len(rows), H] of the
    given logical rows.  ``lm_head``: the output kind (see the header).
    """
    if lm_head not in LM_HEAD_KINDS:
        raise ValueError(f"lm_head must be one of {LM_HEAD_KINDS}")
    if branches is None:
        branches = list(layout.branches())
    rows: List[int] = []
    for b in branches:
        rows.append(b.last_row)
        rows.extend(range(b.node_row0, b.node_row0 + len(b.trie.prefixes)))
    rows = sorted(set(rows))
    at = {r: i for i, r in enumerate(rows)}
    z = logits(W, hidden(rows))
    if lm_head == "bf16":
        z = round_to_bf16(z)
    lse_v = logsumexp(z)
    lse = {r: float(lse_v[at[r]]) for r in rows}

    def z_at(r, t):
        return float(z[at[r], t])

    out = {}
    for b in branches:
        lp = option_logprobs(b, lse, z_at)
        out[(b.input_no, b.question)] = BranchScores(lp, renormalise(lp), residual(lp))
    return out


def join_floors(layout: Layout, scores: Dict[Tuple[int, int], BranchScores]) -> None:
    """floor_p = p of the same question's floor branch; lift = p - floor_p."""
    floor_of = {}
    for n, li in enumerate(layout.inputs):
        if li.kind == "floor":
            floor_of[li.ident] = n
    for (n, q), s in scores.items():
        if layout.inputs[n].kind != "input":
            continue
        f = scores.get((floor_of.get(q, -1), q))
        if f is None:
            continue
        s.floor_p = f.p.copy()
        s.lift = s.p - f.p
