"""Branch attention, computed two plain ways in float64 (oracle).

TEST INFRASTRUCTURE ONLY -- see the package header.

What is computed: every token attends to its own content and the causal prefix
of its own branch (and, for an option trie node, the node's own prefix chain),
never to another branch or another input.  The pages state the result, not the
kernel: the content is read once and every question is a branch of the same
pass, and the answers are the same as asking each question as its own prompt
over a prefix cache [PyPI "spinf-serve 0.1.1", "What it does"; "Speed and
scale": "for the same answers"; article "Bulk classification and decision
inference on one GPU", benchmark paragraph].  So the plain definition is: row x
equals the last row of ordinary causal softmax attention over x's root path.

Readings (the pages are silent): the softmax scale is 1/sqrt(head_dim) unless
given; with grouped query heads, query head h reads key/value head
h // (Hq / Hkv) (consecutive groups).

Form (i)  ``attention_input``: for each input, causal attention over its
          content; for each branch, causal attention over content + template,
          keeping the template rows; for each trie node, attention over its
          root path.
Form (ii) ``attention_dense``: one masked softmax over all logical rows with a
          dense mask written from the structural rule (same input; content keys
          causal for content rows, all content for branch rows; template keys
          of the own branch, causal for template rows; trie-node keys that are
          prefixes of the row's own node).  Small problems only.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional

import numpy as np

from .tree import Layout, LInput, root_path


def causal_attention_tail(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Textbook causal attention for the last m positions of a sequence.

    q [m, Hq, d]: queries at positions n-m .. n-1; k, v [n, Hkv, d].
    Returns [m, Hq, d]; query i sees keys 0 .. n-m+i.
    """
    m, hq, d = q.shape
    n, hkv, _ = k.shape
    g = hq // hkv
    pos = np.arange(n - m, n)
    allowed = np.arange(n)[None, :] <= pos[:, None]
    out = np.empty((m, hq, d), dtype=np.float64)
    for h in range(hq):
        kh = k[:, h // g, :]
        vh = v[:, h // g, :]
        s = (q[:, h, :] @ kh.T) * scale
        s = np.where(allowed, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ vh
    return out


def attention_input(layout: Layout, li: LInput, q: np.ndarray, k: np.ndarray, v: np.ndarray,
                    scale: Optional[float] = None, branches: Optional[Iterable[int]] = None,
                    content: bool = True) -> np.ndarray:
    """Form (i) for one logical input.

    q, k, v hold the input's own rows (index 0 = ``li.first_row``), float64.
    ``branches``: indices of the branches to compute (default all); rows not
    computed are NaN.  ``content``: also compute the content rows.
    """
    n = q.shape[0]
    hq, d = q.shape[1], q.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.full((n, hq, d), np.nan)
    C = li.C
    base = li.first_row
    if content and C > 0:
        out[:C] = causal_attention_tail(q[:C], k[:C], v[:C], scale)
    want = range(len(li.branches)) if branches is None else branches
    for bi in want:
        b = li.branches[bi]
        # content then the whole template (shared tokens first): every template
        # token attends causally along this sequence
        tmpl = np.asarray(b.template_rows, np.int64) - base
        seq = np.r_[0:C, tmpl]
        out[tmpl] = causal_attention_tail(q[tmpl], k[seq], v[seq], scale)
        for ni in range(len(b.trie.prefixes)):
            x = b.node_row0 + ni
            path = np.asarray(root_path(layout, x)) - base
            out[x - base:x - base + 1] = causal_attention_tail(q[x - base:x - base + 1], k[path], v[path], scale)
    return out


def dense_mask(layout: Layout) -> np.ndarray:
    """Mask[i, j] = row i attends to row j, from the structural rule."""
    N = layout.n_rows
    kind = layout.row_kind
    inp = layout.row_input
    br = layout.row_branch
    pos = layout.row_pos
    prefix = {}
    for li_no, li in enumerate(layout.inputs):
        for bi, b in enumerate(li.branches):
            for ni, p in enumerate(b.trie.prefixes):
                prefix[b.node_row0 + ni] = p
    tp = layout.row_tprefix
    M = np.zeros((N, N), dtype=bool)
    for i in range(N):
        for j in range(N):
            if inp[i] != inp[j]:
                continue
            if kind[j] == 0:
                M[i, j] = (pos[j] <= pos[i]) if kind[i] == 0 else True
            elif kind[j] == 1 and br[j] < 0:
                # a shared template token: seen by the shared tokens whose prefix
                # extends its own, and by the template tokens and trie nodes of
                # every question whose template starts with its prefix and goes
                # on past it (a question's last token is never shared)
                if kind[i] == 0 or len(tp[j]) > len(tp[i]) or tp[i][:len(tp[j])] != tp[j]:
                    continue
                if br[i] >= 0:
                    full = len(layout.inputs[inp[i]].branches[br[i]].template_rows)
                    M[i, j] = len(tp[j]) < full
                else:
                    M[i, j] = True
            elif kind[j] == 1:
                if kind[i] == 0 or br[i] != br[j]:
                    continue
                M[i, j] = (pos[j] <= pos[i]) if kind[i] == 1 else True
            else:
                if kind[i] != 2 or br[i] != br[j]:
                    continue
                pi, pj = prefix[i], prefix[j]
                M[i, j] = len(pj) <= len(pi) and pi[:len(pj)] == pj
    return M


def attention_dense(layout: Layout, q: np.ndarray, k: np.ndarray, v: np.ndarray,
                    scale: Optional[float] = None, mask: Optional[np.ndarray] = None) -> np.ndarray:
    """Form (ii): masked softmax over all logical rows (small problems)."""
    N, hq, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if mask is None:
        mask = dense_mask(layout)
    out = np.empty((N, hq, d))
    for h in range(hq):
        s = (q[:, h, :] @ k[:, h // g, :].T) * scale
        s = np.where(mask, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, h // g, :]
    return out
