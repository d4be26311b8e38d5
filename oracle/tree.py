"""The logical token tree of a scoring problem (oracle).

TEST INFRASTRUCTURE ONLY -- see the package header.

What the pages fix, restated:
  * one input is a content read once, with every question laid out as a branch
    of that read; a question's template stops at the position of its answer
    [PyPI "spinf-serve 0.1.1", "What it does": Scoring; Many questions, one read];
  * templates and options are compiled to token tries, and scoring is one packed
    forward over them [PyPI, "Layout": protocol/compiler/packer/scorer];
  * the floor is the same question asked of empty content [PyPI, "What it
    does"; article "Bulk classification and decision inference on one GPU",
    the paragraph after the response example].

Readings taken where the pages are silent (listed with the others in the design
notes): the row in front of the answer slot -- the template's last token --
predicts an option's first token; an option of n tokens feeds its n-1 proper
prefixes as trie nodes, shared by options with a common prefix; "empty
content" is a content of zero tokens.

Every logical token has a parent in the tree; its root path (the tokens it
attends to, itself last) is the chain of ancestors:
  content token t     -> content token t-1 (t = 0: none)
  template token 0    -> last content token (C = 0: none)
  template token j    -> template token j-1
  trie node, depth 1  -> last template token
  trie node, depth k  -> the trie node of its first k-1 tokens

Template tries [PyPI "Layout": the engine compiles templates into token
tries; "What it does": placeholder values expand one template into many
questions].  When the
templates' token ids are given, the questions of one input share the tokens
of common template prefixes.  Reading taken: a prefix of a question's template
up to (not including) its last token is shared when at least two of the
input's questions start with it; the last token -- the answer slot -- is
always the question's own.  A shared token is one logical token (one row, one
set of activations) whose parent is the shared token before it (or the last
content token); a question's own template tokens follow its last shared token.
Logical rows of an input: the content, then for each question in order the
shared tokens of its template not yet numbered, its own template tokens and
its option-trie nodes.  Without template token ids nothing is shared.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Tuple

import numpy as np


@dataclasses.dataclass
class Trie:
    """Proper prefixes of one question's options, in first-appearance order."""
    prefixes: List[tuple]
    index: Dict[tuple, int]
    # per option: list of (source, token); source -1 = template's last token,
    # else a node index; step k predicts token k of the option from source k
    chains: List[List[Tuple[int, int]]]


def build_trie(options: List[tuple]) -> Trie:
    prefixes: List[tuple] = []
    index: Dict[tuple, int] = {}
    for o in options:
        for k in range(1, len(o)):
            p = tuple(o[:k])
            if p not in index:
                index[p] = len(prefixes)
                prefixes.append(p)
    chains = []
    for o in options:
        steps = []
        for k in range(len(o)):
            src = -1 if k == 0 else index[tuple(o[:k])]
            steps.append((src, int(o[k])))
        chains.append(steps)
    return Trie(prefixes, index, chains)


@dataclasses.dataclass
class LBranch:
    input_no: int         # logical input number (row-numbering order)
    question: int
    first_row: int        # logical row of the question's first own template token
    L: int                # own template tokens (the whole template when nothing is shared)
    node_row0: int        # logical row of trie node 0
    trie: Trie
    is_floor: bool
    stem_rows: List[int] = dataclasses.field(default_factory=list)  # shared template tokens, in order

    @property
    def template_rows(self) -> List[int]:
        """Logical rows of the whole template, in order (shared, then own)."""
        return list(self.stem_rows) + list(range(self.first_row, self.first_row + self.L))

    @property
    def last_row(self) -> int:
        return self.first_row + self.L - 1

    def row_of(self, src: int) -> int:
        return self.last_row if src < 0 else self.node_row0 + src


@dataclasses.dataclass
class LInput:
    kind: str             # "input" | "floor"
    ident: int            # input index, or question id for a floor
    first_row: int
    C: int
    branches: List[LBranch]


@dataclasses.dataclass
class Layout:
    inputs: List[LInput]
    n_rows: int
    parent: np.ndarray    # int64 [n_rows], -1 = root
    # per row: (logical input number, kind code, branch index within input or -1,
    #           position: content index / template index / node index)
    row_input: np.ndarray
    row_kind: np.ndarray  # 0 content, 1 template, 2 trie node
    row_branch: np.ndarray  # branch index within the input; -1 for content and shared template tokens
    row_pos: np.ndarray   # content index / template index / trie node index
    # per row: the template token ids from the template's start through this
    # row (template rows), the whole template (trie nodes), None (content);
    # only when template token ids are given
    row_tprefix: list = None

    def branches(self):
        for li in self.inputs:
            for b in li.branches:
                yield b


def build_layout(problem, floors: bool = True) -> Layout:
    """Logical rows of every input (then one floor input per distinct asked
    question when ``floors``), with their tree parents."""
    tries = {}

    def trie_of(q):
        if q not in tries:
            opts = []
            for o in range(int(problem.opt_off[q]), int(problem.opt_off[q + 1])):
                opts.append(tuple(int(t) for t in problem.tok[problem.tok_off[o]:problem.tok_off[o + 1]]))
            tries[q] = build_trie(opts)
        return tries[q]

    plan = []
    for i in range(len(problem.content_len)):
        qs = [int(q) for q in problem.branch_q[problem.branch_off[i]:problem.branch_off[i + 1]]]
        plan.append(("input", i, int(problem.content_len[i]), qs))
    if floors:
        for q in sorted(set(int(q) for q in problem.branch_q)):
            plan.append(("floor", q, 0, [q]))

    has_tmpl = getattr(problem, "tmpl_tok", None) is not None

    def template(q):
        off = int(np.sum(problem.q_len[:q]))
        return tuple(int(x) for x in problem.tmpl_tok[off:off + int(problem.q_len[q])])

    parent, r_in, r_kind, r_br, r_pos, r_tp = [], [], [], [], [], []
    inputs = []
    row = 0
    for n, (kind, ident, C, qs) in enumerate(plan):
        li = LInput(kind, ident, row, C, [])
        for t in range(C):
            parent.append(row + t - 1 if t > 0 else -1)
            r_in.append(n); r_kind.append(0); r_br.append(-1); r_pos.append(t); r_tp.append(None)
        row += C
        last_content = li.first_row + C - 1 if C > 0 else -1
        # shared template prefixes: those at least two of the input's
        # questions start with, never including a question's last token
        shared = [0] * len(qs)
        if has_tmpl:
            count = {}
            for q in qs:
                T = template(q)
                for k in range(1, len(T)):
                    count[T[:k]] = count.get(T[:k], 0) + 1
            for bi, q in enumerate(qs):
                T = template(q)
                s = 0
                while s < len(T) - 1 and count[T[:s + 1]] >= 2:
                    s += 1
                shared[bi] = s
        stem_row = {}
        for bi, q in enumerate(qs):
            L = int(problem.q_len[q])
            T = template(q) if has_tmpl else None
            s = shared[bi]
            stem = []
            for k in range(1, s + 1):
                p = T[:k]
                if p not in stem_row:
                    stem_row[p] = row
                    parent.append(stem_row[T[:k - 1]] if k > 1 else last_content)
                    r_in.append(n); r_kind.append(1); r_br.append(-1); r_pos.append(k - 1); r_tp.append(p)
                    row += 1
                stem.append(stem_row[p])
            tr = trie_of(q)
            own = L - s
            b = LBranch(n, q, row, own, row + own, tr, kind == "floor", stem)
            for j in range(own):
                parent.append(row + j - 1 if j > 0 else (stem[-1] if stem else last_content))
                r_in.append(n); r_kind.append(1); r_br.append(bi); r_pos.append(s + j)
                r_tp.append(T[:s + j + 1] if has_tmpl else None)
            for ni, p in enumerate(tr.prefixes):
                par = b.last_row if len(p) == 1 else b.node_row0 + tr.index[p[:-1]]
                parent.append(par)
                r_in.append(n); r_kind.append(2); r_br.append(bi); r_pos.append(ni)
                r_tp.append(T if has_tmpl else None)
            row += own + len(tr.prefixes)
            li.branches.append(b)
        inputs.append(li)
    return Layout(inputs, row, np.asarray(parent, np.int64), np.asarray(r_in, np.int64),
                  np.asarray(r_kind, np.int64), np.asarray(r_br, np.int64), np.asarray(r_pos, np.int64),
                  r_tp if has_tmpl else None)


def root_path(layout: Layout, x: int) -> List[int]:
    """Logical rows row x attends to, root first, x last."""
    path = []
    while x >= 0:
        path.append(int(x))
        x = int(layout.parent[x])
    return path[::-1]


def scored_rows(layout: Layout) -> List[int]:
    """Rows whose next-token distribution is needed: each template's last token
    and every trie node."""
    out = []
    for b in layout.branches():
        out.append(b.last_row)
        out.extend(range(b.node_row0, b.node_row0 + len(b.trie.prefixes)))
    return out
