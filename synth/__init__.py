"""Seeded synthetic workloads for the branch-packed scoring pass.

This module only *draws inputs*: problem structure (content lengths, question
lengths, option token ids) and activations (Q/K/V per logical token, hidden
states per logical token, lm-head weights).  It holds none of the method's
arithmetic: no attention, no softmax, no scoring, no packing.  Both the oracle
tests and the GPU path consume what it draws.

Logical problem (the shape of a scoring request once tokenised):
  * input i has a content of ``content_len[i]`` tokens and asks the questions
    ``branch_q[branch_off[i]:branch_off[i+1]]``;
  * question q has a template of ``q_len[q]`` tokens (the last one is the row
    in front of the answer slot) and options ``opt_off[q]:opt_off[q+1]``;
  * option o is the token sequence ``tok[tok_off[o]:tok_off[o+1]]``.

Logical row numbering (the data-layout convention every side uses to address
activations): inputs in order, then -- when floors are requested -- one floor
input per distinct asked question, in ascending question id.  Inside one input:
its content rows, then for every branch in order the template rows followed by
the option-trie nodes of that question.  Trie nodes are the distinct proper
prefixes of the options, numbered in order of first appearance when the options
are walked in order and each option's prefixes by increasing length.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import numpy as np

__all__ = [
    "Problem", "Dims", "Workload", "CONFIGS", "make_workload", "make_problem",
    "count_trie_nodes", "logical_inputs", "seed_for", "STREAM_INPUT",
    "STREAM_FLOOR", "STREAM_LM_HEAD", "STREAM_CALIB", "STREAM_HIDDEN",
    "ModelDims", "model_weights", "embed_block", "embed_table", "stack_fp8_scales",
]

STREAM_INPUT, STREAM_FLOOR, STREAM_LM_HEAD, STREAM_CALIB, STREAM_HIDDEN = 0, 1, 2, 3, 4
STREAM_MODEL, STREAM_EMBED, STREAM_TOKEN_EMBED = 5, 6, 7


@dataclasses.dataclass
class Problem:
    content_len: np.ndarray   # int32 [n_inputs]
    branch_off: np.ndarray    # int32 [n_inputs + 1]
    branch_q: np.ndarray      # int32 [n_branches]
    q_len: np.ndarray         # int32 [n_questions]
    opt_off: np.ndarray       # int32 [n_questions + 1]
    tok_off: np.ndarray       # int32 [n_options + 1]
    tok: np.ndarray           # int32 [n_option_tokens]
    vocab: int
    # template token ids, question after question (q_len[q] each); None: the
    # templates' tokens are not given and no template tokens are shared
    tmpl_tok: Optional[np.ndarray] = None

    @property
    def n_inputs(self) -> int:
        return int(self.content_len.shape[0])

    @property
    def n_questions(self) -> int:
        return int(self.q_len.shape[0])

    def options_of(self, q: int) -> List[tuple]:
        out = []
        for o in range(int(self.opt_off[q]), int(self.opt_off[q + 1])):
            out.append(tuple(int(t) for t in self.tok[self.tok_off[o]:self.tok_off[o + 1]]))
        return out

    def questions_of(self, i: int) -> List[int]:
        return [int(q) for q in self.branch_q[self.branch_off[i]:self.branch_off[i + 1]]]

    def template_of(self, q: int) -> tuple:
        """Template token ids of question q (requires tmpl_tok)."""
        off = int(np.sum(self.q_len[:q]))
        return tuple(int(t) for t in self.tmpl_tok[off:off + int(self.q_len[q])])

    def subset(self, inputs: Sequence[int]) -> "Problem":
        """The same questions, asked only by the listed inputs (in that order)."""
        cl = np.asarray([self.content_len[i] for i in inputs], np.int32)
        bq, off = [], [0]
        for i in inputs:
            bq.extend(self.questions_of(i))
            off.append(len(bq))
        return Problem(cl, np.asarray(off, np.int32), np.asarray(bq, np.int32),
                       self.q_len, self.opt_off, self.tok_off, self.tok, self.vocab, self.tmpl_tok)


@dataclasses.dataclass
class Dims:
    hq: int
    hkv: int
    head_dim: int
    hidden: int
    vocab: int
    dtype: str                # "f32" | "bf16" | "fp8"


@dataclasses.dataclass
class Workload:
    name: str
    cfg_seed: int
    problem: Problem
    dims: Dims
    budgets: List[int]
    floors: bool = True
    # id of each logical input: ("input", i) or ("floor", q)
    inputs: Optional[List[tuple]] = None


def count_trie_nodes(options: Sequence[tuple]) -> int:
    """Number of distinct proper prefixes of the option sequences (array sizing only)."""
    seen = set()
    for o in options:
        for k in range(1, len(o)):
            seen.add(tuple(o[:k]))
    return len(seen)


def logical_inputs(problem: Problem, floors: bool) -> List[tuple]:
    """Logical inputs in row-numbering order: ("input", i) then ("floor", q)."""
    out = [("input", i) for i in range(problem.n_inputs)]
    if floors:
        asked = sorted(set(int(q) for q in problem.branch_q))
        out += [("floor", q) for q in asked]
    return out


def input_rows(problem: Problem, which: tuple) -> int:
    """Logical rows owned by one logical input (content + templates + trie nodes)
    when no template tokens are shared; an upper bound otherwise (activation
    blocks are drawn at this size and a layout uses their first rows)."""
    kind, idx = which
    if kind == "input":
        qs = problem.questions_of(idx)
        c = int(problem.content_len[idx])
    else:
        qs = [idx]
        c = 0
    return c + sum(int(problem.q_len[q]) + count_trie_nodes(problem.options_of(q)) for q in qs)


def seed_for(cfg_seed: int, stream: int, ident: int) -> int:
    """A 63-bit seed from numpy's SeedSequence([cfg_seed, stream, ident])."""
    st = np.random.SeedSequence([int(cfg_seed), int(stream), int(ident)]).generate_state(2, np.uint32)
    return int((int(st[0]) << 31) ^ int(st[1])) & ((1 << 63) - 1)


# ----------------------------------------------------------------------------- problems

def _csr(lists):
    off = [0]
    flat = []
    for l in lists:
        flat.extend(l)
        off.append(len(flat))
    return np.asarray(off, np.int32), np.asarray(flat, np.int32)


def _single_token_options(rng, n_opts, vocab):
    ids = rng.choice(vocab, size=n_opts, replace=False)
    return [(int(t),) for t in ids]


def _prefix_free(opts):
    s = set(opts)
    if len(s) != len(opts):
        return False
    for o in opts:
        for k in range(1, len(o)):
            if tuple(o[:k]) in s:
                return False
    return True


def _label_options(rng, n_opts, max_len, vocab, lead_pool=3):
    """Multi-token labels; first tokens share a small pool so tries branch."""
    pool = rng.choice(vocab, size=lead_pool, replace=False)
    while True:
        opts = []
        for _ in range(n_opts):
            n = int(rng.integers(1, max_len + 1))
            first = int(pool[rng.integers(0, lead_pool)])
            rest = [int(t) for t in rng.integers(0, vocab, size=n - 1)]
            opts.append(tuple([first] + rest))
        if _prefix_free(opts):
            return opts


def _assemble(content_len, asks, q_len, q_opts, vocab, templates=None) -> Problem:
    branch_off, branch_q = _csr(asks)
    opt_counts = [len(o) for o in q_opts]
    opt_off = np.concatenate([[0], np.cumsum(opt_counts)]).astype(np.int32)
    flat_opts = [o for opts in q_opts for o in opts]
    tok_off, tok = _csr(flat_opts)
    tmpl = None
    if templates is not None:
        assert [len(x) for x in templates] == [int(n) for n in q_len]
        tmpl = np.asarray([t for x in templates for t in x], np.int32)
    return Problem(np.asarray(content_len, np.int32), branch_off, branch_q,
                   np.asarray(q_len, np.int32), opt_off, tok_off, tok, int(vocab), tmpl)


def _distinct_seqs(rng, n, max_len, vocab):
    """n token sequences of 1..max_len tokens with distinct first tokens."""
    firsts = rng.choice(vocab, size=n, replace=False)
    return [tuple([int(f)] + [int(x) for x in rng.integers(0, vocab, size=int(rng.integers(0, max_len)))])
            for f in firsts]


def _grid_templates(rng, vocab, lead=(8, 14), n_a=(3, 5), n_b=(3, 5)):
    """One template with two placeholders expanded into a grid of questions:
    lead-in, value of A (1-3 tokens), connector, value of B (1-2 tokens), a
    closing run ending in the answer slot."""
    lead_in = [int(x) for x in rng.integers(0, vocab, size=int(rng.integers(lead[0], lead[1] + 1)))]
    a_vals = _distinct_seqs(rng, int(rng.integers(n_a[0], n_a[1] + 1)), 3, vocab)
    mid = [int(x) for x in rng.integers(0, vocab, size=int(rng.integers(2, 5)))]
    b_vals = _distinct_seqs(rng, int(rng.integers(n_b[0], n_b[1] + 1)), 2, vocab)
    tail = [int(x) for x in rng.integers(0, vocab, size=int(rng.integers(1, 4)))]
    return [tuple(lead_in + list(a) + mid + list(b) + tail) for a in a_vals for b in b_vals]


def make_problem(name: str, cfg_seed: int, **over) -> Problem:
    """Problem structure of a named configuration (see CONFIGS)."""
    rng = np.random.default_rng(np.random.SeedSequence([cfg_seed, 99]))
    if name == "tiny":
        V = over.get("vocab", 1024)
        nq = 4
        q_len = [12] * nq
        q_opts = [_single_token_options(rng, 2, V) for _ in range(nq)]
        return _assemble([64], [list(range(nq))], q_len, q_opts, V)
    if name in ("news", "news2"):
        V = over.get("vocab", 262144)
        n_in = over.get("n_inputs", 24)
        nq = 56
        lo, hi = (14, 26) if name == "news" else (10, 19)
        q_len = rng.integers(lo, hi + 1, size=nq)
        q_opts = [_single_token_options(rng, 2, V) for _ in range(nq)]
        cl = rng.integers(440, 501, size=n_in)
        return _assemble(cl, [list(range(nq))] * n_in, q_len, q_opts, V)
    if name == "moderation":
        V = over.get("vocab", 262144)
        n_in = over.get("n_inputs", 300)
        nq = 106
        q_len = rng.integers(15, 31, size=nq)
        q_opts = [_label_options(rng, int(rng.integers(2, 6)), 3, V) for _ in range(nq)]
        cl = rng.integers(30, 121, size=n_in)
        return _assemble(cl, [list(range(nq))] * n_in, q_len, q_opts, V)
    if name == "extreme":
        V = over.get("vocab", 262144)
        n_in = over.get("n_inputs", 8)
        nq = over.get("n_questions", 1000)
        q_len = rng.integers(10, 21, size=nq)
        q_opts = [_single_token_options(rng, 2, V) for _ in range(nq)]
        cl = [over.get("content", 2000)] * n_in
        return _assemble(cl, [list(range(nq))] * n_in, q_len, q_opts, V)
    if name == "fp8":
        V = over.get("vocab", 262144)
        n_in = over.get("n_inputs", 500)
        nq = 80
        q_len = rng.integers(14, 27, size=nq)
        q_opts = [_single_token_options(rng, 2, V) for _ in range(nq)]
        cl = rng.integers(200, 801, size=n_in)
        asks = []
        for _ in range(n_in):
            k = int(rng.integers(20, 81))
            asks.append(sorted(int(q) for q in rng.choice(nq, size=k, replace=False)))
        return _assemble(cl, asks, q_len, q_opts, V)
    if name == "grid":
        # questions from placeholder templates: every content asks the grids of
        # a few templates, whose questions share lead-ins and partial fillings
        V = over.get("vocab", 262144)
        n_in = over.get("n_inputs", 16)
        templates = []
        for _ in range(over.get("n_templates", 3)):
            templates += _grid_templates(rng, V)
        nq = len(templates)
        q_opts = [_single_token_options(rng, 2, V) for _ in range(nq)]
        cl = rng.integers(over.get("min_content", 200), over.get("max_content", 400) + 1, size=n_in)
        return _assemble(cl, [list(range(nq))] * n_in, [len(x) for x in templates], q_opts, V, templates)
    if name == "random_shared":
        # small random problems whose templates share lead-ins (a pool of two)
        V = over.get("vocab", 64)
        n_in = over.get("n_inputs", 3)
        nq = over.get("n_questions", 6)
        max_c = over.get("max_content", 20)
        leads = [[int(x) for x in rng.integers(0, V, size=int(rng.integers(1, over.get("max_lead", 5) + 1)))]
                 for _ in range(2)]
        templates = []
        for _ in range(nq):
            lead = leads[int(rng.integers(0, 2))][:int(rng.integers(0, over.get("max_lead", 5) + 1))]
            rest = [int(x) for x in rng.integers(0, over.get("tail_vocab", V), size=int(rng.integers(1, 4)))]
            templates.append(tuple(lead + rest))
        q_opts = []
        for _ in range(nq):
            n_o = int(rng.integers(1, over.get("max_options", 3) + 1))
            q_opts.append(_label_options(rng, n_o, over.get("max_option_tokens", 3), V, lead_pool=min(3, V)))
        cl = rng.integers(over.get("min_content", 0), max_c + 1, size=n_in)
        asks = []
        for _ in range(n_in):
            k = int(rng.integers(1, nq + 1))
            asks.append(sorted(int(q) for q in rng.choice(nq, size=k, replace=False)))
        return _assemble(cl, asks, [len(x) for x in templates], q_opts, V, templates)
    if name == "long":
        # inputs at the request limits: one content of max_content tokens (the
        # man page's default limit is 4,096), one of 1,000-2,000 and one of at
        # most 64; templates of 100 to max_query tokens (limit 256), so a
        # branch spans several 32-key chunks; multi-token labels
        V = over.get("vocab", 1000)
        nq = over.get("n_questions", 8)
        q_len = rng.integers(100, over.get("max_query", 256) + 1, size=nq)
        q_opts = [_label_options(rng, int(rng.integers(2, 5)), 3, V) for _ in range(nq)]
        cl = [over.get("max_content", 4096), int(rng.integers(1000, 2001)), int(rng.integers(0, 65))]
        asks = [sorted(int(q) for q in rng.choice(nq, size=int(rng.integers(3, nq + 1)), replace=False))
                for _ in cl]
        return _assemble(cl, asks, q_len, q_opts, V)
    if name == "random":
        # small random problems for oracle self-tests and packer tests
        V = over.get("vocab", 64)
        n_in = over.get("n_inputs", 3)
        nq = over.get("n_questions", 4)
        max_c = over.get("max_content", 20)
        max_l = over.get("max_len", 6)
        q_len = rng.integers(1, max_l + 1, size=nq)
        q_opts = []
        for _ in range(nq):
            n_o = int(rng.integers(1, over.get("max_options", 4) + 1))
            q_opts.append(_label_options(rng, n_o, over.get("max_option_tokens", 3), V,
                                         lead_pool=min(3, V)))
        cl = rng.integers(over.get("min_content", 0), max_c + 1, size=n_in)
        asks = []
        for _ in range(n_in):
            k = int(rng.integers(1, nq + 1))
            asks.append(sorted(int(q) for q in rng.choice(nq, size=k, replace=False)))
        return _assemble(cl, asks, q_len, q_opts, V)
    raise KeyError(name)


CONFIGS: Dict[str, dict] = {
    "tiny": dict(cfg_seed=1, dims=Dims(4, 2, 64, 256, 1024, "f32"), budgets=[16384]),
    "news": dict(cfg_seed=2, dims=Dims(32, 16, 128, 3840, 262144, "bf16"), budgets=[16384]),
    "news2": dict(cfg_seed=2, dims=Dims(32, 16, 128, 3840, 262144, "bf16"), budgets=[16384]),
    "moderation": dict(cfg_seed=3, dims=Dims(32, 16, 128, 3840, 262144, "bf16"), budgets=[16384]),
    "extreme": dict(cfg_seed=4, dims=Dims(32, 8, 128, 3840, 262144, "bf16"), budgets=[16384]),
    "fp8": dict(cfg_seed=5, dims=Dims(32, 8, 128, 3840, 262144, "fp8"), budgets=[8192, 16384, 32768]),
    # template tries (grids of placeholder questions sharing template prefixes)
    "grid": dict(cfg_seed=6, dims=Dims(32, 16, 128, 3840, 262144, "bf16"), budgets=[16384]),
}


def make_workload(name: str, **over) -> Workload:
    c = CONFIGS[name]
    dims = dataclasses.replace(c["dims"], **{k: v for k, v in over.items() if k in ("hq", "hkv", "head_dim", "hidden", "vocab", "dtype")})
    pover = {k: v for k, v in over.items() if k not in ("hq", "hkv", "head_dim", "hidden", "dtype")}
    pover.setdefault("vocab", dims.vocab)
    prob = make_problem(name, c["cfg_seed"], **pover)
    wl = Workload(name, c["cfg_seed"], prob, dims, list(c["budgets"]), floors=True)
    wl.inputs = logical_inputs(prob, wl.floors)
    return wl


# ----------------------------------------------------------------------------- activations

def _torch():
    import torch
    return torch


def input_ident(which: tuple):
    kind, idx = which
    return (STREAM_INPUT, idx) if kind == "input" else (STREAM_FLOOR, idx)


# "sharp" query/key draws for parity tests that must be able to fail on the
# score arithmetic: Q, K ~ N(0, 1), so q.k / sqrt(d) has a standard deviation
# near 1 (the metric draws divide both by sqrt(d) again, which leaves scores
# of std 1/d and a softmax that is almost a plain average), and a few planted
# key rows scaled by SHARP_PLANT, whose scores (std about SHARP_PLANT) often
# rise far above the maximum of the chunks before them.  Planted rows: inside
# the content, the rows whose index is SHARP_CONTENT_AT mod SHARP_CONTENT_EVERY
# (so never in the first 64-key chunk); after the content, the rows whose
# offset from the content end is SHARP_TAIL_AT mod SHARP_TAIL_EVERY (inside a
# template's first chunk of 32 keys, and again in every later one).
SHARP_PLANT = 6.0
SHARP_CONTENT_AT, SHARP_CONTENT_EVERY = 100, 128
SHARP_TAIL_AT, SHARP_TAIL_EVERY = 7, 32


def sharp_plant_rows(content: int, n_rows: int) -> np.ndarray:
    """Boolean mask over a logical input's rows: the planted key rows."""
    r = np.arange(n_rows)
    tail = r - content
    return np.where(r < content, r % SHARP_CONTENT_EVERY == SHARP_CONTENT_AT,
                    tail % SHARP_TAIL_EVERY == SHARP_TAIL_AT)


def activation_block(wl: Workload, which: tuple, device="cpu", peaked: bool = False, sharp: bool = False):
    """Q, K, V [rows, H*, d] (float32, before any dtype cast) and hidden [rows, H]
    for every logical row of one logical input, drawn from its own seed.

    Q, K, V ~ N(0,1)/sqrt(d); hidden ~ N(0,1)/sqrt(H) (``peaked``: N(0,1)).
    ``sharp``: Q, K ~ N(0,1) with planted key rows (see SHARP_PLANT); V and
    hidden as above.  The same seed draws the same normals in every mode.
    """
    torch = _torch()
    stream, ident = input_ident(which)
    n = input_rows(wl.problem, which)
    d = wl.dims
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(wl.cfg_seed, stream, ident))
    s = 1.0 / np.sqrt(d.head_dim)
    sqk = 1.0 if sharp else s
    q = torch.randn((n, d.hq, d.head_dim), generator=g, device=device) * sqk
    k = torch.randn((n, d.hkv, d.head_dim), generator=g, device=device) * sqk
    v = torch.randn((n, d.hkv, d.head_dim), generator=g, device=device) * s
    if sharp:
        c = int(wl.problem.content_len[ident]) if which[0] == "input" else 0
        plant = torch.from_numpy(sharp_plant_rows(c, n)).to(device)
        k[plant] *= SHARP_PLANT
    g2 = torch.Generator(device=device)
    g2.manual_seed(seed_for(wl.cfg_seed, STREAM_HIDDEN, ident if stream == STREAM_INPUT else 10_000_000 + ident))
    h = torch.randn((n, d.hidden), generator=g2, device=device)
    if not peaked:
        h = h / np.sqrt(d.hidden)
    return q, k, v, h


def lm_head(wl: Workload, device="cpu", dtype=None):
    """W [V, H] ~ N(0, 0.02^2), cast to bf16 (RNE) unless ``dtype`` says otherwise."""
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(wl.cfg_seed, STREAM_LM_HEAD, 0))
    w = torch.empty((wl.dims.vocab, wl.dims.hidden), device=device, dtype=torch.float32)
    # row blocks keep peak host memory low for the 262,144 x 3,840 head
    blk = 16384
    for r0 in range(0, wl.dims.vocab, blk):
        r1 = min(wl.dims.vocab, r0 + blk)
        w[r0:r1] = torch.randn((r1 - r0, wl.dims.hidden), generator=g, device=device) * 0.02
    return w.to(dtype if dtype is not None else torch.bfloat16)


def fp8_scales(wl: Workload, calib_tokens: int = 4096, sharp: bool = False):
    """Per-tensor e4m3 scales s = amax / 448 for Q, K, V from a separate seeded
    calibration draw of the same distribution (static calibration); ``sharp``
    calibrates on the sharp draws, planted key rows included (the calibration
    tokens read as one content)."""
    torch = _torch()
    d = wl.dims
    g = torch.Generator()
    g.manual_seed(seed_for(wl.cfg_seed, STREAM_CALIB, 0))
    s = 1.0 / np.sqrt(d.head_dim)
    sqk = 1.0 if sharp else s
    q = torch.randn((calib_tokens, d.hq, d.head_dim), generator=g) * sqk
    k = torch.randn((calib_tokens, d.hkv, d.head_dim), generator=g) * sqk
    v = torch.randn((calib_tokens, d.hkv, d.head_dim), generator=g) * s
    if sharp:
        k[torch.from_numpy(sharp_plant_rows(calib_tokens, calib_tokens))] *= SHARP_PLANT
    return tuple(float(t.abs().max()) / 448.0 for t in (q, k, v))


def to_e4m3(x, scale: float):
    """Quantise x / scale to OCP e4m3fn bytes: saturate to +-448, then round to
    nearest even (torch's float8_e4m3fn cast).  Returns a uint8 tensor."""
    torch = _torch()
    y = (x.float() / scale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return y.view(torch.uint8)


def cast_inputs(wl: Workload, q, k, v, scales=None):
    """Cast float32 Q/K/V to the workload's input dtype.  Returns (q, k, v) as
    float32 (f32 workloads), bfloat16, or uint8 e4m3 bytes (fp8)."""
    torch = _torch()
    dt = wl.dims.dtype
    if dt == "f32":
        return q.float(), k.float(), v.float()
    if dt == "bf16":
        return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    if dt == "fp8":
        sq, sk, sv = scales
        return to_e4m3(q, sq), to_e4m3(k, sk), to_e4m3(v, sv)
    raise ValueError(dt)


# ----------------------------------------------------------------------------- decoder stack

@dataclasses.dataclass
class ModelDims:
    """A decoder stack over the packed pass (synthetic weights)."""
    hidden: int
    hq: int
    hkv: int
    head_dim: int
    ffn: int          # gated MLP width
    layers: int
    rope_base: float = 10000.0
    eps: float = 1e-6


MODEL_CONFIGS = {
    # the news attention shape with a 4x gated MLP
    "news": ModelDims(3840, 32, 16, 128, 15360, 2),
    # small shapes the oracle runs in seconds
    "small": ModelDims(256, 4, 2, 64, 512, 2),
    "small_d128": ModelDims(512, 8, 4, 128, 768, 2),
}


def model_weights(md: ModelDims, seed: int, device="cpu"):
    """Per layer: wq [Hq*d, H], wk / wv [Hkv*d, H], wo [H, Hq*d], wg / wu [F, H],
    wd [H, F], each ~ N(0, 1/fan_in) and cast to bf16 (RNE); RMS gains g_attn,
    g_mlp [H] ~ U(0.5, 1.5) as bf16; and the final gain g_final.  Returns
    (list of per-layer dicts, g_final)."""
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(seed, STREAM_MODEL, 0))
    H, F = md.hidden, md.ffn
    qd, kd = md.hq * md.head_dim, md.hkv * md.head_dim

    def mat(rows, fan_in):
        return (torch.randn((rows, fan_in), generator=g, device=device) / np.sqrt(fan_in)).to(torch.bfloat16)

    def gain():
        return (0.5 + torch.rand((H,), generator=g, device=device)).to(torch.bfloat16)

    layers = []
    for _ in range(md.layers):
        layers.append(dict(wq=mat(qd, H), wk=mat(kd, H), wv=mat(kd, H), wo=mat(H, qd),
                           wg=mat(F, H), wu=mat(F, H), wd=mat(H, F), g_attn=gain(), g_mlp=gain()))
    return layers, gain()


def embed_block(wl: Workload, md: ModelDims, which: tuple, device="cpu"):
    """Input embeddings x0 [rows, H] ~ N(0, 1) (float32) for every logical row
    of one logical input, from its own seed (a stand-in for token embeddings:
    the problem carries no content token ids)."""
    torch = _torch()
    stream, ident = input_ident(which)
    n = input_rows(wl.problem, which)
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(wl.cfg_seed, STREAM_EMBED, ident if stream == STREAM_INPUT else 10_000_000 + ident))
    return torch.randn((n, md.hidden), generator=g, device=device)


def embed_table(md: ModelDims, vocab: int, seed: int, device="cpu"):
    """Embedding rows of decoded tokens: E [vocab, H] ~ N(0, 1), cast to bf16."""
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(seed, STREAM_TOKEN_EMBED, 0))
    return torch.randn((vocab, md.hidden), generator=g, device=device).to(torch.bfloat16)


# static input scales of the fp8 linears: rmsnorm outputs (gains up to 1.5,
# tails to about 5 sigma), attention outputs (convex mixes of v rows) and the
# gated MLP product (heavier tails); values beyond saturate at +-448 * s
FP8_INPUT_AMAX = {"qkv": 8.0, "o": 4.0, "gu": 8.0, "d": 16.0}


def stack_fp8_scales(layers):
    """Per layer the static e4m3 scales of the fp8 linears: s_* = amax(W) / 448
    over each (fused) weight, x_* = FP8_INPUT_AMAX / 448 for its input."""
    torch = _torch()
    out = []
    for L in layers:
        def amax(*ws):
            return max(float(w.float().abs().max()) for w in ws)
        s = dict(s_qkv=amax(L["wq"], L["wk"], L["wv"]) / 448.0, s_o=amax(L["wo"]) / 448.0,
                 s_gu=amax(L["wg"], L["wu"]) / 448.0, s_d=amax(L["wd"]) / 448.0)
        s.update({"x_" + k: v / 448.0 for k, v in FP8_INPUT_AMAX.items()})
        out.append(s)
    return out
