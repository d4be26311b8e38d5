"""The decoder stack around branch attention, in float64 (oracle).

TEST INFRASTRUCTURE ONLY -- see the package header.

What is computed.  The engine runs a whole decoder model over the packed pass
and feeds its last hidden states to the lm head [PyPI "spinf-serve 0.1.1",
"Layout": the engine does one packed forward; models/ holds one stack per
architecture family].  The pages name the model family but not the layer's
equations, so the reading taken is the plain pre-norm decoder layer:

    h  = rmsnorm(x) * g_attn
    q  = rope(h Wq^T),  k = rope(h Wk^T),  v = h Wv^T      (per head)
    x <- x + attention(q, k, v) Wo^T
    h  = rmsnorm(x) * g_mlp
    x <- x + (silu(h Wg^T) * (h Wu^T)) Wd^T

and after the last layer the head reads rmsnorm(x) * g_final.

  * rmsnorm(x) = x / sqrt(mean(x^2) + eps) over the hidden dimension.
  * silu(z) = z / (1 + exp(-z)).
  * rope: the rotary position embedding of Su et al. (RoFormer): within each
    head, the pair of dimensions (2i, 2i+1) is rotated by the angle
    pos * base^(-2i/d); (a, b) -> (a cos t - b sin t, a sin t + b cos t).
  * attention: causal softmax attention with scale 1/sqrt(d), query head h
    reading key/value head h // (Hq/Hkv), as in ``oracle.attention``.
  * positions: a row's position is its index on its own root path (content
    token t at t, template token j at C + j, the trie node of depth k at
    C + L - 1 + k), so each question sees the positions it would have as its
    own prompt -- the pages' "the same answers" as running each question on
    its own [PyPI "Speed and scale"].

fp8 linears (the pages' checkpoints are calibrated static fp8 [man page
"spinf-serve", DESCRIPTION: fp8s]; reading: every linear layer of the stack
quantizes its weight and its input per tensor with static scales,
q8(t, s) = round_to_e4m3(t / s) * s, and multiplies the quantized values
exactly; the fused q/k/v and gate/up weights share one scale each;
attention and the lm head keep their bf16 inputs):

    y = q8(x, s_x) q8(W, s_w)^T

Form (i)  ``forward_input``: the model run over ordinary sequences: the
          content; content + template for each branch (keeping the template
          rows); the root path of each trie node (keeping its last row).
Form (ii) ``forward_dense``: layer by layer over all logical rows at once,
          attention under the dense tree mask of ``oracle.attention``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Iterable, List, Optional

import numpy as np

from .attention import causal_attention_tail, dense_mask
from .numerics import round_to_e4m3, to_f64
from .tree import Layout, LInput, root_path


@dataclasses.dataclass
class Model:
    """float64 weights of the stack; see ``from_synth``."""
    hidden: int
    hq: int
    hkv: int
    head_dim: int
    rope_base: float
    eps: float
    layers: List[dict]
    g_final: np.ndarray
    # per layer, with fp8 linears: weight scales s_qkv, s_o, s_gu, s_d and
    # input scales x_qkv, x_o, x_gu, x_d; None: exact linears
    fp8: Optional[List[dict]] = None

    @staticmethod
    def from_synth(md, layers, g_final, fp8_scales=None) -> "Model":
        return Model(md.hidden, md.hq, md.hkv, md.head_dim, float(md.rope_base), float(md.eps),
                     [{k: to_f64(v) for k, v in L.items()} for L in layers], to_f64(g_final),
                     None if fp8_scales is None else [dict(s) for s in fp8_scales])


def q8(t: np.ndarray, s: float) -> np.ndarray:
    """Per-tensor e4m3 quantization with scale s, as float64 values."""
    return round_to_e4m3(np.asarray(t, np.float64) / s) * s


def _lin(m: Model, li: int, x: np.ndarray, w: np.ndarray, kind: str) -> np.ndarray:
    """x W^T, with the layer's fp8 quantization of both when the model has it."""
    if m.fp8 is None:
        return x @ w.T
    f = m.fp8[li]
    return q8(x, f["x_" + kind]) @ q8(w, f["s_" + kind]).T


def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g over the last axis."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def rope(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """x [n, heads, d], pos [n]: dims (2i, 2i+1) of every head rotated by
    pos * base^(-2i/d)."""
    n, _, d = x.shape
    i = np.arange(d // 2)
    ang = np.asarray(pos, np.float64)[:, None] * base ** (-2.0 * i / d)[None, :]  # [n, d/2]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    a, b = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def _qkv(m: Model, li: int, x: np.ndarray, pos: np.ndarray):
    L = m.layers[li]
    n = x.shape[0]
    h = rms_norm(x, L["g_attn"], m.eps)
    w = np.concatenate([L["wq"], L["wk"], L["wv"]], axis=0)  # one fused linear
    y = _lin(m, li, h, w, "qkv")
    qd, kd = m.hq * m.head_dim, m.hkv * m.head_dim
    q = y[:, :qd].reshape(n, m.hq, m.head_dim)
    k = y[:, qd:qd + kd].reshape(n, m.hkv, m.head_dim)
    v = y[:, qd + kd:].reshape(n, m.hkv, m.head_dim)
    return rope(q, pos, m.rope_base), rope(k, pos, m.rope_base), v


def _mlp(m: Model, li: int, x: np.ndarray) -> np.ndarray:
    L = m.layers[li]
    h = rms_norm(x, L["g_mlp"], m.eps)
    F = L["wg"].shape[0]
    gu = _lin(m, li, h, np.concatenate([L["wg"], L["wu"]], axis=0), "gu")  # one fused linear
    return _lin(m, li, silu(gu[:, :F]) * gu[:, F:], L["wd"], "d")


def decoder_sequence(m: Model, x0: np.ndarray) -> np.ndarray:
    """The stack over one ordinary sequence x0 [n, H] at positions 0 .. n-1.
    Returns the head's input rmsnorm(x) * g_final at every position."""
    x = np.array(x0, dtype=np.float64)
    n = x.shape[0]
    pos = np.arange(n)
    scale = 1.0 / math.sqrt(m.head_dim)
    for li, L in enumerate(m.layers):
        q, k, v = _qkv(m, li, x, pos)
        att = causal_attention_tail(q, k, v, scale).reshape(n, m.hq * m.head_dim)
        x = x + _lin(m, li, att, L["wo"], "o")
        x = x + _mlp(m, li, x)
    return rms_norm(x, m.g_final, m.eps)


def forward_input(m: Model, layout: Layout, li: LInput, x0: np.ndarray,
                  branches: Optional[Iterable[int]] = None, content: bool = True) -> np.ndarray:
    """Form (i) for one logical input: x0 holds its own rows (index 0 =
    ``li.first_row``).  Rows not computed are NaN."""
    n = x0.shape[0]
    out = np.full((n, m.hidden), np.nan)
    base, C = li.first_row, li.C
    if content and C > 0:
        out[:C] = decoder_sequence(m, x0[:C])
    want = range(len(li.branches)) if branches is None else branches
    for bi in want:
        b = li.branches[bi]
        tmpl = np.asarray(b.template_rows, np.int64) - base
        seq = np.r_[0:C, tmpl]
        out[tmpl] = decoder_sequence(m, x0[seq])[C:]
        for ni in range(len(b.trie.prefixes)):
            x = b.node_row0 + ni
            path = np.asarray(root_path(layout, x)) - base
            out[x - base] = decoder_sequence(m, x0[path])[-1]
    return out


def positions(layout: Layout) -> np.ndarray:
    """Each logical row's position: its index on its own root path."""
    return np.array([len(root_path(layout, x)) - 1 for x in range(layout.n_rows)], np.int64)


def forward_dense(m: Model, layout: Layout, x0: np.ndarray) -> np.ndarray:
    """Form (ii): all logical rows layer by layer, attention under the dense
    tree mask.  x0 [n_rows, H] in logical row order.  Small problems only."""
    x = np.array(x0, dtype=np.float64)
    n = x.shape[0]
    pos = positions(layout)
    mask = dense_mask(layout)
    scale = 1.0 / math.sqrt(m.head_dim)
    g = m.hq // m.hkv
    for li, L in enumerate(m.layers):
        q, k, v = _qkv(m, li, x, pos)
        att = np.empty((n, m.hq, m.head_dim))
        for h in range(m.hq):
            s = (q[:, h, :] @ k[:, h // g, :].T) * scale
            s = np.where(mask, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            att[:, h, :] = (p / p.sum(axis=1, keepdims=True)) @ v[:, h // g, :]
        x = x + _lin(m, li, att.reshape(n, -1), L["wo"], "o")
        x = x + _mlp(m, li, x)
    return rms_norm(x, m.g_final, m.eps)
