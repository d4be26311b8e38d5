"""The decoder stack over each pass, for one GPU.

``ForwardJob`` is a ``Job`` whose hidden states are not given but computed:
the caller supplies, per logical input, the input embeddings x0 of its rows
(f32), and the stack's weights; per pass and run the job enqueues, after the
metadata upload:

    x = x0
    per layer:  h = rmsnorm(x) * g_attn                       spb_rmsnorm
                q, k, v = h [Wq; Wk; Wv]^T, RoPE on q and k     spb_linear (QKV_ROPE)
                o = branch attention(q, k, v)                  spb_branch_attention
                x += o Wo^T                                    spb_linear (RESIDUAL)
                h = rmsnorm(x) * g_mlp                          spb_rmsnorm
                a = silu(h Wg^T) * (h Wu^T)                     spb_linear (SILU_GATE)
                x += a Wd^T                                    spb_linear (RESIDUAL)
    hidden = rmsnorm(x) * g_final                               spb_rmsnorm

then the lm head and the floor join as for ``Job``.  Every step runs in
libspb; this module only lays out buffers and orders the calls.
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np

from . import (LINEAR_QKV_ROPE, LINEAR_RESIDUAL, LINEAR_SILU_GATE, Plan, PreparedLinear, PreparedNorm,
               rope_table)
from .driver import Job, PassBuffers


def gate_up_rows(wg, wu):
    """W for the SILU_GATE epilogue: blocks of 64 rows, the 32 gate rows then
    the 32 matching up rows."""
    import torch
    F, K = wg.shape
    return torch.stack([wg.reshape(F // 32, 32, K), wu.reshape(F // 32, 32, K)], dim=1).reshape(2 * F, K).contiguous()


class ForwardJob(Job):
    """All passes of a plan with the decoder stack in front of the head.

    md: model dims (hidden, hq, hkv, head_dim, ffn, layers, rope_base, eps);
    layers: per layer dict of bf16 device tensors wq, wk, wv, wo, wg, wu, wd,
    g_attn, g_mlp; g_final: bf16 [hidden].  n_pos bounds the positions the
    rotary table covers (content + template + option depth)."""

    def __init__(self, plan: Plan, md, layers: List[dict], g_final, vocab: int, device="cuda",
                 batch_head: bool = False, lm_head_kind: int = 0, n_pos: int = 8192):
        import torch
        super().__init__(plan, md.hq, md.hkv, md.head_dim, md.hidden, vocab, torch.bfloat16, torch.bfloat16,
                         torch.bfloat16, device=device, batch_head=batch_head, lm_head_kind=lm_head_kind)
        self.md = md
        self.W = []
        for L in layers:
            self.W.append(dict(
                wqkv=torch.cat([L["wq"], L["wk"], L["wv"]], 0).to(device).contiguous(),
                wo=L["wo"].to(device).contiguous(),
                wgu=gate_up_rows(L["wg"].to(device), L["wu"].to(device)),
                wd=L["wd"].to(device).contiguous(),
                g_attn=L["g_attn"].to(device).contiguous(), g_mlp=L["g_mlp"].to(device).contiguous()))
        self.g_final = g_final.to(device).contiguous()
        self.rope = torch.from_numpy(rope_table(n_pos, md.head_dim, md.rope_base)).to(device)
        self.n_pos = int(n_pos)
        self.lin_marks = None  # optional: per pass, per layer, 4 (begin, end) event pairs

    def _alloc(self, k: int) -> PassBuffers:
        t = self.torch
        buf = super()._alloc(k)
        n = max(1, buf.n_tokens)
        md = self.md
        buf.x0 = t.empty((n, md.hidden), dtype=t.float32, device=self.device)
        buf.x = t.empty((n, md.hidden), dtype=t.float32, device=self.device)
        buf.h = t.empty((n, md.hidden), dtype=t.bfloat16, device=self.device)
        buf.act = t.empty((n, md.ffn), dtype=t.bfloat16, device=self.device)
        pos = self.plan.positions(k)
        if pos.size and int(pos.max()) >= self.n_pos:
            raise ValueError(f"positions up to {int(pos.max())} need n_pos > {self.n_pos}")
        buf.pos = t.zeros(n, dtype=t.int32, device=self.device)
        if pos.size:
            buf.pos[:pos.size] = t.from_numpy(pos).to(self.device)
        return buf

    def fill(self, k: int, buf: PassBuffers, provider, cache):
        """Gathers pass k's input embeddings from the per-input blocks."""
        t = self.torch
        lr, _ = self.plan.rows(k)
        if len(lr) == 0:
            return
        inp = np.searchsorted(self.row_off, lr, side="right") - 1
        off = lr - self.row_off[inp]
        for n in np.unique(inp):
            if n not in cache:
                if len(cache) >= 4:
                    cache.pop(next(iter(cache)))
                cache[n] = provider(int(n))
            x0 = cache[n]
            sel = np.nonzero(inp == n)[0]
            buf.x0.index_copy_(0, t.from_numpy(sel).to(self.device), x0.index_select(0, t.from_numpy(off[sel]).to(self.device)))

    def load(self, provider):
        super().load(provider)
        md = self.md
        self._ops = []
        for buf in self.passes:
            n = buf.n_tokens
            ops = []
            if n > 0:
                x, h = buf.x[:n], buf.h[:n]
                o2 = buf.o.reshape(buf.o.shape[0], -1)[:n]
                for W in self.W:
                    ops.append(PreparedNorm(x, W["g_attn"], h, md.eps))
                    ops.append(PreparedLinear(h, W["wqkv"], LINEAR_QKV_ROPE, q=buf.q[:n], k_out=buf.k[:n],
                                              v=buf.v[:n], hq=md.hq, hkv=md.hkv, head_dim=md.head_dim,
                                              pos=buf.pos[:n], rope=self.rope))
                    ops.append("attention")
                    ops.append(PreparedLinear(o2, W["wo"], LINEAR_RESIDUAL, resid=x))
                    ops.append(PreparedNorm(x, W["g_mlp"], h, md.eps))
                    ops.append(PreparedLinear(h, W["wgu"], LINEAR_SILU_GATE, y=buf.act[:n]))
                    ops.append(PreparedLinear(buf.act[:n], W["wd"], LINEAR_RESIDUAL, resid=x))
                ops.append(PreparedNorm(x, self.g_final, buf.hidden[:n], md.eps))
            self._ops.append(ops)

    def _forward(self, k: int, plan: Plan, stream):
        buf = self.passes[k]
        if buf.n_tokens == 0:
            return
        with self.torch.cuda.stream(stream):
            buf.x.copy_(buf.x0, non_blocking=True)
        marks = None if self.lin_marks is None else self.lin_marks[k]
        li = 0
        for op in self._ops[k]:
            if isinstance(op, str):
                self._attn[k](plan, stream)
            elif isinstance(op, PreparedLinear):
                op(stream, None if marks is None else marks[li])
                li += 1
            else:
                op(stream)

    def hidden_by_logical_row(self, rows):
        """Final hidden rows (host float32 [H]) keyed by logical row; a row
        placed in several passes is returned from each (list)."""
        want = set(int(r) for r in rows)
        out = {}
        for k in range(self.plan.n_passes):
            lr, _ = self.plan.rows(k)
            idx = [i for i, r in enumerate(lr.tolist()) if r in want]
            if not idx:
                continue
            hdn = self.passes[k].hidden[self.torch.tensor(idx, device=self.device)].float().cpu().numpy()
            for j, i in enumerate(idx):
                out.setdefault(int(lr[i]), []).append(hdn[j])
        return out
