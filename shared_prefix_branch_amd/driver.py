"""The engine loop around libspb's calls, for one GPU.

A job is a plan plus activations: the caller supplies, per logical input, its
Q/K/V rows and hidden states (device tensors, already in the pass dtype), and
the lm head.  ``Job`` assembles each pass's token-major buffers from them by
the plan's placement, then per pass enqueues: metadata upload, branch
attention, option scoring.  The host floor join runs after all passes.
Nothing here computes the method: every step runs in libspb.
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np

from . import Plan, branch_attention, score_finalize, score_options, score_workspace_bytes


@dataclasses.dataclass
class PassBuffers:
    n_tokens: int
    q: object
    k: object
    v: object
    o: object
    hidden: object
    meta: object
    workspace: object
    lp: object
    p: object
    residual: object


Provider = Callable[[int], Tuple[object, object, object, object]]


class Job:
    """All passes of a plan, resident on one device."""

    def __init__(self, plan: Plan, hq: int, hkv: int, head_dim: int, hidden_dim: int, vocab: int,
                 qkv_dtype, out_dtype, hidden_dtype, device="cuda", scales=(1.0, 1.0, 1.0)):
        import torch
        self.torch = torch
        self.plan = plan
        self.hq, self.hkv, self.d, self.H, self.V = hq, hkv, head_dim, hidden_dim, vocab
        self.qkv_dtype, self.out_dtype, self.hidden_dtype = qkv_dtype, out_dtype, hidden_dtype
        self.device = device
        self.scales = tuple(scales)
        self.row_off, self.floor_q = plan.inputs()
        self.passes: List[PassBuffers] = []

    def _alloc(self, k: int) -> PassBuffers:
        t = self.torch
        inf = self.plan.info(k)
        n = max(1, inf["n_tokens"])
        dev = self.device
        meta = t.empty(inf["meta_bytes"], dtype=t.uint8, device=dev)
        ws = t.empty(max(256, score_workspace_bytes(self.plan, k, self.V, self.H)), dtype=t.uint8, device=dev)
        return PassBuffers(
            inf["n_tokens"],
            t.empty((n, self.hq, self.d), dtype=self.qkv_dtype, device=dev),
            t.empty((n, self.hkv, self.d), dtype=self.qkv_dtype, device=dev),
            t.empty((n, self.hkv, self.d), dtype=self.qkv_dtype, device=dev),
            t.empty((n, self.hq, self.d), dtype=self.out_dtype, device=dev),
            t.empty((n, self.H), dtype=self.hidden_dtype, device=dev),
            meta, ws,
            t.empty(max(1, inf["n_options"]), dtype=t.float32, device=dev),
            t.empty(max(1, inf["n_options"]), dtype=t.float32, device=dev),
            t.empty(max(1, inf["n_branches"]), dtype=t.float32, device=dev))

    def fill(self, k: int, buf: PassBuffers, provider: Provider, cache: Dict[int, tuple]):
        """Gathers pass k's rows from the per-input activations."""
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
            q, kk, v, h = cache[n]
            sel = np.nonzero(inp == n)[0]
            dst = t.from_numpy(sel).to(self.device)
            src = t.from_numpy(off[sel]).to(self.device)
            buf.q.index_copy_(0, dst, q.index_select(0, src))
            buf.k.index_copy_(0, dst, kk.index_select(0, src))
            buf.v.index_copy_(0, dst, v.index_select(0, src))
            buf.hidden.index_copy_(0, dst, h.index_select(0, src))

    def load(self, provider: Provider):
        """Allocates and fills every pass."""
        cache: Dict[int, tuple] = {}
        self.passes = []
        for k in range(self.plan.n_passes):
            buf = self._alloc(k)
            self.fill(k, buf, provider, cache)
            self.passes.append(buf)

    def run_pass(self, k: int, lm_head, stream=None, attention=True, scoring=True, marks=None):
        """Enqueues pass k.  ``marks``, if given, holds four created events:
        recorded on ``stream`` around the attention kernel (0, 1) and, by the
        library, around the lm-head GEMM kernel (2, 3)."""
        buf = self.passes[k]
        self.plan.upload(k, buf.meta, stream)
        if marks is not None:
            marks[0].record(stream)
        if attention:
            branch_attention(self.plan, k, buf.meta, buf.q, buf.k, buf.v, buf.o, scales=self.scales, stream=stream)
        if marks is not None:
            marks[1].record(stream)
        if scoring:
            score_options(self.plan, k, buf.meta, buf.hidden, lm_head, buf.workspace, buf.lp, buf.p, buf.residual,
                          stream=stream, gemm_events=None if marks is None else (marks[2], marks[3]))

    def run(self, lm_head, stream=None, attention=True, scoring=True, marks=None):
        for k in range(self.plan.n_passes):
            self.run_pass(k, lm_head, stream, attention, scoring, None if marks is None else marks[k])

    def pass_outputs(self, k: int):
        """Host copies of pass k's lp, p, residual."""
        inf = self.plan.info(k)
        b = self.passes[k]
        return (b.lp[:inf["n_options"]].cpu().numpy(), b.p[:inf["n_options"]].cpu().numpy(),
                b.residual[:inf["n_branches"]].cpu().numpy())

    def finalize(self) -> dict:
        outs = [self.pass_outputs(k) for k in range(self.plan.n_passes)]
        return score_finalize(self.plan, [o[0] for o in outs], [o[1] for o in outs], [o[2] for o in outs])

    def attention_by_logical_row(self, rows: Sequence[int]) -> Dict[int, object]:
        """Attention output rows (host float32 [hq, d]) keyed by logical row; a
        content row placed in several passes is returned from each (list)."""
        want = set(int(r) for r in rows)
        out: Dict[int, list] = {}
        for k in range(self.plan.n_passes):
            lr, _ = self.plan.rows(k)
            idx = [i for i, r in enumerate(lr.tolist()) if r in want]
            if not idx:
                continue
            o = self.passes[k].o[self.torch.tensor(idx, device=self.device)].float().cpu().numpy()
            for j, i in enumerate(idx):
                out.setdefault(int(lr[i]), []).append(o[j])
        return out
