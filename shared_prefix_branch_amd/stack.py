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

from . import (LINEAR_F32, LINEAR_QKV_ROPE, LINEAR_RESIDUAL, LINEAR_SILU_GATE, MAX_SLOT_RANGES, Plan,
               PreparedAttention, PreparedLinear, PreparedNorm, beam_step, decode_attention, gather_rows, rope_table,
               topk_lse)
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
                 batch_head: bool = False, lm_head_kind: int = 0, n_pos: int = 8192, keep_kv: bool = False):
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
        self.keep_kv = bool(keep_kv)  # keep every layer's K/V of the pass (for slot decoding)

    def _alloc(self, k: int) -> PassBuffers:
        t = self.torch
        buf = super()._alloc(k)
        n = max(1, buf.n_tokens)
        md = self.md
        buf.x0 = t.empty((n, md.hidden), dtype=t.float32, device=self.device)
        buf.x = t.empty((n, md.hidden), dtype=t.float32, device=self.device)
        buf.h = t.empty((n, md.hidden), dtype=t.bfloat16, device=self.device)
        buf.act = t.empty((n, md.ffn), dtype=t.bfloat16, device=self.device)
        buf.kv = [(buf.k, buf.v)]
        if self.keep_kv:
            for _ in range(1, md.layers):
                buf.kv.append((t.empty_like(buf.k), t.empty_like(buf.v)))
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
        for k, buf in enumerate(self.passes):
            n = buf.n_tokens
            ops = []
            if n > 0:
                x, h = buf.x[:n], buf.h[:n]
                o2 = buf.o.reshape(buf.o.shape[0], -1)[:n]
                for li, W in enumerate(self.W):
                    kk, vv = buf.kv[li % len(buf.kv)]
                    ops.append(PreparedNorm(x, W["g_attn"], h, md.eps))
                    ops.append(PreparedLinear(h, W["wqkv"], LINEAR_QKV_ROPE, q=buf.q[:n], k_out=kk[:n],
                                              v=vv[:n], hq=md.hq, hkv=md.hkv, head_dim=md.head_dim,
                                              pos=buf.pos[:n], rope=self.rope))
                    ops.append(PreparedAttention(k, buf.meta, buf.q, kk, vv, buf.o))
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
            if isinstance(op, PreparedAttention):
                op(plan, stream)
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


class SlotDecoder:
    """Searched decoding of slot questions on the read a ``ForwardJob``
    (built with ``keep_kv=True``) has run: per pass, the B beams of all its
    slots advance together, one decode step per token (see spb_decode.hip).

    slots: per slot a dict(branch=logical branch id, stop=token, mask=row of
    ``masks`` or -1 for the whole vocabulary); embed: bf16 [V, H] embedding
    rows of decoded tokens; lm_head: bf16 [V, H]; masks: int32 [n_masks,
    ceil(V / 32)] allowed-token bit sets (device) or None."""

    def __init__(self, job: ForwardJob, embed, lm_head, slots: List[dict], beams: int, max_tokens: int,
                 masks=None):
        import torch
        t = torch
        self.job, self.embed, self.W = job, embed, lm_head
        self.B, self.T, self.k = int(beams), int(max_tokens), int(beams)
        self.masks = masks
        md, dev = job.md, job.device
        self.by_pass = {}
        for i, s in enumerate(slots):
            info = job.plan.slot(s["branch"])
            self.by_pass.setdefault(info["pass"], []).append((i, s, info))
        self.n_slots = len(slots)
        self._runs = []
        V = lm_head.shape[0]
        for k, items in sorted(self.by_pass.items()):
            S = len(items)
            R = S * self.B
            buf = job.passes[k]
            i32 = dict(dtype=t.int32, device=dev)
            rng = np.zeros((S, MAX_SLOT_RANGES, 2), np.int32)
            nrg = np.zeros(S, np.int32)
            for j, (_, s, info) in enumerate(items):
                nrg[j] = len(info["ranges"])
                rng[j, :nrg[j]] = np.asarray(info["ranges"], np.int32)
            run = dict(
                pass_=k, items=items, S=S, R=R,
                ranges=t.from_numpy(rng).to(dev), n_ranges=t.from_numpy(nrg).to(dev),
                slot_rows=t.tensor([info["row"] for _, _, info in items], **i32),
                slot_pos=t.tensor([info["position"] for _, _, info in items], **i32),
                stop=t.tensor([s["stop"] for _, s, _ in items], **i32),
                mask0=t.tensor([s.get("mask", -1) for _, s, _ in items], **i32),
                stop_r=t.tensor([s["stop"] for _, s, _ in items for _ in range(self.B)], **i32),
                mask_r=t.tensor([s.get("mask", -1) for _, s, _ in items for _ in range(self.B)], **i32),
                h0=t.empty((S, md.hidden), dtype=t.bfloat16, device=dev),
                z0=t.empty((S, V), dtype=t.float32, device=dev),
                ids0=t.empty((S, self.k), **i32), lp0=t.empty((S, self.k), dtype=t.float32, device=dev),
                lse0=t.empty(S, dtype=t.float32, device=dev),
                x=t.empty((R, md.hidden), dtype=t.float32, device=dev),
                h=t.empty((R, md.hidden), dtype=t.bfloat16, device=dev),
                q=t.empty((R, md.hq, md.head_dim), dtype=t.bfloat16, device=dev),
                o=t.empty((R, md.hq, md.head_dim), dtype=t.bfloat16, device=dev),
                act=t.empty((R, md.ffn), dtype=t.bfloat16, device=dev),
                hid=t.empty((R, md.hidden), dtype=t.bfloat16, device=dev),
                z=t.empty((R, V), dtype=t.float32, device=dev),
                ids=t.empty((R, self.k), **i32), lp=t.empty((R, self.k), dtype=t.float32, device=dev),
                lse=t.empty(R, dtype=t.float32, device=dev),
                pos=t.empty(R, **i32), feed=t.empty(R, **i32),
                kdec=[t.empty((self.T * R, md.hkv, md.head_dim), dtype=t.bfloat16, device=dev)
                      for _ in range(md.layers)],
                vdec=[t.empty((self.T * R, md.hkv, md.head_dim), dtype=t.bfloat16, device=dev)
                      for _ in range(md.layers)],
                state=[dict(tok=t.empty((R, self.T), **i32), len=t.empty(R, **i32), fin=t.empty(R, **i32),
                            path=t.empty((R, self.T), **i32), nb=t.empty(S, **i32),
                            score=t.empty(R, dtype=t.float32, device=dev)) for _ in range(2)])
            self._runs.append(run)
            self._prepare(run, buf)

    def _prepare(self, run, buf):
        """Marshals every call of the run once (step 0 and steps 1 .. T-1)."""
        job, md = self.job, self.job.md
        S, R, B = run["S"], run["R"], self.B
        ops0 = [gather_rows(buf.hidden, run["slot_rows"], S, dst_bf16=run["h0"]),
                PreparedLinear(run["h0"], self.W, LINEAR_F32, yf=run["z0"]),
                topk_lse(run["z0"], self.k, run["ids0"], run["lp0"], run["lse0"], masks=self.masks,
                         mask_of_row=run["mask0"] if self.masks is not None else None, stop_of_row=run["stop"]),
                beam_step(S, B, self.k, self.T, 0, run["stop"], run["ids0"], run["lp0"], None, run["state"][0],
                          run["feed"])]
        steps = []
        for st in range(1, self.T):
            cur, nxt = run["state"][(st - 1) % 2], run["state"][st % 2]
            ops = [gather_rows(self.embed, run["feed"], R, dst_f32=run["x"], pos=run["pos"], pos_base=run["slot_pos"],
                               per=B, pos_add=st)]
            for li, W in enumerate(job.W):
                kp, vp = buf.kv[li % len(buf.kv)]
                kd = run["kdec"][li][(st - 1) * R:st * R]
                vd = run["vdec"][li][(st - 1) * R:st * R]
                ops.append(PreparedNorm(run["x"], W["g_attn"], run["h"], md.eps))
                ops.append(PreparedLinear(run["h"], W["wqkv"], LINEAR_QKV_ROPE, q=run["q"], k_out=kd, v=vd,
                                          hq=md.hq, hkv=md.hkv, head_dim=md.head_dim, pos=run["pos"], rope=job.rope))
                ops.append(decode_attention(run["q"], kp, vp, run["kdec"][li], run["vdec"][li], run["o"], B,
                                            run["ranges"], run["n_ranges"], cur["path"], st - 1))
                ops.append(PreparedLinear(run["o"].reshape(R, -1), W["wo"], LINEAR_RESIDUAL, resid=run["x"]))
                ops.append(PreparedNorm(run["x"], W["g_mlp"], run["h"], md.eps))
                ops.append(PreparedLinear(run["h"], W["wgu"], LINEAR_SILU_GATE, y=run["act"]))
                ops.append(PreparedLinear(run["act"], W["wd"], LINEAR_RESIDUAL, resid=run["x"]))
            ops.append(PreparedNorm(run["x"], job.g_final, run["hid"], md.eps))
            ops.append(PreparedLinear(run["hid"], self.W, LINEAR_F32, yf=run["z"]))
            ops.append(topk_lse(run["z"], self.k, run["ids"], run["lp"], run["lse"], masks=self.masks,
                                mask_of_row=run["mask_r"] if self.masks is not None else None,
                                stop_of_row=run["stop_r"]))
            ops.append(beam_step(S, B, self.k, self.T, st, run["stop"], run["ids"], run["lp"], cur, nxt, run["feed"]))
            steps.append(ops)
        run["ops0"], run["steps"] = ops0, steps

    def run(self, stream=None):
        """Enqueues every pass's decoding (after the job's run on the same stream)."""
        for run in self._runs:
            for op in run["ops0"]:
                op(stream)
            for ops in run["steps"]:
                for op in ops:
                    op(stream)

    def results(self) -> List[List[dict]]:
        """Per slot (in the order given): its beams, best first, as dicts
        tokens / lp / finished (host; waits for the device)."""
        out = [None] * self.n_slots
        for run in self._runs:
            st = run["state"][(self.T - 1) % 2]
            tok = st["tok"].cpu().numpy()
            ln = st["len"].cpu().numpy()
            fin = st["fin"].cpu().numpy()
            sc = st["score"].cpu().numpy()
            nb = st["nb"].cpu().numpy()
            for j, (i, s, info) in enumerate(run["items"]):
                beams = []
                for b in range(int(nb[j])):
                    r = j * self.B + b
                    beams.append(dict(tokens=tuple(int(x) for x in tok[r, :ln[r]]), lp=float(sc[r]),
                                      finished=bool(fin[r])))
                out[i] = beams
        return out
