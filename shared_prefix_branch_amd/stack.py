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

then the lm head and the floor join as for ``Job``.  With ``fp8_scales``
the four linears run on e4m3 operands: the weights are quantized once at
load, each input right before its linear (spb_quantize_e4m3), with static
per-tensor scales.  Every step runs in libspb; this module only lays out
buffers and orders the calls.
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np

from . import (LINEAR_F32, LINEAR_QKV_ROPE, LINEAR_RESIDUAL, LINEAR_SILU_GATE, MAX_SLOT_RANGES, Plan,
               PreparedAttention, PreparedLinear, PreparedNorm, beam_step, decode_attention, gather_rows,
               quantize_e4m3, rope_table, topk_lse)
from .driver import Job, PassBuffers


class _Quant:
    """An e4m3 quantization step of ForwardJob's op list (marshalled once)."""

    def __init__(self, src, dst, scale):
        self.call = quantize_e4m3(src, dst, scale)


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
                 batch_head: bool = False, lm_head_kind: int = 0, n_pos: int = 8192, keep_kv: bool = False,
                 fp8_scales: Optional[List[dict]] = None, head_rows: int = 0):
        import torch
        super().__init__(plan, md.hq, md.hkv, md.head_dim, md.hidden, vocab, torch.bfloat16, torch.bfloat16,
                         torch.bfloat16, device=device, batch_head=batch_head, lm_head_kind=lm_head_kind,
                         head_rows=head_rows)
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
        self.fp8 = fp8_scales
        if fp8_scales is not None:
            # weights to e4m3 once, with their per-tensor scales
            for W, s in zip(self.W, fp8_scales):
                for name, key in (("wqkv", "qkv"), ("wo", "o"), ("wgu", "gu"), ("wd", "d")):
                    q = torch.empty(W[name].shape, dtype=torch.uint8, device=device)
                    quantize_e4m3(W[name], q, s["s_" + key])()
                    W[name + "8"] = q
                torch.cuda.synchronize()
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
        if self.fp8 is not None:  # e4m3 copies of the linears' inputs
            buf.h8 = t.empty((n, md.hidden), dtype=t.uint8, device=self.device)
            buf.o8 = t.empty((n, md.hq * md.head_dim), dtype=t.uint8, device=self.device)
            buf.a8 = t.empty((n, md.ffn), dtype=t.uint8, device=self.device)
        buf.kv = [(buf.k, buf.v)]
        if self.keep_kv:
            # every layer's K/V, all passes in one buffer per layer (slot decoding
            # reads the prefixes of every pass's slots from it in one launch)
            o, rows = self.kv_off[k], buf.k.shape[0]
            buf.kv = [(K[o:o + rows], V[o:o + rows]) for K, V in self.kv_global]
            buf.k, buf.v = buf.kv[0]
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
        t = self.torch
        md = self.md
        if self.keep_kv:
            rows = [max(1, self.plan.info(k)["n_tokens"]) for k in range(self.plan.n_passes)]
            self.kv_off = np.r_[0, np.cumsum(rows)].astype(np.int64).tolist()
            shape = (self.kv_off[-1], md.hkv, md.head_dim)
            self.kv_global = [(t.empty(shape, dtype=t.bfloat16, device=self.device),
                               t.empty(shape, dtype=t.bfloat16, device=self.device)) for _ in range(md.layers)]
        super().load(provider)
        self._ops = []
        for k, buf in enumerate(self.passes):
            n = buf.n_tokens
            ops = []
            if n > 0:
                x, h = buf.x[:n], buf.h[:n]
                o2 = buf.o.reshape(buf.o.shape[0], -1)[:n]
                for li, W in enumerate(self.W):
                    kk, vv = buf.kv[li % len(buf.kv)]
                    lin_in = self._lin_inputs(buf, li, n, ops)
                    ops.append(PreparedNorm(x, W["g_attn"], h, md.eps))
                    xin, wq, sc = lin_in("qkv", h, W)
                    ops.append(PreparedLinear(xin, wq, LINEAR_QKV_ROPE, q=buf.q[:n], k_out=kk[:n],
                                              v=vv[:n], hq=md.hq, hkv=md.hkv, head_dim=md.head_dim,
                                              pos=buf.pos[:n], rope=self.rope, fp8_scales=sc))
                    ops.append(PreparedAttention(k, buf.meta, buf.q, kk, vv, buf.o))
                    xin, wq, sc = lin_in("o", o2, W)
                    ops.append(PreparedLinear(xin, wq, LINEAR_RESIDUAL, resid=x, fp8_scales=sc))
                    ops.append(PreparedNorm(x, W["g_mlp"], h, md.eps))
                    xin, wq, sc = lin_in("gu", h, W)
                    ops.append(PreparedLinear(xin, wq, LINEAR_SILU_GATE, y=buf.act[:n], fp8_scales=sc))
                    xin, wq, sc = lin_in("d", buf.act[:n], W)
                    ops.append(PreparedLinear(xin, wq, LINEAR_RESIDUAL, resid=x, fp8_scales=sc))
                ops.append(PreparedNorm(x, self.g_final, buf.hidden[:n], md.eps))
            self._ops.append(ops)

    def _lin_inputs(self, buf, li: int, n: int, ops: list):
        """For a linear of layer li: (its input operand, its weight, fp8 scales
        or None); with fp8 it first appends the quantization of the input."""
        names = {"qkv": "wqkv", "o": "wo", "gu": "wgu", "d": "wd"}
        dst = {"qkv": "h8", "o": "o8", "gu": "h8", "d": "a8"}

        def f(kind, x, W):
            if self.fp8 is None:
                return x, W[names[kind]], None
            s = self.fp8[li]
            xq = getattr(buf, dst[kind])[:n]
            ops.append(_Quant(x, xq, s["x_" + kind]))
            return xq, W[names[kind] + "8"], (s["x_" + kind], s["s_" + kind])
        return f

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
            elif isinstance(op, _Quant):
                op.call(stream)
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
    (built with ``keep_kv=True``) has run: the B beams of every slot, of every
    pass, advance together, one decode step per token (see spb_decode.hip).

    slots: per slot a dict(branch=logical branch id, stop=token, mask=row of
    ``masks`` or -1 for the whole vocabulary); embed: bf16 [V, H] embedding
    rows of decoded tokens; lm_head: bf16 [V, H]; masks: int32 [n_masks,
    ceil(V / 32)] allowed-token bit sets (device) or None."""

    def __init__(self, job: ForwardJob, embed, lm_head, slots: List[dict], beams: int, max_tokens: int,
                 masks=None):
        import torch
        t = torch
        if not job.keep_kv:
            raise ValueError("slot decoding needs a ForwardJob built with keep_kv=True")
        if job.fp8 is not None:
            raise ValueError("slot decoding runs the bf16 stack")
        self.job, self.embed, self.W = job, embed, lm_head
        self.B, self.T, self.k = int(beams), int(max_tokens), int(beams)
        self.masks = masks
        md, dev = job.md, job.device
        items = []
        for i, s in enumerate(slots):
            items.append((i, s, job.plan.slot(s["branch"])))
        items.sort(key=lambda it: (it[2]["pass"], it[0]))  # slots grouped by pass
        self.items = items
        S = len(items)
        R = S * self.B
        V = lm_head.shape[0]
        i32 = dict(dtype=t.int32, device=dev)
        rng = np.zeros((S, MAX_SLOT_RANGES, 2), np.int32)
        nrg = np.zeros(S, np.int32)
        for j, (_, s, info) in enumerate(items):
            nrg[j] = len(info["ranges"])
            rng[j, :nrg[j]] = np.asarray(info["ranges"], np.int32)
            rng[j, :nrg[j], 0] += job.kv_off[info["pass"]]
        self.S, self.R = S, R
        f32 = dict(dtype=t.float32, device=dev)
        bf = dict(dtype=t.bfloat16, device=dev)
        self.buf = dict(
            ranges=t.from_numpy(rng).to(dev), n_ranges=t.from_numpy(nrg).to(dev),
            slot_pos=t.tensor([info["position"] for _, _, info in items], **i32),
            stop=t.tensor([s["stop"] for _, s, _ in items], **i32),
            mask0=t.tensor([s.get("mask", -1) for _, s, _ in items], **i32),
            stop_r=t.tensor([s["stop"] for _, s, _ in items for _ in range(self.B)], **i32),
            mask_r=t.tensor([s.get("mask", -1) for _, s, _ in items for _ in range(self.B)], **i32),
            h0=t.empty((S, md.hidden), **bf), z0=t.empty((S, V), **f32),
            ids0=t.empty((S, self.k), **i32), lp0=t.empty((S, self.k), **f32), lse0=t.empty(S, **f32),
            x=t.empty((R, md.hidden), **f32), h=t.empty((R, md.hidden), **bf),
            q=t.empty((R, md.hq, md.head_dim), **bf), o=t.empty((R, md.hq, md.head_dim), **bf),
            act=t.empty((R, md.ffn), **bf), hid=t.empty((R, md.hidden), **bf), z=t.empty((R, V), **f32),
            ids=t.empty((R, self.k), **i32), lp=t.empty((R, self.k), **f32), lse=t.empty(R, **f32),
            pos=t.empty(R, **i32), feed=t.empty(R, **i32),
            kdec=[t.empty((self.T * R, md.hkv, md.head_dim), **bf) for _ in range(md.layers)],
            vdec=[t.empty((self.T * R, md.hkv, md.head_dim), **bf) for _ in range(md.layers)],
            state=[dict(tok=t.empty((R, self.T), **i32), len=t.empty(R, **i32), fin=t.empty(R, **i32),
                        path=t.empty((R, self.T), **i32), nb=t.empty(S, **i32), score=t.empty(R, **f32))
                   for _ in range(2)])
        self._prepare()

    def _prepare(self):
        """Marshals every call once: step 0 and steps 1 .. T-1."""
        job, md, b = self.job, self.job.md, self.buf
        S, R, B = self.S, self.R, self.B
        ops0 = []
        j = 0
        while j < S:  # the slots' template rows, pass by pass, into h0
            k = self.items[j][2]["pass"]
            j1 = j
            while j1 < S and self.items[j1][2]["pass"] == k:
                j1 += 1
            rows = self.job.torch.tensor([self.items[x][2]["row"] for x in range(j, j1)], dtype=self.job.torch.int32,
                                         device=job.device)
            ops0.append(gather_rows(job.passes[k].hidden, rows, j1 - j, dst_bf16=b["h0"][j:j1]))
            j = j1
        masked = self.masks is not None
        ops0 += [PreparedLinear(b["h0"], self.W, LINEAR_F32, yf=b["z0"]),
                 topk_lse(b["z0"], self.k, b["ids0"], b["lp0"], b["lse0"], masks=self.masks,
                          mask_of_row=b["mask0"] if masked else None, stop_of_row=b["stop"]),
                 beam_step(S, B, self.k, self.T, 0, b["stop"], b["ids0"], b["lp0"], None, b["state"][0], b["feed"])]
        steps = []
        for st in range(1, self.T):
            cur, nxt = b["state"][(st - 1) % 2], b["state"][st % 2]
            ops = [gather_rows(self.embed, b["feed"], R, dst_f32=b["x"], pos=b["pos"], pos_base=b["slot_pos"],
                               per=B, pos_add=st)]
            for li, W in enumerate(job.W):
                kp, vp = job.kv_global[li]
                kd = b["kdec"][li][(st - 1) * R:st * R]
                vd = b["vdec"][li][(st - 1) * R:st * R]
                ops.append(PreparedNorm(b["x"], W["g_attn"], b["h"], md.eps))
                ops.append(PreparedLinear(b["h"], W["wqkv"], LINEAR_QKV_ROPE, q=b["q"], k_out=kd, v=vd,
                                          hq=md.hq, hkv=md.hkv, head_dim=md.head_dim, pos=b["pos"], rope=job.rope))
                ops.append(decode_attention(b["q"], kp, vp, b["kdec"][li], b["vdec"][li], b["o"], B,
                                            b["ranges"], b["n_ranges"], cur["path"], st - 1))
                ops.append(PreparedLinear(b["o"].reshape(R, -1), W["wo"], LINEAR_RESIDUAL, resid=b["x"]))
                ops.append(PreparedNorm(b["x"], W["g_mlp"], b["h"], md.eps))
                ops.append(PreparedLinear(b["h"], W["wgu"], LINEAR_SILU_GATE, y=b["act"]))
                ops.append(PreparedLinear(b["act"], W["wd"], LINEAR_RESIDUAL, resid=b["x"]))
            ops.append(PreparedNorm(b["x"], job.g_final, b["hid"], md.eps))
            ops.append(PreparedLinear(b["hid"], self.W, LINEAR_F32, yf=b["z"]))
            ops.append(topk_lse(b["z"], self.k, b["ids"], b["lp"], b["lse"], masks=self.masks,
                                mask_of_row=b["mask_r"] if masked else None, stop_of_row=b["stop_r"]))
            ops.append(beam_step(S, B, self.k, self.T, st, b["stop"], b["ids"], b["lp"], cur, nxt, b["feed"]))
            steps.append(ops)
        self._ops0, self._steps = ops0, steps

    def run(self, stream=None):
        """Enqueues the decoding of every slot (after the job's run on the same stream)."""
        for op in self._ops0:
            op(stream)
        for ops in self._steps:
            for op in ops:
                op(stream)

    def results(self) -> List[List[dict]]:
        """Per slot (in the order given): its beams, best first, as dicts
        tokens / lp / finished (host; waits for the device)."""
        st = self.buf["state"][(self.T - 1) % 2]
        tok = st["tok"].cpu().numpy()
        ln = st["len"].cpu().numpy()
        fin = st["fin"].cpu().numpy()
        sc = st["score"].cpu().numpy()
        nb = st["nb"].cpu().numpy()
        out = [None] * len(self.items)
        for j, (i, s, info) in enumerate(self.items):
            beams = []
            for bb in range(int(nb[j])):
                r = j * self.B + bb
                beams.append(dict(tokens=tuple(int(x) for x in tok[r, :ln[r]]), lp=float(sc[r]),
                                  finished=bool(fin[r])))
            out[i] = beams
        return out
