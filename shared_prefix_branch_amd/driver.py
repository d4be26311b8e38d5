"""The engine loop around libspb's calls, for one GPU.

A job is a plan plus activations: the caller supplies, per logical input, its
Q/K/V rows and hidden states (device tensors, already in the pass dtype), and
the lm head.  ``Job`` assembles each pass's token-major buffers from them by
the plan's placement, then per pass enqueues: metadata upload, branch
attention, option scoring.  The host floor join runs after all passes.
Nothing here computes the method: every step runs in libspb.

Transfers and pipelining: every pass's metadata is staged in pinned host
memory and uploaded on a copy stream; pass k's upload waits only until the
previous run's pass k has finished with the buffer, and pass k's kernels wait
only for that upload, so uploads overlap other passes' kernels.  All passes
write their option scores into one device buffer, copied back in one transfer
at the end of the run; results are double-buffered, so a caller may enqueue
run i+1 before it joins run i and the GPU never waits on the host.

Head groups: by default each pass has its own lm-head launch.  With
``head_rows`` > 0, consecutive passes whose scored rows total at most
``head_rows`` share one launch, made after the last of them has run its
attention, so W streams once per group instead of once per pass (a pass with
more rows than that is a group of its own); ``batch_head`` puts every pass in
one group.  The scores are bit-identical to the per-pass head.
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np

from . import (Plan, PreparedAttention, PreparedScore, PreparedScoreBatch, SpbError, score_batch_workspace_bytes,
               score_finalize, score_workspace_bytes)


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
    lp: object        # score outputs of the result slot the last run wrote
    p: object
    residual: object
    slots: list = None  # per result slot: (lp, p, residual) device views


Provider = Callable[[int], Tuple[object, object, object, object]]


class Job:
    """All passes of a plan, resident on one device."""

    def __init__(self, plan: Plan, hq: int, hkv: int, head_dim: int, hidden_dim: int, vocab: int,
                 qkv_dtype, out_dtype, hidden_dtype, device="cuda", scales=(1.0, 1.0, 1.0),
                 batch_head: bool = False, lm_head_kind: int = 0, head_rows: int = 0, fp8_dma: bool = True):
        import torch
        self.torch = torch
        self.plan = plan
        self.hq, self.hkv, self.d, self.H, self.V = hq, hkv, head_dim, hidden_dim, vocab
        self.qkv_dtype, self.out_dtype, self.hidden_dtype = qkv_dtype, out_dtype, hidden_dtype
        self.device = device
        self.scales = tuple(scales)
        self.row_off, self.floor_q = plan.inputs()
        self.passes: List[PassBuffers] = []
        self.copy_stream = None
        self._set = 0                  # pinned metadata set staged last
        self._set_done = [None, None]  # per metadata set: event after its last upload
        self._slot = 1                 # result slot of the last run
        self._slot_plan = [None, None]
        self._slot_done = [None, None]  # per result slot: event after its copy back
        self._pass_done: List = []      # per pass: event after the last run's kernels
        self._head = None               # lm head the prepared score calls point at
        self._attn: List = []
        self._score: List = []
        self.batch_head = bool(batch_head)
        self.head_rows = int(head_rows)
        self.lm_head_kind = int(lm_head_kind)
        # e4m3 inputs: attention widens V into a workspace and copies K/V
        # asynchronously (fp8_dma), else it stages them through registers
        self.fp8_dma = bool(fp8_dma)
        if self.batch_head and plan.n_passes > 64:
            raise ValueError("batch_head covers at most 64 passes")
        self.grouped = self.batch_head or self.head_rows > 0
        self.head_groups = self._group_passes(plan)
        self._shapes = [tuple(plan.info(k)[f] for f in self._SHAPE_FIELDS) for k in range(plan.n_passes)]

    def _group_passes(self, plan: Plan) -> List[List[int]]:
        """The passes of each lm-head launch, in pass order."""
        n = plan.n_passes
        if self.batch_head:
            return [list(range(n))]
        if self.head_rows <= 0:
            return [[k] for k in range(n)]
        groups: List[List[int]] = []
        cur: List[int] = []
        rows = 0
        for k in range(n):
            m = plan.info(k)["n_scored_rows"]
            if cur and (rows + m > self.head_rows or len(cur) == 64):  # 64: the batch call's pass limit
                groups.append(cur)
                cur, rows = [], 0
            cur.append(k)
            rows += m
        if cur:
            groups.append(cur)
        return groups

    # -- buffers ---------------------------------------------------------------
    def _result_sizes(self):
        out = []
        for k in range(self.plan.n_passes):
            inf = self.plan.info(k)
            out.append((max(1, inf["n_options"]), max(1, inf["n_branches"])))
        return out

    def _alloc(self, k: int) -> PassBuffers:
        t = self.torch
        inf = self.plan.info(k)
        n = max(1, inf["n_tokens"])
        dev = self.device
        meta = t.empty(inf["meta_bytes"], dtype=t.uint8, device=dev)
        ws_bytes = 256 if self.grouped else max(256, score_workspace_bytes(self.plan, k, self.V, self.H,
                                                                              self.lm_head_kind))
        ws = t.empty(ws_bytes, dtype=t.uint8, device=dev)
        return PassBuffers(
            inf["n_tokens"],
            t.empty((n, self.hq, self.d), dtype=self.qkv_dtype, device=dev),
            t.empty((n, self.hkv, self.d), dtype=self.qkv_dtype, device=dev),
            t.empty((n, self.hkv, self.d), dtype=self.qkv_dtype, device=dev),
            t.empty((n, self.hq, self.d), dtype=self.out_dtype, device=dev),
            t.empty((n, self.H), dtype=self.hidden_dtype, device=dev),
            meta, ws, None, None, None, [])

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
        t = self.torch
        cache: Dict[int, tuple] = {}
        sizes = self._result_sizes()
        total = sum(2 * no + nb for no, nb in sizes)
        self.results = [t.empty(total, dtype=t.float32, device=self.device) for _ in range(2)]
        self.results_host = [t.empty(total, dtype=t.float32, pin_memory=True) for _ in range(2)]
        # two pinned metadata sets: the next batch is staged into one while
        # the other may still be uploading
        self.meta_host = [[t.empty(self.plan.info(k)["meta_bytes"], dtype=t.uint8, pin_memory=True)
                           for k in range(self.plan.n_passes)] for _ in range(2)]
        self.passes = []
        off = 0
        for k in range(self.plan.n_passes):
            buf = self._alloc(k)
            no, nb = sizes[k]
            for r in range(2):
                res = self.results[r]
                buf.slots.append((res[off:off + no], res[off + no:off + 2 * no], res[off + 2 * no:off + 2 * no + nb]))
            buf.lp, buf.p, buf.residual = buf.slots[0]
            off += 2 * no + nb
            self.fill(k, buf, provider, cache)
            self.passes.append(buf)
        # one attention workspace serves every pass: their kernels run in order on one stream
        self.att_ws = None
        if self.fp8_dma and self.qkv_dtype in (t.uint8, getattr(t, "float8_e4m3fn", t.uint8)):
            from . import FP8_E4M3, attention_workspace_bytes
            nb = max(attention_workspace_bytes(self.plan, k, FP8_E4M3, self.hkv, self.d)
                     for k in range(self.plan.n_passes))
            self.att_ws = t.empty(max(256, nb), dtype=t.uint8, device=self.device)
        self._attn = [PreparedAttention(k, b.meta, b.q, b.k, b.v, b.o, scales=self.scales, workspace=self.att_ws)
                      for k, b in enumerate(self.passes)]
        if self.grouped:
            # one workspace for every group: their launches run in order on one stream
            nb = max(score_batch_workspace_bytes(self.plan, g, self.V, self.H, self.lm_head_kind)
                     for g in self.head_groups)
            self.batch_ws = t.empty(max(256, nb), dtype=t.uint8, device=self.device)
        self._pass_done = [None] * len(self.passes)

    def _prepare_head(self, lm_head):
        if self._head is not lm_head:
            if self.grouped:
                P = self.passes
                self._score = [[PreparedScoreBatch(g, [P[k].meta for k in g], [P[k].hidden for k in g], lm_head,
                                                   self.batch_ws, [P[k].slots[r] for k in g], self.lm_head_kind)
                                for r in range(2)] for g in self.head_groups]
            else:
                self._score = [[PreparedScore(k, b.meta, b.hidden, lm_head, b.workspace, *b.slots[r],
                                              lm_head_kind=self.lm_head_kind)
                                for r in range(2)] for k, b in enumerate(self.passes)]
            self._head = lm_head

    # -- metadata ------------------------------------------------------------
    def stage_host(self, plan: Optional[Plan] = None):
        """Copies a plan's metadata (by default the job's) into the pinned set
        not staged last; host work that can run while the GPU is busy.  The
        plan must have this job's pass shapes.  Returns the token ``run``
        takes."""
        plan = self.plan if plan is None else plan
        self.check_shapes(plan)
        self._set ^= 1
        if self._set_done[self._set] is not None:
            self._set_done[self._set].synchronize()  # its previous upload has left the buffers
        for k in range(plan.n_passes):
            plan.meta_copy(k, self.meta_host[self._set][k])
        return plan, self._set

    _SHAPE_FIELDS = ("n_tokens", "n_options", "n_branches", "n_scored_rows", "meta_bytes")

    def check_shapes(self, plan: Plan):
        """Raises SpbError unless ``plan`` has the pass shapes this job's
        buffers were sized for (rows, options, branches, scored rows and
        metadata bytes of every pass)."""
        if plan is self.plan:  # the job's own plan, or one staged (and checked) before
            return
        if plan.n_passes != len(self._shapes):
            raise SpbError(-4, f"the plan has {plan.n_passes} passes, this job {len(self._shapes)}")
        for k in range(plan.n_passes):
            got = tuple(plan.info(k)[f] for f in self._SHAPE_FIELDS)
            if got != self._shapes[k]:
                raise SpbError(-4, f"pass {k}: the plan's {dict(zip(self._SHAPE_FIELDS, got))} differ from this "
                                   f"job's {dict(zip(self._SHAPE_FIELDS, self._shapes[k]))}")

    def _upload(self, which: int, stream):
        """Uploads pinned set ``which`` on the copy stream, pass k after the
        previous run's pass-k kernels (which read the old metadata); returns
        one event per pass."""
        t = self.torch
        if self.copy_stream is None:
            self.copy_stream = t.cuda.Stream(device=self.device)
        cs = self.copy_stream
        events = []
        with t.cuda.stream(cs):
            for k in range(len(self.passes)):
                if self._pass_done[k] is not None:
                    cs.wait_event(self._pass_done[k])
                else:
                    cs.wait_stream(stream)
                self.passes[k].meta.copy_(self.meta_host[which][k], non_blocking=True)
                ev = t.cuda.Event()
                ev.record(cs)
                events.append(ev)
        if events:
            self._set_done[which] = events[-1]
        return events

    # -- running -------------------------------------------------------------
    def run(self, lm_head, stream=None, attention=True, scoring=True, marks=None, staged=None):
        """Enqueues every pass of a plan, then the copy of its scores back.
        ``staged``: a ``stage_host`` token (the plan to run and its pinned
        metadata); None stages the job's plan now.  ``marks``, if given, holds
        per pass four created events: recorded on ``stream`` around the
        attention kernel (0, 1) and, by the library, around the lm-head GEMM
        kernel (2, 3); with head groups, events 2, 3 of entry g time the
        launch of group g."""
        t = self.torch
        stream = stream if stream is not None else t.cuda.current_stream()
        if staged is None:
            staged = self.stage_host()
        plan, which = staged
        self.plan = plan
        self._prepare_head(lm_head)
        r = self._slot ^ 1
        if self._slot_done[r] is not None:
            self._slot_done[r].synchronize()  # its previous copy back has landed
        uploaded = self._upload(which, stream)
        gi = 0
        for k, buf in enumerate(self.passes):
            stream.wait_event(uploaded[k])
            mk = None if marks is None else marks[k]
            if mk is not None:
                mk[0].record(stream)
            if attention:
                self._forward(k, plan, stream)
            if mk is not None:
                mk[1].record(stream)
            if not self.grouped:
                if scoring:
                    self._score[k][r](plan, stream, None if mk is None else (mk[2], mk[3]))
                done = t.cuda.Event()
                done.record(stream)
                self._pass_done[k] = done
            elif k == self.head_groups[gi][-1]:
                if scoring:
                    mg = None if marks is None else marks[gi]
                    self._score[gi][r](plan, stream, None if mg is None else (mg[2], mg[3]))
                done = t.cuda.Event()
                done.record(stream)
                for kk in self.head_groups[gi]:
                    self._pass_done[kk] = done
                gi += 1
            buf.lp, buf.p, buf.residual = buf.slots[r]
        with t.cuda.stream(stream):
            self.results_host[r].copy_(self.results[r], non_blocking=True)
        ev = t.cuda.Event()
        ev.record(stream)
        self._slot, self._slot_plan[r], self._slot_done[r] = r, plan, ev

    def _forward(self, k: int, plan: Plan, stream):
        """Pass k's rows up to the hidden states the head reads: here branch
        attention alone (the hidden states are given)."""
        self._attn[k](plan, stream)

    def finalize(self, slot: Optional[int] = None, copy: bool = False) -> dict:
        """Waits for a run's scores (by default the last run's) and joins the
        floors on the host.  copy: fetch the slot's device scores again (after
        the caller rewrote them)."""
        t = self.torch
        r = self._slot if slot is None else slot
        if copy:
            stream = t.cuda.current_stream()
            with t.cuda.stream(stream):
                self.results_host[r].copy_(self.results[r], non_blocking=True)
            stream.synchronize()
        else:
            self._slot_done[r].synchronize()
        plan = self._slot_plan[r]
        host = self.results_host[r].numpy()
        lps, ps, rs = [], [], []
        off = 0
        for k, (no, nb) in enumerate(self._result_sizes()):
            inf = plan.info(k)
            lps.append(host[off:off + inf["n_options"]])
            ps.append(host[off + no:off + no + inf["n_options"]])
            rs.append(host[off + 2 * no:off + 2 * no + inf["n_branches"]])
            off += 2 * no + nb
        return score_finalize(plan, lps, ps, rs)

    @property
    def last_slot(self) -> int:
        return self._slot

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
