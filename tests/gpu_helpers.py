"""Helpers for the GPU tests: run a workload through libspb and through the
oracle on the same seeded inputs, and compare."""
from __future__ import annotations

import dataclasses
import math
import sys
from typing import Dict, List, Optional, Sequence

import numpy as np

import synth
import shared_prefix_branch_amd as spb
from shared_prefix_branch_amd.driver import Job
from oracle import attention as OA
from oracle import numerics as ON
from oracle import scoring as OS
from oracle import tree as OT

TOL = {"f32": 2e-2, "bf16": 2e-2, "fp8": 1e-1}
# The scores' tolerance follows the hidden rows that feed the head: bf16 (or f32
# rounded to bf16) in every configuration, the fp8 one included, whose fp8
# inputs are only Q, K and V.
SCORE_TOL = 2e-2
# A guarded comparison must reject a planted wrong answer by at least this
# factor over its tolerance, else the comparison could not fail and the test
# says so.
GUARD = 5.0


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class Case:
    """One workload (or a subset of its inputs) packed at one budget and run on the GPU."""

    def __init__(self, wl: synth.Workload, budget: int, inputs: Optional[Sequence[int]] = None,
                 floors: bool = True, peaked: bool = False, device: str = "cuda", gen_device: str = "cuda",
                 chained: bool = False, cache: Optional[dict] = None, batch_head: bool = False,
                 lm_head_kind: int = 0, head_rows: int = 0, sharp: bool = False, fp8_dma: bool = True):
        import torch
        self.torch = torch
        self.wl = wl
        self.inputs = list(range(wl.problem.n_inputs)) if inputs is None else list(inputs)
        self.prob = wl.problem if inputs is None else wl.problem.subset(self.inputs)
        self.floors = floors
        self.peaked = peaked
        self.sharp = sharp
        self.device = device
        self.gen_device = gen_device
        self.plan = spb.pack_pass(self.prob, token_budget=budget, floors=floors)
        # logical input number -> identity of its seeded activations
        ids = [("input", i) for i in self.inputs]
        if floors:
            ids += [("floor", q) for q in sorted(set(int(q) for q in self.prob.branch_q))]
        self.ids = ids
        self.dims = wl.dims
        self.scales = synth.fp8_scales(wl, sharp=sharp) if wl.dims.dtype == "fp8" else (1.0, 1.0, 1.0)
        self._blocks: Dict[tuple, tuple] = {} if cache is None else cache  # activations by identity
        self.batch_head = batch_head
        self.head_rows = head_rows
        self.lm_head_kind = lm_head_kind
        self.fp8_dma = fp8_dma

    # -- inputs --------------------------------------------------------------
    def block(self, ident):
        """Cast activations of one logical input, on the GPU (cached)."""
        if ident not in self._blocks:
            q, k, v, h = synth.activation_block(self.wl, ident, device=self.gen_device, peaked=self.peaked,
                                                sharp=self.sharp)
            qc, kc, vc = synth.cast_inputs(self.wl, q, k, v, self.scales)
            hc = h.float() if self.dims.dtype == "f32" else h.to(self.torch.bfloat16)
            self._blocks[ident] = tuple(t.to(self.device) for t in (qc, kc, vc, hc))
        return self._blocks[ident]

    def provider(self, n: int):
        return self.block(self.ids[n])

    # -- GPU -------------------------------------------------------------------
    def run(self, W):
        t = self.torch
        d = self.dims
        qkv = {"f32": t.float32, "bf16": t.bfloat16, "fp8": t.uint8}[d.dtype]
        out = t.float32 if d.dtype == "f32" else t.bfloat16
        hid = t.float32 if d.dtype == "f32" else t.bfloat16
        self.job = Job(self.plan, d.hq, d.hkv, d.head_dim, d.hidden, d.vocab, qkv, out, hid,
                       device=self.device, scales=self.scales, batch_head=self.batch_head,
                       lm_head_kind=self.lm_head_kind, head_rows=self.head_rows, fp8_dma=self.fp8_dma)
        self.job.load(self.provider)
        self.job.run(W)
        t.cuda.synchronize()
        self.res = self.job.finalize()
        return self.res

    def branch_results(self):
        """Per content branch (input number, question) -> (lp, p, residual, floor_p, lift) numpy."""
        res = self.res
        out = {}
        pos = 0
        b = 0
        for n, i in enumerate(self.inputs):
            for q in self.prob.questions_of(n):
                k = int(self.prob.opt_off[q + 1] - self.prob.opt_off[q])
                out[(n, q)] = tuple(res[f][pos:pos + k].copy() for f in ("lp", "p")) + \
                    (float(res["residual"][b]),) + tuple(res[f][pos:pos + k].copy() for f in ("floor_p", "lift"))
                pos += k
                b += 1
        return out

    # -- oracle ----------------------------------------------------------------
    def oracle_inputs(self, n):
        """The oracle's float64 inputs of logical input n: what the boundary
        computes on.  f32 Q, K and V are taken rounded to bf16 (RNE), as the
        library rounds them on load; at O(1) scores that rounding alone moves
        attention rows by a few percent, more than the tolerance.  Hidden rows
        are rounded per lm-head kind in oracle_scores."""
        q, k, v, h = self.block(self.ids[n])
        sq, sk, sv = self.scales
        q, k, v = ON.to_f64(q, sq), ON.to_f64(k, sk), ON.to_f64(v, sv)
        if self.dims.dtype == "f32":
            q, k, v = ON.round_to_bf16(q), ON.round_to_bf16(k), ON.round_to_bf16(v)
        return (q, k, v, ON.to_f64(h))


def rel_l2_rows(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max over (row, head) of ||gpu - ref|| / ||ref||."""
    num = np.linalg.norm(gpu - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    return float(np.max(num / np.maximum(den, 1e-30)))


def check_attention(case: Case, inputs: Sequence[int] = None, branches_per_input: int = None, rng=None,
                    guard: bool = False):
    """GPU attention rows vs the oracle's per-sequence form; returns the max error.

    ``guard``: also compute the oracle with every query zeroed -- a plain
    average of V over the same keys, what a kernel that dropped QK^T would
    return -- and require it to miss the oracle by GUARD times the tolerance
    on some row, so that the comparison can fail on the score arithmetic."""
    lay = OT.build_layout(case.prob, floors=case.floors)
    tol = TOL[case.dims.dtype]
    worst = 0.0
    wrong = 0.0
    todo = range(len(lay.inputs)) if inputs is None else inputs
    for n in todo:
        li = lay.inputs[n]
        q, k, v, _ = case.oracle_inputs(n)
        if branches_per_input is not None and len(li.branches) > branches_per_input:
            bs = sorted(rng.choice(len(li.branches), size=branches_per_input, replace=False).tolist())
        else:
            bs = list(range(len(li.branches)))
        ref = OA.attention_input(lay, li, q, k, v, branches=bs, content=True)
        rows = [r for r in range(ref.shape[0]) if not np.isnan(ref[r, 0, 0])]
        if guard:
            flat = OA.attention_input(lay, li, np.zeros_like(q), k, v, branches=bs, content=True)
            wrong = max(wrong, max(rel_l2_rows(flat[r][None], ref[r][None]) for r in rows))
        got = case.job.attention_by_logical_row([li.first_row + r for r in rows])
        for r in rows:
            outs = got[li.first_row + r]
            for o in outs[1:]:  # a re-staged content row is bit-identical in every pass
                assert np.array_equal(o, outs[0]), f"re-staged row {li.first_row + r} differs between passes"
            e = rel_l2_rows(outs[0][None], ref[r][None])
            worst = max(worst, e)
    assert worst <= tol, f"attention rel err {worst} > {tol}"
    if guard:
        assert wrong >= GUARD * tol, \
            f"guard: the plain V average is only {wrong:.3g} from the oracle (tolerance {tol}); the test cannot fail"
    return worst


KIND_NAME = {0: "f32out", 1: "bf16", 2: "fp32"}


def oracle_scores(case: Case, W, branch_keys: Sequence[tuple] = None, wrong: str = None):
    """Oracle scores (with floors joined) for content branches keyed (input number, question),
    for the case's lm-head kind.  The f32out and bf16 heads take f32 hidden rows
    rounded to bf16 (the library rounds them on load); the fp32 head takes them
    as they are.

    ``wrong`` plants a mistake into the oracle's inputs, for the guards:
    "flat" zeroes the hidden rows (constant logits), "neighbour" scores every
    option token's successor in the vocabulary (a one-off gather)."""
    prob = case.prob
    if wrong == "neighbour":
        prob = dataclasses.replace(prob, tok=((prob.tok.astype(np.int64) + 1) % prob.vocab).astype(np.int32))
    elif wrong not in (None, "flat"):
        raise ValueError(wrong)
    lay = OT.build_layout(prob, floors=case.floors)
    hid_cache = {}
    kind = KIND_NAME[case.lm_head_kind]

    def hidden(rows):
        out = []
        for r in rows:
            n = int(lay.row_input[r])
            if n not in hid_cache:
                h = case.oracle_inputs(n)[3]
                hid_cache[n] = h if kind == "fp32" else ON.round_to_bf16(h)
                if wrong == "flat":
                    hid_cache[n] = np.zeros_like(hid_cache[n])
            out.append(hid_cache[n][r - lay.inputs[n].first_row])
        return np.stack(out)

    branches = []
    want = None if branch_keys is None else set(branch_keys)
    floors_needed = set()
    for b in lay.branches():
        key = (b.input_no, b.question)
        if lay.inputs[b.input_no].kind == "input" and (want is None or key in want):
            branches.append(b)
            floors_needed.add(b.question)
    for b in lay.branches():
        if b.is_floor and b.question in floors_needed:
            branches.append(b)
    sc = OS.score_branches(lay, hidden, W, branches, lm_head=kind)
    OS.join_floors(lay, sc)
    return {k: v for k, v in sc.items() if lay.inputs[k[0]].kind == "input"}


def score_errors(got: dict, ref: dict) -> dict:
    """Per field, the largest error of ``got`` against ``ref`` (both keyed like
    oracle_scores; ``got`` values are (lp, p, residual, floor_p, lift))."""
    err = {"lp": 0.0, "p": 0.0, "residual": 0.0, "floor_p": 0.0, "lift": 0.0}
    for key, s in ref.items():
        lp, p, r, fp, lift = got[key]
        err["lp"] = max(err["lp"], float(np.max(np.abs(lp - s.lp) / np.abs(s.lp))))
        err["p"] = max(err["p"], float(np.max(np.abs(p - s.p))))
        err["residual"] = max(err["residual"], abs(r - s.residual))
        if s.floor_p is not None and fp is not None:
            err["floor_p"] = max(err["floor_p"], float(np.max(np.abs(fp - s.floor_p))))
            err["lift"] = max(err["lift"], float(np.max(np.abs(lift - s.lift))))
    return err


def check_scores(case: Case, ref: dict, guards: Sequence[dict] = ()):
    """GPU scores vs the oracle's, within SCORE_TOL; the Sigma p = 1 and
    mass + residual = 1 invariants on every compared branch.  Each of
    ``guards`` (oracle scores with a planted mistake, from oracle_scores(...,
    wrong=...)) must miss ``ref`` by GUARD times the tolerance in some field."""
    tol = SCORE_TOL
    got = case.branch_results()
    for key in ref:
        lp, p, r = got[key][:3]
        assert abs(float(np.sum(p)) - 1.0) < 1e-5
        assert abs(float(np.sum(np.exp(lp.astype(np.float64)))) + r - 1.0) < 1e-5
    err = score_errors(got, ref)
    for k, e in err.items():
        assert e <= tol, f"{k} error {e} > {tol}"
    for g in guards:
        ge = score_errors({k: (s.lp, s.p, s.residual, s.floor_p, s.lift) for k, s in g.items()}, ref)
        assert max(ge.values()) >= GUARD * tol, \
            f"guard: a planted mistake is only {ge} from the oracle (tolerance {tol}); the test cannot fail"
    return err


def lm_head(wl, device="cuda"):
    """The seeded bf16 lm head on the device, and the same bytes on the host."""
    W = synth.lm_head(wl, device=device)
    return W, W.cpu()
