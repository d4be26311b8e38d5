"""Benchmark of the packed scoring pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload moderation] [--layers L] [--no-cpu-baseline]

The default workload is the moderation shape (300 contents x 106 questions of
2-5 multi-token labels, 61 passes of 16,384 tokens), the largest of the
configurations that fits one GPU; news, news2, extreme, fp8, tiny and grid are
the others.

A step is one pass of the whole hot path over one batch of synthetic input:
pack the batch into token-budget passes (host C++), and per pass upload the
metadata, run branch attention and the scored-row lm head (GPU); then copy
the option scores back and join the floors (host).  Steps are pipelined: the
host enqueues step i, then packs and stages batch i+1 and joins step i-1's
scores while the GPU runs step i; the last step's join is inside the timed
region.  Inputs (Q/K/V, hidden states, lm head) are resident in HBM before
timing starts.

Prints one JSON line: whole-job packed tokens/s as `value`, plus scored
questions/s, per-kernel timings from HIP events recorded on the launch stream
inside the timed steps, the roofline of the dominant kernel (the lm-head GEMM)
and the oracle timed on the host cores as `cpu_baseline`.  Each lm-head launch
is placed against its own bound (HBM at most 312 scored rows per W stream,
MFMA above); `roofline` aggregates the launches of the bound that takes most
of the head's time, never mixing the two, and `per_launch` lists every
launch's bound and fraction.  Attention reports its MFMA utilisation on
unmasked pairs against the peak of its input dtype (e4m3 Q.K^T with bf16 P.V:
the mixed peak) and its HBM rate against algorithmic bytes.  `traffic` is the
kernel's HBM bytes per launch from the committed counter summary for the
workload in profiles/ (null when the kernel source has changed since).

With --layers L the hidden states are not given: each pass first runs L
decoder layers (synthetic bf16 weights, the news attention shape with a 4x
gated MLP) from seeded input embeddings, and the roofline is that of the
linear-layer GEMM kernel, which then dominates the step.

    python bench.py --copy-calibration

runs only a plain 1 GiB device-to-device copy, three times, for scaling the
FETCH_SIZE / WRITE_SIZE counters.

    python bench.py --mfma-calibration

runs the library's MFMA calibration loop (the head's MFMA with operands in
registers, no memory traffic), with random bf16 operands and with small
integers, on every CU for about 80 ms each, and prints the sustained TFLOP/s:
what the head's MFMA reaches on this chip when nothing else limits it.

    python bench.py --head-sweep 8,16,56,128,256 [--steps K --warmup W]

times the lm head alone (news head shape) at each scored-row count and prints
one JSON line per count with its HBM and MFMA fractions.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
# e4m3 attention: Q.K^T (half the flops) on the fp8 MFMA, P.V on the bf16 one
PEAK_ATT_FP8_TFLOPS = 2.0 / (1.0 / PEAK_FP8_TFLOPS + 1.0 / PEAK_BF16_TFLOPS)   # 3,333
# lm-head ridge in scored rows per W stream: the head does M flop per W byte
HEAD_RIDGE_ROWS = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)   # 312.5
HERE = os.path.dirname(os.path.abspath(__file__))
# the files that define each kernel (a counter summary holds while they match)
KERNEL_SOURCES = {
    "head_lse_kernel": ("shared_prefix_branch_amd/csrc/spb_score.hip", "shared_prefix_branch_amd/csrc/spb_gemm.h",
                        "shared_prefix_branch_amd/csrc/spb_dev.h", "shared_prefix_branch_amd/csrc/spb_head_layout.h"),
    "branch_attention": ("shared_prefix_branch_amd/csrc/spb_attention.hip", "shared_prefix_branch_amd/csrc/spb_dev.h",
                         "shared_prefix_branch_amd/csrc/spb_meta.h"),
}
DEFAULT_CPU_SAMPLE = {"moderation": 20, "fp8": 40}   # contents in the oracle's sample (else all)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="moderation")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--layers", type=int, default=0,
                    help="decoder layers in front of the head (synthetic weights, news model dims); "
                         "0: attention alone with given hidden states")
    ap.add_argument("--fp8", action="store_true",
                    help="with --layers: the linears on e4m3 operands (static per-tensor scales)")
    ap.add_argument("--slots", type=int, default=0,
                    help="with --layers: after the timed steps, decode this many extraction slots (the first "
                         "question of each of the first contents) by beam search and time them")
    ap.add_argument("--beams", type=int, default=4)
    ap.add_argument("--slot-tokens", type=int, default=8)
    ap.add_argument("--no-template-sharing", action="store_true",
                    help="drop the template token ids, so questions share no template prefix")
    ap.add_argument("--cpu-sample-inputs", type=int, default=0,
                    help="contents in the oracle's sample (0: the workload's default, all of them for news, "
                         "tiny and extreme, 20 for moderation, 40 for fp8)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--mfma-calibration", action="store_true")
    ap.add_argument("--head-batch", action="store_true",
                    help="one lm-head launch for all passes of the step (spb_score_options_batch) "
                         "instead of one per pass")
    ap.add_argument("--head-rows", type=int, default=768,
                    help="group consecutive passes into one lm-head launch while their scored rows total at "
                         "most this many (0: one launch per pass); 768 = three row chunks of 256 per "
                         "vocabulary slice, the most that share W lines in one XCD's L2 well")
    ap.add_argument("--lm-head", default="f32out", choices=["f32out", "bf16", "fp32"],
                    help="lm-head output kind (f32out is the default of the engine the pages describe)")
    ap.add_argument("--head-sweep", default="",
                    help="comma-separated scored-row counts: time the lm head alone on the news head shape")
    return ap.parse_args()


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(HERE, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str, mode: str = "per_launch"):
    """HBM bytes per launch of ``kernel`` on ``workload`` from the committed
    counter summary profiles/<kernel>_<workload>_traffic.md, or None when it
    is missing or was taken on other kernel sources."""
    rel = f"profiles/{kernel}_{workload}_traffic.md"
    path = os.path.join(HERE, rel)
    if not os.path.exists(path):
        return None, f"no counter summary for {workload}"
    text = open(path).read()
    m_src = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    m_val = re.search(r"hbm_bytes_per_launch\[" + mode + r"\]:\s*([0-9.eE+]+)", text)
    if not (m_src and m_val):
        return None, "counter summary unreadable"
    if m_src.group(1) != source_hash(kernel):
        return None, "kernel changed since the counters were taken"
    return float(m_val.group(1)), rel


def head_roofline(M, head_ms, hidden: int, vocab: int) -> dict:
    """The lm head's roofline from its launches: M scored rows and event time
    (ms) per launch.  Each launch is placed against its own bound (HBM up to
    HEAD_RIDGE_ROWS rows per W stream, MFMA above); the reported figure
    aggregates the launches of the bound holding most of the head's time and
    never mixes the two."""
    M = np.asarray(M, dtype=np.float64)
    head_ms = np.asarray(head_ms, dtype=np.float64)
    flops = 2.0 * hidden * vocab * M
    nbytes = 2.0 * hidden * vocab + M * hidden * 2.0
    bounds = np.where(M > HEAD_RIDGE_ROWS, "mfma", "hbm")
    fracs = np.where(bounds == "mfma", flops / (head_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                     nbytes / (head_ms * 1e-3) / 1e9 / PEAK_HBM_GBS)
    t_mfma = float(head_ms[bounds == "mfma"].sum())
    bound = "mfma" if t_mfma >= 0.5 * float(head_ms.sum()) else "hbm"
    sel = bounds == bound
    if bound == "mfma":
        ach = float(flops[sel].sum() / (head_ms[sel].sum() * 1e-3) / 1e12)
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_BF16_TFLOPS, 4)}
    else:
        ach = float(nbytes[sel].sum() / (head_ms[sel].sum() * 1e-3) / 1e9)
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4)}
    return {"flops": flops, "bytes": nbytes, "bounds": bounds, "fracs": fracs, "bound": bound, "sel": sel,
            "roof": roof, "time_weighted_frac": round(float((fracs * head_ms).sum() / head_ms.sum()), 4)}


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read_per_copy": n, "bytes_written_per_copy": n, "copies": 3}}),
          flush=True)


def mfma_calibration():
    import torch
    import shared_prefix_branch_amd as spb
    torch.cuda.set_device(0)
    wg, iters = 256, 200000  # one work group of four waves per CU; about 80 ms at the nominal rate
    out = torch.empty(wg * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    flops = wg * 4 * iters * 16 * 32 * 32 * 16 * 2.0
    for random in (True, False):
        for rep in range(3):
            b, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            b.record(stream)
            spb.mfma_calibration(out, wg, iters, random, stream)
            e.record(stream)
            e.synchronize()
            ms = b.elapsed_time(e)
            tf = flops / (ms * 1e-3) / 1e12
            print(json.dumps({"mfma_calibration": {"operands": "random bf16" if random else "small integers",
                                                   "rep": rep, "ms": round(ms, 3), "tflops": round(tf, 1),
                                                   "frac_of_nominal": round(tf / PEAK_BF16_TFLOPS, 4)}}),
                  flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): the path has no multi-GPU leg; "
              "passes are independent and would shard as data parallelism across processes.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.mfma_calibration:
        mfma_calibration()
        return
    if args.head_sweep:
        head_sweep([int(x) for x in args.head_sweep.split(",")], args.steps, args.warmup)
        return
    import torch
    import synth
    import shared_prefix_branch_amd as spb
    from shared_prefix_branch_amd.driver import Job

    dev = "cuda:0"
    torch.cuda.set_device(0)
    wl = synth.make_workload(args.workload)
    d = wl.dims
    budget = wl.budgets[0]
    prob = wl.problem
    if args.no_template_sharing:
        prob = synth.Problem(**{**prob.__dict__, "tmpl_tok": None})

    # ---- inputs resident in HBM
    plan = spb.pack_pass(prob, token_budget=budget)
    info = plan.info()
    ids = synth.logical_inputs(prob, True)
    scales = synth.fp8_scales(wl) if d.dtype == "fp8" else (1.0, 1.0, 1.0)
    qkv_dt = {"bf16": torch.bfloat16, "fp8": torch.uint8, "f32": torch.float32}[d.dtype]
    out_dt = torch.float32 if d.dtype == "f32" else torch.bfloat16
    hid_dt = torch.float32 if d.dtype == "f32" else torch.bfloat16

    def provider(n):
        q, k, v, h = synth.activation_block(wl, ids[n], device=dev)
        qc, kc, vc = synth.cast_inputs(wl, q, k, v, scales)
        return qc, kc, vc, h.to(hid_dt)

    batch_head = args.head_batch and plan.n_passes <= 64
    head_kind = {"f32out": 0, "bf16": 1, "fp32": 2}[args.lm_head]
    md = None
    if args.layers > 0:
        import dataclasses
        from shared_prefix_branch_amd.stack import ForwardJob
        if d.dtype != "bf16":
            raise SystemExit("--layers runs bf16 workloads only")
        md = dataclasses.replace(synth.MODEL_CONFIGS["news"], layers=args.layers, hidden=d.hidden, hq=d.hq,
                                 hkv=d.hkv, head_dim=d.head_dim)
        layers_w, g_final = synth.model_weights(md, wl.cfg_seed, device=dev)
        fp8_scales = synth.stack_fp8_scales(layers_w) if args.fp8 else None
        job = ForwardJob(plan, md, layers_w, g_final, d.vocab, device=dev, batch_head=batch_head,
                         lm_head_kind=head_kind, keep_kv=args.slots > 0, fp8_scales=fp8_scales,
                         head_rows=args.head_rows)
        job.load(lambda n: synth.embed_block(wl, md, ids[n], device=dev))
        del layers_w
    else:
        job = Job(plan, d.hq, d.hkv, d.head_dim, d.hidden, d.vocab, qkv_dt, out_dt, hid_dt, device=dev,
                  scales=scales, batch_head=batch_head, lm_head_kind=head_kind, head_rows=args.head_rows)
        job.load(provider)
    W = synth.lm_head(wl, device=dev)
    torch.cuda.synchronize()

    n_pass = plan.n_passes
    stream = torch.cuda.current_stream()
    questions = int(info["n_content_branches"])
    tokens = int(info["n_tokens"])

    def step(state, marks=None):
        # enqueue every pass of the batch staged last and the copy of its
        # scores back; while the GPU runs them, pack the next batch, stage its
        # metadata in pinned memory and join the previous step's scores
        job.run(W, stream=stream, marks=marks, staged=state["next"])
        slot = job.last_slot
        state["next"] = job.stage_host(spb.pack_pass(prob, token_budget=budget))
        if state["prev"] is not None:
            state["res"] = job.finalize(state["prev"])
        state["prev"] = slot

    def drain(state):
        if state["prev"] is not None:
            state["res"] = job.finalize(state["prev"])
            state["prev"] = None

    # HIP events on the launch stream, created up front (a torch event exists
    # once recorded), recorded inside the timed steps
    marks = [[[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_pass)]
             for _ in range(args.steps)]
    for ms in marks:
        for mk in ms:
            for ev in mk:
                ev.record(stream)
    # with the stack: per step, pass and linear launch (4 per layer), a pair
    # of events the library records around the linear kernel
    n_lin = 4 * args.layers
    lin_marks = [[[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(n_lin)] for _ in range(n_pass)] for _ in range(args.steps)]
    for ms in lin_marks:
        for mk in ms:
            for pair in mk:
                for ev in pair:
                    ev.record(stream)
    torch.cuda.synchronize()

    state = {"next": job.stage_host(spb.pack_pass(prob, token_budget=budget)), "prev": None, "res": None}
    for _ in range(args.warmup):
        step(state)
    drain(state)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if n_lin:
            job.lin_marks = lin_marks[i]
        step(state, marks[i])
    drain(state)   # the last step's scores are joined inside the timed region
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    res = state["res"]
    ms_step = (t1 - t0) * 1e3 / args.steps
    if n_lin:
        job.lin_marks = None

    att_ms = np.zeros(n_pass)
    groups = job.head_groups
    n_head = len(groups)   # lm-head launches per step
    head_ms = np.zeros(n_head)
    for ms in marks:
        for k, mk in enumerate(ms):
            att_ms[k] += mk[0].elapsed_time(mk[1]) / args.steps
            if k < n_head:
                head_ms[k] += mk[2].elapsed_time(mk[3]) / args.steps
    pair_flops = 4.0 * d.head_dim * d.hq
    att_flops = np.array([plan.info(k)["unmasked_pairs"] * pair_flops for k in range(n_pass)])
    # attention's algorithmic bytes: Q, K, V read once, O written once
    b_in = {"bf16": 2, "fp8": 1, "f32": 4}[d.dtype]
    b_out = 4 if d.dtype == "f32" else 2
    att_bytes_tok = (d.hq + 2 * d.hkv) * d.head_dim * b_in + d.hq * d.head_dim * b_out
    att_bytes = np.array([plan.info(k)["n_tokens"] * att_bytes_tok for k in range(n_pass)], dtype=np.float64)
    att_peak = PEAK_ATT_FP8_TFLOPS if d.dtype == "fp8" else PEAK_BF16_TFLOPS
    att_ridge = att_peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    att_tflops = att_flops.sum() / (att_ms.sum() * 1e-3) / 1e12
    att_gbs = att_bytes.sum() / (att_ms.sum() * 1e-3) / 1e9
    att_ai = att_flops.sum() / att_bytes.sum()
    att_bound = "mfma" if att_ai > att_ridge else "hbm"
    M = np.array([sum(plan.info(k)["n_scored_rows"] for k in g) for g in groups], dtype=np.float64)
    hr = head_roofline(M, head_ms, d.hidden, d.vocab)
    head_flops, head_bytes, bounds, fracs = hr["flops"], hr["bytes"], hr["bounds"], hr["fracs"]
    head_tflops = head_flops.sum() / (head_ms.sum() * 1e-3) / 1e12
    head_gbs = head_bytes.sum() / (head_ms.sum() * 1e-3) / 1e9
    head_bound, sel = hr["bound"], hr["sel"]
    stack = None
    if n_lin:
        # linear launches: (n, k) per kind; m = the pass's tokens
        kinds = [("qkv", (md.hq + 2 * md.hkv) * md.head_dim, md.hidden), ("o", md.hidden, md.hq * md.head_dim),
                 ("gate_up", 2 * md.ffn, md.hidden), ("down", md.hidden, md.ffn)]
        lin_ms = np.zeros((n_pass, n_lin))
        for ms in lin_marks:
            for k, mk in enumerate(ms):
                for j, (b, e) in enumerate(mk):
                    lin_ms[k, j] += b.elapsed_time(e) / args.steps
        toks = np.array([plan.info(k)["n_tokens"] for k in range(n_pass)], dtype=np.float64)
        lin_flops = np.array([[2.0 * toks[k] * kinds[j % 4][1] * kinds[j % 4][2] for j in range(n_lin)]
                              for k in range(n_pass)])
        lin_tf = lin_flops.sum() / (lin_ms.sum() * 1e-3) / 1e12
        per_kind = {}
        for j4, (name, n_, k_) in enumerate(kinds):
            js = [j for j in range(n_lin) if j % 4 == j4]
            ms_k = float(lin_ms[:, js].sum())
            per_kind[name] = {"n": n_, "k": k_, "ms": round(ms_k, 4),
                              "tflops": round(float(lin_flops[:, js].sum()) / (ms_k * 1e-3) / 1e12, 2)}
        peak = PEAK_FP8_TFLOPS if args.fp8 else PEAK_BF16_TFLOPS
        stack = {"layers": md.layers, "hidden": md.hidden, "ffn": md.ffn, "linear_dtype": "e4m3" if args.fp8 else "bf16",
                 "forward_ms": round(float(att_ms.sum()), 4),
                 "linear": {"ms": round(float(lin_ms.sum()), 4), "tflops": round(lin_tf, 2),
                            "frac": round(lin_tf / peak, 4), "launches_per_step": int(n_pass * n_lin),
                            "per_kind": per_kind}}
    kernel_name = "head_lse_kernel"
    if head_kind != 0:
        traffic, traffic_src = None, "counters taken for the f32out lm head only"
    elif batch_head or (args.head_rows > 0 and n_head != n_pass):
        traffic, traffic_src = None, "counters taken with one lm-head launch per pass only"
    else:
        traffic, traffic_src = measured_traffic(kernel_name, args.workload)
    roof = dict(hr["roof"])
    roof["traffic"] = None if traffic is None else round(traffic)
    roof["traffic_source"] = traffic_src
    roof["algorithmic_bytes_per_launch"] = round(float(head_bytes.mean()))
    roof["kernel"] = "head_lse_kernel (lm-head GEMM with fused log-sum-exp, in spb_score_options)"
    roof["launches"] = f"{int(sel.sum())} of {n_head} lm-head launches per step are {head_bound}-bound; " \
                       f"achieved is over those"
    # the fp32 head runs three bf16 products per logit term (hi, mid, lo planes of h)
    roof["mfma_products_per_term"] = 3 if head_kind == 2 else 1
    roof["time_weighted_frac"] = hr["time_weighted_frac"]
    roof["per_launch"] = {"ms": [round(x, 4) for x in head_ms], "scored_rows": M.astype(int).tolist(),
                          "bound": bounds.tolist(), "frac": [round(float(x), 4) for x in fracs],
                          "flops_per_scored_row": 2 * d.hidden * d.vocab,
                          "algorithmic_bytes": [int(x) for x in head_bytes]}
    att_traffic, att_traffic_src = measured_traffic("branch_attention", args.workload)

    if stack is not None:
        # the linear layers dominate the step: their GEMM kernel is the roofline
        roof = {"bound": "mfma", "achieved": round(lin_tf, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(lin_tf / peak, 4), "traffic": None,
                "traffic_source": "counters not taken for the linear kernel",
                "kernel": "linear_kernel (decoder-stack GEMMs with fused epilogues, spb_linear)",
                "per_launch": {"ms_mean": round(float(lin_ms.mean()), 4),
                               "flops_mean": float(lin_flops.mean())}}
    line = {
        "metric": "packed tokens/s + scored questions/s per MI355X; attention MFMA util",
        "value": round(tokens / (ms_step * 1e-3), 1),
        "unit": "packed tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "fp8e4m3+bf16", "f32": "f32"}[d.dtype],
        "data": "synthetic (seeded Gaussian activations and lm head)",
        "config": {"workload": f"{args.workload}: {prob.n_inputs} contents x {len(prob.q_len)} questions, "
                               f"token budget {budget}, {n_pass} passes",
                   "packed_tokens": tokens, "questions": questions, "token_budget": budget,
                   "hq": d.hq, "hkv": d.hkv, "head_dim": d.head_dim, "hidden": d.hidden, "vocab": d.vocab,
                   "lm_head": args.lm_head, "lm_head_launches_per_step": n_head,
                   "template_sharing": prob.tmpl_tok is not None, "decoder_layers": args.layers},
        "questions_per_s": round(questions / (ms_step * 1e-3), 1),
        "attention": {"ms": round(float(att_ms.sum()), 4), "tflops": round(att_tflops, 2),
                      "mfma_util": round(att_tflops / att_peak, 4), "mfma_peak": round(att_peak, 1),
                      "gbs": round(att_gbs, 1), "hbm_frac": round(att_gbs / PEAK_HBM_GBS, 4),
                      "arithmetic_intensity": round(att_ai, 1), "bound": att_bound,
                      "roofline_frac": round((att_tflops / att_peak) if att_bound == "mfma"
                                             else (att_gbs / PEAK_HBM_GBS), 4),
                      "algorithmic_bytes_per_launch": round(float(att_bytes.mean())),
                      "traffic": None if att_traffic is None else round(att_traffic),
                      "traffic_source": att_traffic_src,
                      "unmasked_pairs": int(info["unmasked_pairs"])},
        "head": {"ms": round(float(head_ms.sum()), 4), "tflops": round(head_tflops, 2), "gbs": round(head_gbs, 1),
                 "scored_rows": int(M.sum())},
        "roofline": roof,
    }
    if stack is not None:
        line["stack"] = stack
        # the pass's events bracket the whole stack, so attention has no time of its own here
        line["attention"] = {"ms": None, "tflops": None, "mfma_util": None,
                             "unmasked_pairs": int(info["unmasked_pairs"]),
                             "note": "inside the decoder stack: stack.forward_ms covers every layer of each pass"}

    if args.slots > 0 and md is not None and not args.fp8:
        line["slots"] = time_slots(job, wl, md, W, prob, args, ms_step, tokens)
    if not args.no_cpu_baseline:
        if md is not None:
            line["cpu_baseline"] = cpu_baseline_stack(wl, md, W)
        else:
            n_cpu = args.cpu_sample_inputs if args.cpu_sample_inputs > 0 else \
                DEFAULT_CPU_SAMPLE.get(args.workload, prob.n_inputs)
            line["cpu_baseline"] = cpu_baseline(wl, W, scales, min(n_cpu, prob.n_inputs))
    print(json.dumps(line), flush=True)


def head_sweep(ms, steps, warmup):
    """The scored-row lm head alone on the news head shape (262,144 x 3,840
    bf16) for M scored rows: one content-free input with M one-token
    questions of two single-token options, so the pass scores exactly M rows.
    One JSON line per M: GEMM-kernel time from HIP events on the launch
    stream, W streaming rate against HBM peak, and MFMA rate."""
    import torch
    import synth
    import shared_prefix_branch_amd as spb
    wl = synth.make_workload("news")
    V, H = wl.dims.vocab, wl.dims.hidden
    dev = "cuda:0"
    torch.cuda.set_device(0)
    W = synth.lm_head(wl, device=dev)
    stream = torch.cuda.current_stream()
    for M in ms:
        prob = synth.Problem(np.array([0], np.int32), np.array([0, M], np.int32), np.arange(M, dtype=np.int32),
                             np.ones(M, np.int32), np.arange(0, 2 * M + 1, 2, dtype=np.int32),
                             np.arange(2 * M + 1, dtype=np.int32), (np.arange(2 * M) * 97 % V).astype(np.int32), V)
        plan = spb.pack_pass(prob, floors=False)
        inf = plan.info(0)
        assert inf["n_scored_rows"] == M and plan.n_passes == 1
        g = torch.Generator(device=dev)
        g.manual_seed(M)
        hid = (torch.randn((inf["n_tokens"], H), generator=g, device=dev) / H ** 0.5).to(torch.bfloat16)
        meta = torch.empty(inf["meta_bytes"], dtype=torch.uint8, device=dev)
        ws = torch.empty(spb.score_workspace_bytes(plan, 0, V, H), dtype=torch.uint8, device=dev)
        lp = torch.empty(inf["n_options"], device=dev)
        p = torch.empty_like(lp)
        res = torch.empty(inf["n_branches"], device=dev)
        plan.upload(0, meta, stream)
        call = spb.PreparedScore(0, meta, hid, W, ws, lp, p, res)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for e in evs:
            e[0].record(stream)
            e[1].record(stream)
        for _ in range(warmup):
            call(plan, stream)
        for e in evs:
            call(plan, stream, (e[0], e[1]))
        torch.cuda.synchronize()
        ms_k = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
        w_bytes = 2.0 * V * H + 2.0 * H * M
        flops = 2.0 * H * V * M
        gbs = w_bytes / (ms_k * 1e-3) / 1e9
        tfl = flops / (ms_k * 1e-3) / 1e12
        print(json.dumps({"head_sweep": {"scored_rows": M, "ms": round(ms_k, 4), "algorithmic_bytes": int(w_bytes),
                                         "gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
                                         "tflops": round(tfl, 2), "mfma_frac": round(tfl / PEAK_BF16_TFLOPS, 4),
                                         "bound": "hbm" if M <= HEAD_RIDGE_ROWS else "mfma"}}),
              flush=True)


def cpu_baseline(wl, W, scales, n_inputs):
    """The float64 oracle, as it stands, on a bounded sample: the first
    ``n_inputs`` contents with all their questions, plus the floors."""
    import torch
    import synth
    from oracle import attention as OA, numerics as ON, scoring as OS, tree as OT

    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 0) for p in threadpool_info() if p.get("user_api") == "blas"] or
                    [torch.get_num_threads()])
    except Exception:
        cores = torch.get_num_threads()
    sub = wl.problem.subset(list(range(n_inputs)))
    lay = OT.build_layout(sub, floors=True)
    ids = [("input", i) for i in range(n_inputs)] + [("floor", q) for q in sorted(set(int(q) for q in sub.branch_q))]
    Wh = W.cpu()
    acts = []
    for ident in ids:
        q, k, v, h = synth.activation_block(wl, ident, device="cpu")
        qc, kc, vc = synth.cast_inputs(wl, q, k, v, scales)
        sq, sk, sv = scales
        acts.append((ON.to_f64(qc, sq), ON.to_f64(kc, sk), ON.to_f64(vc, sv), ON.to_f64(h.to(torch.bfloat16))))
    t0 = time.perf_counter()
    for n, li in enumerate(lay.inputs):
        q, k, v, _ = acts[n]
        OA.attention_input(lay, li, q, k, v)

    def hidden(rows):
        return np.stack([acts[int(lay.row_input[r])][3][r - lay.inputs[int(lay.row_input[r])].first_row] for r in rows])

    sc = OS.score_branches(lay, hidden, Wh)
    OS.join_floors(lay, sc)
    dt = time.perf_counter() - t0
    qn = len(sub.branch_q)
    return {"value": round(lay.n_rows / dt, 2), "unit": "packed tokens/s", "questions_per_s": round(qn / dt, 3),
            "cores": cores, "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"{n_inputs} contents x {len(wl.problem.q_len)} questions + {len(ids) - n_inputs} floors "
                      f"= {lay.n_rows} tokens, {qn} questions; float64 NumPy, BLAS threads {cores}"}


def time_slots(job, wl, md, W, prob, args, ms_step, tokens):
    """Decodes ``args.slots`` {*} slots (the first question of each of the
    first contents, full vocabulary) on the last step's read, timed with HIP
    events over ``args.steps`` repeats."""
    import torch
    import synth
    from shared_prefix_branch_amd.stack import SlotDecoder
    n = min(args.slots, prob.n_inputs)
    E = synth.embed_table(md, wl.dims.vocab, wl.cfg_seed, device="cuda")
    slots = [dict(branch=int(prob.branch_off[i]), stop=1) for i in range(n)]
    dec = SlotDecoder(job, E, W, slots, args.beams, args.slot_tokens)
    stream = torch.cuda.current_stream()
    dec.run(stream)  # warm-up
    torch.cuda.synchronize()
    b, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b.record(stream)
    for _ in range(args.steps):
        dec.run(stream)
    e.record(stream)
    torch.cuda.synchronize()
    ms = b.elapsed_time(e) / args.steps
    res = dec.results()
    per_slot = ms / n
    per_token = ms_step / tokens  # GPU-and-host time of one packed scoring token in the step
    return {"slots": n, "beams": args.beams, "max_tokens": args.slot_tokens, "ms": round(ms, 4),
            "ms_per_slot": round(per_slot, 4), "scoring_token_equivalents_per_slot": round(per_slot / per_token, 1),
            "decode_steps": args.slot_tokens, "rows_per_step": n * args.beams,
            "example": {"tokens": list(res[0][0]["tokens"]), "lp": round(res[0][0]["lp"], 4)}}


def cpu_baseline_stack(wl, md, W):
    """The float64 oracle's per-sequence forward through the decoder stack and
    the head, on a bounded sample: one content and its first question."""
    import torch
    import synth
    from oracle import forward as OF, numerics as ON, scoring as OS, tree as OT

    cores = torch.get_num_threads()
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 0) for p in threadpool_info() if p.get("user_api") == "blas"] or [cores])
    except Exception:
        pass
    sub = wl.problem.subset([0])
    lay = OT.build_layout(sub, floors=False)
    layers_w, g_final = synth.model_weights(md, wl.cfg_seed)
    m = OF.Model.from_synth(md, layers_w, g_final)
    li = lay.inputs[0]
    x0 = ON.to_f64(synth.embed_block(wl, md, ("input", 0)))
    t0 = time.perf_counter()
    out = OF.forward_input(m, lay, li, x0, branches=[0], content=True)
    b = li.branches[0]
    sc = OS.score_branches(lay, lambda rows: out[np.asarray(rows) - li.first_row], W.cpu(), [b])
    dt = time.perf_counter() - t0
    assert len(sc) == 1
    toks = li.C + len(b.template_rows) + len(b.trie.prefixes)
    return {"value": round(toks / dt, 3), "unit": "packed tokens/s", "questions_per_s": round(1 / dt, 5),
            "cores": cores, "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"one content ({li.C} tokens) and its first question through {md.layers} decoder layers "
                      f"and the head: {toks} tokens, 1 question; float64 NumPy, BLAS threads {cores}"}


if __name__ == "__main__":
    main()
