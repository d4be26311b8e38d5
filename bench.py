"""Benchmark of the packed scoring pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload news] [--no-cpu-baseline]

A step is one pass of the whole hot path over one batch of synthetic input:
pack the batch into token-budget passes (host C++), and per pass upload the
metadata, run branch attention and the scored-row lm head (GPU); then copy
the option scores back and join the floors (host).  The host packs the next
step's batch while the GPU runs the current one.  Inputs (Q/K/V, hidden
states, lm head) are resident in HBM before timing starts.

Prints one JSON line: whole-job packed tokens/s as `value`, plus scored
questions/s, per-kernel timings from HIP events on the launch stream, the
roofline of the dominant kernel (the lm head) and the oracle timed on the
host cores as `cpu_baseline`.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="news")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-inputs", type=int, default=2)
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): the path has no multi-GPU leg; "
              "passes are independent and would shard as data parallelism across processes.", file=sys.stderr)
        sys.exit(2)
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

    job = Job(plan, d.hq, d.hkv, d.head_dim, d.hidden, d.vocab, qkv_dt, out_dt, hid_dt, device=dev, scales=scales)
    job.load(provider)
    W = synth.lm_head(wl, device=dev)
    torch.cuda.synchronize()

    n_pass = plan.n_passes
    stream = torch.cuda.current_stream()
    questions = int(info["n_content_branches"])
    tokens = int(info["n_tokens"])

    def step(next_plan_holder):
        # enqueue every pass, pack the next batch on the host meanwhile,
        # then bring the scores back and join the floors
        p = next_plan_holder[0]
        job.plan = p
        job.run(W, stream=stream)
        next_plan_holder[0] = spb.pack_pass(prob, token_budget=budget)
        res = job.finalize()   # synchronises on the copies back
        return res

    holder = [spb.pack_pass(prob, token_budget=budget)]
    for _ in range(args.warmup):
        step(holder)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        res = step(holder)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps

    # ---- per-kernel timing with HIP events on the launch stream
    reps = max(3, min(10, args.steps))
    att_ms = np.zeros(n_pass)
    head_ms = np.zeros(n_pass)
    for k in range(n_pass):
        buf = job.passes[k]
        plan.upload(k, buf.meta, stream)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        for r in range(reps + 1):
            ev[0].record(stream)
            spb.branch_attention(plan, k, buf.meta, buf.q, buf.k, buf.v, buf.o, scales=scales, stream=stream)
            ev[1].record(stream)
            spb.score_options(plan, k, buf.meta, buf.hidden, W, buf.workspace, buf.lp, buf.p, buf.residual,
                              stream=stream)
            ev[2].record(stream)
            torch.cuda.synchronize()
            if r > 0:
                att_ms[k] += ev[0].elapsed_time(ev[1]) / reps
                head_ms[k] += ev[1].elapsed_time(ev[2]) / reps
    pair_flops = 4.0 * d.head_dim * d.hq
    att_flops = np.array([plan.info(k)["unmasked_pairs"] * pair_flops for k in range(n_pass)])
    M = np.array([plan.info(k)["n_scored_rows"] for k in range(n_pass)], dtype=np.float64)
    head_flops = 2.0 * d.hidden * d.vocab * M
    w_bytes = 2.0 * d.hidden * d.vocab
    head_bytes = w_bytes + M * d.hidden * 2.0
    att_tflops = att_flops.sum() / (att_ms.sum() * 1e-3) / 1e12
    head_tflops = head_flops.sum() / (head_ms.sum() * 1e-3) / 1e12
    head_gbs = head_bytes.sum() / (head_ms.sum() * 1e-3) / 1e9
    head_bound = "mfma" if M.mean() > PEAK_BF16_TFLOPS / PEAK_HBM_GBS else "hbm"
    if head_bound == "mfma":
        roof = {"bound": "mfma", "achieved": round(head_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(head_tflops / PEAK_BF16_TFLOPS, 4), "traffic": None}
    else:
        roof = {"bound": "hbm", "achieved": round(head_gbs, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(head_gbs / PEAK_HBM_GBS, 4), "traffic": None}
    roof["kernel"] = "head_lse_kernel (spb_score_options)"
    roof["per_launch"] = {"ms": [round(x, 4) for x in head_ms], "scored_rows": M.astype(int).tolist(),
                          "flops_per_scored_row": 2 * d.hidden * d.vocab, "w_bytes": int(w_bytes)}

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
                   "hq": d.hq, "hkv": d.hkv, "head_dim": d.head_dim, "hidden": d.hidden, "vocab": d.vocab},
        "questions_per_s": round(questions / (ms_step * 1e-3), 1),
        "attention": {"ms": round(float(att_ms.sum()), 4), "tflops": round(att_tflops, 2),
                      "mfma_util": round(att_tflops / PEAK_BF16_TFLOPS, 4),
                      "unmasked_pairs": int(info["unmasked_pairs"])},
        "head": {"ms": round(float(head_ms.sum()), 4), "tflops": round(head_tflops, 2), "gbs": round(head_gbs, 1),
                 "scored_rows": int(M.sum())},
        "roofline": roof,
    }

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, W, scales, args.cpu_sample_inputs, provider_host=None)
    print(json.dumps(line), flush=True)


def cpu_baseline(wl, W, scales, n_inputs, provider_host=None):
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


if __name__ == "__main__":
    main()
