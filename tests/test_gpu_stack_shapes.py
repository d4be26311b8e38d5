"""GPU parity of the decoder stack at the shapes the benchmark runs (news model
dimensions: hidden 3,840, 32 query / 16 KV heads of 128, a gated MLP of
15,360, two layers), through the C ABI.

Each linear layer is launched at its benchmark shape -- a full pass of rows
(13,000) times QKV with RoPE (8,192 x 3,840), o (3,840 x 4,096), gate/up
(30,720 x 3,840) and down (3,840 x 15,360), tiles dealt over the eight XCD
ranges -- with bf16 and with e4m3 operands, and a seeded sample of rows is
checked against the float64 products; the same rows launched in a smaller
call must give the same bits.  Then a two-layer stack at these dimensions on
a small problem against the oracle's per-sequence forward, bf16 and fp8."""
import math

import numpy as np
import pytest

import synth
from tests.gpu_helpers import check_scores, lm_head, say
from tests.test_gpu_stack import TOL_HIDDEN, TOL_OP, StackCase, _rel_rows

pytestmark = pytest.mark.gpu

M_PASS = 13000          # rows of a full benchmark pass (news: 12,900-16,384 tokens)
N_SAMPLE = 24           # rows checked against float64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import shared_prefix_branch_amd as spb
    spb.lib()


def _dev_normal(shape, scale, seed):
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device="cuda") * scale).to(torch.bfloat16)


def _rows(seed, m=M_PASS):
    rng = np.random.default_rng(seed)
    return np.sort(np.r_[rng.choice(m - 2, size=N_SAMPLE - 2, replace=False), m - 2, m - 1])


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "e4m3"])
@pytest.mark.parametrize("kind", ["qkv", "o", "gate_up", "down"])
def test_linear_at_bench_shape(kind, fp8):
    import torch
    import shared_prefix_branch_amd as spb
    from shared_prefix_branch_amd.stack import gate_up_rows
    from oracle import forward as OF
    from oracle.numerics import to_f64
    md = synth.MODEL_CONFIGS["news"]
    H, F, hq, hkv, d = md.hidden, md.ffn, md.hq, md.hkv, md.head_dim
    n, k = {"qkv": ((hq + 2 * hkv) * d, H), "o": (H, hq * d), "gate_up": (2 * F, H), "down": (H, F)}[kind]
    say(f"case: linear {kind} m={M_PASS} n={n} k={k} {'e4m3' if fp8 else 'bf16'}")
    seed = {"qkv": 10, "o": 20, "gate_up": 30, "down": 40}[kind] + (5 if fp8 else 0)
    x = _dev_normal((M_PASS, k), 1.0, seed)
    w = _dev_normal((n, k), 1.0 / math.sqrt(k), seed + 1)
    rows = _rows(seed)
    xs = to_f64(x[torch.from_numpy(rows).cuda()].cpu())
    wh = w.cpu()
    kw = {}
    if fp8:
        sx = float(x.float().abs().max()) / 448
        sw = float(w.float().abs().max()) / 448
        x8 = torch.empty_like(x, dtype=torch.uint8)
        w8 = torch.empty_like(w, dtype=torch.uint8)
        spb.quantize_e4m3(x, x8, sx)()
        spb.quantize_e4m3(w, w8, sw)()
        xa, wa = x8, w8
        kw["fp8_scales"] = (sx, sw)
        xs = OF.q8(xs, sx)
        wf = OF.q8(to_f64(wh), sw)
    else:
        xa, wa = x, w
        wf = to_f64(wh)
    if kind == "gate_up":
        wa_launch = gate_up_rows(wa[:F], wa[F:])
    else:
        wa_launch = wa
    full = xs @ wf.T   # [N_SAMPLE, n]
    m0 = 5

    def launch(xin):
        mm = xin.shape[0]
        if kind == "qkv":
            pos = torch.arange(mm, dtype=torch.int32, device="cuda") * 3 % 4096
            table = torch.from_numpy(spb.rope_table(4096, d, md.rope_base)).cuda()
            q = torch.empty((mm, hq, d), dtype=torch.bfloat16, device="cuda")
            kk = torch.empty((mm, hkv, d), dtype=torch.bfloat16, device="cuda")
            v = torch.empty((mm, hkv, d), dtype=torch.bfloat16, device="cuda")
            spb.linear(xin, wa_launch, spb.LINEAR_QKV_ROPE, q=q, k_out=kk, v=v, hq=hq, hkv=hkv, head_dim=d,
                       pos=pos, rope=table, **kw)
            return torch.cat([q.reshape(mm, -1), kk.reshape(mm, -1), v.reshape(mm, -1)], dim=1), pos
        if kind == "gate_up":
            y = torch.empty((mm, F), dtype=torch.bfloat16, device="cuda")
            spb.linear(xin, wa_launch, spb.LINEAR_SILU_GATE, y=y, **kw)
            return y, None
        r = torch.zeros((mm, n), dtype=torch.float32, device="cuda")
        spb.linear(xin, wa_launch, spb.LINEAR_RESIDUAL, resid=r, **kw)
        return r, None

    out, pos = launch(xa)
    part, _ = launch(xa[m0:])
    torch.cuda.synchronize()
    got = out[torch.from_numpy(rows).cuda()].float().cpu().double().numpy()
    if kind == "qkv":
        p = pos.cpu().numpy()[rows]
        ref = np.concatenate([OF.rope(full[:, :hq * d].reshape(-1, hq, d), p, md.rope_base).reshape(len(rows), -1),
                              OF.rope(full[:, hq * d:(hq + hkv) * d].reshape(-1, hkv, d), p,
                                      md.rope_base).reshape(len(rows), -1),
                              full[:, (hq + hkv) * d:]], axis=1)
    elif kind == "gate_up":
        ref = OF.silu(full[:, :F]) * full[:, F:]
    else:
        ref = full
    err = _rel_rows(got, ref)
    say(f"  sampled rows rel err {err:.2e}")
    assert err <= TOL_OP
    # a row's bits do not depend on how many rows the launch covers (the
    # QKV positions of the smaller launch differ, so compare V, which has none)
    if kind == "qkv":
        a, b = out[m0:, (hq + hkv) * d:], part[:, (hq + hkv) * d:]
    else:
        a, b = out[m0:], part
    assert torch.equal(a.contiguous().view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32),
                       b.contiguous().view(torch.int16 if b.dtype == torch.bfloat16 else torch.int32))


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "e4m3"])
def test_stack_news_dims_against_oracle(fp8):
    from oracle import scoring as OS
    md = synth.MODEL_CONFIGS["news"]
    wl = synth.make_workload("news", vocab=2000)
    wl.problem = synth.make_problem("random", 64, vocab=2000, n_inputs=2, n_questions=3, min_content=60,
                                    max_content=140, max_len=16, max_options=3, max_option_tokens=2)
    wl.inputs = synth.logical_inputs(wl.problem, True)
    W, Wh = lm_head(wl)
    say(f"case: two-layer stack at news dimensions, {'e4m3' if fp8 else 'bf16'} linears")
    case = StackCase(wl, md, 16384, fp8=fp8)
    case.run(W)
    lay, hid = case.oracle()
    got = case.job.hidden_by_logical_row(list(hid))
    worst = max(_rel_rows(got[r][0][None], ref[None]) for r, ref in hid.items())
    tol = 1e-1 if fp8 else TOL_HIDDEN
    assert worst <= tol, f"hidden rel err {worst}"
    sc = OS.score_branches(lay, lambda rows: np.stack([hid[r] for r in rows]), Wh)
    OS.join_floors(lay, sc)
    ref = {k: v for k, v in sc.items() if lay.inputs[k[0]].kind == "input"}
    if fp8:
        res = case.branch_results()
        e = max(float(np.max(np.abs(res[k][1] - s.p))) for k, s in ref.items())
        assert e <= 1e-1
        es = {"p": e}
    else:
        es = check_scores(case, ref)
    say(f"  hidden rel err {worst:.2e}; scores {es}")
