"""GPU parity of the decoder stack around branch attention, through the C ABI:
the linear-layer epilogues and rmsnorm against the oracle's operations, then
whole packed forwards (layers, head, floors) against the oracle's
per-sequence forward, and batch invariance of the stacked pass."""
import math

import numpy as np
import pytest

import synth
from tests.gpu_helpers import Case, check_scores, lm_head, say
from tests.test_gpu_invariance import _same

pytestmark = pytest.mark.gpu

# Bounds from the rounding points: activations are rounded to bf16 once per
# op (2^-9 relative each), the residual stream is f32.
TOL_OP = 1e-2       # one linear layer or rmsnorm, per row, relative L2
TOL_HIDDEN = 3e-2   # the final hidden rows after the stack, per row, relative L2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import shared_prefix_branch_amd as spb
    spb.lib()


def _rel_rows(got, ref):
    num = np.linalg.norm(got - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    return float(np.max(num / np.maximum(den, 1e-30)))


def _bf16(rng, shape, scale=1.0):
    import torch
    return torch.from_numpy(rng.normal(size=shape) * scale).float().to(torch.bfloat16)


@pytest.mark.parametrize("m,n,k", [(300, 392, 128), (1000, 256, 320), (7, 8, 64)])
def test_linear_bf16_and_residual(m, n, k):
    import torch
    import shared_prefix_branch_amd as spb
    from oracle.numerics import to_f64
    say(f"case: linear m={m} n={n} k={k}")
    rng = np.random.default_rng(m + n + k)
    x, w = _bf16(rng, (m, k)), _bf16(rng, (n, k), 1 / math.sqrt(k))
    ref = to_f64(x) @ to_f64(w).T
    xd, wd = x.cuda(), w.cuda()
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    spb.linear(xd, wd, spb.LINEAR_BF16, y=y)
    r0 = torch.from_numpy(rng.normal(size=(m, n))).float()
    r = r0.cuda()
    spb.linear(xd, wd, spb.LINEAR_RESIDUAL, resid=r)
    torch.cuda.synchronize()
    assert _rel_rows(to_f64(y), ref) <= TOL_OP
    assert _rel_rows(r.cpu().double().numpy() - r0.double().numpy(), ref) <= TOL_OP
    # the residual epilogue adds exactly the bf16 output
    assert torch.equal(r.cpu(), r0 + y.float().cpu())
    # a row's bits do not depend on how many rows the launch covers
    if m > 8:
        y2 = torch.empty((m - 5, n), dtype=torch.bfloat16, device="cuda")
        spb.linear(xd[5:], wd, spb.LINEAR_BF16, y=y2)
        torch.cuda.synchronize()
        assert torch.equal(y2.cpu(), y[5:].cpu())


def test_linear_silu_gate():
    import torch
    import shared_prefix_branch_amd as spb
    from shared_prefix_branch_amd.stack import gate_up_rows
    from oracle import forward as OF
    from oracle.numerics import to_f64
    say("case: linear silu gate m=333 F=320 k=192")
    rng = np.random.default_rng(5)
    m, F, k = 333, 320, 192
    x, wg, wu = _bf16(rng, (m, k)), _bf16(rng, (F, k), 1 / math.sqrt(k)), _bf16(rng, (F, k), 1 / math.sqrt(k))
    y = torch.empty((m, F), dtype=torch.bfloat16, device="cuda")
    spb.linear(x.cuda(), gate_up_rows(wg.cuda(), wu.cuda()), spb.LINEAR_SILU_GATE, y=y)
    torch.cuda.synchronize()
    xf = to_f64(x)
    ref = OF.silu(xf @ to_f64(wg).T) * (xf @ to_f64(wu).T)
    assert _rel_rows(to_f64(y), ref) <= TOL_OP


@pytest.mark.parametrize("hq,hkv,d", [(4, 2, 64), (8, 4, 128), (4, 4, 128)])
def test_linear_qkv_rope(hq, hkv, d):
    import torch
    import shared_prefix_branch_amd as spb
    from oracle import forward as OF
    from oracle.numerics import to_f64
    say(f"case: qkv rope hq={hq} hkv={hkv} d={d}")
    rng = np.random.default_rng(hq * d)
    m, k = 290, 256
    n = (hq + 2 * hkv) * d
    x, w = _bf16(rng, (m, k)), _bf16(rng, (n, k), 1 / math.sqrt(k))
    pos = rng.integers(0, 4000, size=m).astype(np.int32)
    table = torch.from_numpy(spb.rope_table(4096, d, 10000.0)).cuda()
    q = torch.empty((m, hq, d), dtype=torch.bfloat16, device="cuda")
    kk = torch.empty((m, hkv, d), dtype=torch.bfloat16, device="cuda")
    v = torch.empty((m, hkv, d), dtype=torch.bfloat16, device="cuda")
    spb.linear(x.cuda(), w.cuda(), spb.LINEAR_QKV_ROPE, q=q, k_out=kk, v=v, hq=hq, hkv=hkv, head_dim=d,
               pos=torch.from_numpy(pos).cuda(), rope=table)
    torch.cuda.synchronize()
    full = to_f64(x) @ to_f64(w).T
    rq = OF.rope(full[:, :hq * d].reshape(m, hq, d), pos, 10000.0)
    rk = OF.rope(full[:, hq * d:(hq + hkv) * d].reshape(m, hkv, d), pos, 10000.0)
    rv = full[:, (hq + hkv) * d:].reshape(m, hkv, d)
    for got, ref in ((q, rq), (kk, rk), (v, rv)):
        assert _rel_rows(to_f64(got).reshape(m, -1), ref.reshape(m, -1)) <= TOL_OP


def test_rmsnorm():
    import torch
    import shared_prefix_branch_amd as spb
    from oracle import forward as OF
    from oracle.numerics import to_f64
    say("case: rmsnorm rows=77 dim=3840")
    rng = np.random.default_rng(9)
    x = torch.from_numpy(rng.normal(size=(77, 3840)) * 3).float()
    g = torch.from_numpy(rng.uniform(0.5, 1.5, 3840)).float().to(torch.bfloat16)
    out = torch.empty((77, 3840), dtype=torch.bfloat16, device="cuda")
    spb.rmsnorm(x.cuda(), g.cuda(), out, 1e-6)
    torch.cuda.synchronize()
    ref = OF.rms_norm(x.double().numpy(), to_f64(g), 1e-6)
    assert _rel_rows(to_f64(out), ref) <= 4e-3


class StackCase(Case):
    """A Case whose hidden states come from the decoder stack."""

    def __init__(self, wl, md, budget, inputs=None, seed=31, fp8=False, **kw):
        super().__init__(wl, budget, inputs=inputs, **kw)
        self.md = md
        self.layers, self.g_final = synth.model_weights(md, seed)
        self.fp8 = synth.stack_fp8_scales(self.layers) if fp8 else None

    def block(self, ident):
        if ident not in self._blocks:
            self._blocks[ident] = synth.embed_block(self.wl, self.md, ident).to(self.device)
        return self._blocks[ident]

    def run(self, W):
        from shared_prefix_branch_amd.stack import ForwardJob
        t = self.torch
        self.job = ForwardJob(self.plan, self.md, self.layers, self.g_final, self.dims.vocab, device=self.device,
                              fp8_scales=self.fp8)
        self.job.load(self.provider)
        self.job.run(W)
        t.cuda.synchronize()
        self.res = self.job.finalize()
        return self.res

    def oracle(self):
        from oracle import forward as OF, tree as OT
        from oracle.numerics import to_f64
        m = OF.Model.from_synth(self.md, self.layers, self.g_final, self.fp8)
        lay = OT.build_layout(self.prob, floors=self.floors)
        hid = {}
        for n, li in enumerate(lay.inputs):
            x0 = to_f64(self.block(self.ids[n]))
            nrows = int((lay.row_input == n).sum())
            out = OF.forward_input(m, lay, li, x0[:nrows])
            for r in range(nrows):
                hid[li.first_row + r] = out[r]
        return lay, hid


def _stack_case(kind, md_name, budget, seed, n_inputs=3, **over):
    md = synth.MODEL_CONFIGS[md_name]
    wl = synth.make_workload("grid", hq=md.hq, hkv=md.hkv, head_dim=md.head_dim, hidden=md.hidden, vocab=1000,
                             dtype="bf16")
    if kind == "random":
        wl.problem = synth.make_problem("random", seed, vocab=1000, n_inputs=n_inputs, n_questions=4, min_content=20,
                                        max_content=140, max_len=12, max_options=4, max_option_tokens=3)
    else:
        wl.problem = synth.make_problem("random_shared", seed, vocab=1000, n_inputs=n_inputs, n_questions=6,
                                        min_content=0, max_content=120, max_lead=40, tail_vocab=3, max_options=3,
                                        max_option_tokens=3)
    wl.inputs = synth.logical_inputs(wl.problem, True)
    return wl, md


@pytest.mark.parametrize("kind,md_name", [("random", "small"), ("shared", "small_d128")])
def test_stack_parity_against_oracle(kind, md_name):
    from oracle import scoring as OS
    wl, md = _stack_case(kind, md_name, 16384, 61)
    W, Wh = lm_head(wl)
    for budget in ((16384, 150) if kind == "random" else (16384, 120)):
        say(f"case: stack {kind} {md_name} budget {budget}")
        case = StackCase(wl, md, budget)
        case.run(W)
        lay, hid = case.oracle()
        got = case.job.hidden_by_logical_row(list(hid))
        worst = 0.0
        for r, ref in hid.items():
            outs = got[r]
            for o in outs[1:]:
                assert np.array_equal(o, outs[0]), f"re-staged row {r} differs between passes"
            worst = max(worst, _rel_rows(outs[0][None], ref[None]))
        assert worst <= TOL_HIDDEN, f"hidden rel err {worst}"
        sc = OS.score_branches(lay, lambda rows: np.stack([hid[r] for r in rows]), Wh)
        OS.join_floors(lay, sc)
        ref = {k: v for k, v in sc.items() if lay.inputs[k[0]].kind == "input"}
        es = check_scores(case, ref)
        say(f"  passes {case.plan.n_passes}: hidden rel err {worst:.2e}; scores {es}")


def test_stack_packed_spilled_and_alone_bit_identical():
    wl, md = _stack_case("shared", "small", 16384, 62)
    W, _ = lm_head(wl)
    say("case: stack packed vs spilled vs alone")
    cache = {}
    packed = StackCase(wl, md, 16384, cache=cache)
    packed.run(W)
    spilled = StackCase(wl, md, 100, inputs=[2, 0, 1], cache=cache)
    spilled.run(W)
    assert spilled.plan.info()["n_tokens"] > packed.plan.info()["n_tokens"]  # content and stems re-staged

    def by_input(c):
        from oracle import tree as OT
        lay = OT.build_layout(c.prob, floors=c.floors)
        res = c.branch_results()
        out = {}
        for n, i in enumerate(c.inputs):
            li = lay.inputs[n]
            rows = list(range(li.first_row, li.first_row + int((lay.row_input == n).sum())))
            got = c.job.hidden_by_logical_row(rows)
            att = [got[r][0].view(np.uint32).copy() for r in rows]
            sc = {q: tuple(np.asarray(x).view(np.uint32).copy() if isinstance(x, np.ndarray)
                           else np.float32(x).view(np.uint32) for x in res[(n, q)])
                  for q in c.prob.questions_of(n)}
            out[i] = (att, sc)
        return out

    P, S = by_input(packed), by_input(spilled)
    for i in range(3):
        _same(P[i], S[i], f"input {i} spilled")
    alone = StackCase(wl, md, 16384, inputs=[1], cache=cache)
    alone.run(W)
    _same(P[1], by_input(alone)[1], "input 1 alone")


def test_quantize_e4m3_codes_equal_the_oracle_rounding():
    import torch
    import shared_prefix_branch_amd as spb
    from oracle import numerics as ON
    say("case: e4m3 quantize, f32 and bf16 inputs, power-of-two scale")
    rng = np.random.default_rng(3)
    x = (rng.normal(size=4099) * np.exp2(rng.uniform(-12, 12, 4099))).astype(np.float32)
    for src in (torch.from_numpy(x), torch.from_numpy(x).to(torch.bfloat16)):
        q = torch.empty(x.size, dtype=torch.uint8, device="cuda")
        spb.quantize_e4m3(src.cuda(), q, 0.125)()
        torch.cuda.synchronize()
        got = ON.e4m3_bytes_to_f64(q.cpu().numpy())
        want = ON.round_to_e4m3(ON.to_f64(src) / 0.125)
        assert np.array_equal(got, want)


@pytest.mark.parametrize("mode", ["bf16", "residual"])
def test_linear_fp8_against_oracle(mode):
    import torch
    import shared_prefix_branch_amd as spb
    from oracle import forward as OF
    from oracle.numerics import to_f64
    say(f"case: fp8 linear ({mode}) m=300 n=392 k=256")
    rng = np.random.default_rng(11)
    m, n, k = 300, 392, 256
    x, w = _bf16(rng, (m, k)), _bf16(rng, (n, k), 1 / math.sqrt(k))
    sx, sw = float(x.float().abs().max()) / 448, float(w.float().abs().max()) / 448
    x8 = torch.empty((m, k), dtype=torch.uint8, device="cuda")
    w8 = torch.empty((n, k), dtype=torch.uint8, device="cuda")
    spb.quantize_e4m3(x.cuda(), x8, sx)()
    spb.quantize_e4m3(w.cuda(), w8, sw)()
    ref = OF.q8(to_f64(x), sx) @ OF.q8(to_f64(w), sw).T
    if mode == "bf16":
        y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        spb.linear(x8, w8, spb.LINEAR_BF16, y=y, fp8_scales=(sx, sw))
        torch.cuda.synchronize()
        got = to_f64(y)
    else:
        r = torch.zeros((m, n), dtype=torch.float32, device="cuda")
        spb.linear(x8, w8, spb.LINEAR_RESIDUAL, resid=r, fp8_scales=(sx, sw))
        torch.cuda.synchronize()
        got = r.cpu().double().numpy()
    assert _rel_rows(got, ref) <= TOL_OP


TOL_FP8 = 1e-1  # the fp8 tolerance for hidden rows and scores


def test_stack_fp8_parity_and_bit_identity():
    from oracle import scoring as OS
    wl, md = _stack_case("shared", "small_d128", 16384, 63)
    W, Wh = lm_head(wl)
    say("case: fp8 stack, shared templates, packed and spilled")
    cache = {}
    packed = StackCase(wl, md, 16384, fp8=True, cache=cache)
    packed.run(W)
    lay, hid = packed.oracle()
    got = packed.job.hidden_by_logical_row(list(hid))
    worst = max(_rel_rows(got[r][0][None], ref[None]) for r, ref in hid.items())
    assert worst <= TOL_FP8, f"hidden rel err {worst}"
    sc = OS.score_branches(lay, lambda rows: np.stack([hid[r] for r in rows]), Wh)
    OS.join_floors(lay, sc)
    err = {"lp": 0.0, "p": 0.0}
    res = packed.branch_results()
    for key, s in sc.items():
        if lay.inputs[key[0]].kind != "input":
            continue
        lp, p = res[key][0], res[key][1]
        err["lp"] = max(err["lp"], float(np.max(np.abs(lp - s.lp) / np.abs(s.lp))))
        err["p"] = max(err["p"], float(np.max(np.abs(p - s.p))))
    assert err["lp"] <= TOL_FP8 and err["p"] <= TOL_FP8, err
    say(f"  hidden rel err {worst:.2e}; scores {err}")
    spilled = StackCase(wl, md, 135, inputs=[1, 2, 0], fp8=True, cache=cache)
    assert spilled.plan.info()["n_tokens"] > packed.plan.info()["n_tokens"]  # content and stems re-staged
    spilled.run(W)
    rows = list(hid)
    a = packed.job.hidden_by_logical_row(rows)
    b = spilled.job.hidden_by_logical_row(rows)
    # the spilled case numbers logical rows in its own input order: compare by input
    la = packed.plan.inputs()[0]
    lb = spilled.plan.inputs()[0]
    for pos_b, i in enumerate([1, 2, 0]):
        n_rows = int(la[i + 1] - la[i])
        for r in range(n_rows):
            xa = a[int(la[i]) + r][0]
            xb = b[int(lb[pos_b]) + r][0]
            assert np.array_equal(xa.view(np.uint32), xb.view(np.uint32)), (i, r)
