"""The block-sparse prefix-sharing cut on the GPU (run on an MI355X).

Rows from r0 on do not see keys [c0, c1), on top of the mask. With
[prompt; chosen; rejected], a causal mask, r0 = c1 = start of rejected and
c0 = start of chosen, one pass equals the two passes [prompt; chosen] and
[prompt; rejected] (page "Training - design (ORPO, flash-CCE head, prefix
sharing, segmented backward)", section 5.4). With the fourth element of the
cut set, rows from r0 on measure their window at logical positions (the cut
keys do not count), and the equality holds under a window too. Checked
against the fp64 oracle with the cut, and against the GPU's own two-branch
passes.
"""
import numpy as np
import pytest
import torch

import oracle
from sdpa_backward_amd import attention, sdpa_bwd, sdpa_fwd_lse, workspace_bytes
from tests.oracle_pins import rel_fro
from tests.test_parity import DEV, LSE_TOL, TOL, _np
from workloads import MASK_CAUSAL, MASK_NONE, MASK_TWO_SIDED, MASK_WINDOW, Workload, make_inputs

pytestmark = pytest.mark.gpu

CASES = [
    # name, B, Hq, Hkv, Lq, Lk, D, dtype, mask, window, cut
    ("orpo_causal_D256", 1, 4, 2, 900, 900, 256, "bf16", MASK_CAUSAL, 0, (650, 300, 650)),
    ("orpo_causal_D128_B2", 2, 4, 1, 517, 517, 128, "bf16", MASK_CAUSAL, 0, (400, 129, 400)),
    ("orpo_causal_D512", 1, 2, 1, 700, 700, 512, "bf16", MASK_CAUSAL, 0, (500, 200, 500)),
    ("cut_w100_D256", 1, 2, 1, 800, 800, 256, "bf16", MASK_WINDOW, 100, (450, 300, 450)),
    ("cut_two_w64_suffix_D64", 1, 2, 2, 300, 700, 64, "bf16", MASK_TWO_SIDED, 64, (100, 450, 520)),
    ("cut_none_D128", 1, 2, 1, 400, 400, 128, "bf16", MASK_NONE, 0, (200, 0, 64)),
    ("orpo_f16_D256", 1, 2, 1, 600, 600, 256, "f16", MASK_CAUSAL, 0, (450, 200, 450)),
    ("orpo_f32_D64", 1, 2, 1, 120, 120, 64, "f32", MASK_CAUSAL, 0, (90, 40, 90)),
    # the window at logical positions (rows from r0 see the keys before c0 through the band moved back by c1 - c0)
    ("logical_w256_D256", 1, 4, 2, 1200, 1200, 256, "bf16", MASK_WINDOW, 256, (800, 300, 800, True)),
    ("logical_w100_ragged_D128", 1, 2, 1, 1031, 1031, 128, "bf16", MASK_WINDOW, 100, (700, 233, 700, True)),
    ("logical_w300_merged_D64", 1, 2, 2, 700, 700, 64, "bf16", MASK_WINDOW, 300, (500, 300, 330, True)),
    ("logical_two_w64_D256", 1, 2, 1, 600, 600, 256, "bf16", MASK_TWO_SIDED, 64, (450, 100, 300, True)),
    ("logical_w128_D512", 1, 2, 1, 800, 800, 512, "bf16", MASK_WINDOW, 128, (500, 200, 500, True)),
    ("logical_w64_suffix_D256", 1, 2, 2, 300, 700, 256, "bf16", MASK_WINDOW, 64, (150, 300, 550, True)),
    ("logical_causal_D256", 1, 2, 1, 640, 640, 256, "bf16", MASK_CAUSAL, 0, (400, 150, 400, True)),
    ("logical_w90_f16_D256", 1, 2, 1, 650, 650, 256, "f16", MASK_WINDOW, 90, (420, 170, 420, True)),
    ("logical_w20_f32_D64", 1, 2, 1, 150, 150, 64, "f32", MASK_WINDOW, 20, (100, 40, 100, True)),
]


def run_cut(w, inp, cut, scale=None):
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    o, lse = sdpa_fwd_lse(q, k, v, w.mask, w.window, scale, cut=cut)
    dq, dk, dv = sdpa_bwd(q, k, v, o, do, lse, w.mask, w.window, scale, cut=cut)
    torch.cuda.synchronize()
    return {"O": o, "lse": lse, "dQ": dq, "dK": dk, "dV": dv}


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_cut_full(case):
    name, B, Hq, Hkv, Lq, Lk, D, dtype, mask, window, cut = case
    w = Workload(name, B, Hq, Hkv, Lq, D, dtype, mask, window, seed=9950 + Lq, Lk=Lk)
    inp = make_inputs(w)
    gpu = run_cut(w, inp, cut)
    ref = oracle.sdpa_fwd_bwd(inp["q"], inp["k"], inp["v"], inp["do"], w.scale, w.mask, w.window, cut=cut)
    errs = {n: rel_fro(_np(gpu[n]), ref[n]) for n in ("O", "dQ", "dK", "dV")}
    fin = np.isfinite(ref["lse"])
    errs["lse"] = float(np.max(np.abs(_np(gpu["lse"])[fin] - ref["lse"][fin]), initial=0.0))
    print(name, {k: f"{x:.2e}" for k, x in errs.items()}, flush=True)
    for n in ("O", "dQ", "dK", "dV"):
        assert errs[n] <= TOL[dtype], (n, errs[n])
    assert errs["lse"] <= LSE_TOL


def test_shared_prompt_pass_equals_two_branches():
    P, Rc, Rr, D = 400, 230, 270, 256
    L = P + Rc + Rr
    w = Workload("orpo_branches", 1, 4, 2, L, D, "bf16", MASK_CAUSAL, 0, seed=9960)
    inp = {n: t.to(DEV) for n, t in make_inputs(w).items()}
    q, k, v, do = inp["q"], inp["k"], inp["v"], inp["do"]
    cut = (P + Rc, P, P + Rc)
    o, lse = sdpa_fwd_lse(q, k, v, "causal", cut=cut)
    dq, dk, dv = sdpa_bwd(q, k, v, o, do, lse, "causal", cut=cut)
    ia = torch.arange(P + Rc, device=DEV)
    ib = torch.cat([torch.arange(P, device=DEV), torch.arange(P + Rc, L, device=DEV)])
    sel = lambda t, idx: t.index_select(2, idx).contiguous()
    # the branch passes run unsplit, as the cut pass does (calls with a cut
    # never split their key ranges or dK/dV shares): an empty forward
    # workspace and a backward workspace with only the Delta rows, so that
    # tiles and summation order match
    fws = torch.empty(0, dtype=torch.uint8, device=DEV)
    bws = lambda n: torch.empty(workspace_bytes(1, 4, n, D, torch.bfloat16), dtype=torch.uint8, device=DEV)
    oa, la = sdpa_fwd_lse(sel(q, ia), sel(k, ia), sel(v, ia), "causal", workspace=fws)
    ga = sdpa_bwd(sel(q, ia), sel(k, ia), sel(v, ia), oa, sel(do, ia), la, "causal", workspace=bws(P + Rc))
    do_b = sel(do, ib)
    do_b[:, :, :P] = 0
    ob, lb = sdpa_fwd_lse(sel(q, ib), sel(k, ib), sel(v, ib), "causal", workspace=fws)
    gb = sdpa_bwd(sel(q, ib), sel(k, ib), sel(v, ib), ob, do_b, lb, "causal", workspace=bws(P + Rr))
    torch.cuda.synchronize()
    # rows of [prompt; chosen] see the same keys at the same positions: bitwise equal
    assert torch.equal(o[:, :, :P + Rc], oa) and torch.equal(lse[:, :, :P + Rc], la)
    assert torch.equal(dq[:, :, :P + Rc], ga[0])
    # rejected rows and the summed prompt keys: equal to bf16 rounding
    f = lambda t: t.double().cpu().numpy()
    assert rel_fro(f(o[:, :, P + Rc:]), f(ob[:, :, P:])) <= 1e-2
    assert float((lse[:, :, P + Rc:] - lb[:, :, P:]).abs().max()) <= LSE_TOL
    assert rel_fro(f(dq[:, :, P + Rc:]), f(gb[0][:, :, P:])) <= 1e-2
    for n, t in (("dK", dk), ("dV", dv)):
        i = 1 if n == "dK" else 2
        assert rel_fro(f(t[:, :, :P]), f(ga[i][:, :, :P].double() + gb[i][:, :, :P].double())) <= 1e-2, n
        assert rel_fro(f(t[:, :, P:P + Rc]), f(ga[i][:, :, P:])) <= 1e-2, n
        assert rel_fro(f(t[:, :, P + Rc:]), f(gb[i][:, :, P:])) <= 1e-2, n


def test_logical_window_shared_pass_equals_two_branches():
    # with the window at logical positions the shared pass equals the two
    # windowed passes [prompt; chosen] and [prompt; rejected] for any window
    P, Rc, Rr, D, W = 300, 260, 340, 256, 200
    L = P + Rc + Rr
    w = Workload("orpo_branches_w", 1, 4, 2, L, D, "bf16", MASK_WINDOW, W, seed=9965)
    inp = {n: t.to(DEV) for n, t in make_inputs(w).items()}
    q, k, v, do = inp["q"], inp["k"], inp["v"], inp["do"]
    cut = (P + Rc, P, P + Rc, True)
    o, lse = sdpa_fwd_lse(q, k, v, "causal_window", W, cut=cut)
    dq, dk, dv = sdpa_bwd(q, k, v, o, do, lse, "causal_window", W, cut=cut)
    ia = torch.arange(P + Rc, device=DEV)
    ib = torch.cat([torch.arange(P, device=DEV), torch.arange(P + Rc, L, device=DEV)])
    sel = lambda t, idx: t.index_select(2, idx).contiguous()
    oa, la = sdpa_fwd_lse(sel(q, ia), sel(k, ia), sel(v, ia), "causal_window", W)
    ga = sdpa_bwd(sel(q, ia), sel(k, ia), sel(v, ia), oa, sel(do, ia), la, "causal_window", W)
    do_b = sel(do, ib)
    do_b[:, :, :P] = 0
    ob, lb = sdpa_fwd_lse(sel(q, ib), sel(k, ib), sel(v, ib), "causal_window", W)
    gb = sdpa_bwd(sel(q, ib), sel(k, ib), sel(v, ib), ob, do_b, lb, "causal_window", W)
    torch.cuda.synchronize()
    f = lambda t: t.double().cpu().numpy()
    assert rel_fro(f(o[:, :, :P + Rc]), f(oa)) <= 1e-2
    assert rel_fro(f(o[:, :, P + Rc:]), f(ob[:, :, P:])) <= 1e-2
    assert float((lse[:, :, :P + Rc] - la).abs().max()) <= LSE_TOL
    assert float((lse[:, :, P + Rc:] - lb[:, :, P:]).abs().max()) <= LSE_TOL
    assert rel_fro(f(dq[:, :, :P + Rc]), f(ga[0])) <= 1e-2
    assert rel_fro(f(dq[:, :, P + Rc:]), f(gb[0][:, :, P:])) <= 1e-2
    for n, t in (("dK", dk), ("dV", dv)):
        i = 1 if n == "dK" else 2
        assert rel_fro(f(t[:, :, :P]), f(ga[i][:, :, :P].double() + gb[i][:, :, :P].double())) <= 1e-2, n
        assert rel_fro(f(t[:, :, P:P + Rc]), f(ga[i][:, :, P:])) <= 1e-2, n
        assert rel_fro(f(t[:, :, P + Rc:]), f(gb[i][:, :, P:])) <= 1e-2, n


def test_cut_under_autograd():
    w = Workload("cut_autograd", 1, 2, 1, 500, 128, "bf16", MASK_CAUSAL, 0, seed=9970)
    inp = make_inputs(w)
    cut = (350, 150, 350)
    q, k, v = (inp[n].to(DEV).requires_grad_() for n in ("q", "k", "v"))
    o = attention(q, k, v, "causal", cut=cut)
    o.backward(inp["do"].to(DEV))
    ref = oracle.sdpa_fwd_bwd(inp["q"], inp["k"], inp["v"], inp["do"], w.scale, "causal", 0, cut=cut)
    for t, n in ((o, "O"), (q.grad, "dQ"), (k.grad, "dK"), (v.grad, "dV")):
        assert rel_fro(_np(t), ref[n]) <= TOL["bf16"], n
