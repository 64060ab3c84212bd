"""Attention sinks on the GPU (run on an MI355X).

A sink is one logit per query head that joins every row's softmax
normalizer as an extra score with a zero value row (reading of the pages'
"sinks" backward parameter: page "Lab 028 lab detail: Off NVIDIA, you fix the
platform yourself", "What I changed, in plain terms", item 2). Compared with
the fp64 oracle: O, lse, dQ, dK, dV as everywhere, and d sinks (relative
error over the [Hq] vector, same gates). The sink values sit near the rows'
log-normalizers (about log of the number of keys), so they take a visible
share of the probability mass.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from sdpa_backward_amd import attention, sdpa_bwd, sdpa_fwd_lse
from tests.oracle_pins import rel_fro
from tests.test_parity import DEV, LSE_TOL, TOL, _np
from workloads import MASK_CAUSAL, MASK_NONE, MASK_TWO_SIDED, MASK_WINDOW, Workload, make_inputs

pytestmark = pytest.mark.gpu

CASES = [
    # name, B, Hq, Hkv, Lq, Lk, D, dtype, mask, window
    ("causal_D256", 1, 4, 2, 700, 700, 256, "bf16", MASK_CAUSAL, 0),
    ("w128_D128_B2", 2, 4, 1, 500, 500, 128, "bf16", MASK_WINDOW, 128),
    ("two_w50_suffix_D512", 1, 2, 1, 300, 900, 512, "bf16", MASK_TWO_SIDED, 50),
    ("none_D64", 1, 4, 4, 256, 256, 64, "bf16", MASK_NONE, 0),
    ("prefix_causal_D256", 1, 2, 1, 600, 250, 256, "bf16", MASK_CAUSAL, 0),   # rows with no key: lse = sink
    ("f16_w64_D256", 1, 4, 2, 400, 400, 256, "f16", MASK_WINDOW, 64),
    ("f32_causal_D64", 2, 2, 1, 100, 100, 64, "f32", MASK_CAUSAL, 0),
    ("f32_prefix_D128", 1, 2, 2, 90, 40, 128, "f32", MASK_CAUSAL, 0),
    ("f32_w30_D256", 1, 2, 1, 120, 120, 256, "f32", MASK_WINDOW, 30),
]


def sink_values(Hq, Lk, seed):
    g = torch.Generator().manual_seed(seed)
    return (math.log(max(Lk, 2)) + 2.0 * torch.randn(Hq, generator=g)).float()


def run_sinks(w, inp, sinks):
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    s = sinks.to(DEV)
    o, lse = sdpa_fwd_lse(q, k, v, w.mask, w.window, w.scale, sinks=s)
    dq, dk, dv, ds = sdpa_bwd(q, k, v, o, do, lse, w.mask, w.window, w.scale, sinks=s)
    torch.cuda.synchronize()
    return {"O": o, "lse": lse, "dQ": dq, "dK": dk, "dV": dv, "dSinks": ds}


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_sinks_full(case):
    name, B, Hq, Hkv, Lq, Lk, D, dtype, mask, window = case
    w = Workload(name, B, Hq, Hkv, Lq, D, dtype, mask, window, seed=9900 + Lq, Lk=Lk)
    inp = make_inputs(w)
    sinks = sink_values(Hq, Lk, w.seed)
    gpu = run_sinks(w, inp, sinks)
    ref = oracle.sdpa_fwd_bwd(inp["q"], inp["k"], inp["v"], inp["do"], w.scale, w.mask, w.window,
                              sinks=sinks.double().numpy())
    errs = {n: rel_fro(_np(gpu[n]), ref[n]) for n in ("O", "dQ", "dK", "dV", "dSinks")}
    errs["lse"] = float(np.max(np.abs(_np(gpu["lse"]) - ref["lse"])))
    print(name, {k: f"{x:.2e}" for k, x in errs.items()}, flush=True)
    for n in ("O", "dQ", "dK", "dV", "dSinks"):
        assert errs[n] <= TOL[dtype], (n, errs[n])
    assert errs["lse"] <= LSE_TOL
    if Lq > Lk and mask == MASK_CAUSAL:   # rows before every key: lse is the sink itself, O and dQ are 0
        e = Lq - Lk
        assert torch.allclose(gpu["lse"][:, :, :e].cpu(), sinks[None, :, None].expand(B, Hq, e), atol=1e-6)
        assert torch.all(gpu["O"][:, :, :e] == 0).item() and torch.all(gpu["dQ"][:, :, :e] == 0).item()


def test_sink_at_minus_infinity_is_no_sink_bitwise():
    w = Workload("sink_inf", 2, 4, 2, 333, 256, "bf16", MASK_WINDOW, 100, seed=9901)
    inp = make_inputs(w)
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    # calls with sinks never split the forward's key ranges: the reference
    # forward runs unsplit too (an empty workspace)
    o, lse = sdpa_fwd_lse(q, k, v, w.mask, w.window, workspace=torch.empty(0, dtype=torch.uint8, device=DEV))
    dq, dk, dv = sdpa_bwd(q, k, v, o, do, lse, w.mask, w.window)
    g = run_sinks(w, inp, torch.full((4,), -math.inf))
    for a, n in ((o, "O"), (lse, "lse"), (dq, "dQ"), (dk, "dK"), (dv, "dV")):
        assert torch.equal(a, g[n]), n
    assert torch.all(g["dSinks"] == 0).item()


def test_sinks_under_autograd():
    w = Workload("sink_autograd", 1, 4, 2, 300, 128, "bf16", MASK_CAUSAL, 0, seed=9902)
    inp = make_inputs(w)
    sinks = sink_values(4, 300, 9902)
    q, k, v = (inp[n].to(DEV).requires_grad_() for n in ("q", "k", "v"))
    s = sinks.to(DEV).requires_grad_()
    o = attention(q, k, v, w.mask, w.window, w.scale, sinks=s)
    o.backward(inp["do"].to(DEV))
    ref = oracle.sdpa_fwd_bwd(inp["q"], inp["k"], inp["v"], inp["do"], w.scale, w.mask, w.window,
                              sinks=sinks.double().numpy())
    for t, n in ((o, "O"), (q.grad, "dQ"), (k.grad, "dK"), (v.grad, "dV"), (s.grad, "dSinks")):
        e = rel_fro(_np(t), ref[n])
        assert e <= TOL["bf16"], (n, e)
