"""The backward that keeps dS for a bounded band (run on an MI355X).

For 16-bit inputs at D = 256 whose key blocks fill the GPU (at least 256
blocks of 128 keys), a band at most 2304 keys wide (sliding windows, the
two-sided window up to about 1080) and the
full workspace of sdpa_bwd_workspace_bytes_ex, the dK/dV pass also writes
dS^T for the band and dQ = scale dS K is formed from it, instead of a dQ pass
that recomputes S and dP. Every case here takes that path (checked through
the workspace sizes) and is compared with the fp64 oracle over whole tensors,
and with the same call given only the Delta workspace (no band buffer): dK
and dV come from the same kernel on both paths, dQ from two different
summation orders, so both sit within the gates of the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from sdpa_backward_amd import bwd_workspace_bytes, sdpa_bwd, sdpa_fwd_lse, workspace_bytes
from tests.oracle_pins import rel_fro
from tests.test_parity import DEV, LSE_TOL, TOL, _np
from workloads import MASK_CAUSAL, MASK_TWO_SIDED, MASK_WINDOW, Workload, make_inputs

pytestmark = pytest.mark.gpu

CASES = [
    # name, B, Hq, Hkv, Lq, Lk, dtype, mask, window
    ("w100_g2", 2, 32, 16, 1024, 1024, "bf16", MASK_WINDOW, 100),
    ("w1024_ragged_mha", 2, 16, 16, 1000, 1000, "bf16", MASK_WINDOW, 1024),
    ("causal_short_g2", 2, 32, 16, 1024, 1024, "bf16", MASK_CAUSAL, 0),
    ("w333_f16", 2, 32, 16, 1024, 1024, "f16", MASK_WINDOW, 333),
    ("twosided_w300", 2, 32, 16, 1024, 1024, "bf16", MASK_TWO_SIDED, 300),
    ("w1_zero_grads", 2, 32, 16, 1024, 1024, "bf16", MASK_WINDOW, 1),
    ("w64_g4", 4, 32, 8, 1024, 1024, "bf16", MASK_WINDOW, 64),
    ("suffix_w256", 1, 32, 16, 512, 2048, "bf16", MASK_WINDOW, 256),
    ("w700_ragged_1900", 1, 32, 16, 1900, 2048, "bf16", MASK_WINDOW, 700),
    ("w130_L1153", 2, 32, 16, 1153, 1153, "bf16", MASK_WINDOW, 130),
    ("twosided_w1024_34tiles", 1, 16, 16, 2304, 2304, "bf16", MASK_TWO_SIDED, 1024),
]


def _run(w, inp, ws_bytes):
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    o, lse = sdpa_fwd_lse(q, k, v, w.mask, w.window, w.scale)
    ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=DEV)
    ws.fill_(255)   # NaN bit patterns: a band entry read before it was written would show
    dq, dk, dv = sdpa_bwd(q, k, v, o, do, lse, w.mask, w.window, w.scale, workspace=ws)
    torch.cuda.synchronize()
    return {"O": o, "lse": lse, "dQ": dq, "dK": dk, "dV": dv}


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_band_path_matches_oracle(case):
    name, B, Hq, Hkv, Lq, Lk, dtype, mask, window = case
    w = Workload(name, B, Hq, Hkv, Lq, 256, dtype, mask, window, seed=15000 + Lq + window, Lk=Lk)
    assert B * Hkv * -(-Lk // 128) >= 256, "the case must run the 16-key dK/dV kernel"
    inp = make_inputs(w)
    dt = w.torch_dtype
    small = workspace_bytes(B, Hq, Lq, 256, dt)
    full = bwd_workspace_bytes(B, Hq, Hq // Hkv, Lq, Lk, 256, dt, mask, window)
    assert full > small, "the case must keep dS for its band"
    band = _run(w, inp, full)
    plain = _run(w, inp, small)
    ref = oracle.sdpa_fwd_bwd(inp["q"], inp["k"], inp["v"], inp["do"], w.scale, w.mask, w.window)
    tol = TOL[dtype]
    errs = {n: rel_fro(_np(band[n]), ref[n]) for n in ("O", "dQ", "dK", "dV") if np.linalg.norm(ref[n]) > 0}
    fin = np.isfinite(ref["lse"])
    errs["lse"] = float(np.max(np.abs(_np(band["lse"])[fin] - ref["lse"][fin]), initial=0.0))
    errs["dQ_vs_plain"] = rel_fro(_np(band["dQ"]), _np(plain["dQ"])) if torch.any(plain["dQ"] != 0) else 0.0
    print(name, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for n in ("dQ", "dK", "dV"):
        assert torch.isfinite(band[n]).all(), n
    if window == 1:   # only the diagonal: dQ and dK are exactly zero in exact arithmetic
        ref2 = oracle.sdpa_fwd_bwd(inp["q"], inp["k"], inp["v"], inp["do"], w.scale, w.mask, 2)
        for n in ("dQ", "dK"):
            assert np.linalg.norm(_np(band[n])) <= 1e-2 * np.linalg.norm(ref2[n]), n
    for n in ("O", "dQ", "dK", "dV"):
        if n in errs:
            assert errs[n] <= tol, (n, errs[n])
    assert errs["lse"] <= LSE_TOL
    # same dK/dV kernel on both paths, Delta summed in another order (at window
    # 1 the dQ and dK of both are rounding noise around an exact zero, checked above)
    if window != 1:
        assert errs["dQ_vs_plain"] <= tol
    for n in ("dK", "dV") if window != 1 else ("dV",):
        e = rel_fro(_np(band[n]), _np(plain[n]))
        assert e <= 2e-3, (n, e)


def test_band_path_is_deterministic():
    w = Workload("det", 2, 32, 16, 1024, 256, "bf16", MASK_WINDOW, 200, seed=15500)
    inp = make_inputs(w)
    full = bwd_workspace_bytes(2, 32, 2, 1024, 1024, 256, torch.bfloat16, MASK_WINDOW, 200)
    a = _run(w, inp, full)
    b = _run(w, inp, full)
    for n in ("dQ", "dK", "dV"):
        assert torch.equal(a[n], b[n]), n
