"""The key-range split of small problems (run on an MI355X).

When the query tiles of a 16-bit call give at most 128 workgroups, the
forward and the dQ pass split each query tile's key tiles into 2 or 4 ranges,
one workgroup each, and a combine pass merges the fp32 partials (the forward's
with their used max and row sum). Every case here takes that path (checked
through the workspace sizes); it is compared with the fp64 oracle over whole
tensors, and with the same calls run unsplit (an empty forward workspace, and
a backward workspace that holds only the Delta rows). The two differ only in
fp32 summation order before the final rounding to the input type. Outputs
start as NaN, so every element must be written.
"""
import numpy as np
import pytest
import torch

import oracle
from sdpa_backward_amd import bwd_workspace_bytes, fwd_workspace_bytes, sdpa_bwd, sdpa_fwd_lse, workspace_bytes
from tests.oracle_pins import rel_fro
from tests.test_parity import DEV, LSE_TOL, TOL, _np
from workloads import MASK_CAUSAL, MASK_NONE, MASK_TWO_SIDED, MASK_WINDOW, Workload, make_inputs

pytestmark = pytest.mark.gpu

CASES = [
    # name, B, Hq, Hkv, Lq, Lk, D, dtype, mask, window, shares
    ("causal_L2048_D256_h8kv4", 1, 8, 4, 2048, 2048, 256, "bf16", MASK_CAUSAL, 0, 2),
    ("causal_L1024_D512_h2kv1", 1, 2, 1, 1024, 1024, 512, "bf16", MASK_CAUSAL, 0, 4),   # empty shares early on
    ("nomask_ragged1000_D128", 1, 4, 2, 1000, 1000, 128, "bf16", MASK_NONE, 0, 4),
    ("suffix300_of_1700_D64_f16", 2, 4, 1, 300, 1700, 64, "f16", MASK_CAUSAL, 0, 4),
    ("rows_without_keys_D256", 1, 4, 2, 900, 500, 256, "bf16", MASK_CAUSAL, 0, 4),   # rows 0..399 see no key
    ("twosided300_D256_mha", 1, 8, 8, 1500, 1500, 256, "bf16", MASK_TWO_SIDED, 300, 2),
    ("window64_L2048_D256", 1, 8, 2, 2048, 2048, 256, "bf16", MASK_WINDOW, 64, 2),
]


def _nan_like(t):
    return torch.full_like(t, float("nan"))


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_split_matches_oracle_and_unsplit(case):
    name, B, Hq, Hkv, Lq, Lk, D, dtype, mask, window, shares = case
    w = Workload(name, B, Hq, Hkv, Lq, D, dtype, mask, window, seed=16000 + Lq + D, Lk=Lk)
    dt = w.torch_dtype
    rows = B * Hq * Lq
    assert fwd_workspace_bytes(B, Hq, Hq // Hkv, Lq, Lk, D, dt, mask, window) == shares * rows * (D + 2) * 4
    inp = make_inputs(w)
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))

    def fwd(ws):
        o, lse = _nan_like(q), torch.full((B, Hq, Lq), float("nan"), device=DEV)
        return sdpa_fwd_lse(q, k, v, mask, window, w.scale, out=o, lse=lse, workspace=ws)

    def bwd(o, lse, ws_bytes):
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
        out = (_nan_like(q), _nan_like(k), _nan_like(v))
        return sdpa_bwd(q, k, v, o, do, lse, mask, window, w.scale, workspace=ws, out=out)

    o_s, lse_s = fwd(None)   # the binding allocates the split's workspace
    o_u, lse_u = fwd(torch.empty(0, dtype=torch.uint8, device=DEV))
    full = bwd_workspace_bytes(B, Hq, Hq // Hkv, Lq, Lk, D, dt, mask, window)
    g_s = bwd(o_s, lse_s, full)
    g_u = bwd(o_u, lse_u, workspace_bytes(B, Hq, Lq, D, dt))
    torch.cuda.synchronize()
    ref = oracle.sdpa_fwd_bwd(inp["q"], inp["k"], inp["v"], inp["do"], w.scale, mask, window)
    got = {"O": o_s, "dQ": g_s[0], "dK": g_s[1], "dV": g_s[2]}
    for n, t in got.items():
        assert torch.isfinite(t).all(), n
    errs = {n: rel_fro(_np(t), ref[n]) for n, t in got.items() if np.linalg.norm(ref[n]) > 0}
    fin = np.isfinite(ref["lse"])
    lse = _np(lse_s)
    errs["lse"] = float(np.max(np.abs(lse[fin] - ref["lse"][fin]), initial=0.0))
    errs["O_vs_unsplit"] = rel_fro(_np(o_s), _np(o_u))
    errs["lse_vs_unsplit"] = float(np.max(np.abs(lse[fin] - _np(lse_u)[fin]), initial=0.0))
    errs["dQ_vs_unsplit"] = rel_fro(_np(g_s[0]), _np(g_u[0]))
    print(name, {n: f"{e:.2e}" for n, e in errs.items()}, flush=True)
    tol = TOL[dtype]
    for n in ("O", "dQ", "dK", "dV"):
        if n in errs:
            assert errs[n] <= tol, (n, errs[n])
    assert errs["lse"] <= LSE_TOL
    # rows with no key: O exactly 0, lse -inf, as unsplit
    assert np.array_equal(np.isfinite(lse), fin)
    assert torch.equal(torch.isfinite(lse_u), torch.isfinite(lse_s))
    if not fin.all():
        assert not _np(o_s)[~fin].any() and not _np(g_s[0])[~fin].any()
    # split vs unsplit: fp32 summation order only, then one rounding to the
    # input type (a few units of its roundoff, relative)
    assert errs["O_vs_unsplit"] <= tol / 2
    assert errs["lse_vs_unsplit"] <= 1e-5
    assert errs["dQ_vs_unsplit"] <= tol / 2


def test_split_is_deterministic():
    w = Workload("det", 1, 8, 4, 2048, 256, "bf16", MASK_CAUSAL, 0, seed=16500)
    inp = make_inputs(w)
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    runs = []
    for _ in range(2):
        o, lse = sdpa_fwd_lse(q, k, v, w.mask, 0, w.scale)
        runs.append((o, lse) + tuple(sdpa_bwd(q, k, v, o, do, lse, w.mask, 0, w.scale)))
    torch.cuda.synchronize()
    for a, b in zip(*runs):
        assert torch.equal(a, b)
