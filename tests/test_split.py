"""The small-problem dK/dV split on the GPU (run on an MI355X).

When a call's key blocks (128 keys per kv head and batch) number fewer than
256, the backward may split each key block's query tiles over 2, 4 or 8
workgroups that write fp32 shares of dK and dV into the workspace, summed in a
fixed order afterwards. Given sdpa_bwd_workspace_bytes(...) bytes it runs
unsplit; given sdpa_bwd_workspace_bytes_ex(...) bytes it splits (and so does
the dQ pass's key range when the query tiles are as few). Both must match the
fp64 oracle, and each other up to fp32 summation order.
"""
import pytest
import torch

import oracle
from sdpa_backward_amd import bwd_workspace_bytes, sdpa_bwd, sdpa_fwd_lse, workspace_bytes
from tests.oracle_pins import rel_fro
from tests.test_parity import DEV, TOL, _np
from workloads import MASK_CAUSAL, MASK_TWO_SIDED, MASK_WINDOW, Workload, make_inputs

pytestmark = pytest.mark.gpu

CASES = [
    # name, B, Hq, Hkv, Lq, Lk, D, dtype, mask, window  (shares: from the key-block count)
    ("c1_causal_D256_8x4", 1, 8, 4, 2048, 2048, 256, "bf16", MASK_CAUSAL, 0),         # 64 blocks: 4 shares
    ("w128_D128_B2", 2, 4, 2, 1500, 1500, 128, "bf16", MASK_WINDOW, 128),            # 48 blocks: 8 shares
    ("suffix_D64_g4", 1, 8, 2, 700, 1900, 64, "bf16", MASK_CAUSAL, 0),              # 30 blocks: 8 shares
    ("two_sided_ragged_D256", 1, 4, 4, 1031, 1031, 256, "f16", MASK_TWO_SIDED, 77),  # 36 blocks: 8 shares
    ("causal_D128_128blk", 1, 32, 16, 1024, 1024, 128, "bf16", MASK_CAUSAL, 0),      # 128 blocks: 2 shares
]


def _run(w, inp, ws_bytes):
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    o, lse = sdpa_fwd_lse(q, k, v, w.mask, w.window, w.scale)
    ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=DEV)
    dq, dk, dv = sdpa_bwd(q, k, v, o, do, lse, w.mask, w.window, w.scale, workspace=ws)
    torch.cuda.synchronize()
    return {"dQ": dq, "dK": dk, "dV": dv}


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_split_matches_unsplit_and_oracle(case):
    name, B, Hq, Hkv, Lq, Lk, D, dtype, mask, window = case
    w = Workload(name, B, Hq, Hkv, Lq, D, dtype, mask, window, seed=9800 + Lq, Lk=Lk)
    inp = make_inputs(w)
    dt = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    small = workspace_bytes(B, Hq, Lq, D, dt)
    big = bwd_workspace_bytes(B, Hq, Hq // Hkv, Lq, Lk, D, dt, mask, window)
    assert big > small, "the case must take the split"
    one = _run(w, inp, small)
    split = _run(w, inp, big)
    ref = oracle.sdpa_fwd_bwd(inp["q"], inp["k"], inp["v"], inp["do"], w.scale, w.mask, w.window)
    errs = {}
    # the full workspace also splits the dQ pass's key ranges (fp32 partials
    # summed in another order) when the query tiles are as few
    errs["dQ"] = (rel_fro(_np(split["dQ"]), ref["dQ"]), rel_fro(_np(split["dQ"]), _np(one["dQ"])))
    for n in ("dK", "dV"):
        errs[n] = (rel_fro(_np(split[n]), ref[n]), rel_fro(_np(split[n]), _np(one[n])))
    print(name, {k: f"{a:.2e}/{b:.2e}" for k, (a, b) in errs.items()}, flush=True)
    for n, (to_ref, to_one) in errs.items():
        assert to_ref <= TOL[dtype], (n, to_ref)
        assert to_one <= 4e-3, (n, to_one)   # a few outputs one 16-bit unit apart (fp32 sums reordered)
