"""Peak device memory of one forward + backward is linear in L (run on an MI355X).

The library allocates nothing: outputs and the backward workspace are torch
tensors, so torch's peak-allocation counter sees every byte. Above the inputs,
one fwd+bwd holds exactly O, lse, dQ, dK, dV and the workspace (one fp32 row
statistic per query row); the test checks that sum and that doubling L doubles
it, for the sliding-window geometry (window 1024) and the causal global one.
The shapes are large enough (at least 256 key blocks, or D = 512) that the
small-problem dK/dV split, whose fp32 shares are linear in L too but sized by
the block count, stays off.
"""
import pytest
import torch

from sdpa_backward_amd import bwd_workspace_bytes, sdpa_bwd, sdpa_fwd_lse
from workloads import MASK_CAUSAL, MASK_WINDOW, Workload, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def peak_above_inputs(w):
    inp = {n: x.to(DEV) for n, x in make_inputs(w).items()}
    q, k, v, do = inp["q"], inp["k"], inp["v"], inp["do"]
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    base = torch.cuda.memory_allocated(DEV)
    torch.cuda.reset_peak_memory_stats(DEV)
    o, lse = sdpa_fwd_lse(q, k, v, w.mask, w.window, w.scale)
    dq, dk, dv = sdpa_bwd(q, k, v, o, do, lse, w.mask, w.window, w.scale)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated(DEV) - base
    outs = sum(t.numel() * t.element_size() for t in (o, lse, dq, dk, dv))
    expect = outs + bwd_workspace_bytes(w.B, w.Hq, w.Hq // w.Hkv, w.L, w.Lkv, w.D, q.dtype)
    del inp, q, k, v, do, o, lse, dq, dk, dv
    torch.cuda.empty_cache()
    return peak, expect


@pytest.mark.parametrize("geom", ["window1024_D256", "causal_D512"])
def test_peak_memory_is_linear_in_L(geom):
    if geom == "window1024_D256":
        make = lambda L: Workload(f"mem_w_{L}", 1, 16, 8, L, 256, "bf16", MASK_WINDOW, 1024, seed=7400)
        Ls = (4096, 8192, 16384, 32768)
    else:
        make = lambda L: Workload(f"mem_c_{L}", 1, 4, 1, L, 512, "bf16", MASK_CAUSAL, 0, seed=7401)
        Ls = (2048, 4096, 8192, 16384)
    peaks = []
    for L in Ls:
        peak, expect = peak_above_inputs(make(L))
        print(geom, L, peak, expect, flush=True)
        # torch rounds each allocation up to 512 bytes
        assert expect <= peak <= expect + 8 * 512, (L, peak, expect)
        peaks.append(peak)
    for a, b in zip(peaks, peaks[1:]):
        assert abs(b / a - 2.0) < 0.01, peaks
