"""Peak device memory of one forward + backward is linear in L (run on an MI355X).

The library allocates nothing: outputs and the backward workspace are torch
tensors, so torch's peak-allocation counter sees every byte. Above the inputs,
one fwd+bwd holds exactly O, lse, dQ, dK, dV and the backward workspace; the
test checks that sum and that doubling L doubles it, at the two attention
layer shapes the pages measure (page "Lab 028 lab detail: Off NVIDIA, you fix
the platform yourself", section "Build log, 2026-10-21", peak-memory table:
32 q-heads with 16 kv heads at D = 256 under a 1024-key causal window, and the
causal D = 512 layer, here with the benchmark's 16 q-heads and 4 kv heads), at
the pages' lengths up to 32,768 tokens. Values do not matter for memory, so
the inputs are drawn on the GPU. Every length has at least 256 key blocks per
call (or D = 512), so the small-problem dK/dV split, whose fp32 shares are
linear in L too but sized by the block count, stays off.
"""
import pytest
import torch

from sdpa_backward_amd import bwd_workspace_bytes, sdpa_bwd, sdpa_fwd_lse
from workloads import MASK_CAUSAL, MASK_WINDOW

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

GEOMS = {
    # name: (Hq, Hkv, D, mask, window, lengths)
    "window1024_h32kv16_D256": (32, 16, 256, MASK_WINDOW, 1024, (4096, 8192, 16384, 32768)),
    "causal_h16kv4_D512": (16, 4, 512, MASK_CAUSAL, 0, (2048, 4096, 8192, 16384, 32768)),
}


def peak_above_inputs(Hq, Hkv, D, mask, window, L, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    mk = lambda H: torch.randn(1, H, L, D, generator=g, device=DEV, dtype=torch.float32).to(torch.bfloat16)
    q, k, v, do = mk(Hq), mk(Hkv), mk(Hkv), mk(Hq)
    scale = D ** -0.5
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    base = torch.cuda.memory_allocated(DEV)
    torch.cuda.reset_peak_memory_stats(DEV)
    o, lse = sdpa_fwd_lse(q, k, v, mask, window, scale)
    dq, dk, dv = sdpa_bwd(q, k, v, o, do, lse, mask, window, scale)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated(DEV) - base
    outs = sum(t.numel() * t.element_size() for t in (o, lse, dq, dk, dv))
    ws = bwd_workspace_bytes(1, Hq, Hq // Hkv, L, L, D, q.dtype, mask, window)
    finite = all(bool(torch.isfinite(t).all()) for t in (o, dq, dk, dv))
    del q, k, v, do, o, lse, dq, dk, dv
    torch.cuda.empty_cache()
    return peak, outs + ws, ws, finite


@pytest.mark.parametrize("geom", list(GEOMS))
def test_peak_memory_is_linear_in_L(geom):
    Hq, Hkv, D, mask, window, Ls = GEOMS[geom]
    peaks = []
    for i, L in enumerate(Ls):
        peak, expect, ws, finite = peak_above_inputs(Hq, Hkv, D, mask, window, L, 7400 + i)
        print(f"{geom} L={L}: peak above inputs {peak / 1e9:.3f} GB (outputs + workspace {expect / 1e9:.3f} GB, "
              f"workspace {ws / 1e9:.3f} GB)", flush=True)
        assert finite, L
        # torch's allocator counts a tensor at a multiple of 512 bytes, and one
        # above 1 MiB at its whole segment (2 MiB granularity) unless more than
        # 1 MiB of it is left over: at most 1 MiB more for each of the six tensors
        assert expect <= peak <= expect + 6 * 2**20, (L, peak, expect)
        peaks.append(peak)
    for a, b in zip(peaks, peaks[1:]):
        assert abs(b / a - 2.0) < 0.01, peaks
