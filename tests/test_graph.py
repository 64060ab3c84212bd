"""Forward and backward captured in one HIP graph (run on an MI355X).

The library allocates nothing, sets nothing with memset and never
synchronizes, so a caller can capture a whole step (forward, then backward)
into a graph and replay it. Each case captures sdpa_fwd_lse and sdpa_bwd with
preallocated outputs and workspaces, replays the graph three times with eager
work and synchronizations in between (the outputs are overwritten with NaN
before each replay), and checks every replay bitwise against the eager calls:
the kernels are deterministic. The cases cover the three backward plans (the
dS band path, the small-problem splits, and the dQ pass that recomputes the
scores) and the forward's key-range split.
"""
import pytest
import torch

from sdpa_backward_amd import bwd_workspace_bytes, fwd_workspace_bytes, sdpa_bwd, sdpa_fwd_lse
from tests.test_parity import DEV
from workloads import MASK_CAUSAL, MASK_WINDOW, Workload, make_inputs

pytestmark = pytest.mark.gpu

CASES = [
    # band path: wide dense D = 256 call under a window
    Workload("graph_band", 2, 32, 16, 1024, 256, "bf16", MASK_WINDOW, 200, seed=17001),
    # small problem: forward / dQ key-range split and dK/dV shares
    Workload("graph_split", 1, 8, 4, 2048, 256, "bf16", MASK_CAUSAL, 0, seed=17002),
    # dQ pass recomputing the scores, 16-key dK/dV at D = 512
    Workload("graph_d512", 1, 16, 4, 1024, 512, "f16", MASK_CAUSAL, 0, seed=17003),
]


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_graph_replays_match_eager(w):
    inp = {n: t.to(DEV) for n, t in make_inputs(w).items()}
    q, k, v, do = inp["q"], inp["k"], inp["v"], inp["do"]
    dt = q.dtype
    o, dq = torch.empty_like(q), torch.empty_like(q)
    dk, dv = torch.empty_like(k), torch.empty_like(v)
    lse = torch.empty(w.B, w.Hq, w.L, dtype=torch.float32, device=DEV)
    fws = torch.empty(fwd_workspace_bytes(w.B, w.Hq, w.group, w.L, w.Lkv, w.D, dt, w.mask, w.window),
                      dtype=torch.uint8, device=DEV)
    bws = torch.empty(max(1, bwd_workspace_bytes(w.B, w.Hq, w.group, w.L, w.Lkv, w.D, dt, w.mask, w.window)),
                      dtype=torch.uint8, device=DEV)

    def step():
        sdpa_fwd_lse(q, k, v, w.mask, w.window, w.scale, out=o, lse=lse, workspace=fws)
        sdpa_bwd(q, k, v, o, do, lse, w.mask, w.window, w.scale, workspace=bws, out=(dq, dk, dv))

    outs = (o, lse, dq, dk, dv)
    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()   # a call on the capture stream before capturing
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        for t in outs:
            t.fill_(float("nan"))
        noise = torch.randn(1 << 20, device=DEV).sum()   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, a, b in zip(("O", "lse", "dQ", "dK", "dV"), outs, want):
            assert torch.equal(a, b), (w.name, r, n)
        assert torch.isfinite(noise)
