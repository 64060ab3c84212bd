"""The allocation-free backward (run on an MI355X).

sdpa_bwd_noalloc is sdpa_bwd with the library's fixed per-GPU scratch in
place of a workspace. Two calls in a row, the second on a smaller problem
(so the scratch holds the first call's data when the second starts), are
each compared with sdpa_bwd on the same inputs given a workspace of the
same size as that scratch (same plan: results bitwise equal) and with the
fp64 oracle. Called through the C ABI with ctypes.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from sdpa_backward_amd import _lib, sdpa_bwd, sdpa_fwd_lse
from tests.oracle_pins import rel_fro
from tests.test_parity import DEV, TOL, _np
from workloads import MASK_CAUSAL, MASK_WINDOW, Workload, make_inputs

pytestmark = pytest.mark.gpu

SCRATCH = 64 << 20   # SDPA_NOALLOC_SCRATCH_BYTES


def _noalloc_abi(q, k, v, o, do, lse, w):
    lib = _lib.load()
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    st = lib.sdpa_bwd_noalloc(P(q), P(k), P(v), P(o), P(do), P(lse), P(dq), P(dk), P(dv), w.B, w.Hq, w.group,
                              w.L, w.Lkv, w.D, _lib.DTYPE[q.dtype], _lib.MASK[w.mask],
                              w.window if "window" in w.mask else 0, w.scale,
                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lib.sdpa_status_string(st)
    return dq, dk, dv


def test_noalloc_two_calls_match_sdpa_bwd():
    cases = [
        # the dS band buffer (32 MiB) fits the scratch: band plan
        Workload("noalloc_band", 2, 32, 16, 1024, 256, "bf16", MASK_WINDOW, 100, seed=16001),
        # smaller: the small-problem split fits: split plan
        Workload("noalloc_split", 1, 4, 2, 300, 128, "bf16", MASK_CAUSAL, 0, seed=16002),
    ]
    for w in cases:
        print("case", w.name, flush=True)
        inp = make_inputs(w)
        q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
        o, lse = sdpa_fwd_lse(q, k, v, w.mask, w.window, w.scale)
        got = _noalloc_abi(q, k, v, o, do, lse, w)
        ws = torch.empty(SCRATCH, dtype=torch.uint8, device=DEV)
        want = sdpa_bwd(q, k, v, o, do, lse, w.mask, w.window, w.scale, workspace=ws)
        torch.cuda.synchronize()
        ref = oracle.sdpa_fwd_bwd(inp["q"], inp["k"], inp["v"], inp["do"], w.scale, w.mask, w.window)
        for n, a, b in zip(("dQ", "dK", "dV"), got, want):
            e = rel_fro(_np(a), ref[n])
            print(w.name, n, f"vs oracle {e:.2e}", flush=True)
            assert torch.equal(a, b), (w.name, n)
            assert e <= TOL[w.dtype], (w.name, n, e)
