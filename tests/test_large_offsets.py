"""Tensors whose element offsets pass 2^31 (run on an MI355X).

Q, O, dO, dQ of [1, 32, 2^20, 128] hold 2^32 elements each (8 GiB in bf16), so
every 32-bit element index would wrap inside the last heads. The window (128)
makes the attention local, which is what lets the fp64 oracle check it: row
i depends only on keys (i - 128, i], so on any stretch [s, s + 3W) of the
sequence the rows and keys in [s + W, s + 3W) (rows) and [s + W, s + 2W)
(keys) have all their inputs inside the stretch, and the oracle run on the
stretch alone gives their exact values. Stretches are taken at the start,
middle and end of the sequence, and every q-head (group 32: one kv head) is
compared.
"""
import numpy as np
import pytest
import torch

import oracle
from sdpa_backward_amd import sdpa_bwd, sdpa_fwd_lse
from tests.oracle_pins import rel_fro
from workloads import MASK_WINDOW

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_offsets_beyond_2_pow_31():
    B, Hq, Hkv, L, D, W = 1, 32, 1, 1 << 20, 128, 128
    scale = D ** -0.5
    g = torch.Generator(device=DEV).manual_seed(7500)
    q = torch.randn(B, Hq, L, D, generator=g, device=DEV, dtype=torch.bfloat16)
    k = torch.randn(B, Hkv, L, D, generator=g, device=DEV, dtype=torch.bfloat16)
    v = torch.randn(B, Hkv, L, D, generator=g, device=DEV, dtype=torch.bfloat16)
    do = torch.randn(B, Hq, L, D, generator=g, device=DEV, dtype=torch.bfloat16)
    assert q.numel() == 1 << 32
    o, lse = sdpa_fwd_lse(q, k, v, MASK_WINDOW, W, scale)
    dq, dk, dv = sdpa_bwd(q, k, v, o, do, lse, MASK_WINDOW, W, scale)
    torch.cuda.synchronize()
    for s in (0, L // 2 - W, L - 3 * W):
        sl = slice(s, s + 3 * W)
        sub = {n: t[:, :, sl].cpu() for n, t in (("q", q), ("k", k), ("v", v), ("do", do))}
        ref = oracle.sdpa_fwd_bwd(sub["q"], sub["k"], sub["v"], sub["do"], scale, MASK_WINDOW, W)
        rows = slice(W, 3 * W) if s > 0 else slice(0, 3 * W)   # a stretch at 0 has no earlier keys
        keys = slice(W, 2 * W) if s > 0 else slice(0, 2 * W)
        got = {"O": o[:, :, sl][:, :, rows], "dQ": dq[:, :, sl][:, :, rows],
               "dK": dk[:, :, sl][:, :, keys], "dV": dv[:, :, sl][:, :, keys]}
        errs = {n: rel_fro(t.double().cpu().numpy(), ref[n][:, :, rows if n in ("O", "dQ") else keys])
                for n, t in got.items()}
        errs["lse"] = float(np.max(np.abs(lse[:, :, sl][:, :, rows].double().cpu().numpy() - ref["lse"][:, :, rows])))
        print("stretch", s, {n: f"{e:.2e}" for n, e in errs.items()}, flush=True)
        for n in ("O", "dQ", "dK", "dV"):
            assert errs[n] <= 1e-2, (s, n, errs[n])
        assert errs["lse"] <= 1e-4, (s, errs["lse"])
