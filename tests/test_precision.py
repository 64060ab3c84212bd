"""Accuracy under peaked softmax at scale 1.0 (run on an MI355X).

The pages' layers attend at scale 1.0 with head-0 scores reaching 20 to 27;
there, score tiles held in bf16 cost 5-7 % relative error in dQ, and fp32
S / dP tiles brought it to 0.5-1.5 % (dQ), 0.4-0.7 % (dK), 0.28 % (dV) with
cosines of 0.9999 or better (page "Lab 028 lab detail: Off NVIDIA, you fix the
platform yourself", sections "fp32 gradient truth" (layer level) and "fp32
score tiles"). The kernels keep S, the softmax state and dP in fp32 and round
only P and dS to bf16 as MFMA operands, so they should sit in the second
regime.

Synthetic stand-in for the pages' activations (their data and weights are not
available): Q, K i.i.d. N(0, sigma^2) with sigma^2 = 7.5 / sqrt(D), so a score
<q, k> has standard deviation 7.5 and each row's largest scores over ~1000
keys land around 20-27; V, dO i.i.d. N(0, 1); bf16 and fp16 inputs.
Reported, as in the pages' table: cosine and relative L2 error of dQ, dK, dV
against the fp64 oracle on the same rounded inputs, per geometry (sliding layer: D = 256, window
1024; full layer: D = 512, causal, GQA group 4).
"""
import numpy as np
import pytest
import torch

import oracle
from tests.oracle_pins import rel_fro
from tests.test_parity import DEV, _np, run
from workloads import MASK_CAUSAL, MASK_WINDOW, Workload

pytestmark = pytest.mark.gpu

GEOMS = [
    # name, Hq, Hkv, L, D, mask, window
    ("sliding_D256_w1024", 4, 2, 2048, 256, MASK_WINDOW, 1024),
    ("full_D512_causal", 4, 1, 2048, 512, MASK_CAUSAL, 0),
]


def peaked_inputs(w, seed):
    """Q, K with score standard deviation 7.5 at scale 1; V, dO standard normal (input dtype)."""
    g = torch.Generator().manual_seed(seed)
    sigma = (7.5 / w.D ** 0.5) ** 0.5
    q = torch.randn(1, w.Hq, w.L, w.D, generator=g) * sigma
    k = torch.randn(1, w.Hkv, w.L, w.D, generator=g) * sigma
    v = torch.randn(1, w.Hkv, w.L, w.D, generator=g)
    do = torch.randn(1, w.Hq, w.L, w.D, generator=g)
    return {n: t.to(w.torch_dtype) for n, t in (("q", q), ("k", k), ("v", v), ("do", do))}


def cosine(a, b):
    a, b = a.ravel(), b.ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


# relative-error gates per input type: (dQ, dK / dV / O); bf16 as in the
# pages' fp32-tile regime, fp16 scaled by its 8x smaller unit roundoff
GATES = {"bf16": (2e-2, 1e-2), "f16": (4e-3, 2e-3)}


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("geom", GEOMS, ids=[g[0] for g in GEOMS])
def test_peaked_scores_scale_one(geom, dtype):
    name, Hq, Hkv, L, D, mask, window = geom
    w = Workload(f"{name}_{dtype}", 1, Hq, Hkv, L, D, dtype, mask, window, seed=9000 + D)
    inp = peaked_inputs(w, w.seed)
    # the workload is what it claims: head-0 row maxima of the allowed scores reach 20-27
    q0 = inp["q"][0, 0].double()
    k0 = inp["k"][0, 0].double()
    S = q0 @ k0.T
    i = torch.arange(L)[:, None]
    j = torch.arange(L)[None, :]
    ok = (j <= i) & ((j > i - window) if mask == MASK_WINDOW else True)
    rowmax = S.masked_fill(~ok, float("-inf")).max(dim=1).values[L // 2:]
    print(name, "head-0 row max of scores: median %.1f, 90th pct %.1f" %
          (rowmax.median().item(), rowmax.quantile(0.9).item()), flush=True)
    assert 18.0 <= rowmax.median().item() <= 30.0

    gpu = run(w, inp, scale=1.0)
    ref = oracle.sdpa_fwd_bwd(inp["q"], inp["k"], inp["v"], inp["do"], 1.0, w.mask, w.window)
    cos = {n: cosine(_np(gpu[n]), ref[n]) for n in ("O", "dQ", "dK", "dV")}
    rel = {n: rel_fro(_np(gpu[n]), ref[n]) for n in ("O", "dQ", "dK", "dV")}
    lse = float(np.max(np.abs(_np(gpu["lse"]) - ref["lse"])))
    print(f"| {name} | {dtype} inputs; fp32 S/dP tiles, {dtype} P/dS operands | "
          f"{cos['dQ']:.5f} / {cos['dK']:.5f} / {cos['dV']:.5f} | "
          f"{100 * rel['dQ']:.2f}% / {100 * rel['dK']:.2f}% / {100 * rel['dV']:.2f}% | "
          f"O {100 * rel['O']:.2f}%, lse {lse:.1e} |", flush=True)
    # gates: the pages' fp32-tile regime for bf16 (cosine >= 0.9999; relative
    # error at most 2 % on dQ, 1 % on dK, dV and O), lse as everywhere else
    gq, g = GATES[dtype]
    for n in ("dQ", "dK", "dV", "O"):
        assert cos[n] >= 0.9999, (n, cos[n])
    assert rel["dQ"] <= gq and rel["dK"] <= g and rel["dV"] <= g and rel["O"] <= g, rel
    assert lse <= 1e-4
