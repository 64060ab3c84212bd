"""A seeded parity sweep over random problems (run on an MI355X).

Modelled on the pages' own parity sweep of the windowed backward (page "Lab
028 lab detail: Off NVIDIA, you fix the platform yourself", section "Gradient
parity": fp32 / fp16 / bf16, head dims 64 to 512, GQA ratios, lengths with
queries shorter than keys, windows from 1 up, causal and not): 160 small
cases (keys below 700, 400 at D = 512) and 24 longer ones (300 to 3000 keys,
1500 at D = 512; windows up to 5000). Every case
draws its shape, mask, window, dtype, layout and optional sinks / cut from a
seeded generator, runs forward and backward through the library and is
compared with the fp64 oracle: O and dV within the dtype's relative gate, lse
within 1e-4 where finite, the same -inf / exact zeros where the oracle has
them, and dQ, dK, d sinks within the gate plus the error their conditioning
allows (below). Head counts stay small so the whole sweep runs in a few minutes.

Why dQ, dK and d sinks get a conditioning term: they depend on
Delta_i = <dO_i, O_i>, which the backward forms from the forward's O rounded
to the input type (as the pages' backward uses its forward's output).
Rounding to nearest moves each O element by a uniform fraction of at most
u / 2 (u: the input type's unit roundoff), so Delta_i moves by about
dD_i = u / (2 sqrt 3) * sqrt(sum_d (dO_id O_id)^2) (the spread of that sum);
that moves dQ_i by scale * dD_i * ||sum_j P_ij k_j||, dK by
scale * P^T (dD * Q), d sinks by sum_i p_i dD_i. With few keys per row,
dP - Delta cancels and three times this spread can exceed the plain gate; it
is computed from the oracle alone (attention with K as the values gives
sum_j P_ij k_j; the dV of a backward with dO replaced by dD * Q gives
P^T (dD * Q)). d sinks, a sum over rows of terms of both signs, is held to
the summation bound tol * sum_i |p_i Delta_i| rather than tol * |d sinks|.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from sdpa_backward_amd import sdpa_bwd, sdpa_fwd_lse
from tests.oracle_pins import rel_fro
from tests.test_parity import DEV, LSE_TOL, TOL

pytestmark = pytest.mark.gpu

N_CASES = 160
DTYPES = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def draw(rng):
    dtype = rng.choice(["bf16", "bf16", "f16", "f32"])
    D = int(rng.choice([64, 128, 256, 512]))
    Hkv = int(rng.choice([1, 2, 4]))
    group = int(rng.choice([1, 2, 4]))
    B = int(rng.choice([1, 1, 2]))
    Lk = int(rng.integers(1, 700 if D <= 256 else 400))
    Lq = int(rng.choice([Lk, Lk, int(rng.integers(1, Lk + 1)), int(rng.integers(1, 2 * Lk + 2))]))
    mask = str(rng.choice(["causal", "causal_window", "window", "none"]))
    window = int(rng.choice([1, 2, 7, 64, 100, 129, 1000, 5000])) if "window" in mask else 0
    scale = float(rng.choice([D ** -0.5, D ** -0.5, 1.0, 0.3]))
    layout = str(rng.choice(["bhld", "bhld", "blhd"]))
    sinks = bool(rng.random() < 0.25)
    cut = None
    if rng.random() < 0.2 and Lk > 4 and Lq > 1:
        c0 = int(rng.integers(0, Lk - 1))
        c1 = int(rng.integers(c0 + 1, Lk + 1))
        cut = (int(rng.integers(0, Lq + 1)), c0, c1)
    return dict(dtype=dtype, D=D, Hq=Hkv * group, Hkv=Hkv, B=B, Lq=Lq, Lk=Lk, mask=mask, window=window,
                scale=scale, layout=layout, sinks=sinks, cut=cut)


def inputs(c, seed):
    g = torch.Generator().manual_seed(seed)
    t = lambda H, L: torch.randn(c["B"], H, L, c["D"], generator=g).to(DTYPES[c["dtype"]])
    q, k, v, do = t(c["Hq"], c["Lq"]), t(c["Hkv"], c["Lk"]), t(c["Hkv"], c["Lk"]), t(c["Hq"], c["Lq"])
    sinks = (math.log(max(c["Lk"], 2)) + torch.randn(c["Hq"], generator=g)).float() if c["sinks"] else None
    return q, k, v, do, sinks


def on_gpu(x, layout):
    x = x.to(DEV)
    return x.transpose(1, 2).contiguous().transpose(1, 2) if layout == "blhd" else x


def draw_long(rng):
    """Longer sequences, as in the pages' sweep (lengths 300 to 3000, queries
    shorter than keys, windows up to 5000), at few heads so the fp64 oracle
    stays within seconds per case."""
    dtype = str(rng.choice(["bf16", "bf16", "f16", "f32"]))
    D = int(rng.choice([64, 128, 256, 256, 512]))
    Hkv = int(rng.choice([1, 2]))
    group = int(rng.choice([1, 2, 4]))
    Lk = int(rng.integers(300, 1500 if D == 512 else 3001))
    Lq = int(rng.choice([Lk, int(rng.integers(1, Lk + 1)), int(rng.integers(1, Lk + 1))]))
    mask = str(rng.choice(["causal", "causal_window", "causal_window", "window", "none"]))
    window = int(rng.choice([1, 64, 333, 1000, 2048, 5000])) if "window" in mask else 0
    scale = float(rng.choice([D ** -0.5, D ** -0.5, 1.0]))
    return dict(dtype=dtype, D=D, Hq=Hkv * group, Hkv=Hkv, B=1, Lq=Lq, Lk=Lk, mask=mask, window=window,
                scale=scale, layout=str(rng.choice(["bhld", "bhld", "blhd"])), sinks=bool(rng.random() < 0.2),
                cut=None)


N_LONG = 24
CASES = [draw(np.random.default_rng(12000 + i)) for i in range(N_CASES)]
CASES += [draw_long(np.random.default_rng(14000 + i)) for i in range(N_LONG)]


@pytest.mark.parametrize("i", range(N_CASES + N_LONG))
def test_sweep_case(i):
    c = CASES[i]
    q, k, v, do, sinks = inputs(c, 13000 + i)
    ref = oracle.sdpa_fwd_bwd(q, k, v, do, c["scale"], c["mask"], c["window"],
                              sinks=None if sinks is None else sinks.double().numpy(), cut=c["cut"])
    qg, kg, vg, dog = (on_gpu(x, c["layout"]) for x in (q, k, v, do))
    sg = None if sinks is None else sinks.to(DEV)
    o, lse = sdpa_fwd_lse(qg, kg, vg, c["mask"], c["window"], c["scale"], sinks=sg, cut=c["cut"])
    grads = sdpa_bwd(qg, kg, vg, o, dog, lse, c["mask"], c["window"], c["scale"], sinks=sg, cut=c["cut"])
    torch.cuda.synchronize()
    got = {"O": o, "dQ": grads[0], "dK": grads[1], "dV": grads[2]}
    if sinks is not None:
        got["dSinks"] = grads[3]
    f = lambda t: t.detach().to("cpu", torch.float64).numpy()
    tol = TOL[c["dtype"]]
    errs = {n: rel_fro(f(t), ref[n]) for n, t in got.items()}
    lse_ref, lse_got = ref["lse"], f(lse)
    fin = np.isfinite(lse_ref)
    print(i, c, {n: f"{e:.1e}" for n, e in errs.items()}, flush=True)
    assert np.array_equal(np.isfinite(lse_got), fin), "rows with no key differ"
    assert float(np.max(np.abs(lse_got[fin] - lse_ref[fin]), initial=0.0)) <= LSE_TOL
    # error the rounded O may put into Delta (per row), carried into dQ, dK, d sinks
    u = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "f32": 2.0 ** -24}[c["dtype"]]
    q64, k64, do64 = (x.double().numpy() for x in (q, k, do))
    d_delta = u / (2 * math.sqrt(3)) * np.sqrt(np.sum((do64 * ref["O"]) ** 2, axis=-1))  # [B, Hq, Lq]
    kw = dict(sinks=None if sinks is None else sinks.double().numpy(), cut=c["cut"])
    pk, _ = oracle.sdpa_forward(q64, k64, k64, c["scale"], c["mask"], c["window"], **kw)   # sum_j P_ij k_j
    cond = {"dQ": c["scale"] * np.linalg.norm(d_delta[..., None] * pk)}
    pt = oracle.sdpa_fwd_bwd(q64, k64, k64, d_delta[..., None] * q64, c["scale"], c["mask"], c["window"], **kw)
    cond["dK"] = c["scale"] * np.linalg.norm(pt["dV"])                            # P^T (dDelta * Q)
    bound = {n: tol * np.linalg.norm(ref[n]) + 3 * cond.get(n, 0.0) for n in ("O", "dQ", "dK", "dV")}
    if sinks is not None:
        p_sink = np.exp(sinks.double().numpy()[None, :, None] - ref["lse"])       # [B, Hq, Lq]
        bound["dSinks"] = np.linalg.norm(tol * np.sum(np.abs(p_sink * ref["Delta"]), axis=(0, 2)) +
                                         3 * np.sqrt(np.sum((p_sink * d_delta) ** 2, axis=(0, 2))))
    for n in got:
        err = float(np.linalg.norm(f(got[n]) - ref[n]))
        assert err <= bound[n], (n, err / max(float(np.linalg.norm(ref[n])), 1e-300), err, bound[n])
