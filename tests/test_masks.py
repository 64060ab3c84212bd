"""GPU parity of the mask variants (run on an MI355X): no mask, the window on
both sides of the diagonal, and queries that are the last Lq of Lk key
positions (Lq < Lk), plus more queries than keys (Lq > Lk), where the first
rows see no key at all.

Each case runs through the C ABI and is compared with the fp64 oracle on the
same inputs: relative Frobenius error per tensor (1e-2 bf16, 2e-3 fp16, 1e-5
fp32), lse
max-abs 1e-4 on rows that have keys; rows with no key must hold exactly
O = 0, lse = -inf, dQ = 0, and keys that no row sees exactly dK = dV = 0
(page "Lab 028 lab detail: Off NVIDIA, you fix the platform yourself",
"What I changed, in plain terms", items 3-5: the non-causal window, and keys
behind every query's window when the queries are a suffix of the keys).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from sdpa_backward_amd import sdpa_bwd, sdpa_fwd_lse
from tests.oracle_pins import rel_fro
from tests.test_parity import DEV, LSE_TOL, TOL, _check_poison, _np, _poisoned_outputs, run
from workloads import BY_NAME, MASK_CAUSAL, MASK_NONE, MASK_TWO_SIDED, MASK_WINDOW, Workload, make_inputs

pytestmark = pytest.mark.gpu

CASES = [
    # name, Hq, Hkv, Lq, Lk, D, dtype, mask, window
    ("none_D64", 2, 1, 200, 200, 64, "bf16", MASK_NONE, 0),
    ("none_ragged_D256", 4, 2, 333, 333, 256, "bf16", MASK_NONE, 0),
    ("none_D512_g2", 2, 1, 300, 300, 512, "bf16", MASK_NONE, 0),
    ("two_w64_D128", 4, 2, 500, 500, 128, "bf16", MASK_TWO_SIDED, 64),
    ("two_w100_D256", 2, 1, 700, 700, 256, "bf16", MASK_TWO_SIDED, 100),
    ("two_w37_D512", 2, 1, 400, 400, 512, "bf16", MASK_TWO_SIDED, 37),
    ("two_w2_D64", 2, 2, 130, 130, 64, "bf16", MASK_TWO_SIDED, 2),
    ("suffix_causal_D256", 4, 2, 300, 1000, 256, "bf16", MASK_CAUSAL, 0),
    ("suffix_w128_D256", 4, 2, 250, 1300, 256, "bf16", MASK_WINDOW, 128),
    ("suffix_two_w200_D128", 2, 1, 333, 1111, 128, "bf16", MASK_TWO_SIDED, 200),
    ("suffix_none_D64", 2, 2, 100, 777, 64, "bf16", MASK_NONE, 0),
    ("suffix_causal_D512", 2, 1, 200, 600, 512, "bf16", MASK_CAUSAL, 0),
    ("suffix_w100_D512", 2, 1, 150, 900, 512, "bf16", MASK_WINDOW, 100),
    ("one_query_D256", 2, 1, 1, 1000, 256, "bf16", MASK_CAUSAL, 0),
    ("prefix_causal_D256", 2, 1, 700, 300, 256, "bf16", MASK_CAUSAL, 0),
    ("prefix_two_w50_D128", 2, 1, 500, 260, 128, "bf16", MASK_TWO_SIDED, 50),
    ("prefix_none_D512", 2, 1, 300, 100, 512, "bf16", MASK_NONE, 0),
    ("one_key_D128", 2, 1, 1000, 1, 128, "bf16", MASK_CAUSAL, 0),
    ("f32_none_D64", 2, 1, 100, 100, 64, "f32", MASK_NONE, 0),
    ("f32_two_w9_D128", 2, 2, 90, 90, 128, "f32", MASK_TWO_SIDED, 9),
    ("f32_suffix_w17_D64", 2, 1, 50, 130, 64, "f32", MASK_WINDOW, 17),
    ("f32_prefix_causal_D64", 2, 1, 90, 40, 64, "f32", MASK_CAUSAL, 0),
    ("f16_none_D128", 2, 1, 300, 300, 128, "f16", MASK_NONE, 0),
    ("f16_two_w80_D256", 2, 1, 400, 400, 256, "f16", MASK_TWO_SIDED, 80),
    ("f16_suffix_w64_D512", 2, 1, 150, 700, 512, "f16", MASK_WINDOW, 64),
    ("f16_prefix_causal_D64", 2, 2, 300, 120, 64, "f16", MASK_CAUSAL, 0),
    # D = 256 calls whose keys each see >= 2048 rows and whose band is too wide
    # to keep dS: the dK/dV pass runs 8-wave workgroups (128 keys)
    ("none_wide_8wave_D256", 16, 16, 2400, 2400, 256, "bf16", MASK_NONE, 0),
    ("suffix_causal_8wave_D256_g2", 32, 16, 2200, 2600, 256, "bf16", MASK_CAUSAL, 0),
    # 16-key dK/dV pass with the dS band: keys below 1601 are behind every
    # window, so their blocks are zeroed by the launcher and not visited
    ("suffix_w200_wide_D256", 32, 16, 300, 2100, 256, "bf16", MASK_WINDOW, 200),
]


def workload(case, seed=8000):
    name, Hq, Hkv, Lq, Lk, D, dtype, mask, window = case
    return Workload(name, 1, Hq, Hkv, Lq, D, dtype, mask, window, seed=seed + Lq + 7 * Lk, Lk=Lk)


def check(w, gpu, ref, tol=None):
    """Relative errors over whole tensors, exact zeros / -inf where the oracle has them."""
    tol = TOL[w.dtype] if tol is None else tol
    lse_ref = ref["lse"]
    empty = ~np.isfinite(lse_ref)                      # rows with no allowed key
    lse = _np(gpu["lse"])
    assert np.all(lse[empty] == -np.inf), "rows with no key must get lse = -inf"
    assert np.all(np.isfinite(lse[~empty])), "rows with keys must get a finite lse"
    for n in ("O", "dQ"):
        assert np.all(_np(gpu[n])[empty] == 0.0), f"{n} of rows with no key must be exactly 0"
    unseen = np.all(ref["dK"] == 0.0, axis=-1) & np.all(ref["dV"] == 0.0, axis=-1)
    for n in ("dK", "dV"):
        assert np.all(_np(gpu[n])[unseen] == 0.0), f"{n} of keys no row sees must be exactly 0"
    errs = {n: rel_fro(_np(gpu[n]), ref[n]) for n in ("O", "dQ", "dK", "dV")}
    errs["lse"] = float(np.max(np.abs(lse[~empty] - lse_ref[~empty]), initial=0.0))
    print(w.name, {k: f"{v:.2e}" for k, v in errs.items()}, f"empty rows {int(empty.sum())}",
          f"unseen keys {int(unseen.sum())}", flush=True)
    for n in ("O", "dQ", "dK", "dV"):
        assert errs[n] <= tol, (n, errs[n])
    assert errs["lse"] <= LSE_TOL, errs["lse"]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_mask_variants_full(case):
    w = workload(case)
    inp = make_inputs(w)
    bufs, views = _poisoned_outputs(w)
    gpu = run(w, inp, out=[views[n] for n in ("O", "lse", "dQ", "dK", "dV")])
    _check_poison(w, bufs, views)
    ref = oracle.sdpa_fwd_bwd(inp["q"], inp["k"], inp["v"], inp["do"], w.scale, w.mask, w.window)
    check(w, gpu, ref)


def test_scale_one_two_sided_suffix():
    w = Workload("two_suffix_scale1", 1, 4, 2, 300, 256, "bf16", MASK_TWO_SIDED, 150, seed=8100, Lk=800)
    inp = make_inputs(w)
    ref = oracle.sdpa_fwd_bwd(inp["q"], inp["k"], inp["v"], inp["do"], 1.0, w.mask, w.window)
    check(w, run(w, inp, scale=1.0), ref)


@pytest.mark.parametrize("Lq,Lk", [(500, 500), (300, 900), (700, 250)])
def test_wide_two_sided_window_equals_no_mask_bitwise(Lq, Lk):
    w = Workload("wide2", 1, 4, 2, Lq, 256, "bf16", MASK_NONE, 0, seed=8200, Lk=Lk)
    inp = make_inputs(w)
    a = run(w, inp)
    for W in (Lq + Lk, 2**31 - 1):
        b = run(w.with_(mask=MASK_TWO_SIDED, window=W), inp)
        for n in ("O", "lse", "dQ", "dK", "dV"):
            assert torch.equal(a[n], b[n]), (W, n)


def test_window_at_least_Lk_equals_causal_bitwise_suffix():
    w = Workload("wbig_suffix", 1, 4, 2, 300, 128, "bf16", MASK_CAUSAL, 0, seed=8300, Lk=700)
    inp = make_inputs(w)
    a = run(w, inp)
    for W in (700, 2**31 - 1):
        b = run(w.with_(mask=MASK_WINDOW, window=W), inp)
        for n in ("O", "lse", "dQ", "dK", "dV"):
            assert torch.equal(a[n], b[n]), (W, n)


def test_window_one_same_for_both_kinds_bitwise():
    w = Workload("w1both", 1, 4, 2, 200, 256, "bf16", MASK_WINDOW, 1, seed=8400, Lk=450)
    inp = make_inputs(w)
    a = run(w, inp)
    b = run(w.with_(mask=MASK_TWO_SIDED), inp)
    for n in ("O", "lse", "dQ", "dK", "dV"):
        assert torch.equal(a[n], b[n]), n


@pytest.mark.parametrize("dtype,D", [("bf16", 256), ("bf16", 512), ("f32", 64)])
def test_no_keys_and_no_rows(dtype, D):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    # rows but no keys: O = 0, lse = -inf, dQ = 0 over NaN-filled outputs
    q = torch.randn(1, 4, 70, D, device=DEV).to(tdt)
    k = torch.empty(1, 2, 0, D, dtype=tdt, device=DEV)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((1, 4, 70), float("nan"), device=DEV)
    sdpa_fwd_lse(q, k, k, "causal", out=o, lse=lse)
    dq = torch.full_like(q, float("nan"))
    dk, dv = torch.empty_like(k), torch.empty_like(k)
    sdpa_bwd(q, k, k, o, q, lse, "causal", out=(dq, dk, dv))
    torch.cuda.synchronize()
    assert torch.all(o == 0).item() and torch.all(lse == -math.inf).item() and torch.all(dq == 0).item()
    # keys but no rows: dK = dV = 0 over NaN-filled outputs
    q0 = torch.empty(1, 4, 0, D, dtype=tdt, device=DEV)
    k = torch.randn(1, 2, 90, D, device=DEV).to(tdt)
    lse0 = torch.empty(1, 4, 0, device=DEV)
    dk, dv = torch.full_like(k, float("nan")), torch.full_like(k, float("nan"))
    for mask, W in (("none", 0), ("causal", 0), ("window", 5)):
        sdpa_bwd(q0, k, k, q0, q0, lse0, mask, W, out=(torch.empty_like(q0), dk, dv))
        torch.cuda.synchronize()
        assert torch.all(dk == 0).item() and torch.all(dv == 0).item(), mask


def _sample(n_total, rng, fixed, n=20):
    idx = set(i for i in fixed if 0 <= i < n_total)
    idx.update(int(x) for x in rng.integers(0, n_total, n))
    return np.array(sorted(idx))


@pytest.mark.parametrize("name", [w.name for w in BY_NAME.values() if w.name.startswith(
    ("bf16_twosided", "bf16_window1024_Lq", "bf16_nomask", "bf16_window1024_L16384_D256_h4"))])
def test_variant_workloads_sampled(name):
    """The benchmark's variant and one-GPU-share workloads, in its launch configuration: sampled
    rows (O, lse, dQ) and keys (dK, dV) against the oracle, which computes them
    one by one; NaN-filled outputs must be fully overwritten."""
    w = BY_NAME[name]
    inp = make_inputs(w)
    bufs, views = _poisoned_outputs(w)
    gpu = run(w, inp, out=[views[n] for n in ("O", "lse", "dQ", "dK", "dV")])
    _check_poison(w, bufs, views)
    rng = np.random.default_rng(w.seed)
    Lq, Lk = w.L, w.Lkv
    got = {n: [] for n in ("O", "lse", "dQ", "dK", "dV")}
    ref = {n: [] for n in got}
    for h in sorted({0, w.Hq // 2 + 1, w.Hq - 1}):
        rows = _sample(Lq, rng, [0, 1, 31, 32, 63, 64, 1023, 1024, Lq // 2, Lq - 2, Lq - 1])
        r = oracle.sampled_rows(inp["q"], inp["k"], inp["v"], inp["do"], w.scale, w.mask, w.window, 0, h, rows)
        for n in ("O", "lse", "dQ"):
            got[n].append(_np(gpu[n][0, h][torch.as_tensor(rows, device=DEV)]))
            ref[n].append(r[n])
    off = Lk - Lq
    key_fixed = [0, 1, 63, 64, off - 1024, off - 1023, off, off + 1, Lk // 2, Lk - 1025, Lk - 2, Lk - 1]
    for g in sorted({0, w.Hkv - 1}):
        keys = _sample(Lk, rng, key_fixed, n=6)
        r = oracle.sampled_keys(inp["q"], inp["k"], inp["v"], inp["do"], w.scale, w.mask, w.window, 0, g, keys)
        for n in ("dK", "dV"):
            got[n].append(_np(gpu[n][0, g][torch.as_tensor(keys, device=DEV)]))
            ref[n].append(r[n])
    errs = {}
    for n in got:
        a, b = np.concatenate(got[n]), np.concatenate(ref[n])
        errs[n] = float(np.max(np.abs(a - b))) if n == "lse" else rel_fro(a, b)
    print(w.name, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for n in ("O", "dQ", "dK", "dV"):
        assert errs[n] <= TOL[w.dtype], (n, errs[n])
    assert errs["lse"] <= LSE_TOL
    if off > w.window > 0 and w.mask == MASK_WINDOW:
        # keys behind every query's window: exactly zero gradients
        dead = off - w.window + 1
        assert torch.all(gpu["dK"][:, :, :dead] == 0).item() and torch.all(gpu["dV"][:, :, :dead] == 0).item()
