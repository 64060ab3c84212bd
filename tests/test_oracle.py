"""CPU-only pins of the fp64 oracle (no GPU, no HIP library).

The oracle is trusted only because of these checks, none of which reuses its
own formulas: a hand-derived worked example, pure-Python brute force,
central finite differences, float64 autograd of a plain forward, the library
SDPA routine, exact invariants, and mutation tests that plant plausible
mistakes into a copy of the oracle and require a pin to catch each one.
"""
import math
import os
import types

import numpy as np
import pytest
import torch

import oracle
from oracle import sdpa_oracle
from tests import oracle_pins as pins
from workloads import CONFIGS, make_inputs

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


# ---------------------------------------------------------------- golden / brute force
def test_worked_example_golden():
    assert pins.pin_golden(sdpa_oracle) <= 1e-14


def test_bruteforce_forward_tiny():
    assert pins.pin_brute(sdpa_oracle) <= 1e-12


# ---------------------------------------------------------------- finite differences
FD_CASES = [
    # Hq, Hkv, L, D, scale, mask, window
    (1, 1, 1, 1, 1.0, "causal", 0),
    (1, 1, 2, 4, 0.5, "causal", 0),
    (2, 1, 7, 4, 0.5, "causal", 0),
    (2, 2, 7, 8, 1 / math.sqrt(8), "causal", 0),
    (4, 1, 13, 4, 3.0, "causal", 0),
    (4, 2, 13, 1, 1.0, "causal_window", 1),
    (2, 1, 13, 4, 1.0, "causal_window", 2),
    (4, 4, 16, 8, 1 / math.sqrt(8), "causal_window", 3),
    (2, 2, 16, 4, 3.0, "causal_window", 5),
    (4, 1, 16, 4, 0.5, "causal_window", 16),
    (1, 1, 7, 8, 1.0, "causal_window", 14),
    (4, 2, 16, 8, 1.0, "causal_window", 5),
]


@pytest.mark.parametrize("case", FD_CASES, ids=[str(c) for c in FD_CASES])
def test_finite_differences_exhaustive(case):
    Hq, Hkv, L, D, s, mask, W = case
    assert pins.fd_error(sdpa_oracle, Hq, Hkv, L, D, s, mask, W) <= 1e-7


@pytest.mark.parametrize("mask,window", [("causal", 0), ("causal_window", 40)])
def test_finite_differences_directional_tiny_config_shape(mask, window):
    # the tiny fp32 workload's geometry: Hq=2, Hkv=1, L=128, D=64, scale 1/8
    assert pins.fd_directional_error(sdpa_oracle, 2, 1, 128, 64, 0.125, mask, window) <= 1e-7


# ---------------------------------------------------------------- independent autograd
def _cfg_inputs(w, **shrink):
    w = w.with_(**shrink) if shrink else w
    t = make_inputs(w)
    return [t[n].to(torch.float64).numpy() for n in ("q", "k", "v", "do")], w


@pytest.mark.parametrize("which,shrink", [
    (0, {}),
    (1, {}),
    (2, {"Hq": 4, "Hkv": 1, "L": 1024}),      # global layer geometry (D=512, group 4), shortened
    (3, {"Hq": 4, "Hkv": 2, "L": 1500, "window": 300}),  # sliding geometry, several windows
    (4, {"Hq": 2, "Hkv": 1, "L": 777, "window": 129}),   # ragged length, window not a power of 2
])
def test_autograd_independent(which, shrink):
    (q, k, v, do), w = _cfg_inputs(CONFIGS[which], **shrink)
    err = pins.autograd_error(sdpa_oracle, q, k, v, do, w.scale, w.mask, w.window)
    assert err <= 1e-12, err


def test_library_sdpa_forward():
    import torch.nn.functional as F
    for which, shrink in ((0, {}), (1, {"L": 1024}), (3, {"Hq": 4, "Hkv": 2, "L": 700, "window": 100})):
        (q, k, v, do), w = _cfg_inputs(CONFIGS[which], **shrink)
        O, lse = oracle.sdpa_forward(q, k, v, w.scale, w.mask, w.window)
        L = w.L
        i = torch.arange(L)[:, None]
        j = torch.arange(L)[None, :]
        ok = j <= i
        if w.mask == "causal_window":
            ok = ok & (j > i - w.window)
        ref = F.scaled_dot_product_attention(
            torch.tensor(q), torch.tensor(k), torch.tensor(v), attn_mask=ok, scale=w.scale, enable_gqa=True)
        assert pins.rel_fro(O, ref.numpy()) <= 1e-12
        if w.mask == "causal":
            ref2 = F.scaled_dot_product_attention(
                torch.tensor(q), torch.tensor(k), torch.tensor(v), is_causal=True, scale=w.scale, enable_gqa=True)
            assert pins.rel_fro(O, ref2.numpy()) <= 1e-12


# ---------------------------------------------------------------- invariants
def _rand(Hq=4, Hkv=2, L=37, D=8, seed=5):
    return pins.tiny_inputs(Hq, Hkv, L, D, seed)


def test_softmax_rows_sum_to_one():
    q, k, v, do = _rand()
    ones = np.ones_like(v)
    for mask, W in (("causal", 0), ("causal_window", 5), ("causal_window", 1)):
        O, _ = oracle.sdpa_forward(q, k, ones, 0.7, mask, W)
        assert np.max(np.abs(O - 1.0)) <= 1e-14


def test_ds_rows_sum_to_zero():
    # equal keys: dQ_i = s * sum_j dS_ij * k = 0 because every dS row sums to zero
    q, k, v, do = _rand()
    k[:] = k[:, :, :1, :]
    for mask, W in (("causal", 0), ("causal_window", 6)):
        res = oracle.sdpa_fwd_bwd(q, k, v, do, 0.9, mask, W)
        assert np.max(np.abs(res["dQ"])) <= 1e-13
        # and lse_i = s<q_i, k> + log(number of allowed keys)
        n = np.array([min(i + 1, W) if mask == "causal_window" else i + 1 for i in range(q.shape[2])])
        g = np.repeat(np.arange(k.shape[1]), q.shape[1] // k.shape[1])
        ref = 0.9 * np.einsum("hid,hd->hi", q[0], k[0, g, 0, :]) + np.log(n)[None]
        assert np.max(np.abs(res["lse"][0] - ref)) <= 1e-13


@pytest.mark.parametrize("W", [37, 38, 2**31 - 1])
def test_window_at_least_L_is_causal_bitwise(W):
    q, k, v, do = _rand()
    a = oracle.sdpa_fwd_bwd(q, k, v, do, 0.8, "causal", 0)
    b = oracle.sdpa_fwd_bwd(q, k, v, do, 0.8, "causal_window", W)
    for n in a:
        assert np.array_equal(a[n], b[n]), n


def test_gqa_equals_mha_with_repeated_kv():
    q, k, v, do = _rand(Hq=6, Hkv=2)
    group = 3
    a = oracle.sdpa_fwd_bwd(q, k, v, do, 0.6, "causal_window", 7)
    kk = np.repeat(k, group, axis=1)
    vv = np.repeat(v, group, axis=1)
    b = oracle.sdpa_fwd_bwd(q, kk, vv, do, 0.6, "causal_window", 7)
    for n in ("O", "lse", "dQ"):
        assert np.max(np.abs(a[n] - b[n])) <= 1e-13
    for n in ("dK", "dV"):
        summed = b[n].reshape(1, 2, group, *b[n].shape[2:]).sum(axis=2)
        assert np.max(np.abs(a[n] - summed)) <= 1e-13
    # group 1 is plain multi-head attention
    c = oracle.sdpa_fwd_bwd(q[:, :2], k, v, do[:, :2], 0.6, "causal", 0)
    d = oracle.sdpa_fwd_bwd(q[:, :1], k[:, :1], v[:, :1], do[:, :1], 0.6, "causal", 0)
    for n in c:
        assert np.allclose(c[n][:, :1], d[n], atol=1e-13, rtol=0), n


def test_masked_keys_contribute_exactly_zero():
    q, k, v, do = _rand()
    L, W = q.shape[2], 5
    i = 20
    base = oracle.sdpa_fwd_bwd(q, k, v, do, 0.7, "causal_window", W)
    for j in (0, i - W, i + 1, L - 1):   # behind the window, and above the diagonal
        k2, v2 = k.copy(), v.copy()
        k2[:, :, j] += 3.0
        v2[:, :, j] -= 2.0
        pert = oracle.sdpa_fwd_bwd(q, k2, v2, do, 0.7, "causal_window", W)
        for n in ("O", "lse", "dQ"):
            assert np.array_equal(base[n][:, :, i], pert[n][:, :, i]), (n, j)


def test_window_one_identity():
    q, k, v, do = _rand()
    s = 1.3
    res = oracle.sdpa_fwd_bwd(q, k, v, do, s, "causal_window", 1)
    g = np.repeat(np.arange(2), 2)
    assert np.array_equal(res["O"][0], v[0, g])
    assert np.allclose(res["lse"][0], s * np.sum(q[0] * k[0, g], axis=-1), atol=1e-14, rtol=0)
    # zero up to fp64 rounding: dS_ii = P_ii * (dP_ii - Delta_i) with dP_ii and
    # Delta_i = <dO_i, v_i> summed in different orders
    assert np.max(np.abs(res["dQ"])) <= 1e-13
    assert np.max(np.abs(res["dK"])) <= 1e-13
    assert np.allclose(res["dV"][0], do[0].reshape(2, 2, *do.shape[2:]).sum(axis=1), atol=1e-14, rtol=0)


def test_gradient_sums():
    q, k, v, do = _rand()
    for mask, W in (("causal", 0), ("causal_window", 4)):
        res = oracle.sdpa_fwd_bwd(q, k, v, do, 0.7, mask, W)
        assert np.max(np.abs(res["dK"].sum(axis=2))) <= 1e-12
        ref = do[0].reshape(2, 2, *do.shape[2:]).sum(axis=(1, 2))
        assert np.max(np.abs(res["dV"][0].sum(axis=1) - ref)) <= 1e-12


def test_key_shift_and_scale_equivalence():
    q, k, v, do = _rand()
    s = 0.7
    base = oracle.sdpa_fwd_bwd(q, k, v, do, s, "causal_window", 6)
    c = np.linspace(-1, 1, k.shape[-1])
    sh = oracle.sdpa_fwd_bwd(q, k + c, v, do, s, "causal_window", 6)
    assert np.max(np.abs(sh["O"] - base["O"])) <= 1e-13
    assert np.max(np.abs(sh["lse"] - base["lse"] - s * (q @ c))) <= 1e-12
    a = 2.5
    sc = oracle.sdpa_fwd_bwd(a * q, k, v, do, s / a, "causal_window", 6)
    assert np.max(np.abs(sc["O"] - base["O"])) <= 1e-13
    assert np.max(np.abs(sc["lse"] - base["lse"])) <= 1e-13
    assert np.max(np.abs(sc["dQ"] * a - base["dQ"])) <= 1e-13


def test_row_blocking_changes_nothing():
    q, k, v, do = _rand(L=50)
    a = oracle.sdpa_fwd_bwd(q, k, v, do, 0.7, "causal_window", 9, row_block=7)
    b = oracle.sdpa_fwd_bwd(q, k, v, do, 0.7, "causal_window", 9, row_block=1024)
    for n in a:
        assert np.max(np.abs(a[n] - b[n])) <= 1e-13


def test_sampled_rows_and_keys_match_full():
    q, k, v, do = _rand(Hq=4, Hkv=2, L=60)
    for mask, W in (("causal", 0), ("causal_window", 11)):
        full = oracle.sdpa_fwd_bwd(q, k, v, do, 0.7, mask, W)
        rows = np.array([0, 13, 59])
        r = oracle.sampled_rows(q, k, v, do, 0.7, mask, W, 0, 3, rows)
        for n in ("O", "lse", "dQ"):
            assert np.max(np.abs(r[n] - full[n][0, 3, rows])) <= 1e-13
        keys = np.array([0, 30, 59])
        kk = oracle.sampled_keys(q, k, v, do, 0.7, mask, W, 0, 1, keys, row_block=17)
        for n in ("dK", "dV"):
            assert np.max(np.abs(kk[n] - full[n][0, 1, keys])) <= 1e-12


# ---------------------------------------------------------------- mutation tests
MUTATIONS = [
    ("dS = P * (dP - delta[:, None])", "dS = P * (dP + delta[:, None])"),          # wrong sign
    ("dS = P * (dP - delta[:, None])", "dS = P * dP"),                              # dropped term
    ('out["dK"] = scale * (dS.T @ qb)', 'out["dK"] = scale * (dS.T @ dob)'),       # wrong operand
    ('out["dK"] = scale * (dS.T @ qb)', 'out["dK"] = (dS.T @ qb)'),                 # dropped scale
    ('out["dQ"] = scale * (dS @ k_g)', 'out["dQ"] = scale * (dS @ v_g)'),           # wrong operand
    ('out["dV"] = P.T @ dob', 'out["dV"] = dS.T @ dob'),                             # P vs dS
    ("dP = dob @ v_g.T", "dP = dob @ k_g.T"),                                        # wrong operand
    ("ok &= j >= i + diag_off - window + 1", "ok &= j > i + diag_off - window + 1"),  # window off by one
    ("ok = j <= i + diag_off", "ok = j < i + diag_off"),                             # diagonal excluded
    ("g = h // group\n            for r0 in range(0, Lq, row_block):\n                rows = np.arange(r0, min(Lq, r0 + row_block))\n                res = head_rows(q[b, h], k[b, g], v[b, g], do[b, h]",
     "g = h % Hkv\n            for r0 in range(0, Lq, row_block):\n                rows = np.arange(r0, min(Lq, r0 + row_block))\n                res = head_rows(q[b, h], k[b, g], v[b, g], do[b, h]"),  # GQA map
    ("lse = m_safe + np.log(tot)", "lse = m_safe + np.log(tot + 1e-3)"),          # wrong normaliser
    ("S = scale * (qb @ k_g.T)", "S = scale * (qb @ k_g.T) + 1e-4"),                # biased scores (lse)
]


def _mutant(old, new):
    src = open(sdpa_oracle.__file__).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new, 1), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _pins_catch(mod):
    failures = []
    try:
        if pins.pin_golden(mod) > 1e-14:
            failures.append("golden")
    except Exception:
        failures.append("golden-raised")
    try:
        if pins.pin_brute(mod) > 1e-12:
            failures.append("brute")
    except Exception:
        failures.append("brute-raised")
    for case in [(4, 2, 9, 4, 0.8, "causal_window", 3), (2, 1, 7, 4, 0.5, "causal", 0)]:
        try:
            if pins.fd_error(mod, *case) > 1e-7:
                failures.append(f"fd{case}")
        except Exception:
            failures.append("fd-raised")
    return failures


@pytest.mark.parametrize("old,new", MUTATIONS, ids=[f"m{i}" for i in range(len(MUTATIONS))])
def test_pins_catch_planted_mistake(old, new):
    assert _pins_catch(_mutant(old, new)), f"no pin caught mutation {new!r}"


def test_unmutated_oracle_passes_the_same_pins():
    assert _pins_catch(sdpa_oracle) == []
