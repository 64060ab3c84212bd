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
from workloads import BY_NAME, make_inputs

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
    (2, 1, 7, 4, 0.5, "none", 0),
    (2, 2, 13, 4, 1.0, "window", 1),
    (4, 2, 13, 4, 0.8, "window", 3),
    (2, 1, 16, 8, 3.0, "window", 16),
]
# queries the last Lq of Lk positions, and more queries than keys
FD_CASES_QK = [
    # Hq, Hkv, Lq, Lk, D, scale, mask, window
    (2, 1, 5, 13, 4, 0.7, "causal", 0),
    (2, 2, 7, 16, 4, 1.0, "causal_window", 3),
    (2, 1, 4, 13, 4, 0.9, "window", 3),
    (2, 1, 6, 9, 4, 0.6, "none", 0),
    (2, 1, 13, 7, 4, 0.8, "causal", 0),
    (2, 1, 13, 7, 4, 1.1, "window", 2),
]


@pytest.mark.parametrize("case", FD_CASES, ids=[str(c) for c in FD_CASES])
def test_finite_differences_exhaustive(case):
    Hq, Hkv, L, D, s, mask, W = case
    assert pins.fd_error(sdpa_oracle, Hq, Hkv, L, D, s, mask, W) <= 1e-7


@pytest.mark.parametrize("case", FD_CASES_QK, ids=[str(c) for c in FD_CASES_QK])
def test_finite_differences_exhaustive_lq_ne_lk(case):
    Hq, Hkv, Lq, Lk, D, s, mask, W = case
    assert pins.fd_error(sdpa_oracle, Hq, Hkv, Lq, D, s, mask, W, Lk=Lk) <= 1e-7


@pytest.mark.parametrize("mask,window", [("causal", 0), ("causal_window", 40)])
def test_finite_differences_directional_tiny_config_shape(mask, window):
    # the tiny fp32 workload's geometry: Hq=2, Hkv=1, L=128, D=64, scale 1/8
    assert pins.fd_directional_error(sdpa_oracle, 2, 1, 128, 64, 0.125, mask, window) <= 1e-7


# ---------------------------------------------------------------- independent autograd
def _cfg_inputs(w, **shrink):
    w = w.with_(**shrink) if shrink else w
    t = make_inputs(w)
    return [t[n].to(torch.float64).numpy() for n in ("q", "k", "v", "do")], w


@pytest.mark.parametrize("name,shrink", [
    ("tiny_fp32_causal_L128_D64_gqa2", {}),
    ("bf16_causal_gqa_L2048_D256_h8kv4", {}),
    ("bf16_causal_global_L8192_D512_h16kv4", {"Hq": 4, "Hkv": 1, "L": 1024}),      # global layer geometry (D=512, group 4), shortened
    ("bf16_window1024_L16384_D256_h32kv16", {"Hq": 4, "Hkv": 2, "L": 1500, "window": 300}),  # sliding geometry, several windows
    ("bf16_window1024_ragged_L30553_D256_h32kv16", {"Hq": 2, "Hkv": 1, "L": 777, "window": 129}),   # ragged length, window not a power of 2
])
def test_autograd_independent(name, shrink):
    (q, k, v, do), w = _cfg_inputs(BY_NAME[name], **shrink)
    err = pins.autograd_error(sdpa_oracle, q, k, v, do, w.scale, w.mask, w.window)
    assert err <= 1e-12, err


@pytest.mark.parametrize("Lq,Lk,mask,window", [
    (300, 300, "none", 0),
    (300, 300, "window", 64),
    (200, 700, "causal", 0),
    (200, 700, "causal_window", 96),
    (200, 700, "window", 96),
    (150, 400, "none", 0),
    (700, 200, "none", 0),
    (500, 260, "window", 300),
])
def test_autograd_independent_more_masks(Lq, Lk, mask, window):
    q, k, v, do = pins.tiny_inputs(4, 2, Lq, 32, 77, Lk)
    err = pins.autograd_error(sdpa_oracle, q, k, v, do, 32 ** -0.5, mask, window)
    assert err <= 1e-12, err


def test_library_sdpa_forward():
    import torch.nn.functional as F
    for name, shrink in (("tiny_fp32_causal_L128_D64_gqa2", {}), ("bf16_causal_gqa_L2048_D256_h8kv4", {"L": 1024}),
                         ("bf16_window1024_L16384_D256_h32kv16", {"Hq": 4, "Hkv": 2, "L": 700, "window": 100})):
        (q, k, v, do), w = _cfg_inputs(BY_NAME[name], **shrink)
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


def test_library_sdpa_no_mask_and_lower_right_causal():
    # no mask: the library routine with no attention mask at all; queries as a
    # suffix of the keys: the library's lower-right causal bias
    import warnings

    import torch.nn.functional as F
    from torch.nn.attention.bias import causal_lower_right
    for Lq, Lk in ((100, 100), (60, 250), (250, 60)):
        q, k, v, _ = pins.tiny_inputs(4, 2, Lq, 16, 78, Lk)
        tq, tk, tv = torch.tensor(q), torch.tensor(k), torch.tensor(v)
        O, _ = oracle.sdpa_forward(q, k, v, 0.3, "none", 0)
        ref = F.scaled_dot_product_attention(tq, tk, tv, scale=0.3, enable_gqa=True)
        assert pins.rel_fro(O, ref.numpy()) <= 1e-12
        if Lq <= Lk:
            with warnings.catch_warnings():
                warnings.simplefilter("ignore")
                bias = causal_lower_right(Lq, Lk)._materialize("cpu")
            O, _ = oracle.sdpa_forward(q, k, v, 0.3, "causal", 0)
            rep = lambda x: x.repeat_interleave(2, dim=1)
            ref = F.scaled_dot_product_attention(tq, rep(tk), rep(tv), attn_mask=bias, scale=0.3)
            assert pins.rel_fro(O, ref.numpy()) <= 1e-12


# ---------------------------------------------------------------- sinks
SINK_FD = [
    # Hq, Hkv, Lq, Lk, D, scale, mask, window, sinks
    (2, 1, 7, 7, 4, 0.7, "causal", 0, (0.4, -1.2)),
    (2, 2, 9, 9, 4, 1.0, "causal_window", 3, (2.5, 0.0)),
    (2, 1, 5, 11, 4, 0.9, "window", 2, (-0.5, 1.0)),
    (2, 1, 9, 4, 4, 0.8, "causal", 0, (1.0, 0.2)),       # rows with no key
    (2, 1, 6, 6, 4, 0.6, "none", 0, (3.0, -3.0)),
]


@pytest.mark.parametrize("case", SINK_FD, ids=[str(c) for c in SINK_FD])
def test_sinks_finite_differences(case):
    Hq, Hkv, Lq, Lk, D, s, mask, W, sinks = case
    assert pins.fd_error(sdpa_oracle, Hq, Hkv, Lq, D, s, mask, W, Lk=Lk, sinks=sinks) <= 1e-7


@pytest.mark.parametrize("mask,window,Lq,Lk", [("causal_window", 64, 300, 300), ("none", 0, 200, 350),
                                               ("causal", 0, 400, 150)])
def test_sinks_autograd_independent(mask, window, Lq, Lk):
    q, k, v, do = pins.tiny_inputs(4, 2, Lq, 32, 79, Lk)
    sinks = np.array([0.5, -2.0, 3.0, 1.25])
    err = pins.autograd_error(sdpa_oracle, q, k, v, do, 32 ** -0.5, mask, window, sinks)
    assert err <= 1e-12, err


def test_sink_at_minus_infinity_is_no_sink_bitwise():
    q, k, v, do = pins.tiny_inputs(4, 2, 30, 8, 80, 41)
    a = oracle.sdpa_fwd_bwd(q, k, v, do, 0.7, "window", 5)
    b = oracle.sdpa_fwd_bwd(q, k, v, do, 0.7, "window", 5, sinks=np.full(4, -np.inf))
    for n in a:
        assert np.array_equal(a[n], b[n]), n
    assert np.all(b["dSinks"] == 0)


def test_sink_takes_mass_without_value():
    # with sinks, lse = log(exp(lse0) + exp(sink)) and O = O0 * exp(lse0 - lse)
    q, k, v, do = pins.tiny_inputs(2, 1, 25, 8, 81, 25)
    sinks = np.array([1.0, -0.5])
    a = oracle.sdpa_fwd_bwd(q, k, v, do, 0.9, "causal", 0)
    b = oracle.sdpa_fwd_bwd(q, k, v, do, 0.9, "causal", 0, sinks=sinks)
    lse = np.logaddexp(a["lse"], sinks[None, :, None])
    assert np.max(np.abs(b["lse"] - lse)) <= 1e-13
    assert np.max(np.abs(b["O"] - a["O"] * np.exp(a["lse"] - lse)[..., None])) <= 1e-13


# ---------------------------------------------------------------- prefix-sharing cut
@pytest.mark.parametrize("case", [(2, 1, 10, 4, 0.8, "causal", 0, (7, 3, 7)),
                                  (2, 2, 12, 4, 1.0, "causal_window", 4, (8, 4, 8)),
                                  (2, 1, 9, 4, 0.6, "none", 0, (5, 1, 4))], ids=["causal", "cwin", "none"])
def test_cut_finite_differences(case):
    Hq, Hkv, L, D, s, mask, W, cut = case
    assert pins.fd_error(sdpa_oracle, Hq, Hkv, L, D, s, mask, W, cut=cut) <= 1e-7


def test_cut_autograd_independent():
    q, k, v, do = pins.tiny_inputs(4, 2, 300, 32, 82)
    err = pins.autograd_error(sdpa_oracle, q, k, v, do, 32 ** -0.5, "causal", 0, cut=(220, 100, 220))
    assert err <= 1e-12, err


@pytest.mark.parametrize("P,Rc,Rr", [(40, 25, 30), (1, 7, 9), (50, 1, 1)])
def test_prefix_sharing_equals_two_branches(P, Rc, Rr):
    # One pass over [prompt; chosen; rejected] with the rejected rows cut off
    # from the chosen keys equals two causal passes, [prompt; chosen] and
    # [prompt; rejected], row for row; the prompt's keys collect the gradient
    # of both branches (dO of the prompt rows counted once, in the first).
    L = P + Rc + Rr
    q, k, v, do = pins.tiny_inputs(4, 2, L, 8, 83)
    cut = (P + Rc, P, P + Rc)
    sh = oracle.sdpa_fwd_bwd(q, k, v, do, 0.7, "causal", 0, cut=cut)
    a_idx = np.arange(P + Rc)
    b_idx = np.concatenate([np.arange(P), np.arange(P + Rc, L)])
    br_a = oracle.sdpa_fwd_bwd(q[:, :, a_idx], k[:, :, a_idx], v[:, :, a_idx], do[:, :, a_idx], 0.7, "causal", 0)
    do_b = do[:, :, b_idx].copy()
    do_b[:, :, :P] = 0.0
    br_b = oracle.sdpa_fwd_bwd(q[:, :, b_idx], k[:, :, b_idx], v[:, :, b_idx], do_b, 0.7, "causal", 0)
    for n in ("O", "lse", "dQ"):
        assert np.max(np.abs(sh[n][:, :, :P + Rc] - br_a[n])) <= 1e-13, n
        assert np.max(np.abs(sh[n][:, :, P + Rc:] - br_b[n][:, :, P:])) <= 1e-13, n
    for n in ("dK", "dV"):
        assert np.max(np.abs(sh[n][:, :, :P] - br_a[n][:, :, :P] - br_b[n][:, :, :P])) <= 1e-13, n
        assert np.max(np.abs(sh[n][:, :, P:P + Rc] - br_a[n][:, :, P:])) <= 1e-13, n
        assert np.max(np.abs(sh[n][:, :, P + Rc:] - br_b[n][:, :, P:])) <= 1e-13, n


@pytest.mark.parametrize("mask,W,P,Rc,Rr", [("causal_window", 6, 20, 9, 14), ("causal_window", 1, 5, 3, 4),
                                             ("causal_window", 40, 12, 7, 9), ("causal", 0, 10, 6, 8)])
def test_logical_window_prefix_sharing_equals_two_branches(mask, W, P, Rc, Rr):
    # With the window at logical positions, one pass over [prompt; chosen;
    # rejected] equals the two windowed passes over [prompt; chosen] and
    # [prompt; rejected] row for row (prompt keys collect both branches'
    # gradient), for any window: this is what the position reset is for.
    L = P + Rc + Rr
    q, k, v, do = pins.tiny_inputs(4, 2, L, 8, 84)
    sh = oracle.sdpa_fwd_bwd(q, k, v, do, 0.7, mask, W, cut=(P + Rc, P, P + Rc, True))
    a_idx = np.arange(P + Rc)
    b_idx = np.concatenate([np.arange(P), np.arange(P + Rc, L)])
    br_a = oracle.sdpa_fwd_bwd(q[:, :, a_idx], k[:, :, a_idx], v[:, :, a_idx], do[:, :, a_idx], 0.7, mask, W)
    do_b = do[:, :, b_idx].copy()
    do_b[:, :, :P] = 0.0
    br_b = oracle.sdpa_fwd_bwd(q[:, :, b_idx], k[:, :, b_idx], v[:, :, b_idx], do_b, 0.7, mask, W)
    for n in ("O", "lse", "dQ"):
        assert np.max(np.abs(sh[n][:, :, :P + Rc] - br_a[n])) <= 1e-13, n
        assert np.max(np.abs(sh[n][:, :, P + Rc:] - br_b[n][:, :, P:])) <= 1e-13, n
    for n in ("dK", "dV"):
        assert np.max(np.abs(sh[n][:, :, :P] - br_a[n][:, :, :P] - br_b[n][:, :, :P])) <= 1e-13, n
        assert np.max(np.abs(sh[n][:, :, P:P + Rc] - br_a[n][:, :, P:])) <= 1e-13, n
        assert np.max(np.abs(sh[n][:, :, P + Rc:] - br_b[n][:, :, P:])) <= 1e-13, n


def test_physical_window_cut_differs_from_the_branches():
    # the plain cut keeps the window at physical positions: a rejected row
    # near the start of its block then reaches fewer prompt keys than in its
    # own branch (the chosen block sits in between), so the two readings differ
    P, Rc, Rr, W = 20, 9, 14, 12
    L = P + Rc + Rr
    q, k, v, _ = pins.tiny_inputs(2, 1, L, 8, 85)
    phys = oracle.sdpa_forward(q, k, v, 0.7, "causal_window", W, cut=(P + Rc, P, P + Rc))[1]
    logi = oracle.sdpa_forward(q, k, v, 0.7, "causal_window", W, cut=(P + Rc, P, P + Rc, True))[1]
    assert np.max(np.abs(phys[:, :, :P + Rc] - logi[:, :, :P + Rc])) == 0.0
    assert np.max(np.abs(phys[:, :, P + Rc:] - logi[:, :, P + Rc:])) > 1e-3


@pytest.mark.parametrize("mask,W", [("causal", 0), ("none", 0)])
def test_logical_cut_without_window_is_the_plain_cut(mask, W):
    # without a window the position of a prompt key does not matter to a row
    # after it (causal) or to any row (no mask): both readings agree exactly
    q, k, v, do = pins.tiny_inputs(2, 1, 30, 8, 86)
    a = oracle.sdpa_fwd_bwd(q, k, v, do, 0.8, mask, W, cut=(18, 7, 18))
    b = oracle.sdpa_fwd_bwd(q, k, v, do, 0.8, mask, W, cut=(18, 7, 18, True))
    for n in ("O", "lse", "dQ", "dK", "dV"):
        assert np.array_equal(a[n], b[n]), n


def test_logical_cut_finite_differences():
    assert pins.fd_error(sdpa_oracle, 2, 1, 13, 4, 0.9, "causal_window", 3, cut=(8, 3, 8, True)) <= 1e-7
    assert pins.fd_error(sdpa_oracle, 2, 2, 12, 4, 0.8, "window", 3, cut=(7, 2, 6, True)) <= 1e-7


def test_logical_cut_autograd_independent():
    q, k, v, do = pins.tiny_inputs(4, 2, 260, 32, 87)
    err = pins.autograd_error(sdpa_oracle, q, k, v, do, 32 ** -0.5, "causal_window", 40,
                              cut=(180, 90, 180, True))
    assert err <= 1e-12, err


# ---------------------------------------------------------------- invariants
def _rand(Hq=4, Hkv=2, L=37, D=8, seed=5, Lk=None):
    return pins.tiny_inputs(Hq, Hkv, L, D, seed, Lk)


@pytest.mark.parametrize("mask,window", [("causal", 0), ("causal_window", 7), ("window", 5), ("none", 0)])
def test_queries_as_suffix_of_keys(mask, window):
    # Lq < Lk: query row i is row i + Lk - Lq of the square problem over all Lk
    # positions; its outputs are that row's, and dK/dV are the square problem's
    # with dO zero on the rows that are not queries.
    Lq, Lk = 11, 30
    q, k, v, do = _rand(L=Lk, seed=21)
    do_sq = do.copy()
    do_sq[:, :, : Lk - Lq] = 0.0
    sq = oracle.sdpa_fwd_bwd(q, k, v, do_sq, 0.7, mask, window)
    sub = oracle.sdpa_fwd_bwd(q[:, :, Lk - Lq:], k, v, do[:, :, Lk - Lq:], 0.7, mask, window)
    for n in ("O", "lse", "dQ"):
        assert np.max(np.abs(sub[n] - sq[n][:, :, Lk - Lq:])) <= 1e-13, n
    for n in ("dK", "dV"):
        assert np.max(np.abs(sub[n] - sq[n])) <= 1e-13, n


def test_more_queries_than_keys_leaves_rows_empty():
    # Lq > Lk under a causal mask: the first Lq - Lk rows have no key at or
    # before their position; they get O = 0, lse = -inf and contribute nothing
    Lq, Lk = 20, 8
    q, k, v, do = _rand(L=Lq, Lk=Lk, seed=22)
    res = oracle.sdpa_fwd_bwd(q, k, v, do, 0.7, "causal", 0)
    e = Lq - Lk
    assert np.all(res["lse"][:, :, :e] == -np.inf) and np.all(np.isfinite(res["lse"][:, :, e:]))
    assert np.all(res["O"][:, :, :e] == 0) and np.all(res["dQ"][:, :, :e] == 0)
    tail = oracle.sdpa_fwd_bwd(q[:, :, e:], k, v, do[:, :, e:], 0.7, "causal", 0)
    for n in ("dK", "dV"):
        assert np.array_equal(res[n], tail[n]), n


def test_two_sided_window_is_time_reversal_symmetric():
    # reversing the order of the positions maps the band |i - j| < W onto itself
    q, k, v, do = _rand(L=29, seed=23)
    f = lambda x: x[:, :, ::-1].copy()
    a = oracle.sdpa_fwd_bwd(q, k, v, do, 0.8, "window", 6)
    b = oracle.sdpa_fwd_bwd(f(q), f(k), f(v), f(do), 0.8, "window", 6)
    for n in ("O", "lse", "dQ", "dK", "dV"):
        assert np.max(np.abs(f(b[n]) - a[n])) <= 1e-13, n   # axis 2 is the position axis of every tensor
    # the causal window is not symmetric: its reversal looks ahead instead
    c = oracle.sdpa_fwd_bwd(f(q), f(k), f(v), f(do), 0.8, "causal_window", 6)
    d = oracle.sdpa_fwd_bwd(q, k, v, do, 0.8, "causal_window", 6)
    assert np.max(np.abs(f(c["O"]) - d["O"])) > 1e-3


@pytest.mark.parametrize("Lq,Lk", [(37, 37), (20, 37), (37, 20)])
def test_wide_two_sided_window_is_no_mask_bitwise(Lq, Lk):
    q, k, v, do = _rand(L=Lq, Lk=Lk, seed=24)
    a = oracle.sdpa_fwd_bwd(q, k, v, do, 0.8, "none", 0)
    for W in (Lq + Lk, 2**31 - 1):
        b = oracle.sdpa_fwd_bwd(q, k, v, do, 0.8, "window", W)
        for n in a:
            assert np.array_equal(a[n], b[n]), (W, n)


def test_window_one_is_self_for_both_window_kinds():
    q, k, v, do = _rand(L=15, Lk=24, seed=25)
    a = oracle.sdpa_fwd_bwd(q, k, v, do, 1.2, "causal_window", 1)
    b = oracle.sdpa_fwd_bwd(q, k, v, do, 1.2, "window", 1)
    for n in a:
        assert np.array_equal(a[n], b[n]), n
    g = np.repeat(np.arange(2), 2)
    assert np.array_equal(a["O"][0], v[0, g, 24 - 15:])


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


@pytest.mark.parametrize("Lq,Lk", [(60, 60), (45, 80), (80, 45)])
def test_sampled_rows_and_keys_match_full(Lq, Lk):
    q, k, v, do = _rand(Hq=4, Hkv=2, L=Lq, Lk=Lk)
    for mask, W in (("causal", 0), ("causal_window", 11), ("window", 9), ("none", 0)):
        full = oracle.sdpa_fwd_bwd(q, k, v, do, 0.7, mask, W)
        rows = np.array([0, 13, Lq - 1])
        r = oracle.sampled_rows(q, k, v, do, 0.7, mask, W, 0, 3, rows)
        for n in ("O", "lse", "dQ"):
            assert np.array_equal(np.isfinite(r[n]), np.isfinite(full[n][0, 3, rows]))
            fin = np.isfinite(r[n])
            assert np.max(np.abs(r[n][fin] - full[n][0, 3, rows][fin])) <= 1e-13
        keys = np.array([0, 30, Lk - 1])
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
    ("ok = ok & (d >= 0) & (d < window)", "ok = ok & (d >= 0) & (d <= window)"),     # window off by one
    ("ok = ok & (d >= 0)\n", "ok = ok & (d > 0)\n"),                                # diagonal excluded
    ("ok = ok & (d > -window) & (d < window)", "ok = ok & (d >= -window) & (d < window)"),  # two-sided, one too many
    ("ok = ok & (d > -window) & (d < window)", "ok = ok & (d >= 0) & (d < window)"),  # two-sided read as causal
    ("d = i + (Lk - Lq) - j", "d = i + (Lq - Lk) - j"),                              # diagonal offset sign
    ("d = i + (Lk - Lq) - j", "d = i - j"),                                          # top-left alignment
    ("nonempty = tot > 0", "nonempty = tot >= 0"),                                   # empty rows -> NaN
    ("ok = ok & ~((i >= r0) & (j >= c0) & (j < c1))", "ok = ok & ~((i > r0) & (j >= c0) & (j < c1))"),  # cut rows off by one
    ("ok = ok & ~((i >= r0) & (j >= c0) & (j < c1))", "ok = ok & ~((i >= r0) & (j >= c0) & (j <= c1))"),  # cut keys too wide
    ("d = np.where((i >= r0) & (j < c0), d - (c1 - c0), d)",
     "d = np.where((i >= r0) & (j < c0), d - (c1 - c0) + 1, d)"),                   # logical shift off by one
    ("d = np.where((i >= r0) & (j < c0), d - (c1 - c0), d)",
     "d = np.where((i >= r0) & (j < c0), d + (c1 - c0), d)"),                       # logical shift sign
    ("d = np.where((i >= r0) & (j < c0), d - (c1 - c0), d)",
     "d = np.where((i >= r0) & (j >= c1), d - (c1 - c0), d)"),                      # shift on the wrong side
    ('out["dSink"] = float(np.sum(P_sink * (0.0 - delta)))', 'out["dSink"] = float(np.sum(P_sink * delta))'),  # sink sign
    ("np.full((len(rows), 1), float(sink))", "np.full((len(rows), 1), 2 * float(sink))"),  # sink logit scaled
    ("ok = np.concatenate([ok, np.ones((len(rows), 1), dtype=bool)], axis=1)",
     "ok = np.concatenate([ok, np.zeros((len(rows), 1), dtype=bool)], axis=1)"),      # sink dropped
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
        if not pins.pin_golden(mod) <= 1e-14:
            failures.append("golden")
    except Exception:
        failures.append("golden-raised")
    try:
        if not pins.pin_brute(mod) <= 1e-12:
            failures.append("brute")
    except Exception:
        failures.append("brute-raised")
    for case in [(4, 2, 9, 4, 0.8, "causal_window", 3), (2, 1, 7, 4, 0.5, "causal", 0),
                 (2, 1, 5, 3, 0.8, "window", 2, 0, 9)]:
        try:
            if not pins.fd_error(mod, *case) <= 1e-7:
                failures.append(f"fd{case}")
        except Exception:
            failures.append("fd-raised")
    try:
        if not pins.fd_error(mod, 2, 1, 6, 3, 0.8, "causal", 0, sinks=(0.5, -1.0)) <= 1e-7:
            failures.append("fd-sinks")
    except Exception:
        failures.append("fd-sinks-raised")
    return failures


@pytest.mark.parametrize("old,new", MUTATIONS, ids=[f"m{i}" for i in range(len(MUTATIONS))])
def test_pins_catch_planted_mistake(old, new):
    assert _pins_catch(_mutant(old, new)), f"no pin caught mutation {new!r}"


def test_unmutated_oracle_passes_the_same_pins():
    assert _pins_catch(sdpa_oracle) == []
