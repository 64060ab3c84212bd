"""GPU parity of the HIP path against the fp64 oracle (run on an MI355X).

Inputs come from workloads.make_inputs (seeded, CPU), are copied to the GPU,
run through the C ABI (sdpa_fwd_lse then sdpa_bwd), and compared with the
oracle on the same values upcast to fp64. Gates: per-tensor relative
Frobenius error <= 1e-2 (bf16) / 2e-3 (fp16) / 1e-5 (fp32) on O, dQ, dK, dV,
and lse max-abs error <= 1e-4. The fp16 gate keeps the bf16 gate's ratio to
the unit roundoff: 1e-2 is about 2.6 u for bf16 (u = 2^-8), and 2.6 u for
fp16 (u = 2^-11) is 1.3e-3, rounded up to 2e-3; P, dS and the outputs are
rounded to the input type, everything else stays fp32. At the three large
workloads the oracle computes one whole kv group (every row of its q-heads,
every key of its kv head) and samples of every other head, and the GPU run
uses the same launch configuration as the benchmark.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from sdpa_backward_amd import sdpa_bwd, sdpa_fwd_lse
from tests.oracle_pins import rel_fro
from workloads import BY_NAME, MASK_CAUSAL, MASK_WINDOW, Workload, make_inputs

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "f16": 2e-3, "f32": 1e-5}
LSE_TOL = 1e-4
DEV = "cuda:0"


def _np(t):
    return t.detach().to("cpu", torch.float64).numpy()


def run(w, inp, window=None, out=None, scale=None):
    window = w.window if window is None else window
    scale = w.scale if scale is None else scale
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    o, lse = sdpa_fwd_lse(q, k, v, w.mask, window, scale, *(out[:2] if out else (None, None)))
    dq, dk, dv = sdpa_bwd(q, k, v, o, do, lse, w.mask, window, scale, out=out[2:] if out else None)
    torch.cuda.synchronize()
    return {"O": o, "lse": lse, "dQ": dq, "dK": dk, "dV": dv}


def check_full(w, gpu, ref, tol=None):
    tol = TOL[w.dtype] if tol is None else tol
    tol = tol if isinstance(tol, dict) else {n: tol for n in ("O", "dQ", "dK", "dV")}
    errs = {n: rel_fro(_np(gpu[n]), ref[n]) for n in ("O", "dQ", "dK", "dV")}
    errs["lse"] = float(np.max(np.abs(_np(gpu["lse"]) - ref["lse"]))) if ref["lse"].size else 0.0
    print(w.name, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for n in ("O", "dQ", "dK", "dV"):
        assert errs[n] <= tol[n], (n, errs[n])
    assert errs["lse"] <= LSE_TOL, errs["lse"]
    return errs


def oracle_full(w, inp, window=None, scale=None):
    window = w.window if window is None else window
    scale = w.scale if scale is None else scale
    return oracle.sdpa_fwd_bwd(inp["q"], inp["k"], inp["v"], inp["do"], scale, w.mask, window)


# ------------------------------------------------------------------ small shapes, full comparison
SMALL = [
    # name, Hq, Hkv, L, D, dtype, mask, window
    ("L1", 2, 1, 1, 64, "bf16", MASK_CAUSAL, 0),
    ("L7", 2, 1, 7, 64, "bf16", MASK_CAUSAL, 0),
    ("ragged129_D128", 4, 2, 129, 128, "bf16", MASK_CAUSAL, 0),
    ("w63_D256", 4, 1, 300, 256, "bf16", MASK_WINDOW, 63),
    ("w64_D256_g4", 8, 2, 513, 256, "bf16", MASK_WINDOW, 64),
    ("w65_D256_mha", 2, 2, 255, 256, "bf16", MASK_WINDOW, 65),
    ("w3_D128", 2, 1, 777, 128, "bf16", MASK_WINDOW, 3),
    ("wL_D64", 4, 4, 1000, 64, "bf16", MASK_WINDOW, 1000),
    ("w1000_D256", 2, 1, 1500, 256, "bf16", MASK_WINDOW, 1000),
    ("causal_D512_g4", 4, 1, 600, 512, "bf16", MASK_CAUSAL, 0),
    ("w200_D512", 2, 1, 1100, 512, "bf16", MASK_WINDOW, 200),
    ("g8_D256", 8, 1, 400, 256, "bf16", MASK_CAUSAL, 0),
    ("f32_D64", 2, 1, 128, 64, "f32", MASK_CAUSAL, 0),
    ("f32_w17_D128", 4, 2, 100, 128, "f32", MASK_WINDOW, 17),
    ("f32_ragged_D64", 2, 2, 33, 64, "f32", MASK_WINDOW, 5),
    ("f32_causal_D256", 2, 1, 150, 256, "f32", MASK_CAUSAL, 0),
    ("f32_w40_D512_g2", 4, 2, 97, 512, "f32", MASK_WINDOW, 40),
    ("f16_causal_D64", 2, 1, 200, 64, "f16", MASK_CAUSAL, 0),
    ("f16_ragged_D128", 4, 2, 129, 128, "f16", MASK_CAUSAL, 0),
    ("f16_w63_D256", 4, 1, 300, 256, "f16", MASK_WINDOW, 63),
    ("f16_w1000_D256", 2, 1, 1500, 256, "f16", MASK_WINDOW, 1000),
    ("f16_causal_D512_g4", 4, 1, 600, 512, "f16", MASK_CAUSAL, 0),
    ("f16_w200_D512", 2, 1, 1100, 512, "f16", MASK_WINDOW, 200),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_shapes_full(case):
    name, Hq, Hkv, L, D, dtype, mask, window = case
    w = Workload(name, 1, Hq, Hkv, L, D, dtype, mask, window, seed=7000 + L)
    inp = make_inputs(w)
    check_full(w, run(w, inp), oracle_full(w, inp))


def test_scale_one_and_three():
    # scale is an arbitrary positive float applied before masking/softmax
    w = Workload("scale", 1, 4, 2, 333, 256, "bf16", MASK_WINDOW, 100, seed=7100)
    inp = make_inputs(w)
    for s in (1.0, 0.3):
        check_full(w, run(w, inp, scale=s), oracle_full(w, inp, scale=s))


# ------------------------------------------------------------------ the five workloads
SMALL = ["tiny_fp32_causal_L128_D64_gqa2", "bf16_causal_gqa_L2048_D256_h8kv4"]
LARGE = ["bf16_causal_global_L8192_D512_h16kv4", "bf16_window1024_L16384_D256_h32kv16", "bf16_window1024_ragged_L30553_D256_h32kv16"]


@pytest.mark.parametrize("name", SMALL)
def test_small_workloads_full(name):
    w = BY_NAME[name]
    inp = make_inputs(w)
    check_full(w, run(w, inp), oracle_full(w, inp))


def test_second_seed_draw():
    for name in SMALL:
        w = BY_NAME[name]
        inp = make_inputs(w, seed=w.seed + 1000)
        check_full(w, run(w, inp), oracle_full(w, inp))


RISING = [
    # name, Hq, Hkv, L, D, mask, window
    ("rising_causal_D256", 2, 1, 1024, 256, MASK_CAUSAL, 0),
    ("rising_w300_D128", 2, 2, 1000, 128, MASK_WINDOW, 300),
    ("rising_causal_D512", 2, 1, 700, 512, MASK_CAUSAL, 0),
    ("rising_w100_D64", 2, 1, 900, 64, MASK_WINDOW, 100),
]


def _rounded_path_grads(w, inp, ref):
    """dQ and dK from the oracle's arithmetic with only the roundings that any
    attention on 16-bit matrix-core operands makes before those products: the
    forward's O formed from P rounded to the input type and itself rounded to
    it, Delta_i = <dO_i, O_i> from that O, and dS rounded to the input type as
    an operand. Everything else stays fp64. Used to size the gate of a case
    that amplifies these roundings, never as a reference."""
    rnd = lambda x: torch.from_numpy(x).float().to(w.torch_dtype).double().numpy()
    q, k, v, do = (_np(inp[n]) for n in ("q", "k", "v", "do"))
    dq, dk = np.zeros_like(q), np.zeros_like(k)
    rows = np.arange(w.L)
    ok = oracle.allowed_block(rows, w.L, w.Lkv, w.mask, w.window)
    for h in range(w.Hq):
        g = h // w.group
        S = w.scale * (q[0, h] @ k[0, g].T)
        P = np.where(ok, np.exp(np.where(ok, S, 0.0) - ref["lse"][0, h][:, None]), 0.0)
        delta = np.sum(do[0, h] * rnd(rnd(P) @ v[0, g]), axis=1)
        dS = rnd(P * (do[0, h] @ v[0, g].T - delta[:, None]))
        dq[0, h] = w.scale * (dS @ k[0, g])
        dk[0, g] += w.scale * (dS.T @ q[0, h])
    return dq, dk


@pytest.mark.parametrize("case", RISING, ids=[c[0] for c in RISING])
def test_rising_scores_force_rescales(case):
    """Scores that grow along the key axis by about 8 (natural log units) per
    64 keys: the running row max of the forward pass rises past its headroom on
    almost every key tile, so the accumulator rescale runs again and again.
    Every query shares a direction u; key j carries (j / L) * alpha * u.

    O, lse and dV (what the rescale touches) keep the usual gates. With u in
    every key, dQ_i = scale sum_j dS_ij k_j (and dK) cancel heavily, so the
    bf16 rounding of dS and of O (through Delta) is amplified: their gate is
    the error that those roundings alone leave in an otherwise exact
    computation (measured here on the same inputs), plus the usual 1e-2."""
    name, Hq, Hkv, L, D, mask, window = case
    w = Workload(name, 1, Hq, Hkv, L, D, "bf16", mask, window, seed=7300 + D)
    g = torch.Generator().manual_seed(w.seed)
    u = torch.randn(D, generator=g)
    u = u / u.norm() * math.sqrt(D)
    alpha = 8.0 * (L / 64) / math.sqrt(D)   # score rise over the whole sequence: about 8 L / 64
    ramp = (torch.arange(L, dtype=torch.float32) / L)[:, None] * alpha
    inp = {
        "q": (torch.randn(1, Hq, L, D, generator=g) * 0.5 + u).to(torch.bfloat16),
        "k": (torch.randn(1, Hkv, L, D, generator=g) * 0.5 + ramp * u).to(torch.bfloat16),
        "v": torch.randn(1, Hkv, L, D, generator=g).to(torch.bfloat16),
        "do": torch.randn(1, Hq, L, D, generator=g).to(torch.bfloat16),
    }
    ref = oracle_full(w, inp)
    dq_r, dk_r = _rounded_path_grads(w, inp, ref)
    floor = {"dQ": rel_fro(dq_r, ref["dQ"]), "dK": rel_fro(dk_r, ref["dK"])}
    print(name, "error of the rounded-operand arithmetic:", {k: f"{x:.2e}" for k, x in floor.items()}, flush=True)
    tol = {"O": 1e-2, "dV": 1e-2, "dQ": floor["dQ"] + 1e-2, "dK": floor["dK"] + 1e-2}
    check_full(w, run(w, inp), ref, tol=tol)


def _sample_rows(L, rng, n):
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 1023, 1024, L // 2, L - 2, L - 1]
    rows = set(r for r in fixed if 0 <= r < L)
    rows.update(int(x) for x in rng.integers(0, L, n))
    return np.array(sorted(rows))


def _sample_key_pair(w, rng):
    """Two adjacent keys (the rows that see them, at most window + 1 or the causal
    tail, stay cheap for the oracle)."""
    L = w.L
    j = int(rng.integers(L - 1024, L - 1)) if w.mask == MASK_CAUSAL else int(rng.integers(0, L - 1))
    return np.array([j, j + 1])


def _poisoned_outputs(w):
    """Output buffers prefilled with NaN, each followed by a canary tail."""
    shapes = {"O": (w.B, w.Hq, w.L, w.D), "lse": (w.B, w.Hq, w.L), "dQ": (w.B, w.Hq, w.L, w.D),
              "dK": (w.B, w.Hkv, w.Lkv, w.D), "dV": (w.B, w.Hkv, w.Lkv, w.D)}
    bufs, views = {}, {}
    for n, shp in shapes.items():
        dt = torch.float32 if n == "lse" else w.torch_dtype
        numel = math.prod(shp)
        buf = torch.full((numel + 4096,), float("nan"), dtype=dt, device=DEV)
        buf[numel:] = 12345.0
        bufs[n] = buf
        views[n] = buf[:numel].view(shp)
    return bufs, views


def _check_poison(w, bufs, views):
    for n, v in views.items():
        assert not torch.isnan(v).any().item(), f"{n} has unwritten (NaN) elements"
        assert torch.all(bufs[n][v.numel():] == 12345.0).item(), f"{n} canary tail overwritten"


@pytest.mark.parametrize("name", LARGE)
def test_large_workloads(name):
    """The three large workloads in the benchmark's launch configuration.

    * One whole kv group (the last) against the oracle: every row of its
      q-heads for O, lse and dQ, every key of its kv head for dK and dV, each
      gated as a per-tensor relative Frobenius error over that group.
    * Every other head too, on samples: rows of every q-head (O, lse, dQ) and
      two adjacent keys of every kv head (dK, dV, from every row and q-head
      that sees them), pooled into one relative error per tensor.
    * Whole-tensor properties: NaN-poisoned outputs are all written, canary
      tails untouched, and the column sums of dV and dK match their closed
      forms (sum_j dV_j = sum of the group's dO rows, sum_j dK_j = 0).
    """
    w = BY_NAME[name]
    inp = make_inputs(w)
    bufs, views = _poisoned_outputs(w)
    gpu = run(w, inp, out=[views[n] for n in ("O", "lse", "dQ", "dK", "dV")])
    _check_poison(w, bufs, views)
    tol = TOL[w.dtype]

    g = w.Hkv - 1
    hs = slice(g * w.group, (g + 1) * w.group)
    ref = oracle.sdpa_fwd_bwd(inp["q"][:, hs], inp["k"][:, g:g + 1], inp["v"][:, g:g + 1], inp["do"][:, hs],
                              w.scale, w.mask, w.window)
    errs = {n: rel_fro(_np(gpu[n][:, hs]), ref[n]) for n in ("O", "dQ")}
    errs.update({n: rel_fro(_np(gpu[n][:, g:g + 1]), ref[n]) for n in ("dK", "dV")})
    errs["lse"] = float(np.max(np.abs(_np(gpu["lse"][:, hs]) - ref["lse"])))
    print(w.name, f"kv group {g} (q-heads {hs.start}..{hs.stop - 1}), whole:",
          {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for n in ("O", "dQ", "dK", "dV"):
        assert errs[n] <= tol, ("group", n, errs[n])
    assert errs["lse"] <= LSE_TOL, ("group", errs["lse"])

    rng = np.random.default_rng(w.seed)
    got = {n: [] for n in ("O", "lse", "dQ", "dK", "dV")}
    want = {n: [] for n in got}
    for h in range(w.Hq):
        if hs.start <= h < hs.stop:
            continue
        rows = _sample_rows(w.L, rng, 6)
        r = oracle.sampled_rows(inp["q"], inp["k"], inp["v"], inp["do"], w.scale, w.mask, w.window, 0, h, rows)
        for n in ("O", "lse", "dQ"):
            got[n].append(_np(gpu[n][0, h][torch.as_tensor(rows, device=DEV)]))
            want[n].append(r[n])
    for gg in range(w.Hkv - 1):
        keys = _sample_key_pair(w, rng)
        r = oracle.sampled_keys(inp["q"], inp["k"], inp["v"], inp["do"], w.scale, w.mask, w.window, 0, gg, keys)
        for n in ("dK", "dV"):
            got[n].append(_np(gpu[n][0, gg][torch.as_tensor(keys, device=DEV)]))
            want[n].append(r[n])
    serr = {}
    for n in got:
        a, b = np.concatenate(got[n]), np.concatenate(want[n])
        serr[n] = float(np.max(np.abs(a - b))) if n == "lse" else rel_fro(a, b)
    print(w.name, "other heads, sampled:", {k: f"{v:.2e}" for k, v in serr.items()}, flush=True)
    for n in ("O", "dQ", "dK", "dV"):
        assert serr[n] <= tol, ("sampled", n, serr[n])
    assert serr["lse"] <= LSE_TOL, ("sampled", serr["lse"])

    # every softmax row sums to one, so sum_j dV_{g,j} = sum over the group's
    # heads and rows of dO
    dv_sum = gpu["dV"].double().sum(dim=2)
    do_sum = inp["do"].to(DEV).double().view(w.B, w.Hkv, w.group, w.L, w.D).sum(dim=(2, 3))
    rel = (torch.linalg.norm(dv_sum - do_sum) / torch.linalg.norm(do_sum)).item()
    print("dV column-sum identity rel err", f"{rel:.2e}", flush=True)
    assert rel <= 1e-2
    # and every dS row sums to zero, so sum_j dK_{g,j} = 0: measured against
    # the size of dK (the backward's Delta comes from the bf16 O, so this only
    # holds to bf16 rounding)
    dk_sum = gpu["dK"].double().sum(dim=2)
    rel_k = (torch.linalg.norm(dk_sum) / torch.linalg.norm(gpu["dK"].double())).item()
    print("dK column-sum identity rel err", f"{rel_k:.2e}", flush=True)
    assert rel_k <= 1e-2


# ------------------------------------------------------------------ invariants on the GPU
def test_window_one_identity_gpu():
    w = Workload("w1", 1, 4, 2, 300, 256, "bf16", MASK_WINDOW, 1, seed=7200)
    inp = make_inputs(w)
    g1 = run(w, inp)
    ref = oracle_full(w, inp)
    ref2 = oracle_full(w, inp, window=2)
    for n in ("O", "dV"):
        assert rel_fro(_np(g1[n]), ref[n]) <= 1e-2
    # true dQ and dK are zero at window 1: measure against the window-2 scale
    for n in ("dQ", "dK"):
        assert np.linalg.norm(_np(g1[n])) <= 1e-2 * np.linalg.norm(ref2[n])
    assert np.max(np.abs(_np(g1["lse"]) - ref["lse"])) <= LSE_TOL


def test_window_at_least_L_equals_causal_bitwise():
    w = Workload("wbig", 1, 4, 2, 700, 256, "bf16", MASK_CAUSAL, 0, seed=7300)
    inp = make_inputs(w)
    a = run(w, inp)
    for W in (700, 701, 2**31 - 1):
        b = run(w.with_(mask=MASK_WINDOW, window=W), inp)
        for n in ("O", "lse", "dQ", "dK", "dV"):
            assert torch.equal(a[n], b[n]), (W, n)


def test_masked_keys_do_not_change_outputs():
    w = Workload("mk", 1, 2, 1, 400, 256, "bf16", MASK_WINDOW, 50, seed=7400)
    inp = make_inputs(w)
    base = run(w, inp)
    i = 300
    pert = dict(inp)
    k2, v2 = inp["k"].clone(), inp["v"].clone()
    for j in (0, 100, i - 50, i + 1, 399):   # behind the window and above the diagonal of row i
        k2[:, :, j] += 3.0
        v2[:, :, j] -= 2.0
    pert["k"], pert["v"] = k2, v2
    p = run(w, pert)
    for n in ("O", "lse"):
        assert torch.equal(base[n][:, :, i], p[n][:, :, i]), n
    assert rel_fro(_np(p["dQ"][:, :, i]), _np(base["dQ"][:, :, i])) <= 1e-6


def test_determinism():
    w = BY_NAME["bf16_causal_gqa_L2048_D256_h8kv4"]
    inp = make_inputs(w)
    a = run(w, inp)
    b = run(w, inp)
    # no atomics anywhere: every output is bitwise reproducible
    for n in ("O", "lse", "dQ", "dK", "dV"):
        assert torch.equal(a[n], b[n]), n


def test_empty_sequence_is_a_no_op():
    q = torch.empty(1, 2, 0, 64, dtype=torch.bfloat16, device=DEV)
    k = torch.empty(1, 1, 0, 64, dtype=torch.bfloat16, device=DEV)
    o, lse = sdpa_fwd_lse(q, k, k, "causal")
    dq, dk, dv = sdpa_bwd(q, k, k, o, q, lse, "causal")
    assert o.numel() == 0 and dq.numel() == 0 and dk.numel() == 0


def test_binding_errors_are_raised():
    from sdpa_backward_amd import SdpaError
    q = torch.zeros(1, 2, 16, 96, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(1, 1, 16, 96, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(SdpaError):
        sdpa_fwd_lse(q, k, k, "causal")          # D = 96 is not built
    q = torch.zeros(1, 2, 16, 64, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(1, 1, 16, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(SdpaError):
        sdpa_fwd_lse(q, k, k, "causal_window", 0)
    with pytest.raises(SdpaError):
        sdpa_fwd_lse(q, k, k, "window", 0)
    with pytest.raises(ValueError):
        sdpa_fwd_lse(q, k, k, "sliding")       # not a mask name
