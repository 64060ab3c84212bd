"""Pins for the fp64 oracle: checks against facts that do not come from the
oracle itself. Each pin takes the oracle module as an argument so the same
checks can be run against deliberately broken copies of it (mutation tests).

Pins:
  golden       hand-derived worked example (tests/golden/worked_L2_D1.json)
  brute        pure-Python loops over the definition (forward: O, lse)
  fd           central finite differences of l = sum(dO * O) (dQ, dK, dV, dSinks)
  autograd     torch float64 autograd of a plain matmul/softmax forward
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _num(x):
    if isinstance(x, str):
        env = {"ln2": math.log(2), "ln3": math.log(3), "ln4": math.log(4)}
        return float(eval(x, {"__builtins__": {}}, env))  # fixture-only arithmetic on ln constants
    if isinstance(x, list):
        return [_num(y) for y in x]
    return float(x)


def load_golden():
    with open(os.path.join(GOLDEN, "worked_L2_D1.json")) as f:
        return json.load(f)


def pin_golden(mod, tol=1e-14):
    """Max abs error of the oracle against the hand-derived worked example."""
    g = load_golden()
    inp = {k: np.array(_num(v)) for k, v in g["inputs"].items() if k in ("q", "k", "v", "do")}
    inp = {k: v[None] for k, v in inp.items()}  # add B=1
    worst = 0.0
    for case, mask, window in (("causal", "causal", 0), ("window1", "causal_window", 1)):
        res = mod.sdpa_fwd_bwd(inp["q"], inp["k"], inp["v"], inp["do"], g["inputs"]["scale"], mask, window)
        for name in ("O", "lse", "dQ", "dK", "dV"):
            ref = np.array(_num(g[case][name]))[None]
            worst = max(worst, float(np.max(np.abs(res[name] - ref))))
    return worst


def brute_forward(q, k, v, scale, mask, window, sinks=None, cut=None):
    """O and lse from the definition with Python loops and math.exp (no numpy linear algebra).

    Query row i sits at key position i + Lk - Lq (queries are the last Lq of
    the Lk positions); a row with no allowed key gets O = 0, lse = -inf (or
    lse = its head's sink logit when sinks are given: the sink adds exp(sink)
    to every row's normalizer and nothing to O)."""
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    group = Hq // Hkv
    O = np.zeros((B, Hq, Lq, D))
    lse = np.zeros((B, Hq, Lq))
    for b in range(B):
        for h in range(Hq):
            g = h // group
            for i in range(Lq):
                pos = i + Lk - Lq
                # logical cut: a row from cut[0] on and the keys from cut[2] on
                # move back by the cut's length (the response restarts right
                # after the prompt); the keys before cut[1] keep their place
                logical = cut is not None and len(cut) > 3 and cut[3] and i >= cut[0]
                sh = cut[2] - cut[1] if logical else 0
                where = (lambda j: j - sh if j >= cut[2] else j) if logical else (lambda j: j)
                p = pos - sh
                if mask == "none":
                    keys = list(range(Lk))
                elif mask == "causal":
                    keys = [j for j in range(Lk) if where(j) <= p]
                elif mask == "causal_window":
                    keys = [j for j in range(Lk) if p - window < where(j) <= p]
                else:  # "window": both sides of the diagonal
                    keys = [j for j in range(Lk) if abs(where(j) - p) < window]
                if cut is not None and i >= cut[0]:   # rows from cut[0] on skip keys [cut[1], cut[2])
                    keys = [j for j in keys if not cut[1] <= j < cut[2]]
                sink = None if sinks is None else float(sinks[h])
                if not keys:
                    lse[b, h, i] = -math.inf if sink is None else sink
                    continue
                s = [scale * sum(float(q[b, h, i, d]) * float(k[b, g, j, d]) for d in range(D)) for j in keys]
                mx = max(s) if sink is None else max(max(s), sink)
                z = sum(math.exp(x - mx) for x in s) + (0.0 if sink is None else math.exp(sink - mx))
                lse[b, h, i] = mx + math.log(z)
                for d in range(D):
                    O[b, h, i, d] = sum(math.exp(x - lse[b, h, i]) * float(v[b, g, j, d]) for x, j in zip(s, keys))
    return O, lse


def tiny_inputs(Hq, Hkv, L, D, seed, Lk=None):
    """Seeded N(0, 1) fp64 inputs; L query rows and Lk (default L) keys."""
    Lk = L if Lk is None else Lk
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, Hq, L, D))
    k = rng.standard_normal((1, Hkv, Lk, D))
    v = rng.standard_normal((1, Hkv, Lk, D))
    do = rng.standard_normal((1, Hq, L, D))
    return q, k, v, do


# Hq, Hkv, Lq, Lk, D, scale, mask, window
BRUTE_CASES = [
    (2, 1, 7, 7, 3, 0.7, "causal", 0),
    (4, 2, 9, 9, 4, 1.0, "causal_window", 3),
    (2, 2, 6, 6, 2, 3.0, "causal_window", 1),
    (3, 1, 5, 5, 5, 0.45, "causal_window", 2),
    (2, 1, 6, 6, 3, 0.9, "none", 0),
    (2, 2, 8, 8, 3, 0.8, "window", 3),
    (2, 1, 4, 9, 3, 0.6, "causal", 0),          # queries the last 4 of 9 positions
    (2, 1, 5, 11, 2, 1.1, "causal_window", 3),
    (2, 1, 4, 10, 3, 0.5, "window", 2),
    (2, 1, 3, 7, 2, 0.7, "none", 0),
    (2, 1, 9, 4, 3, 0.8, "causal", 0),          # more queries than keys: the first rows see nothing
    (2, 2, 8, 5, 2, 1.3, "window", 2),
]
# [prompt 3; chosen 4; rejected 3] and a cut inside a suffix-query problem
BRUTE_CUT_CASES = [
    ((2, 1, 10, 10, 3, 0.8, "causal", 0), (7, 3, 7)),
    ((2, 2, 6, 11, 2, 1.2, "causal_window", 4), (3, 2, 6)),
    ((2, 1, 8, 8, 3, 0.6, "none", 0), (4, 0, 3)),
    # the window at logical positions: [prompt 3; chosen 4; rejected 4], window 3 and 5
    ((2, 1, 11, 11, 3, 0.9, "causal_window", 3), (7, 3, 7, True)),
    ((2, 2, 11, 11, 2, 0.7, "causal_window", 5), (7, 3, 7, True)),
    ((2, 1, 9, 9, 3, 1.1, "window", 3), (6, 2, 5, True)),
]
# the same kind of cases with sink logits (per head)
BRUTE_SINK_CASES = [
    ((2, 1, 7, 7, 3, 0.7, "causal", 0), (0.5, -1.0)),
    ((2, 2, 6, 9, 2, 1.1, "window", 2), (2.0, -0.3)),
    ((2, 1, 9, 4, 3, 0.8, "causal", 0), (1.5, 0.0)),      # rows with no key: lse = sink
]


def pin_brute(mod, cases=None):
    """Max abs error of oracle O/lse against brute force over a few tiny cases (lse -inf must match)."""
    cases = cases or ([(c, None, None) for c in BRUTE_CASES] + [(c, sk, None) for c, sk in BRUTE_SINK_CASES] +
                      [(c, None, cut) for c, cut in BRUTE_CUT_CASES])
    worst = 0.0
    for n, (case, sinks, cut) in enumerate(cases):
        Hq, Hkv, Lq, Lk, D, s, mask, W = case
        q, k, v, _ = tiny_inputs(Hq, Hkv, Lq, D, 100 + n, Lk)
        kw = {}
        if sinks is not None:
            kw["sinks"] = np.array(sinks, dtype=np.float64)
        if cut is not None:
            kw["cut"] = cut
        O, lse = mod.sdpa_forward(q, k, v, s, mask, W, **kw)
        Ob, lb = brute_forward(q, k, v, s, mask, W, kw.get("sinks"), cut)
        if not np.all(np.isfinite(O)):
            return math.inf
        fin = np.isfinite(lb)
        if not np.array_equal(np.isfinite(lse), fin) or np.any(lse[~fin] != lb[~fin]):
            return math.inf
        worst = max(worst, float(np.max(np.abs(O - Ob))), float(np.max(np.abs(lse[fin] - lb[fin]), initial=0.0)))
    return worst


def fd_error(mod, Hq, Hkv, L, D, scale, mask, window, seed=0, Lk=None, sinks=None, cut=None):
    """max|FD - analytic| / max|analytic| over every coordinate of Q, K and V (and the sinks)."""
    q, k, v, do = tiny_inputs(Hq, Hkv, L, D, seed, Lk)
    kw = {} if sinks is None else {"sinks": np.asarray(sinks, dtype=np.float64)}
    ckw = {} if cut is None else {"cut": cut}
    res = mod.sdpa_fwd_bwd(q, k, v, do, scale, mask, window, **kw, **ckw)
    grads = {"q": res["dQ"], "k": res["dK"], "v": res["dV"]}
    base = {"q": q, "k": k, "v": v}
    if sinks is not None:
        grads["sinks"] = res["dSinks"]
        base["sinks"] = kw["sinks"]

    def loss(a):
        extra = {} if sinks is None else {"sinks": a["sinks"]}
        O, _ = mod.sdpa_forward(a["q"], a["k"], a["v"], scale, mask, window, **extra, **ckw)
        return float(np.sum(do * O))

    worst = 0.0
    scale_ref = max(float(np.max(np.abs(g))) for g in grads.values())
    for name in base:
        x = base[name]
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            x0 = x[idx]
            h = 1e-6 * max(1.0, abs(x0))
            xp = x.copy()
            xp[idx] = x0 + h
            xm = x.copy()
            xm[idx] = x0 - h
            fd[idx] = (loss(dict(base, **{name: xp})) - loss(dict(base, **{name: xm}))) / (2 * h)
        worst = max(worst, float(np.max(np.abs(fd - grads[name]))))
    return worst / scale_ref


def fd_directional_error(mod, Hq, Hkv, L, D, scale, mask, window, ndir=16, seed=0):
    """Directional central differences along random unit directions in (Q, K, V) jointly."""
    q, k, v, do = tiny_inputs(Hq, Hkv, L, D, seed)
    res = mod.sdpa_fwd_bwd(q, k, v, do, scale, mask, window)
    rng = np.random.default_rng(seed + 1)

    def loss(qq, kk, vv):
        O, _ = mod.sdpa_forward(qq, kk, vv, scale, mask, window)
        return float(np.sum(do * O))

    worst = 0.0
    for _ in range(ndir):
        u = [rng.standard_normal(x.shape) for x in (q, k, v)]
        nrm = math.sqrt(sum(float(np.sum(x * x)) for x in u))
        u = [x / nrm for x in u]
        h = 1e-6
        lp = loss(q + h * u[0], k + h * u[1], v + h * u[2])
        lm = loss(q - h * u[0], k - h * u[1], v - h * u[2])
        fd = (lp - lm) / (2 * h)
        an = float(np.sum(res["dQ"] * u[0]) + np.sum(res["dK"] * u[1]) + np.sum(res["dV"] * u[2]))
        gn = math.sqrt(sum(float(np.sum(res[n] ** 2)) for n in ("dQ", "dK", "dV")))
        worst = max(worst, abs(fd - an) / gn)
    return worst


def torch_mask(Lq, Lk, mask, window, cut=None):
    """Allowed pairs [Lq, Lk] built from torch's own band routines: tril keeps
    j <= i + diagonal and triu keeps j >= i + diagonal, with the diagonal moved
    Lk - Lq to the right (queries are the last Lq key positions)."""
    ones = torch.ones(Lq, Lk, dtype=torch.bool)
    off = Lk - Lq
    if mask == "none":
        ok = ones
    elif mask == "causal":
        ok = torch.tril(ones, diagonal=off)
    elif mask == "causal_window":
        ok = torch.tril(ones, diagonal=off) & torch.triu(ones, diagonal=off - window + 1)
    elif mask == "window":
        ok = torch.tril(ones, diagonal=off + window - 1) & torch.triu(ones, diagonal=off - window + 1)
    else:
        raise ValueError(mask)
    if cut is not None:   # a zeroed block: rows cut[0].. against keys cut[1]..cut[2]-1
        ok = ok.clone()
        if len(cut) > 3 and cut[3]:
            # logical window: rows cut[0].. see the keys before cut[1] through the
            # band of a sequence without the cut keys (diagonal cut[2]-cut[1] lower)
            shifted = torch_mask(Lq, Lk - (cut[2] - cut[1]), mask, window)
            ok[cut[0]:, :cut[1]] = shifted[cut[0]:, :cut[1]]
        ok[cut[0]:, cut[1]:cut[2]] = False
    return ok


def torch_plain(q, k, v, do, scale, mask, window, sinks=None, cut=None):
    """float64 autograd of the plain forward: matmul -> -inf mask -> softmax -> matmul
    (every row must have an allowed key, or a sink). Sinks: one more score
    column per head, concatenated after masking, whose value row is zero."""
    q = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    k = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    v = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    group = q.shape[1] // k.shape[1]
    kk = k.repeat_interleave(group, dim=1)
    vv = v.repeat_interleave(group, dim=1)
    ok = torch_mask(q.shape[2], k.shape[2], mask, window, cut)
    S = scale * torch.matmul(q, kk.transpose(-1, -2).contiguous())
    S = S.masked_fill(~ok, float("-inf"))
    if sinks is not None:
        sk = torch.tensor(sinks, dtype=torch.float64, requires_grad=True)
        col = sk.view(1, -1, 1, 1).expand(S.shape[0], S.shape[1], S.shape[2], 1)
        S = torch.cat([S, col], dim=-1)
        vv = torch.cat([vv, torch.zeros_like(vv[:, :, :1])], dim=2)
    else:
        assert bool(ok.any(dim=1).all()), "a row with no allowed key"
    lse = torch.logsumexp(S, dim=-1)
    O = torch.matmul(torch.softmax(S, dim=-1), vv)
    O.backward(torch.tensor(do, dtype=torch.float64))
    out = {"O": O.detach().numpy(), "lse": lse.detach().numpy(), "dQ": q.grad.numpy(),
           "dK": k.grad.numpy(), "dV": v.grad.numpy()}
    if sinks is not None:
        out["dSinks"] = sk.grad.numpy()
    return out


def rel_fro(x, ref):
    den = float(np.linalg.norm(ref))
    num = float(np.linalg.norm(np.asarray(x) - ref))
    return num / den if den > 0 else num


def autograd_error(mod, q, k, v, do, scale, mask, window, sinks=None, cut=None):
    kw = {} if sinks is None else {"sinks": np.asarray(sinks, dtype=np.float64)}
    if cut is not None:
        kw["cut"] = cut
    res = mod.sdpa_fwd_bwd(q, k, v, do, scale, mask, window, **kw)
    ref = torch_plain(q, k, v, do, scale, mask, window, sinks, cut)
    names = ("O", "lse", "dQ", "dK", "dV") + (() if sinks is None else ("dSinks",))
    return max(rel_fro(res[n], ref[n]) for n in names)
