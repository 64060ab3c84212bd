"""Plain fp64 CPU oracle for masked scaled-dot-product attention: forward with
per-row logsumexp, and the closed-form gradient (dQ, dK, dV).

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of bench.py use it. It shares no code with the HIP library.

What is computed, and where the pages define it
------------------------------------------------
* The forward keeps each row's logsumexp, the normalizer of its softmax, for
  the backward to reuse (page "Lab 028 lab detail: Off NVIDIA, you fix the
  platform yourself", section "What I changed, in plain terms", item 1). The
  backward rebuilds P from the scores and that lse and forms P and dS per
  element (same page, section "2026-10-21", "What the code says";
  page "Training - design (ORPO, flash-CCE head, prefix sharing, segmented
  backward)", section 6, which lists a fused backward that stores per-row LSE
  and recomputes P).
* Masks: above the causal diagonal P is zero; a window additionally zeroes P
  where the key index is below ``i + diag_off - window_size + 1`` (Lab 028
  page, "Plan for the build", step 4, and "What I changed", items 3-4). A
  window without the causal mask is read as a band on both sides of the
  query's diagonal: a key at distance ``window_size`` or more from it, ahead
  or behind, is masked (same page, "What I changed", items 3 and 4, where the
  non-causal window also drops the tiles wholly ahead). With queries a suffix of the keys,
  ``diag_off = Lk - Lq`` (same page, item 5(b), and the parity cases with
  ``qL < kL``). No mask: every key.
* Block-sparse cut: the prefix-sharing forward runs one pass over
  [prompt; chosen; rejected] under a mask that is causal except that the
  rejected rows never see the chosen tokens (page "Training - design (ORPO,
  flash-CCE head, prefix sharing, segmented backward)", section 5.4); here a
  cut (r0, c0, c1) removes keys [c0, c1) from rows r0 onwards, on top of any
  mask. The same section cuts its sliding window at logical positions (each
  response restarts right after the prompt, by its block-wise position
  reset): with a fourth element ``logical`` true, rows r0 onwards measure
  their distance to a key before c0 as if the cut keys were not there, i.e.
  from the key's position plus c1 - c0. With r0 = c1 that makes every
  rejected row's mask the mask of the pass over [prompt; rejected] alone.
* Sinks: the backward the pages patch also takes attention sinks as a
  parameter (Lab 028 page, "What I changed", item 2). Reading: one logit per
  query head that joins every row's softmax normalizer as an extra score
  with a zero value row (see head_rows).
* GQA: query head h reads kv head ``h // group`` (page "MiniCPM5 Decode
  Megakernel - end-to-end build plan (handoff)", section 4.1, per-layer stage 5).

The pages name these pieces but never print the gradient formulas, so the
oracle writes out the textbook chain rule of the plain definition:

    S   = scale * Q K^T                        (all keys, one row at a time)
    S_ij = -inf where (i, j) is not allowed
    lse_i = logsumexp_j S_ij                   (natural log)
    P   = exp(S - lse)                         (exactly 0 where masked)
    O   = P V
    dP  = dO V^T
    Delta_i = <dO_i, O_i>                      (= sum_j P_ij dP_ij)
    dS  = P * (dP - Delta)
    dQ  = scale * dS K
    dK  = scale * dS^T Q      (summed over the q-heads of the kv group)
    dV  = P^T dO              (summed over the q-heads of the kv group)

The score matrix is materialised in full-width row blocks (``row_block`` query
rows x every key). Softmax rows are independent, so row blocking changes no
value; nothing else is blocked, fused or reordered.

Readings where the pages are silent: lse uses the natural log; a row with no
allowed key (possible only when Lq > Lk under a causal mask, or with no keys
at all) gets lse = -inf, O = 0 and zero gradients; ``window >= Lk`` is
identical to plain causal, and a two-sided window of at least Lq + Lk keys is
identical to no mask.

Pins: tests/test_oracle.py checks this module against central finite
differences, an independent float64 autograd of the plain forward (its mask
built from torch's tril/triu), the library SDPA routine (causal, no mask, and
its lower-right causal bias for queries that are a suffix of the keys),
pure-Python brute force on tiny inputs, a hand-derived worked example and
exact invariants.
"""
from __future__ import annotations

import numpy as np

MASKS = ("none", "causal", "causal_window", "window")


def allowed(i, j, Lq: int, Lk: int, mask: str, window: int, cut=None):
    """True where query row i may attend key j (numpy broadcasting over i, j).

    With d = i + diag_off - j, diag_off = Lk - Lq (the query's diagonal sits
    diag_off keys to the right of its row index):
      none:          every key
      causal:        d >= 0
      causal_window: 0 <= d < window
      window:        -window < d < window   (both sides, diagonal included)
    Keys outside [0, Lk) and rows outside [0, Lq) do not exist.

    cut = (r0, c0, c1): additionally, rows i >= r0 do not see keys
    c0 <= j < c1 (the block-sparse prefix-sharing mask: with the sequence
    [prompt; chosen; rejected], r0 = c1 = start of rejected and c0 = start of
    chosen, so the rejected rows never see the chosen tokens).
    cut = (r0, c0, c1, logical) with logical true: besides, for rows i >= r0
    a key j < c0 sits at position j + (c1 - c0) in the distance d above (the
    cut keys do not count), so a window reaches that far further back.
    """
    if mask not in MASKS:
        raise ValueError(f"unknown mask {mask!r}")
    if mask in ("causal_window", "window") and window < 1:
        raise ValueError("window must be >= 1")
    i = np.asarray(i, dtype=np.int64)
    j = np.asarray(j, dtype=np.int64)
    ok = (i >= 0) & (i < Lq) & (j >= 0) & (j < Lk)
    d = i + (Lk - Lq) - j
    if cut is not None and len(cut) > 3 and cut[3]:
        r0, c0, c1 = cut[:3]
        d = np.where((i >= r0) & (j < c0), d - (c1 - c0), d)
    if mask == "causal":
        ok = ok & (d >= 0)
    elif mask == "causal_window":
        ok = ok & (d >= 0) & (d < window)
    elif mask == "window":
        ok = ok & (d > -window) & (d < window)
    if cut is not None:
        r0, c0, c1 = cut[:3]
        ok = ok & ~((i >= r0) & (j >= c0) & (j < c1))
    return ok


def allowed_block(rows: np.ndarray, Lq: int, Lk: int, mask: str, window: int, cut=None) -> np.ndarray:
    """Boolean [len(rows), Lk]: the allowed pairs of these query rows."""
    return allowed(np.asarray(rows)[:, None], np.arange(Lk)[None, :], Lq, Lk, mask, window, cut)


def rows_attending(keys, Lq: int, Lk: int, mask: str, window: int, cut=None) -> np.ndarray:
    """Sorted query rows that attend at least one of ``keys`` (for sampled key gradients)."""
    rows = np.arange(Lq)
    hit = np.zeros(Lq, dtype=bool)
    for j in np.asarray(keys):
        hit |= allowed(rows, int(j), Lq, Lk, mask, window, cut)
    return rows[hit]


def _softmax_rows(S: np.ndarray, ok: np.ndarray):
    """Masked row softmax in fp64: returns (P, lse). Empty rows: P = 0, lse = -inf."""
    S = np.where(ok, S, -np.inf)
    m = S.max(axis=1)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    with np.errstate(under="ignore"):
        E = np.exp(S - m_safe[:, None])        # exp(-inf) = 0 at masked entries
    tot = E.sum(axis=1)
    with np.errstate(divide="ignore"):
        lse = m_safe + np.log(tot)              # log(0) = -inf for an empty row
    nonempty = tot > 0
    P = np.zeros_like(S)
    P[nonempty] = np.exp(S[nonempty] - lse[nonempty, None])
    return P, lse


def head_rows(q_h, k_g, v_g, do_h, scale, mask, window, rows, want_grad=True, sink=None, cut=None):
    """Forward (and, with ``do_h``, backward) for one q-head and a set of query rows.

    q_h, do_h: [Lq, D]; k_g, v_g: [Lk, D] (fp64). Returns a dict with
    O[rows], lse[rows], Delta[rows] and, if want_grad, dQ[rows] plus the
    additive contributions of these rows to dK and dV ([Lk, D] each).

    ``sink``: this head's sink logit, or None. It is one more score column,
    allowed for every row, whose value row is zero: it enters every row's
    softmax normalizer and takes probability mass without adding to O. Its
    gradient is the chain rule through that column, dS_sink = P_sink (0 - Delta),
    returned summed over the rows as "dSink".
    """
    Lq, Lk = q_h.shape[0], k_g.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    ok = allowed_block(rows, Lq, Lk, mask, window, cut)
    qb = q_h[rows]
    S = scale * (qb @ k_g.T)
    if sink is not None:
        S = np.concatenate([S, np.full((len(rows), 1), float(sink))], axis=1)
        ok = np.concatenate([ok, np.ones((len(rows), 1), dtype=bool)], axis=1)
    P, lse = _softmax_rows(S, ok)
    if sink is not None:
        P, P_sink = P[:, :Lk], P[:, Lk]
    O = P @ v_g
    out = {"O": O, "lse": lse}
    if not want_grad:
        return out
    dob = do_h[rows]
    dP = dob @ v_g.T
    delta = np.sum(dob * O, axis=1)
    dS = P * (dP - delta[:, None])
    out["Delta"] = delta
    out["dQ"] = scale * (dS @ k_g)
    out["dK"] = scale * (dS.T @ qb)
    out["dV"] = P.T @ dob
    if sink is not None:
        out["dSink"] = float(np.sum(P_sink * (0.0 - delta)))
    return out


def _f64(x):
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch  # local: torch is only needed to unwrap tensors
        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def sdpa_forward(q, k, v, scale, mask="causal", window=0, row_block=1024, sinks=None, cut=None):
    """O [B,Hq,Lq,D] and lse [B,Hq,Lq] for inputs [B,H,L,D] (any float dtype, upcast to fp64).

    sinks: optional [Hq] sink logits (see head_rows)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    sinks = None if sinks is None else _f64(sinks)
    B, Hq, Lq, D = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv
    O = np.zeros_like(q)
    lse = np.zeros((B, Hq, Lq))
    for b in range(B):
        for h in range(Hq):
            g = h // group
            for r0 in range(0, Lq, row_block):
                rows = np.arange(r0, min(Lq, r0 + row_block))
                res = head_rows(q[b, h], k[b, g], v[b, g], None, scale, mask, window, rows, want_grad=False,
                                sink=None if sinks is None else sinks[h], cut=cut)
                O[b, h, rows] = res["O"]
                lse[b, h, rows] = res["lse"]
    return O, lse


def sdpa_fwd_bwd(q, k, v, do, scale, mask="causal", window=0, row_block=1024, sinks=None, cut=None):
    """Forward and closed-form backward. Returns dict O, lse, Delta, dQ, dK, dV (fp64 numpy),
    and dSinks [Hq] when sinks [Hq] are given."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    sinks = None if sinks is None else _f64(sinks)
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv
    O = np.zeros_like(q)
    lse = np.zeros((B, Hq, Lq))
    delta = np.zeros((B, Hq, Lq))
    dQ = np.zeros_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    dSinks = np.zeros(Hq)
    for b in range(B):
        for h in range(Hq):
            g = h // group
            for r0 in range(0, Lq, row_block):
                rows = np.arange(r0, min(Lq, r0 + row_block))
                res = head_rows(q[b, h], k[b, g], v[b, g], do[b, h], scale, mask, window, rows,
                                sink=None if sinks is None else sinks[h], cut=cut)
                O[b, h, rows] = res["O"]
                lse[b, h, rows] = res["lse"]
                delta[b, h, rows] = res["Delta"]
                dQ[b, h, rows] = res["dQ"]
                dK[b, g] += res["dK"]
                dV[b, g] += res["dV"]
                if sinks is not None:
                    dSinks[h] += res["dSink"]
    out = {"O": O, "lse": lse, "Delta": delta, "dQ": dQ, "dK": dK, "dV": dV}
    if sinks is not None:
        out["dSinks"] = dSinks
    return out


def sampled_rows(q, k, v, do, scale, mask, window, b, h, rows, sinks=None, cut=None):
    """O, lse and dQ of selected query rows of head (b, h), from the full key range."""
    group = q.shape[1] // k.shape[1]
    g = h // group
    qh, kg, vg, doh = _f64(q[b, h]), _f64(k[b, g]), _f64(v[b, g]), _f64(do[b, h])
    res = head_rows(qh, kg, vg, doh, scale, mask, window, rows, sink=None if sinks is None else _f64(sinks)[h],
                    cut=cut)
    return {"O": res["O"], "lse": res["lse"], "dQ": res["dQ"]}


def sampled_keys(q, k, v, do, scale, mask, window, b, g, keys, row_block=1024, sinks=None, cut=None):
    """dK, dV of selected keys of kv head (b, g): every row that attends them, every q-head of the group."""
    Hq, Lq = q.shape[1], q.shape[2]
    Lk = k.shape[2]
    group = Hq // k.shape[1]
    rows = rows_attending(keys, Lq, Lk, mask, window, cut)
    kg, vg = _f64(k[b, g]), _f64(v[b, g])
    dK = np.zeros_like(kg)
    dV = np.zeros_like(vg)
    for h in range(g * group, (g + 1) * group):
        qh, doh = _f64(q[b, h]), _f64(do[b, h])
        for r0 in range(0, len(rows), row_block):
            rr = rows[r0:r0 + row_block]
            res = head_rows(qh, kg, vg, doh, scale, mask, window, rr,
                            sink=None if sinks is None else _f64(sinks)[h], cut=cut)
            dK += res["dK"]
            dV += res["dV"]
    keys = np.asarray(keys)
    return {"dK": dK[keys], "dV": dV[keys]}
