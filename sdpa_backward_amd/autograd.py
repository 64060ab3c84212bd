"""torch.autograd wrapper of the library: attention(q, k, v) as a differentiable
op whose forward keeps the per-row logsumexp and whose backward is sdpa_bwd.

The forward saves q, k, v, O and lse (O(L) extra memory: O and one float per
query row); the backward rebuilds P from them one tile at a time. lse gets no
gradient. Inputs are [B, H, L, D] views with contiguous rows (a projection
output in [B, L, H, D] layout passes as ``t.transpose(1, 2)`` with no copy).
"""
from __future__ import annotations

import torch

from ._lib import sdpa_bwd, sdpa_fwd_lse


class SDPAFunction(torch.autograd.Function):
    """O = softmax(scale * Q K^T + mask) V with the library's forward and backward
    (and optional per-head sink logits in every row's normalizer)."""

    @staticmethod
    def forward(ctx, q, k, v, mask="causal", window=0, scale=None, sinks=None, cut=None):
        o, lse = sdpa_fwd_lse(q, k, v, mask, window, scale, sinks=sinks, cut=cut)
        ctx.save_for_backward(q, k, v, o, lse, sinks)
        ctx.cfg = (mask, window, scale, cut)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse, sinks = ctx.saved_tensors
        mask, window, scale, cut = ctx.cfg
        # The incoming gradient is often an expanded view: o.sum().backward()
        # hands over strides (0, 0, 0, 0), a loss weighted by a broadcast vector
        # a zero row stride. The library reads rows of D contiguous elements
        # with one row stride shared by q and dO, so such views become a
        # contiguous copy in q's layout.
        if do.stride(3) != 1 or 0 in do.stride() or do.stride(2) != q.stride(2):
            do = torch.empty_like(q).copy_(do)  # q's strides when q is dense, else contiguous
        grads = sdpa_bwd(q, k, v, o, do, lse, mask, window, scale, sinks=sinks, cut=cut)
        dsinks = grads[3] if sinks is not None else None
        return grads[0], grads[1], grads[2], None, None, None, dsinks, None


def attention(q, k, v, mask="causal", window=0, scale=None, sinks=None, cut=None):
    """Differentiable attention over [B, H, L, D] tensors (q: Hq heads, k/v: Hkv heads, Hq % Hkv == 0);
    sinks: optional float32 [Hq] logits (differentiable); cut: optional (r0, c0, c1), rows from r0 on do
    not see keys [c0, c1) (prefix sharing: [prompt; chosen; rejected] with r0 = c1 = start of rejected,
    c0 = start of chosen); (r0, c0, c1, True) also measures the window of rows from r0 on at logical
    positions (the cut keys do not count)."""
    return SDPAFunction.apply(q, k, v, mask, window, scale, sinks, cut)
