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
    """O = softmax(scale * Q K^T + mask) V with the library's forward and backward."""

    @staticmethod
    def forward(ctx, q, k, v, mask="causal", window=0, scale=None):
        o, lse = sdpa_fwd_lse(q, k, v, mask, window, scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.cfg = (mask, window, scale)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        mask, window, scale = ctx.cfg
        dq, dk, dv = sdpa_bwd(q, k, v, o, do, lse, mask, window, scale)
        return dq, dk, dv, None, None, None


def attention(q, k, v, mask="causal", window=0, scale=None):
    """Differentiable attention over [B, H, L, D] tensors (q: Hq heads, k/v: Hkv heads, Hq % Hkv == 0)."""
    return SDPAFunction.apply(q, k, v, mask, window, scale)
