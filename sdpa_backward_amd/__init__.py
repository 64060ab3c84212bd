"""MI355X (gfx950) memory-efficient scaled-dot-product attention: forward with
per-row logsumexp and tiled dQ/dK/dV backward with GQA, under causal, causal
sliding-window, two-sided window or no mask, with the queries optionally the
last Lq of Lk key positions. The compute lives in the HIP library libsdpa.so (C ABI in
include/sdpa.h); this package is its thin Python binding.
"""
from ._lib import (SdpaError, bwd_workspace_bytes, fwd_workspace_bytes, load, sdpa_bwd, sdpa_fwd_lse,  # noqa: F401
                   workspace_bytes)
from .autograd import SDPAFunction, attention  # noqa: F401

__all__ = ["sdpa_fwd_lse", "sdpa_bwd", "workspace_bytes", "bwd_workspace_bytes", "fwd_workspace_bytes", "load",
           "SdpaError", "attention", "SDPAFunction"]
