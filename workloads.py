"""Seeded synthetic workloads for the attention forward/backward path.

This module holds shapes and seeded random inputs only: no attention arithmetic.
Both the CPU oracle tests and the HIP-path tests/bench draw their inputs here,
so the two sides see bit-identical tensors.

Shapes follow the attention layers of a long-context LoRA step (32 query heads;
global causal layers with D=512 and 4 KV heads; sliding layers with a 1024-key
window, D=256 and 16 KV heads; a 30,553-token example), as described on the
page "Lab 028 lab detail: Off NVIDIA, you fix the platform yourself", section
"2026-10-21" (starting point and probe table) and its model-step table.

Recipe (every config): a CPU torch.Generator seeded with ``seed``; draw
Q, K, V, dO in that order with ``torch.randn`` in float32 (i.i.d. N(0, 1));
cast to bfloat16 (round-to-nearest-even) for the bf16 configs, keep float32
for the fp32 config. Layout [B, H, L, D] contiguous; Q and dO carry Hq heads,
K and V carry Hkv = Hq / group heads. The softmax scale is 1/sqrt(D) rounded
to float32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Optional

import torch

MASK_NONE = "none"
MASK_CAUSAL = "causal"
MASK_WINDOW = "causal_window"      # window keys up to and including the diagonal
MASK_TWO_SIDED = "window"          # window - 1 keys on either side of the diagonal, no causal mask


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    L: int
    D: int
    dtype: str          # "bf16", "f16" or "f32"
    mask: str           # MASK_NONE, MASK_CAUSAL, MASK_WINDOW or MASK_TWO_SIDED
    window: int = 0     # window size (diagonal included); 0 without a window
    seed: int = 1000
    Lk: Optional[int] = None  # keys (default L); the L queries are the last L of the Lk positions

    @property
    def Lkv(self) -> int:
        return self.L if self.Lk is None else self.Lk

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    @property
    def scale(self) -> float:
        return float(torch.tensor(1.0 / math.sqrt(self.D), dtype=torch.float32))

    @property
    def torch_dtype(self):
        return {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[self.dtype]

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads of this path, smallest first.
WORKLOADS = [
    Workload("tiny_fp32_causal_L128_D64_gqa2", 1, 2, 1, 128, 64, "f32", MASK_CAUSAL, 0, 1000),
    Workload("bf16_causal_gqa_L2048_D256_h8kv4", 1, 8, 4, 2048, 256, "bf16", MASK_CAUSAL, 0, 1001),
    Workload("bf16_causal_global_L8192_D512_h16kv4", 1, 16, 4, 8192, 512, "bf16", MASK_CAUSAL, 0, 1002),
    Workload("bf16_window1024_L16384_D256_h32kv16", 1, 32, 16, 16384, 256, "bf16", MASK_WINDOW, 1024, 1003),
    Workload("bf16_window1024_ragged_L30553_D256_h32kv16", 1, 32, 16, 30553, 256, "bf16", MASK_WINDOW, 1024, 1004),
]
# The variants beside them, at the sliding layers' geometry: the window on
# both sides of the diagonal, the queries as the last quarter of the key
# positions (keys behind every query's window must get zero gradients), and
# no mask at all (page "Lab 028 lab detail: Off NVIDIA, you fix the platform
# yourself", "What I changed, in plain terms", items 3-5).
VARIANTS = [
    Workload("bf16_twosided_window1024_L16384_D256_h32kv16", 1, 32, 16, 16384, 256, "bf16", MASK_TWO_SIDED, 1024, 1005),
    Workload("bf16_window1024_Lq4096_Lk16384_D256_h32kv16", 1, 32, 16, 4096, 256, "bf16", MASK_WINDOW, 1024, 1006,
             Lk=16384),
    Workload("bf16_nomask_L4096_D256_h32kv16", 1, 32, 16, 4096, 256, "bf16", MASK_NONE, 0, 1007),
]
# One GPU's share of the L = 16384 window layer when it is split over eight:
# by kv-heads (2 of 16, with their 4 q-heads), or by sequence (a 2048-query
# chunk with the 1023 keys before it that its window reaches, a halo the left
# neighbour would send).
SHARES = [
    Workload("bf16_window1024_L16384_D256_h4kv2", 1, 4, 2, 16384, 256, "bf16", MASK_WINDOW, 1024, 1008),
    Workload("bf16_window1024_Lq2048_Lk3071_D256_h32kv16", 1, 32, 16, 2048, 256, "bf16", MASK_WINDOW, 1024, 1009,
             Lk=3071),
]
BY_NAME = {w.name: w for w in WORKLOADS + VARIANTS + SHARES}


def make_inputs(w: Workload, seed: Optional[int] = None) -> dict:
    """Seeded CPU tensors q, k, v, do in the workload's dtype, layout [B, H, L, D]."""
    g = torch.Generator(device="cpu").manual_seed(w.seed if seed is None else seed)
    shapes = {
        "q": (w.B, w.Hq, w.L, w.D),
        "k": (w.B, w.Hkv, w.Lkv, w.D),
        "v": (w.B, w.Hkv, w.Lkv, w.D),
        "do": (w.B, w.Hq, w.L, w.D),
    }
    out = {}
    for name in ("q", "k", "v", "do"):
        x = torch.randn(shapes[name], dtype=torch.float32, generator=g)
        out[name] = x.to(w.torch_dtype).contiguous()
    return out
