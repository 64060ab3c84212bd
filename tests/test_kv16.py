"""The 16-key dK/dV kernel at D = 256 on the GPU (run on an MI355X).

Dense 16-bit calls at D = 256 whose key blocks (128 keys per kv head and
batch) number at least 256 run their dK/dV pass with 16-key waves on
v_mfma_f32_16x16x32 (D = 512 always does; its cases live in the other
files). Checked against the fp64 oracle, and against the 32-key kernel,
which a strided copy of the same tensors takes. With a band at most 2304 keys
wide the dense call also keeps dS for the band and forms dQ from it, while the
strided copy recomputes S and dP for dQ: the two dQ agree to fp32 summation
order and dS rounding.
"""
import numpy as np
import pytest
import torch

import oracle
from sdpa_backward_amd import sdpa_bwd, sdpa_fwd_lse
from tests.oracle_pins import rel_fro
from tests.test_parity import DEV, TOL, _np
from workloads import MASK_CAUSAL, MASK_TWO_SIDED, MASK_WINDOW, Workload, make_inputs

pytestmark = pytest.mark.gpu

CASES = [
    # name, B, Hq, Hkv, Lq, Lk, D, dtype, mask, window   (key blocks: ceil(Lk / 128) * Hkv * B >= 256)
    ("mha64_causal_L512", 1, 64, 64, 512, 512, 256, "bf16", MASK_CAUSAL, 0),
    ("gqa2_w100_ragged_L1000", 1, 64, 32, 1000, 1000, 256, "bf16", MASK_WINDOW, 100),
    ("B2_two_sided_suffix", 2, 32, 16, 300, 1000, 256, "f16", MASK_TWO_SIDED, 77),
    ("gqa4_causal_f16_L1024", 1, 128, 32, 1024, 1024, 256, "f16", MASK_CAUSAL, 0),
    ("more_rows_than_keys", 1, 64, 64, 700, 512, 256, "bf16", MASK_CAUSAL, 0),   # 188 rows see no key
    ("window_one", 1, 64, 64, 512, 512, 256, "bf16", MASK_WINDOW, 1),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_kv16_d256(case):
    name, B, Hq, Hkv, Lq, Lk, D, dtype, mask, window = case
    assert -(-Lk // 128) * Hkv * B >= 256
    w = Workload(name, B, Hq, Hkv, Lq, D, dtype, mask, window, seed=9850 + Lq, Lk=Lk)
    inp = make_inputs(w)
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    o, lse = sdpa_fwd_lse(q, k, v, w.mask, w.window, w.scale)
    dq, dk, dv = sdpa_bwd(q, k, v, o, do, lse, w.mask, w.window, w.scale)
    # the same values in a [B, L, H, D] layout: the strided instantiation, 32-key waves
    blhd = lambda t: t.transpose(1, 2).contiguous().transpose(1, 2)
    g2 = sdpa_bwd(blhd(q), blhd(k), blhd(v), blhd(o), blhd(do), lse, w.mask, w.window, w.scale)
    torch.cuda.synchronize()
    ref = oracle.sdpa_fwd_bwd(inp["q"], inp["k"], inp["v"], inp["do"], w.scale, w.mask, w.window)
    errs = {n: rel_fro(_np(t), ref[n]) for n, t in (("dK", dk), ("dV", dv), ("dQ", dq))}
    cross = {"dK": rel_fro(_np(dk), _np(g2[1])), "dV": rel_fro(_np(dv), _np(g2[2])),
             "dQ": rel_fro(_np(dq), _np(g2[0]))}
    print(name, {k_: f"{x:.2e}" for k_, x in errs.items()}, {k_: f"{x:.2e}" for k_, x in cross.items()}, flush=True)
    for n, e in errs.items():
        assert e <= TOL[dtype], (n, e)
    if mask == MASK_WINDOW and window == 1:
        # one key per row: P = 1 and dP equals Delta, so dK is exactly zero and
        # both kernels return fp32 cancellation noise, summed over d in different
        # orders; bound the difference absolutely instead of relatively
        for n, t, r in (("dK", dk, g2[1]), ("dQ", dq, g2[0])):
            assert float(np.linalg.norm(_np(t) - _np(r))) <= TOL[dtype], cross
            cross.pop(n)
    for n, e in cross.items():
        assert e <= 4e-3, (n, e)   # two kernels, same rounding points, fp32 sums in another order
