"""Batches, strided layouts and the autograd wrapper (run on an MI355X).

* B > 1 against the fp64 oracle (every batch entry has its own inputs).
* Strided tensors: [B, L, H, D] projection outputs seen as [B, H, L, D]
  views, slices of one fused QKV buffer, and padded rows give results
  bitwise equal to the same values laid out contiguously (the kernels do the
  same arithmetic; only addresses change).
* attention() under torch.autograd, and a synthetic single attention layer
  (random weights, seeded inputs: x -> Q, K, V projections -> attention ->
  output projection) whose gradients are compared with the same layer in
  float64 on the CPU with the oracle as its attention (the way a LoRA trainer
  calls the op: page "Lab 028 lab detail: Off NVIDIA, you fix the platform
  yourself", "Model step", where the sliding layers call the windowed op).
"""
import numpy as np
import pytest
import torch

import oracle
from sdpa_backward_amd import attention, sdpa_bwd, sdpa_fwd_lse, workspace_bytes
from tests.oracle_pins import rel_fro
from tests.test_parity import DEV, LSE_TOL, TOL, _np, check_full, oracle_full, run
from workloads import MASK_CAUSAL, MASK_NONE, MASK_TWO_SIDED, MASK_WINDOW, Workload, make_inputs

pytestmark = pytest.mark.gpu

BATCH = [
    # name, B, Hq, Hkv, L, Lk, D, dtype, mask, window
    ("B2_causal_D128", 2, 4, 2, 300, 300, 128, "bf16", MASK_CAUSAL, 0),
    ("B3_w64_D256", 3, 2, 1, 400, 400, 256, "bf16", MASK_WINDOW, 64),
    ("B2_suffix_two_w50_D512", 2, 2, 1, 150, 500, 512, "bf16", MASK_TWO_SIDED, 50),
    ("B2_none_f16_D64", 2, 4, 4, 200, 200, 64, "f16", MASK_NONE, 0),
    ("B2_f32_w9_D64", 2, 2, 1, 90, 90, 64, "f32", MASK_WINDOW, 9),
]


@pytest.mark.parametrize("case", BATCH, ids=[c[0] for c in BATCH])
def test_batches(case):
    name, B, Hq, Hkv, L, Lk, D, dtype, mask, window = case
    w = Workload(name, B, Hq, Hkv, L, D, dtype, mask, window, seed=9500 + L, Lk=Lk)
    inp = make_inputs(w)
    check_full(w, run(w, inp), oracle_full(w, inp))


def _layouts(x, kind, H, pad=64):
    """The same [B, H, L, D] values as a strided view of another buffer."""
    B, _, L, D = x.shape
    if kind == "blhd":       # projection output [B, L, H, D]
        buf = x.transpose(1, 2).contiguous()
        return buf.transpose(1, 2)
    if kind == "padded":     # rows of D + pad elements, heads interleaved by rows
        buf = torch.zeros(B, L, H, D + pad, dtype=x.dtype, device=x.device)
        buf[..., :D] = x.transpose(1, 2)
        return buf[..., :D].transpose(1, 2)
    raise ValueError(kind)


def _fused_qkv(q, k, v):
    """q, k, v as slices of one [B, L, Hq + 2 Hkv, D] buffer (a fused QKV projection)."""
    B, Hq, L, D = q.shape
    Hkv = k.shape[1]
    buf = torch.cat([q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2)], dim=2).contiguous()
    return (buf[:, :, :Hq].transpose(1, 2), buf[:, :, Hq:Hq + Hkv].transpose(1, 2),
            buf[:, :, Hq + Hkv:].transpose(1, 2))


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("kind", ["blhd", "padded", "fused"])
def test_strided_equals_contiguous_bitwise(kind, dtype):
    D = 64 if dtype == "f32" else 256
    w = Workload(f"strided_{kind}", 2, 4, 2, 333, D, dtype, MASK_WINDOW, 100, seed=9600, Lk=333)
    inp = {n: t.to(DEV) for n, t in make_inputs(w).items()}
    q, k, v, do = inp["q"], inp["k"], inp["v"], inp["do"]
    # strided calls never take the small-problem splits (key ranges of the
    # forward and dQ pass, dK/dV shares; their partials are summed in another
    # order): the contiguous reference runs unsplit too
    o, lse = sdpa_fwd_lse(q, k, v, w.mask, w.window, workspace=torch.empty(0, dtype=torch.uint8, device=DEV))
    ws = torch.empty(max(1, workspace_bytes(2, 4, 333, D, q.dtype)), dtype=torch.uint8, device=DEV)
    dq, dk, dv = sdpa_bwd(q, k, v, o, do, lse, w.mask, w.window, workspace=ws)
    if kind == "fused":
        qs, ks, vs = _fused_qkv(q, k, v)
    else:
        qs, ks, vs = _layouts(q, kind, 4), _layouts(k, kind, 2), _layouts(v, kind, 2)
    dos = _layouts(do, "blhd", 4)
    assert not qs.is_contiguous() and not ks.is_contiguous()
    o2, lse2 = sdpa_fwd_lse(qs, ks, vs, w.mask, w.window)
    dq2, dk2, dv2 = sdpa_bwd(qs, ks, vs, o2, dos, lse2, w.mask, w.window)
    torch.cuda.synchronize()
    if kind == "blhd":   # a dense strided input keeps its layout in the outputs
        assert o2.stride() == qs.stride() and dk2.stride() == ks.stride()
    for a, b, n in ((o, o2, "O"), (lse, lse2, "lse"), (dq, dq2, "dQ"), (dk, dk2, "dK"), (dv, dv2, "dV")):
        assert torch.equal(a, b.contiguous()), n


def test_autograd_matches_oracle():
    w = Workload("autograd", 2, 4, 2, 257, 128, "bf16", MASK_WINDOW, 77, seed=9700, Lk=300)
    inp = make_inputs(w)
    q, k, v = (inp[n].to(DEV).requires_grad_() for n in ("q", "k", "v"))
    o = attention(q, k, v, w.mask, w.window)
    o.backward(inp["do"].to(DEV))
    ref = oracle_full(w, inp)
    errs = {n: rel_fro(_np(t), ref[n]) for n, t in (("O", o), ("dQ", q.grad), ("dK", k.grad), ("dV", v.grad))}
    print("autograd", {k: f"{x:.2e}" for k, x in errs.items()}, flush=True)
    for n, e in errs.items():
        assert e <= TOL["bf16"], (n, e)


@pytest.mark.parametrize("loss", ["sum", "row_weighted", "head_summed"])
def test_autograd_expanded_upstream_gradient(loss):
    """Losses whose gradient reaches attention() as an expanded view: o.sum()
    gives dO strides (0, 0, 0, 0), a row-weighted sum over D a zero stride
    along D, a sum over heads a zero head stride. The backward must give the
    oracle's gradients for the dO those views stand for."""
    w = Workload(f"autograd_{loss}", 2, 4, 2, 300, 256, "bf16", MASK_WINDOW, 90, seed=9710)
    inp = make_inputs(w)
    q, k, v = (inp[n].to(DEV).requires_grad_() for n in ("q", "k", "v"))
    o = attention(q, k, v, w.mask, w.window)
    g = torch.Generator().manual_seed(9711)
    if loss == "sum":
        do = torch.ones(o.shape, dtype=torch.float64)
        o.sum().backward()
    elif loss == "row_weighted":
        wr = torch.randn(w.L, generator=g).to(torch.bfloat16)
        (o.sum(-1) * wr.to(DEV)).sum().backward()
        do = wr.double()[:, None].expand(o.shape)
    else:
        wh = torch.randn(w.L, w.D, generator=g).to(torch.bfloat16)
        (o.sum(1) * wh.to(DEV)).sum().backward()
        do = wh.double()[None, None].expand(o.shape)
    ref = oracle.sdpa_fwd_bwd(inp["q"], inp["k"], inp["v"], do.contiguous().numpy(), w.scale, w.mask, w.window)
    errs = {n: rel_fro(_np(t), ref[n]) for n, t in (("dQ", q.grad), ("dK", k.grad), ("dV", v.grad))}
    print("autograd", loss, {k: f"{x:.2e}" for k, x in errs.items()}, flush=True)
    # the expanded dO holds exact values (ones, or the bf16 weights times ones)
    for n, e in errs.items():
        assert e <= TOL["bf16"], (n, e)


class _OracleAttention(torch.autograd.Function):
    """fp64 CPU attention through the oracle (reference side of the layer test)."""

    @staticmethod
    def forward(ctx, q, k, v, mask, window, scale):
        O, _ = oracle.sdpa_forward(q.numpy(), k.numpy(), v.numpy(), scale, mask, window)
        ctx.save_for_backward(q, k, v)
        ctx.cfg = (mask, window, scale)
        return torch.from_numpy(O)

    @staticmethod
    def backward(ctx, do):
        q, k, v = ctx.saved_tensors
        mask, window, scale = ctx.cfg
        r = oracle.sdpa_fwd_bwd(q.numpy(), k.numpy(), v.numpy(), do.numpy(), scale, mask, window)
        return torch.from_numpy(r["dQ"]), torch.from_numpy(r["dK"]), torch.from_numpy(r["dV"]), None, None, None


def _layer(x, Wq, Wk, Wv, Wo, Hq, Hkv, D, mask, window, attn):
    """One attention layer: projections in [B, L, H, D] layout, attention on
    the [B, H, L, D] views, output projection; 2-D matmuls only."""
    B, L, E = x.shape
    x2 = x.reshape(B * L, E)
    q = (x2 @ Wq).view(B, L, Hq, D).transpose(1, 2)
    k = (x2 @ Wk).view(B, L, Hkv, D).transpose(1, 2)
    v = (x2 @ Wv).view(B, L, Hkv, D).transpose(1, 2)
    o = attn(q, k, v, mask, window, D ** -0.5)
    return (o.transpose(1, 2).reshape(B * L, Hq * D) @ Wo).view(B, L, E)


@pytest.mark.parametrize("mask,window", [(MASK_WINDOW, 128), (MASK_CAUSAL, 0), (MASK_TWO_SIDED, 64)])
def test_single_attention_layer_gradients(mask, window):
    B, L, E, Hq, Hkv, D = 2, 384, 512, 8, 4, 128
    g = torch.Generator().manual_seed(9800)
    x = torch.randn(B, L, E, generator=g).to(torch.bfloat16)
    Ws = [(torch.randn(E, n, generator=g) * E ** -0.5).to(torch.bfloat16)
          for n in (Hq * D, Hkv * D, Hkv * D)]
    Wo = (torch.randn(Hq * D, E, generator=g) * (Hq * D) ** -0.5).to(torch.bfloat16)
    gy = torch.randn(B, L, E, generator=g).to(torch.bfloat16)
    params = [x, *Ws, Wo]

    gpu = [t.to(DEV).requires_grad_() for t in params]
    y = _layer(*gpu, Hq, Hkv, D, mask, window, lambda q, k, v, m, w, s: attention(q, k, v, m, w, s))
    y.backward(gy.to(DEV))
    ref = [t.double().requires_grad_() for t in params]
    yr = _layer(*ref, Hq, Hkv, D, mask, window, _OracleAttention.apply)
    yr.backward(gy.double())
    names = ("dx", "dWq", "dWk", "dWv", "dWo")
    errs = {"y": rel_fro(_np(y), yr.detach().numpy())}
    errs.update({n: rel_fro(_np(a.grad), b.grad.numpy()) for n, a, b in zip(names, gpu, ref)})
    cos = {n: float(np.dot(_np(a.grad).ravel(), b.grad.numpy().ravel()) /
                    (np.linalg.norm(_np(a.grad)) * np.linalg.norm(b.grad.numpy())))
           for n, a, b in zip(names, gpu, ref)}
    print("layer", mask, {k: f"{x:.2e}" for k, x in errs.items()}, "cos", {k: f"{x:.6f}" for k, x in cos.items()},
          flush=True)
    # every tensor crosses several bf16 roundings (the projections' outputs, the
    # attention's inputs and outputs, P and dS inside it): 2e-2 relative, and
    # the gradients point the same way
    for n, e in errs.items():
        assert e <= 2e-2, (n, e)
    for n, c in cos.items():
        assert c >= 0.9998, (n, c)
