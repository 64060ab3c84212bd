"""ctypes binding of libsdpa.so: argument marshalling only.

Every step of the attention forward and backward runs in the HIP library.
This module checks tensor dtypes, shapes, devices and strides, allocates
outputs and the backward workspace with torch (torch owns device memory and
streams), and passes raw device pointers, element strides and the current HIP
stream. There is no CPU path: if the library is missing or a call fails, it
raises.

Tensors are seen as [B, H, L, D] and may be strided views (for example
``x.view(B, L, H, D).transpose(1, 2)`` of a projection output, or slices of a
fused QKV buffer); the D elements of a row must be contiguous. The kernels
read K and V (and Q and dO) with one set of row offsets, so when the two of a
pair have different row strides the binding hands the library contiguous
copies of both (the only copies it ever makes).
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsdpa.so")

SDPA_OK = 0
STATUS = {0: "SDPA_OK", -1: "SDPA_ERR_INVALID_ARG", -2: "SDPA_ERR_UNSUPPORTED", -3: "SDPA_ERR_WORKSPACE",
          -4: "SDPA_ERR_LAUNCH", -5: "SDPA_ERR_SCRATCH_LIMIT"}
DTYPE = {torch.bfloat16: 0, torch.float32: 1, torch.float16: 2}
MASK = {"none": 0, "causal": 1, "causal_window": 2, "window": 3}

EXPORTS = ("sdpa_fwd_lse", "sdpa_fwd_lse_ex", "sdpa_fwd_lse_ws", "sdpa_fwd_workspace_bytes", "sdpa_bwd",
           "sdpa_bwd_ex", "sdpa_bwd_timed", "sdpa_bwd_noalloc", "sdpa_bwd_workspace_bytes",
           "sdpa_bwd_workspace_bytes_ex", "sdpa_status_string", "sdpa_abi_version")

_lib = None


class SdpaStrides(ctypes.Structure):
    """sdpa_strides: element strides of one [B, H, L, D] tensor."""
    _fields_ = [("b", ctypes.c_int64), ("h", ctypes.c_int64), ("l", ctypes.c_int64)]


class SdpaExt(ctypes.Structure):
    """sdpa_ext: strides, sinks / d sinks and the block-sparse cut of the *_ex calls."""
    _fields_ = [("strides", ctypes.POINTER(SdpaStrides)), ("sinks", ctypes.c_void_p), ("dsinks", ctypes.c_void_p),
                ("cut_row", ctypes.c_int32), ("cut_key_lo", ctypes.c_int32), ("cut_key_hi", ctypes.c_int32),
                ("cut_logical", ctypes.c_int32)]


class SdpaError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} returned {STATUS.get(status, status)}: {msg}")
        self.status = status


def load(path: str = LIB_PATH):
    """Load libsdpa.so and declare its signatures. Raises if it has not been built."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m sdpa_backward_amd.build`")
    lib = ctypes.CDLL(path)
    p, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    dims = [i32, i32, i32, i32, i32, i32, i32, i32, i32, f32]  # B Hq group Lq Lk D dtype mask window scale
    ext = ctypes.POINTER(SdpaExt)
    lib.sdpa_fwd_lse.argtypes = [p, p, p, p, p] + dims + [p]
    lib.sdpa_fwd_lse_ex.argtypes = [p, p, p, p, p] + dims + [ext, p]
    lib.sdpa_fwd_lse_ws.argtypes = [p, p, p, p, p, p, sz] + dims + [p]
    lib.sdpa_bwd.argtypes = [p, p, p, p, p, p, p, p, p, p, sz] + dims + [p]
    lib.sdpa_bwd_ex.argtypes = [p, p, p, p, p, p, p, p, p, p, sz] + dims + [ext, p]
    lib.sdpa_bwd_timed.argtypes = [p, p, p, p, p, p, p, p, p, p, sz] + dims + [p, ctypes.POINTER(ctypes.c_void_p)]
    lib.sdpa_bwd_noalloc.argtypes = [p, p, p, p, p, p, p, p, p] + dims + [p]
    for f in ("sdpa_fwd_lse", "sdpa_fwd_lse_ex", "sdpa_fwd_lse_ws", "sdpa_bwd", "sdpa_bwd_ex", "sdpa_bwd_timed",
              "sdpa_bwd_noalloc"):
        getattr(lib, f).restype = ctypes.c_int
    lib.sdpa_fwd_workspace_bytes.argtypes = [i32] * 9
    lib.sdpa_fwd_workspace_bytes.restype = sz
    lib.sdpa_bwd_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.sdpa_bwd_workspace_bytes.restype = sz
    lib.sdpa_bwd_workspace_bytes_ex.argtypes = [i32] * 9
    lib.sdpa_bwd_workspace_bytes_ex.restype = sz
    lib.sdpa_status_string.argtypes = [ctypes.c_int]
    lib.sdpa_status_string.restype = ctypes.c_char_p
    lib.sdpa_abi_version.argtypes = []
    lib.sdpa_abi_version.restype = ctypes.c_int
    if path == LIB_PATH:
        _lib = lib
    return lib


def _check(fn, status):
    if status != SDPA_OK:
        raise SdpaError(fn, status, load().sdpa_status_string(status).decode())


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _strides(*ts):
    arr = (SdpaStrides * len(ts))()
    for a, t in zip(arr, ts):
        a.b, a.h, a.l = t.stride(0), t.stride(1), t.stride(2)
    return arr


def _rows_ok(t):
    """The D elements of a row are contiguous (any stride is fine for a single element)."""
    return t.dim() == 4 and (t.stride(3) == 1 or t.shape[3] <= 1)


def _validate(q, k, v, extra=()):
    """(B, Hq, group, Lq, Lk, D) of q [B, Hq, Lq, D] and k, v [B, Hkv, Lk, D]."""
    for name, t in (("q", q), ("k", k), ("v", v), *extra):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.dtype != q.dtype:
            raise ValueError(f"{name} has dtype {t.dtype}, q has {q.dtype}")
        if not _rows_ok(t):
            raise ValueError(f"{name} must be [B, H, L, D] with contiguous rows (stride 1 along D)")
    if q.dtype not in DTYPE:
        raise ValueError(f"unsupported dtype {q.dtype}")
    B, Hq, Lq, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    Hkv, Lk = k.shape[1], k.shape[2]
    if Hkv == 0 or Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, Hq, Hq // Hkv, Lq, Lk, D


def _same_rows(a, b):
    """a, b with one row stride (the library reads the pair with shared offsets)."""
    if a.stride(2) == b.stride(2):
        return a, b
    return a.contiguous(), b.contiguous()


def _sinks_arg(sinks, q, Hq):
    """Sink logits as a 16-byte-aligned float32 [Hq] device tensor (or None)."""
    if sinks is None:
        return None
    if sinks.device != q.device or sinks.dtype != torch.float32 or sinks.shape != (Hq,):
        raise ValueError(f"sinks must be float32 [Hq={Hq}] on {q.device}")
    if not sinks.is_contiguous() or sinks.data_ptr() % 16:
        sinks = sinks.clone()
    return sinks


def _ext(strides, sinks=None, dsinks=None, cut=None):
    e = SdpaExt()
    e.strides = strides
    e.sinks = None if sinks is None else sinks.data_ptr()
    e.dsinks = None if dsinks is None else dsinks.data_ptr()
    if cut is not None:
        if len(cut) not in (3, 4):
            raise ValueError("cut is (r0, c0, c1) or (r0, c0, c1, logical)")
        e.cut_row, e.cut_key_lo, e.cut_key_hi = (int(x) for x in cut[:3])
        e.cut_logical = int(bool(cut[3])) if len(cut) == 4 else 0
    return ctypes.byref(e), e   # (the struct stays referenced until the call returns)


def _mask_args(mask, window):
    if mask not in MASK:
        raise ValueError(f"mask must be one of {tuple(MASK)}")
    return MASK[mask], int(window) if mask in ("causal_window", "window") else 0


def default_scale(D):
    return 1.0 / math.sqrt(D)


def _out_like(t, out):
    o = torch.empty_like(t) if out is None else out   # keeps t's strides when t is dense
    if o.shape != t.shape or o.dtype != t.dtype or not _rows_ok(o):
        raise ValueError("output buffer must match its input's shape and dtype, rows contiguous")
    return o


def fwd_workspace_bytes(B, Hq, group, Lq, Lk, D, dtype, mask="causal", window=0):
    """Workspace with which the forward splits each query tile's key range (small problems; 0: no split)."""
    m, w = _mask_args(mask, window)
    return int(load().sdpa_fwd_workspace_bytes(B, Hq, group, Lq, Lk, D, DTYPE[dtype], m, w))


def sdpa_fwd_lse(q, k, v, mask="causal", window=0, scale=None, out=None, lse=None, sinks=None, cut=None,
                 workspace=None):
    """O [B,Hq,Lq,D] (q.dtype) and lse [B,Hq,Lq] (float32, natural log).

    k, v are [B, Hkv, Lk, D]; with Lk != Lq the queries are the last Lq key
    positions. mask: "none", "causal", "causal_window" (window keys up to the
    diagonal) or "window" (window - 1 keys either side of it). sinks: optional
    float32 [Hq] logits that join every row's softmax normalizer. cut:
    optional (r0, c0, c1), rows from r0 on do not see keys [c0, c1) (the
    prefix-sharing mask), or (r0, c0, c1, True): besides, rows from r0 on
    place the keys before c0 at their position plus c1 - c0 (the window at
    logical positions). O takes q's strides when q is dense (e.g. a
    [B, L, H, D] layout stays one). workspace: device bytes for the key-range
    split of small problems (contiguous tensors, no sinks, no cut); None
    allocates fwd_workspace_bytes(...) of them, an empty tensor runs unsplit."""
    B, Hq, group, L, Lk, D = _validate(q, k, v)
    sinks = _sinks_arg(sinks, q, Hq)
    k, v = _same_rows(k, v)
    scale = default_scale(D) if scale is None else float(scale)
    m, w = _mask_args(mask, window)
    o = _out_like(q, out)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=q.device) if lse is None else lse
    if lse.shape != (B, Hq, L) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be float32 [B, Hq, L]")
    if sinks is None and cut is None and all(t.is_contiguous() for t in (q, k, v, o)):
        if workspace is None:
            need = fwd_workspace_bytes(B, Hq, group, L, Lk, D, q.dtype, mask, window)
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device) if need > 0 else None
        nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        st = load().sdpa_fwd_lse_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                    _ptr(workspace) if nbytes > 0 else ctypes.c_void_p(0), nbytes, B, Hq, group, L,
                                    Lk, D, DTYPE[q.dtype], m, w, scale, _stream(q.device))
        _check("sdpa_fwd_lse_ws", st)
        return o, lse
    ext, _keep = _ext(_strides(q, k, v, o), sinks, cut=cut)
    st = load().sdpa_fwd_lse_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, group, L, Lk, D,
                                DTYPE[q.dtype], m, w, scale, ext, _stream(q.device))
    _check("sdpa_fwd_lse_ex", st)
    return o, lse


def workspace_bytes(B, Hq, L, D, dtype):
    """Workspace of the backward without the small-problem dK/dV split (the Delta rows)."""
    return int(load().sdpa_bwd_workspace_bytes(B, Hq, L, D, DTYPE[dtype]))


def bwd_workspace_bytes(B, Hq, group, Lq, Lk, D, dtype, mask="causal", window=0):
    """Workspace with which the backward runs its fastest plan for this shape and mask: it may
    also split a small problem's dK/dV pass, or keep dS for a bounded (windowed) band."""
    m, w = _mask_args(mask, window)
    return int(load().sdpa_bwd_workspace_bytes_ex(B, Hq, group, Lq, Lk, D, DTYPE[dtype], m, w))


def sdpa_bwd(q, k, v, o, do, lse, mask="causal", window=0, scale=None, workspace=None, out=None,
             events=None, sinks=None, cut=None):
    """dQ, dK, dV for the forward sdpa_fwd_lse(q, k, v, mask, window, scale) returned (o, lse);
    with ``sinks`` (the forward's), also d sinks: (dq, dk, dv, dsinks).

    Gradients take the strides of q, k, v when those are dense. ``events``:
    optional four raw hipEvent_t handles recorded before the first kernel and
    after each of the three passes (sdpa_bwd_timed; contiguous tensors, no
    sinks, no cut)."""
    B, Hq, group, L, Lk, D = _validate(q, k, v, (("o", o), ("do", do)))
    sinks = _sinks_arg(sinks, q, Hq)
    dsinks = None if sinks is None else torch.empty(Hq, dtype=torch.float32, device=q.device)
    if o.shape != q.shape or do.shape != q.shape:
        raise ValueError("o and do must match q")
    if lse.shape != (B, Hq, L) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be float32 [B, Hq, L]")
    scale = default_scale(D) if scale is None else float(scale)
    m, w = _mask_args(mask, window)
    need = bwd_workspace_bytes(B, Hq, group, L, Lk, D, q.dtype, mask, window)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if out is None:
        dq, dk, dv = _out_like(q, None), _out_like(k, None), _out_like(v, None)
    else:
        dq, dk, dv = (_out_like(t, x) for t, x in zip((q, k, v), out))
    k, v = _same_rows(k, v)
    q, do = _same_rows(q, do)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
            _ptr(workspace), workspace.numel(), B, Hq, group, L, Lk, D, DTYPE[q.dtype], m, w, scale)
    if events is None:
        ext, _keep = _ext(_strides(q, k, v, o, do, dq, dk, dv), sinks, dsinks, cut)
        _check("sdpa_bwd_ex", load().sdpa_bwd_ex(*args, ext, _stream(q.device)))
    else:
        if sinks is not None or cut is not None or not all(t.is_contiguous() for t in (q, k, v, o, do, dq, dk, dv)):
            raise ValueError("the timed backward takes contiguous tensors, no sinks and no cut")
        if len(events) != 4:
            raise ValueError("events: four hipEvent_t handles")
        arr = (ctypes.c_void_p * 4)(*events)
        _check("sdpa_bwd_timed", load().sdpa_bwd_timed(*args, _stream(q.device), arr))
    return (dq, dk, dv) if sinks is None else (dq, dk, dv, dsinks)


def sdpa_bwd_noalloc(q, k, v, o, do, lse, mask="causal", window=0, scale=None, out=None):
    """sdpa_bwd through the allocation-free entry point (the library's fixed per-GPU scratch, no
    workspace): contiguous tensors; ``out`` = (dq, dk, dv) buffers, or None to allocate them here."""
    B, Hq, group, L, Lk, D = _validate(q, k, v, (("o", o), ("do", do)))
    if not all(t.is_contiguous() for t in (q, k, v, o, do, lse)):
        raise ValueError("sdpa_bwd_noalloc takes contiguous tensors")
    scale = default_scale(D) if scale is None else float(scale)
    m, w = _mask_args(mask, window)
    dq, dk, dv = (torch.empty_like(t) for t in (q, k, v)) if out is None else out
    if not all(x.is_contiguous() and x.shape == t.shape and x.dtype == t.dtype for x, t in zip((dq, dk, dv), (q, k, v))):
        raise ValueError("output buffers must be contiguous and match q, k, v")
    st = load().sdpa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk),
                                 _ptr(dv), B, Hq, group, L, Lk, D, DTYPE[q.dtype], m, w, scale, _stream(q.device))
    _check("sdpa_bwd_noalloc", st)
    return dq, dk, dv
