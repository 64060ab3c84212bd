"""CPU-side checks of the C ABI: the library loads, exports every function
include/sdpa.h declares, and every argument error is reported by status code
before anything is launched (so no GPU is needed)."""
import ctypes
import os
import re

import pytest

from sdpa_backward_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdpa.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3
BF16, F32, F16 = 0, 1, 2
NONE, CAUSAL, WINDOW, TWO_SIDED = 0, 1, 2, 3
FAKE = 0x10000  # aligned, never dereferenced: validation fails or returns before any launch


def header_functions(path=HEADER):
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sdpa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from sdpa_backward_amd import build
        build.build()
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert set(names) == set(_lib.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_probe_library_exports_its_header():
    from sdpa_backward_amd import build
    path = build.PROBE_LIB
    if not os.path.exists(path):
        build.build()
    probe = ctypes.CDLL(path)
    names = header_functions(os.path.join(ROOT, "include", "sdpa_probe.h"))
    assert names == ["sdpa_probe_mfma_bf16", "sdpa_probe_mfma_bf16_flop"], names
    for n in names:
        assert hasattr(probe, n), n
    probe.sdpa_probe_mfma_bf16_flop.restype = ctypes.c_double
    probe.sdpa_probe_mfma_bf16_flop.argtypes = [ctypes.c_int32, ctypes.c_int32]
    assert probe.sdpa_probe_mfma_bf16_flop(10, 3) == 10 * 4 * 8 * 3 * 32768
    probe.sdpa_probe_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    assert probe.sdpa_probe_mfma_bf16(None, 1, 1, None) == -1   # rejected before any launch
    assert probe.sdpa_probe_mfma_bf16(ctypes.c_void_p(FAKE), 0, 1, None) == -1


def test_version_and_status_strings(lib):
    assert lib.sdpa_abi_version() == 500
    for code in (OK, INVALID, UNSUPPORTED, WORKSPACE, -4, 99):
        assert isinstance(lib.sdpa_status_string(code), bytes)
    assert lib.sdpa_status_string(OK) == b"ok"


def test_workspace_is_linear_in_L(lib):
    ws = [lib.sdpa_bwd_workspace_bytes(1, 32, L, 256, BF16) for L in (4096, 8192, 16384, 32768)]
    assert ws[0] > 0
    for a, b in zip(ws, ws[1:]):
        assert abs(b - 2 * a) <= 512   # alignment slack only
    # Delta only: one float per query row
    assert lib.sdpa_bwd_workspace_bytes(1, 32, 16384, 256, BF16) == 32 * 16384 * 4
    assert lib.sdpa_bwd_workspace_bytes(1, 2, 128, 64, F32) == 1024
    assert lib.sdpa_bwd_workspace_bytes(0, 32, 16384, 256, BF16) == 0
    assert lib.sdpa_bwd_workspace_bytes(1, 32, 16384, 100, BF16) == 0   # unsupported D
    assert lib.sdpa_bwd_workspace_bytes(1, 32, 16384, 256, 7) == 0       # unknown dtype
    assert lib.sdpa_bwd_workspace_bytes(1, 32, 16384, 256, F16) == 32 * 16384 * 4


def fwd(lib, B=1, Hq=4, group=2, Lq=64, Lk=64, D=64, dtype=BF16, mask=CAUSAL, window=0, scale=0.125,
        ptrs=(FAKE,) * 5):
    """sdpa_fwd_lse; pointer order q, k, v, o, lse."""
    return lib.sdpa_fwd_lse(*[ctypes.c_void_p(p) for p in ptrs], B, Hq, group, Lq, Lk, D, dtype, mask, window,
                            scale, None)


def bwd(lib, B=1, Hq=4, group=2, Lq=64, Lk=64, D=64, dtype=BF16, mask=CAUSAL, window=0, scale=0.125,
        ptrs=(FAKE,) * 9, ws=FAKE, ws_bytes=1 << 40):
    """sdpa_bwd; pointer order q, k, v, o, dO, lse, dq, dk, dv."""
    return lib.sdpa_bwd(*[ctypes.c_void_p(p) for p in ptrs], ctypes.c_void_p(ws), ws_bytes, B, Hq, group, Lq,
                        Lk, D, dtype, mask, window, scale, None)


@pytest.mark.parametrize("kw,expect", [
    ({"dtype": 3}, INVALID),
    ({"dtype": -1}, INVALID),
    ({"mask": 4}, INVALID),
    ({"mask": -1}, INVALID),
    ({"B": -1}, INVALID),
    ({"Lq": -5}, INVALID),
    ({"Lk": -5}, INVALID),
    ({"Hq": -4}, INVALID),
    ({"D": 0}, INVALID),
    ({"group": 0}, INVALID),
    ({"Hq": 6, "group": 4}, INVALID),
    ({"mask": WINDOW, "window": 0}, INVALID),
    ({"mask": TWO_SIDED, "window": 0}, INVALID),
    ({"mask": TWO_SIDED, "window": -3}, INVALID),
    ({"scale": 0.0}, INVALID),
    ({"scale": -1.0}, INVALID),
    ({"scale": float("inf")}, INVALID),
    ({"scale": float("nan")}, INVALID),
    ({"D": 96}, UNSUPPORTED),
    ({"D": 1024}, UNSUPPORTED),
    ({"dtype": F32, "D": 32}, UNSUPPORTED),
    ({"dtype": F16, "D": 96}, UNSUPPORTED),
    ({"Hq": 70000, "group": 1}, UNSUPPORTED),
    ({"Lq": 1 << 29, "Lk": (1 << 29) + 1}, UNSUPPORTED),   # row / key indices plus offsets must fit int32
])
def test_argument_errors(lib, kw, expect):
    assert fwd(lib, **kw) == expect
    assert bwd(lib, **kw) == expect


def test_null_and_misaligned_pointers(lib):
    for n in range(5):
        p = [FAKE] * 5
        p[n] = 0
        assert fwd(lib, ptrs=p) == INVALID
        p[n] = FAKE + 2
        assert fwd(lib, ptrs=p) == INVALID
    for n in range(9):
        p = [FAKE] * 9
        p[n] = 0
        assert bwd(lib, ptrs=p) == INVALID


def test_workspace_errors(lib):
    need = lib.sdpa_bwd_workspace_bytes(1, 4, 64, 64, BF16)
    assert bwd(lib, ws=0) == WORKSPACE
    assert bwd(lib, ws_bytes=need - 1) == WORKSPACE
    assert bwd(lib, ws=FAKE + 8) == WORKSPACE


def test_empty_problems_launch_nothing(lib):
    for kw in ({"B": 0}, {"Lq": 0, "Lk": 0}, {"Hq": 0}):
        assert fwd(lib, ptrs=(0,) * 5, **kw) == OK
        assert bwd(lib, ptrs=(0,) * 9, ws=0, ws_bytes=0, **kw) == OK
    # no query rows: the forward has nothing to write, whatever the keys
    assert fwd(lib, Lq=0, Lk=64, ptrs=(0,) * 5) == OK


def test_pointers_of_empty_tensors_are_not_checked(lib):
    # no rows but keys: the backward still writes dK, dV (zeros), so those and
    # K, V must be valid while Q, O, dO, lse, dQ may be null; a null one of
    # the four is refused before any launch
    for n in (1, 2, 7, 8):
        p = [0] * 9
        for m in (1, 2, 7, 8):
            p[m] = FAKE
        p[n] = 0
        assert bwd(lib, Lq=0, Lk=64, ptrs=p, ws=0, ws_bytes=0) == INVALID
    # keys but no rows in the forward: returns before looking at any pointer
    assert fwd(lib, Lq=0, Lk=64, ptrs=(0, FAKE + 2, 0, 0, 0)) == OK
    # rows but no keys: Q, O, lse (forward) must be valid
    for n in (0, 3, 4):
        p = [FAKE, 0, 0, FAKE, FAKE]
        p[n] = 0
        assert fwd(lib, Lk=0, ptrs=p) == INVALID
    # ... and Q, O, dO, lse, dQ (backward), with the workspace
    for n in (0, 3, 4, 5, 6):
        p = [FAKE, 0, 0, FAKE, FAKE, FAKE, FAKE, 0, 0]
        p[n] = 0
        assert bwd(lib, Lk=0, ptrs=p) == INVALID
    assert bwd(lib, Lk=0, ptrs=[FAKE, 0, 0, FAKE, FAKE, FAKE, FAKE, 0, 0], ws=0) == WORKSPACE


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        _lib.sdpa_fwd_lse(q, q[:, :1].contiguous(), q[:, :1].contiguous())


def _st(*triples):
    arr = (_lib.SdpaStrides * len(triples))()
    for a, (b, h, l) in zip(arr, triples):
        a.b, a.h, a.l = b, h, l
    return arr


def _x(strides=None, sinks=None, dsinks=None, cut=(0, 0, 0), logical=0):
    e = _lib.SdpaExt()
    e.strides = strides
    e.sinks, e.dsinks = sinks, dsinks
    e.cut_row, e.cut_key_lo, e.cut_key_hi = cut
    e.cut_logical = logical
    return ctypes.byref(e), e


def test_extension_errors(lib):
    # q [1, 4, 64, 64], k/v [1, 2, 64, 64]; a dense [B, L, H, D] layout is valid
    # (validated, then rejected here only by a null pointer so nothing launches)
    B, Hq, Hkv, L, D = 1, 4, 2, 64, 64
    blhd_q, blhd_kv = (L * Hq * D, D, Hq * D), (L * Hkv * D, D, Hkv * D)
    p0 = [FAKE] * 5
    p0[0] = 0
    args = (B, Hq, 2, L, L, D, BF16, CAUSAL, 0, 0.125)
    good, _k1 = _x(_st(blhd_q, blhd_kv, blhd_kv, blhd_q))
    assert lib.sdpa_fwd_lse_ex(*[ctypes.c_void_p(x) for x in p0], *args, good, None) == INVALID
    p = [ctypes.c_void_p(FAKE)] * 5
    for bad in (_st(blhd_q, blhd_kv, blhd_kv, (0, D, D - 8)),          # row stride below D
                _st(blhd_q, blhd_kv, blhd_kv, (0, D, Hq * D + 4)),     # not a 16-byte multiple
                _st(blhd_q, (-64, D, Hkv * D), blhd_kv, blhd_q),       # negative
                _st(blhd_q, blhd_kv, blhd_kv, (0, D, 1 << 23))):       # row stride too large
        x, _k = _x(bad)
        assert lib.sdpa_fwd_lse_ex(*p, *args, x, None) == INVALID
    # K and V with different row strides: not built
    x, _k = _x(_st(blhd_q, blhd_kv, (0, L * D, D), blhd_q))
    assert lib.sdpa_fwd_lse_ex(*p, *args, x, None) == UNSUPPORTED
    # backward: Q and dO must share their row stride too
    pb = [ctypes.c_void_p(FAKE)] * 9
    ws = (ctypes.c_void_p(FAKE), 1 << 40)
    x, _k = _x(_st(blhd_q, blhd_kv, blhd_kv, blhd_q, (0, L * D, D), blhd_q, blhd_kv, blhd_kv))
    assert lib.sdpa_bwd_ex(*pb, *ws, *args, x, None) == UNSUPPORTED
    # sinks and their gradient come together
    for s_, d_ in ((FAKE, None), (None, FAKE)):
        x, _k = _x(sinks=s_, dsinks=d_)
        assert lib.sdpa_bwd_ex(*pb, *ws, *args, x, None) == INVALID
    # misaligned sinks
    x, _k = _x(sinks=FAKE + 4)
    assert lib.sdpa_fwd_lse_ex(*[ctypes.c_void_p(v) for v in p0], *args, x, None) == INVALID
    # a cut outside the rows / keys
    for cut in ((-1, 0, 5), (10, 5, 3), (10, 0, L + 1), (L + 1, 0, 5), (0, -2, 5)):
        x, _k = _x(cut=cut)
        assert lib.sdpa_fwd_lse_ex(*p, *args, x, None) == INVALID, cut
        assert lib.sdpa_bwd_ex(*pb, *ws, *args, x, None) == INVALID, cut
    # the logical-position flag is 0 or 1
    for lg in (2, -1):
        x, _k = _x(cut=(40, 10, 40), logical=lg)
        assert lib.sdpa_fwd_lse_ex(*p, *args, x, None) == INVALID, lg
        assert lib.sdpa_bwd_ex(*pb, *ws, *args, x, None) == INVALID, lg
    # fp32 rows need 16-byte multiples too: 4 elements
    args32 = (B, Hq, 2, L, L, D, F32, CAUSAL, 0, 0.125)
    x, _k = _x(_st(blhd_q, blhd_kv, blhd_kv, (0, D, Hq * D + 2)))
    assert lib.sdpa_fwd_lse_ex(*p, *args32, x, None) == INVALID


def test_split_workspace_sizes(lib):
    ex9 = lib.sdpa_bwd_workspace_bytes_ex
    ex9.argtypes = [ctypes.c_int32] * 9
    ex9.restype = ctypes.c_size_t
    ex = lambda *a: ex9(*a, CAUSAL, 0)
    delta = lambda B, Hq, Lq: -(-(B * Hq * Lq * 4) // 256) * 256
    # causal L=2048 D=256 8/4: 16 key blocks x 4 kv heads = 64 workgroups -> 4 shares of fp32 dK, dV
    assert ex(1, 8, 2, 2048, 2048, 256, BF16) == delta(1, 8, 2048) + 2 * 4 * 4 * 2048 * 256 * 4
    assert ex(1, 8, 2, 2048, 2048, 256, F16) == ex(1, 8, 2, 2048, 2048, 256, BF16)
    # 8 blocks: capped at 8 shares; 128 blocks: 2 shares; 256 blocks and more: none
    assert ex(1, 2, 2, 500, 1000, 64, BF16) == delta(1, 2, 500) + 2 * 8 * 1 * 1000 * 64 * 4
    assert ex(1, 4, 1, 4096, 4096, 128, BF16) == delta(1, 4, 4096) + 2 * 2 * 1 * 4 * 4096 * 128 * 4
    assert ex(2, 8, 1, 4096, 4096, 128, BF16) == delta(2, 8, 4096)     # 512 blocks
    assert ex(1, 32, 2, 16384, 16384, 256, BF16) == lib.sdpa_bwd_workspace_bytes(1, 32, 16384, 256, BF16)
    # fp32 and D = 512 never split; empty and invalid shapes need nothing
    assert ex(1, 2, 2, 128, 128, 64, F32) == lib.sdpa_bwd_workspace_bytes(1, 2, 128, 64, F32)
    assert ex(1, 16, 4, 2048, 2048, 512, BF16) == lib.sdpa_bwd_workspace_bytes(1, 16, 2048, 512, BF16)
    assert ex(1, 8, 2, 2048, 0, 256, BF16) == delta(1, 8, 2048)
    assert ex(0, 8, 2, 2048, 2048, 256, BF16) == 0
    assert ex(1, 8, 3, 2048, 2048, 256, BF16) == 0


def test_forward_split_workspace_sizes(lib):
    fb = lib.sdpa_fwd_workspace_bytes
    fb.argtypes = [ctypes.c_int32] * 9
    fb.restype = ctypes.c_size_t
    ex = lib.sdpa_bwd_workspace_bytes_ex
    ex.argtypes = [ctypes.c_int32] * 9
    ex.restype = ctypes.c_size_t
    delta = lambda B, Hq, Lq: -(-(B * Hq * Lq * 4) // 256) * 256
    # causal L = 2048, D = 256, 8 q-heads: 16 query tiles of 128 rows x 8 = 128
    # workgroups -> 2 key-range shares of fp32 (O row, used max, row sum)
    assert fb(1, 8, 2, 2048, 2048, 256, BF16, CAUSAL, 0) == 2 * 8 * 2048 * (256 + 2) * 4
    assert fb(1, 8, 2, 2048, 2048, 256, F16, CAUSAL, 0) == 2 * 8 * 2048 * (256 + 2) * 4
    # at most 64 workgroups (D = 512 tiles hold 64 rows: 16 x 2 = 32): 4 shares
    assert fb(1, 2, 1, 1024, 1024, 512, BF16, CAUSAL, 0) == 4 * 2 * 1024 * (512 + 2) * 4
    # the longest query tile needs two key tiles per share: window 64 spans
    # 191 keys (4 tiles of 64) -> 2 shares; window 1 spans 128 keys (3) -> none
    assert fb(1, 8, 2, 2048, 2048, 256, BF16, WINDOW, 64) == 2 * 8 * 2048 * (256 + 2) * 4
    assert fb(1, 8, 2, 2048, 2048, 256, BF16, WINDOW, 1) == 0
    # grids that fill the GPU, fp32, no keys, invalid shapes: none
    assert fb(1, 32, 2, 16384, 16384, 256, BF16, WINDOW, 1024) == 0
    assert fb(2, 8, 1, 2048, 2048, 256, BF16, CAUSAL, 0) == 0   # 256 workgroups
    assert fb(1, 9, 1, 2048, 2048, 256, BF16, CAUSAL, 0) == 0   # 144: two shares would exceed 256
    assert fb(1, 2, 2, 128, 128, 64, F32, CAUSAL, 0) == 0
    assert fb(1, 8, 2, 2048, 0, 256, BF16, CAUSAL, 0) == 0
    assert fb(1, 8, 3, 2048, 2048, 256, BF16, CAUSAL, 0) == 0
    # the backward's dQ pass splits the same way (fp32 dQ rows only); its
    # partials and the dK/dV shares share memory, so the larger one counts
    assert ex(1, 2, 1, 1024, 1024, 512, BF16, CAUSAL, 0) == delta(1, 2, 1024) + 4 * 2 * 1024 * 512 * 4
    assert ex(1, 8, 2, 2048, 2048, 256, BF16, CAUSAL, 0) == delta(1, 8, 2048) + 2 * 4 * 4 * 2048 * 256 * 4


def test_forward_workspace_errors(lib):
    fws = lib.sdpa_fwd_lse_ws
    fws.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_size_t] + [ctypes.c_int32] * 9 + [ctypes.c_float,
                                                                                          ctypes.c_void_p]
    fws.restype = ctypes.c_int
    p = [ctypes.c_void_p(FAKE)] * 5
    dims = (1, 8, 2, 2048, 2048, 256, BF16, CAUSAL, 0, 0.0625)
    # a workspace of nonzero size must be non-null and 16-byte aligned; the
    # shape is checked first
    assert fws(*p, None, 1024, *dims, None) == WORKSPACE
    assert fws(*p, ctypes.c_void_p(FAKE + 8), 1024, *dims, None) == WORKSPACE
    assert fws(*p, None, 1024, 1, 8, 2, 2048, 2048, 256, 3, CAUSAL, 0, 0.0625, None) == INVALID
    assert fws(*[ctypes.c_void_p(0)] * 5, None, 0, 0, 8, 2, 2048, 2048, 256, BF16, CAUSAL, 0, 0.0625, None) == OK


def test_band_workspace_sizes(lib):
    ex = lib.sdpa_bwd_workspace_bytes_ex
    ex.argtypes = [ctypes.c_int32] * 9
    ex.restype = ctypes.c_size_t
    delta = lambda B, Hq, Lq: -(-(B * Hq * Lq * 4) // 256) * 256
    tile = 64 * 128 * 2  # one band tile: 64 keys x 128 rows, 16-bit
    # window 1024 at D = 256 (16-key dK/dV kernel): a block of 128 rows sees
    # keys i0 - 1023 .. i0 + 127, i.e. 18 key tiles of 64, for each of
    # 32 heads x 128 row blocks
    assert ex(1, 32, 2, 16384, 16384, 256, BF16, WINDOW, 1024) == delta(1, 32, 16384) + 32 * 128 * 18 * tile
    assert ex(1, 32, 2, 16384, 16384, 256, F16, WINDOW, 1024) == delta(1, 32, 16384) + 32 * 128 * 18 * tile
    # ragged length: 239 row blocks
    assert ex(1, 32, 2, 30553, 30553, 256, BF16, WINDOW, 1024) == delta(1, 32, 30553) + 32 * 239 * 18 * tile
    # linear in L at a fixed window
    sizes = [ex(1, 32, 2, L, L, 256, BF16, WINDOW, 1024) for L in (4096, 8192, 16384, 32768)]
    assert [b / a for a, b in zip(sizes, sizes[1:])] == [2.0, 2.0, 2.0]
    # window 1: keys i0 .. i0 + 127, 2 tiles
    assert ex(1, 32, 2, 16384, 16384, 256, BF16, WINDOW, 1) == delta(1, 32, 16384) + 32 * 128 * 2 * tile
    # the two-sided window 1024 spans keys i0 - 1023 .. i0 + 127 + 1023: 34 tiles
    assert ex(1, 32, 2, 16384, 16384, 256, BF16, TWO_SIDED, 1024) == delta(1, 32, 16384) + 32 * 128 * 34 * tile
    # bands wider than 9 D = 2304 keys keep no dS: the two-sided window 1100
    # (38 tiles), causal and no mask at long lengths; and only D = 256 keeps it
    assert ex(1, 32, 2, 16384, 16384, 256, BF16, TWO_SIDED, 1100) == delta(1, 32, 16384)
    assert ex(1, 32, 2, 16384, 16384, 256, BF16, WINDOW, 2150) == delta(1, 32, 16384) + 32 * 128 * 36 * tile
    assert ex(1, 32, 2, 16384, 16384, 256, BF16, WINDOW, 2200) == delta(1, 32, 16384)
    assert ex(1, 32, 2, 16384, 16384, 256, BF16, CAUSAL, 0) == delta(1, 32, 16384)
    assert ex(1, 32, 2, 4096, 4096, 256, BF16, NONE, 0) == delta(1, 32, 4096)
    assert ex(1, 32, 2, 16384, 16384, 128, BF16, WINDOW, 1024) == delta(1, 32, 16384)
    assert ex(1, 16, 4, 16384, 16384, 512, BF16, WINDOW, 1024) == delta(1, 16, 16384)
    # short sequences: the band is capped by the key tiles that exist, and the
    # dS buffer only comes with the 16-key kernel (at least 256 key blocks of 128)
    assert ex(2, 16, 1, 1024, 1024, 256, BF16, CAUSAL, 0) == delta(2, 16, 1024) + 2 * 16 * 8 * 16 * tile
    assert ex(1, 8, 2, 2048, 2048, 256, BF16, WINDOW, 100) == delta(1, 8, 2048) + 2 * 4 * 4 * 2048 * 256 * 4
    # the band of one kv head's q-heads must stay under 2 GiB (the dK/dV pass
    # addresses it with 32-bit offsets): group 32 at L = 65536 needs 4.8 GB
    assert ex(1, 64, 32, 65536, 65536, 256, BF16, WINDOW, 1024) == delta(1, 64, 65536)
    assert ex(1, 64, 2, 65536, 65536, 256, BF16, WINDOW, 1024) == delta(1, 64, 65536) + 64 * 512 * 18 * tile


def test_ext_layout_matches_header(tmp_path):
    # the ctypes mirror of sdpa_ext against the C compiler's layout of the header
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "layout.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "sdpa.h"\n'
                   'int main(void) { printf("%zu %zu %zu %zu %zu\\n", sizeof(sdpa_ext), offsetof(sdpa_ext, sinks), '
                   'offsetof(sdpa_ext, dsinks), offsetof(sdpa_ext, cut_row), offsetof(sdpa_ext, cut_logical)); '
                   'return 0; }\n')
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    exe = tmp_path / "layout"
    r = subprocess.run([gcc, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(root, "include"), "-I", "/opt/rocm/include",
                        str(src), "-o", str(exe)], capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("header does not compile on the host: " + r.stderr[-300:])
    got = tuple(int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split())
    E = _lib.SdpaExt
    assert got == (ctypes.sizeof(E), E.sinks.offset, E.dsinks.offset, E.cut_row.offset, E.cut_logical.offset)


def noalloc(lib, B=1, Hq=4, group=2, Lq=64, Lk=64, D=64, dtype=BF16, mask=CAUSAL, window=0, scale=0.125,
            ptrs=(FAKE,) * 9):
    """sdpa_bwd_noalloc; pointer order q, k, v, o, dO, lse, dq, dk, dv."""
    return lib.sdpa_bwd_noalloc(*[ctypes.c_void_p(p) for p in ptrs], B, Hq, group, Lq, Lk, D, dtype, mask, window,
                                scale, None)


def test_noalloc_rejects_before_touching_the_device(lib):
    # argument errors, and a problem whose Delta rows (4 B Hq Lq bytes) exceed the
    # fixed 64 MiB scratch, are refused before the first device call (no GPU here)
    assert noalloc(lib, dtype=7) == INVALID
    assert noalloc(lib, Hq=6, group=4) == INVALID
    assert noalloc(lib, D=96) == UNSUPPORTED
    SCRATCH_LIMIT = -5
    assert 4 * 1 * 64 * 262145 > 64 << 20
    assert noalloc(lib, B=1, Hq=64, group=2, Lq=262145, Lk=262145) == SCRATCH_LIMIT
    assert lib.sdpa_status_string(SCRATCH_LIMIT) != lib.sdpa_status_string(-99)
