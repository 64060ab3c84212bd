// C ABI of the attention library: argument validation, workspace sizing and
// dispatch to the gfx950 kernels. Nothing here allocates device memory.
//
// Unsupported combinations are refused with a status code rather than run on
// another algorithm; the silent fall back to a materialised score matrix is
// the failure the pages measure (page "Lab 028 lab detail: Off NVIDIA, you fix
// the platform yourself", section "2026-10-21", starting point and upstream
// state, where an unsupported window is refused with "NYI").
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "sdpa.h"
#include "common.h"

namespace sdpa {
enum { QS_FWD = 0, QS_DQ = 1 };
template <int D, int MODE, typename E>
hipError_t launch_qs(const void* q, const void* k, const void* v, const void* o, const void* dO, float* lse,
                     float* delta, void* out, const float* sinks, int B, int Hq, int group, int Lq, int Lk, int dlo,
                     int dhi, Cut cut, float scale, const AllStrides& st, int nseg, float* part, hipStream_t stream);
template <int D>
int qs_split_shares(int B, int Hq, int Lq, int Lk, int dlo, int dhi, bool dense);
template <int D, typename E>
hipError_t launch_kv(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                     const float* delta, void* dk, void* dv, int B, int Hq, int group, int Lq, int Lk, int dlo,
                     int dhi, Cut cut, float scale, const AllStrides& st, float* part, int nseg,
                     hipStream_t stream);
template <int D>
int kv_split_shares(int B, int Hq, int group, int Lq, int Lk, bool dense);
template <int D, typename E>
hipError_t launch_kv16(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                       const float* delta, void* dk, void* dv, int B, int Hq, int group, int Lq, int Lk, int dlo,
                       int dhi, Cut cut, float scale, const AllStrides& st, void* dst, int nqb, int nkb,
                       hipStream_t stream);
template <int D, typename E>
hipError_t launch_delta(const void* o, const void* dO, float* delta, long long rows, hipStream_t stream);
template <int D, typename E>
hipError_t launch_dsq(const void* dst, const void* k, void* dq, int B, int Hq, int group, int Lq, int Lk, int dlo,
                      int dhi, int nqb, int nkb, float scale, hipStream_t stream);
template <int D>
hipError_t launch_fwd_f32(const void*, const void*, const void*, void*, float*, int, int, const float*, int, int,
                          int, int, int, Cut, float, const AllStrides&, hipStream_t);
hipError_t launch_dsinks(const float* lse, const float* delta, const float* sinks, float* dsinks, int B, int Hq,
                         int Lq, hipStream_t stream);
template <int D>
hipError_t launch_bwd_f32(const void*, const void*, const void*, const void*, const void*, const float*,
                          void*, void*, void*, float*, int, int, int, int, int, int, int, Cut, float,
                          const AllStrides&, hipStream_t, const hipEvent_t*);

// Optional timing events of a backward: [0] before its first kernel, [1] after
// the first pass, [2] after the dK/dV pass, [3] after the last pass.
hipError_t mark(const hipEvent_t* ev, int i, hipStream_t stream) {
  return ev != nullptr ? hipEventRecord(ev[i], stream) : hipSuccess;
}

// How a 16-bit backward runs (chosen by the host from the shape, the layout
// and the workspace given).
struct BwdPlan {
  bool wide;     // dense, and the key blocks alone fill the GPU: 16-key dK/dV waves at D = 256
  float* part;   // fp32 dK/dV shares of the small-problem split (nseg > 1), or null
  int nseg;
  void* band;    // dS band buffer (bounded band, D = 256, wide), or null
  int nqb, nkb;  // its row blocks and key tiles per block
  float* qpart;  // fp32 dQ partials of the dQ pass's key-range split (qseg > 1), or null
  int qseg;
};

// 16-bit backward.
//   band buffer: Delta pass, dK/dV pass that also writes dS^T for the band,
//                dQ = scale dS K from that buffer (no score recomputed);
//   otherwise:   dQ pass (recomputes S and dP, also writes Delta; each query
//                tile's key range split into qseg shares when qseg > 1), then
//                the dK/dV pass (split into nseg shares summed into part when
//                nseg > 1; part may reuse the dQ partials' memory, which the
//                dQ pass's combine has read by then).
template <int D, typename E>
hipError_t launch_bwd_mfma(const void* q, const void* k, const void* v, const void* o, const void* dO,
                           const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int Hq,
                           int group, int Lq, int Lk, int dlo, int dhi, Cut cut, float scale, const AllStrides& st,
                           const BwdPlan& plan, hipStream_t stream, const hipEvent_t* ev) {
  hipError_t e;
  if ((e = mark(ev, 0, stream)) != hipSuccess) return e;
  if constexpr (D == 256) {
    if (plan.band != nullptr) {
      if ((e = launch_delta<D, E>(o, dO, delta, (long long)B * Hq * Lq, stream)) != hipSuccess) return e;
      if ((e = mark(ev, 1, stream)) != hipSuccess) return e;
      e = launch_kv16<D, E>(q, k, v, dO, lse, delta, dk, dv, B, Hq, group, Lq, Lk, dlo, dhi, cut, scale, st,
                            plan.band, plan.nqb, plan.nkb, stream);
      if (e != hipSuccess) return e;
      if ((e = mark(ev, 2, stream)) != hipSuccess) return e;
      e = launch_dsq<D, E>(plan.band, k, dq, B, Hq, group, Lq, Lk, dlo, dhi, plan.nqb, plan.nkb, scale, stream);
      if (e != hipSuccess) return e;
      return mark(ev, 3, stream);
    }
  }
  e = launch_qs<D, QS_DQ, E>(q, k, v, o, dO, const_cast<float*>(lse), delta, dq, nullptr, B, Hq, group, Lq, Lk, dlo,
                             dhi, cut, scale, st, plan.qseg, plan.qpart, stream);
  if (e != hipSuccess) return e;
  if ((e = mark(ev, 1, stream)) != hipSuccess) return e;
  // 16-key waves (v_mfma_f32_16x16x32): at D = 512 always (32-key waves would
  // not fit their accumulators in registers there), at D = 256 for dense calls
  // whose key blocks fill the GPU (two workgroups per CU; measured faster than
  // the 32-key kernel there); otherwise 32-key waves. The choice depends on
  // the shape and layout only, never on the workspace given.
  if constexpr (D == 512) {
    e = launch_kv16<D, E>(q, k, v, dO, lse, delta, dk, dv, B, Hq, group, Lq, Lk, dlo, dhi, cut, scale, st, nullptr,
                          0, 0, stream);
  } else {
    if (D == 256 && plan.wide)
      e = launch_kv16<256, E>(q, k, v, dO, lse, delta, dk, dv, B, Hq, group, Lq, Lk, dlo, dhi, cut, scale, st,
                              nullptr, 0, 0, stream);
    else
      e = launch_kv<D, E>(q, k, v, dO, lse, delta, dk, dv, B, Hq, group, Lq, Lk, dlo, dhi, cut, scale, st,
                          plan.part, plan.nseg, stream);
  }
  if (e != hipSuccess) return e;
  if ((e = mark(ev, 2, stream)) != hipSuccess) return e;
  return mark(ev, 3, stream);
}
}  // namespace sdpa

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Shape {
  int B, Hq, group, Lq, Lk, D, dtype, mask, window;
  float scale;
  bool no_rows() const { return B == 0 || Hq == 0 || Lq == 0; }
  bool no_keys() const { return B == 0 || Hq == 0 || Lk == 0; }
  // The mask as a band dlo <= j - i <= dhi (query rows are the last Lq of the
  // Lk key positions, so the diagonal sits at j - i = Lk - Lq), clamped to the
  // differences that occur, [-(Lq - 1), Lk - 1]. The window counts the
  // diagonal: causal window [off - W + 1, off]; a window without the causal
  // mask extends the same distance past the diagonal, [off - W + 1, off + W - 1]
  // (page "Lab 028 lab detail: Off NVIDIA, you fix the platform yourself",
  // section "What I changed, in plain terms", items 3-5).
  void band(int& dlo, int& dhi) const {
    const int64_t off = (int64_t)Lk - Lq, lo_min = -((int64_t)Lq - 1), hi_max = (int64_t)Lk - 1;
    int64_t lo = lo_min, hi = hi_max;
    if (mask == SDPA_MASK_CAUSAL) hi = off;
    if (mask == SDPA_MASK_CAUSAL_WINDOW) lo = off - window + 1, hi = off;
    if (mask == SDPA_MASK_WINDOW) lo = off - window + 1, hi = off + window - 1;
    lo = std::max(lo, lo_min);
    hi = std::min(hi, hi_max);
    if (lo > hi) lo = hi_max, hi = lo_min - 1;  // empty band (the kernels see empty row and key ranges)
    dlo = (int)std::max<int64_t>(std::min<int64_t>(lo, INT32_MAX), INT32_MIN);
    dhi = (int)std::max<int64_t>(std::min<int64_t>(hi, INT32_MAX), INT32_MIN);
  }
};

bool d_supported(int dtype, int D) {
  return D == 64 || D == 128 || D == 256 || D == 512;
}

bool windowed(int mask) { return mask == SDPA_MASK_CAUSAL_WINDOW || mask == SDPA_MASK_WINDOW; }

// Shape checks shared by both entry points (pointers are checked by the caller).
int check_shape(const Shape& s) {
  if (s.dtype != SDPA_BF16 && s.dtype != SDPA_F32 && s.dtype != SDPA_F16) return SDPA_ERR_INVALID_ARG;
  if (s.mask != SDPA_MASK_NONE && s.mask != SDPA_MASK_CAUSAL && !windowed(s.mask)) return SDPA_ERR_INVALID_ARG;
  if (s.B < 0 || s.Hq < 0 || s.Lq < 0 || s.Lk < 0 || s.D <= 0 || s.group <= 0) return SDPA_ERR_INVALID_ARG;
  if (s.Hq % s.group != 0) return SDPA_ERR_INVALID_ARG;
  if (windowed(s.mask) && s.window < 1) return SDPA_ERR_INVALID_ARG;
  if (!isfinite(s.scale) || !(s.scale > 0.f)) return SDPA_ERR_INVALID_ARG;
  if (!d_supported(s.dtype, s.D)) return SDPA_ERR_UNSUPPORTED;
  // size limits: the kernels' 1-D grids hold at most 2^31 - 1 workgroups (checked
  // again at launch), head and batch counts stay far below that, and row / key
  // indices plus band offsets stay inside int32
  if (s.Hq > 65535 || s.B > 65535) return SDPA_ERR_UNSUPPORTED;
  if ((int64_t)s.Lq + s.Lk > (int64_t(1) << 30)) return SDPA_ERR_UNSUPPORTED;
  if ((int64_t)s.B * s.Hq * s.Lq > (int64_t(1) << 40) || (int64_t)s.B * s.Hq * s.Lk > (int64_t(1) << 40))
    return SDPA_ERR_UNSUPPORTED;
  return SDPA_OK;
}

size_t workspace_for(const Shape& s) {
  if (s.no_rows()) return 0;
  const size_t rows = (size_t)s.B * s.Hq * s.Lq;
  return align_up(rows * sizeof(float));  // Delta_i = <dO_i, O_i>, one float per query row
}

// Shares of the dK/dV split for a 16-bit call (1: none).
int split_shares(const Shape& s, bool dense) {
  if (s.dtype == SDPA_F32) return 1;
  switch (s.D) {
    case 64: return sdpa::kv_split_shares<64>(s.B, s.Hq, s.group, s.Lq, s.Lk, dense);
    case 128: return sdpa::kv_split_shares<128>(s.B, s.Hq, s.group, s.Lq, s.Lk, dense);
    case 256: return sdpa::kv_split_shares<256>(s.B, s.Hq, s.group, s.Lq, s.Lk, dense);
    default: return 1;
  }
}

bool wide_call(const Shape& s, bool dense) { return s.D == 256 && dense && split_shares(s, dense) == 1; }

// Key-range shares per query tile of the forward and the dQ pass for a 16-bit
// call (1: none), and the bytes of their fp32 partials (the forward's with a
// used max and row sum per row).
int qsplit_shares(const Shape& s, bool dense) {
  if (s.dtype == SDPA_F32 || s.no_rows() || s.no_keys()) return 1;
  int dlo, dhi;
  s.band(dlo, dhi);
  switch (s.D) {
    case 64: return sdpa::qs_split_shares<64>(s.B, s.Hq, s.Lq, s.Lk, dlo, dhi, dense);
    case 128: return sdpa::qs_split_shares<128>(s.B, s.Hq, s.Lq, s.Lk, dlo, dhi, dense);
    case 256: return sdpa::qs_split_shares<256>(s.B, s.Hq, s.Lq, s.Lk, dlo, dhi, dense);
    case 512: return sdpa::qs_split_shares<512>(s.B, s.Hq, s.Lq, s.Lk, dlo, dhi, dense);
    default: return 1;
  }
}

size_t qsplit_bytes(const Shape& s, int nseg, bool forward) {
  if (nseg <= 1) return 0;
  const size_t rows = (size_t)s.B * s.Hq * s.Lq;
  return align_up((size_t)nseg * rows * ((size_t)s.D + (forward ? 2 : 0)) * sizeof(float));
}

// Bytes of the split's fp32 dK and dV shares.
size_t split_bytes(const Shape& s, int nseg) {
  return nseg > 1 ? align_up(2 * (size_t)nseg * s.B * (s.Hq / s.group) * s.Lk * s.D * sizeof(float)) : 0;
}

int64_t floor_div(int64_t a, int64_t b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }

// Whether this shape's dense call keeps dS for its band (16-bit, D = 256, the
// 16-key dK/dV kernel), and the band buffer's geometry and bytes (0: it does
// not). A block of kBandRows rows at i0 sees keys [i0 + dlo, i0 + 127 + dhi]
// (clipped to [0, Lk)); i0 is a multiple of the tile width, so unclipped
// blocks all span floor((127 + dhi) / 64) - floor(dlo / 64) + 1 key tiles and
// clipped ones no more. The buffer is used only when a block's band is at most
// 9 D keys wide, so it never exceeds 9 times the size of Q (at D = 256 a
// causal window of up to about 2150 keys, or the two-sided window 1024):
// memory stays linear in Lq at any length, and wider bands (causal, no mask)
// recompute S and dP for dQ instead.
size_t band_bytes(const Shape& s, int dlo, int dhi, int& nqb, int& nkb) {
  nqb = nkb = 0;
  if (s.dtype == SDPA_F32 || s.D != 256 || s.no_rows() || s.no_keys() || dlo > dhi) return 0;
  const int64_t tiles = floor_div(sdpa::kBandRows - 1 + (int64_t)dhi, sdpa::kBandKeys) -
                        floor_div(dlo, sdpa::kBandKeys) + 1;
  const int64_t n = std::min<int64_t>(tiles, (s.Lk + sdpa::kBandKeys - 1) / sdpa::kBandKeys);
  if (n * sdpa::kBandKeys > 9 * (int64_t)s.D) return 0;
  const int64_t rb = (s.Lq + sdpa::kBandRows - 1) / sdpa::kBandRows;
  // the dK/dV pass addresses the band of one kv head's q-heads with 32-bit offsets
  if ((int64_t)s.group * rb * n * sdpa::kBandKeys * sdpa::kBandRows * 2 >= (int64_t(1) << 31)) return 0;
  nqb = (int)rb;
  nkb = (int)n;
  return align_up((size_t)s.B * s.Hq * nqb * nkb * sdpa::kBandKeys * sdpa::kBandRows * 2);
}

// Whether a dense 16-bit call runs the 16-key dK/dV kernel at D = 256 (its key
// blocks alone fill the GPU, so no split).


int to_status(hipError_t e) { return e == hipSuccess ? SDPA_OK : SDPA_ERR_LAUNCH; }

int elem_bytes(int dtype) { return dtype == SDPA_F32 ? 4 : 2; }

// The block-sparse cut of an extension struct (none: an empty key range).
int take_cut(const Shape& s, const sdpa_ext* ext, sdpa::Cut& cut) {
  cut = {s.Lq, 0, 0, 0};
  if (ext == nullptr || ext->cut_key_lo == ext->cut_key_hi) return SDPA_OK;
  if (ext->cut_key_lo < 0 || ext->cut_key_lo > ext->cut_key_hi || ext->cut_key_hi > s.Lk || ext->cut_row < 0 ||
      ext->cut_row > s.Lq || (ext->cut_logical != 0 && ext->cut_logical != 1))
    return SDPA_ERR_INVALID_ARG;
  const int sh = ext->cut_logical ? ext->cut_key_hi - ext->cut_key_lo : 0;
  cut = {ext->cut_row, ext->cut_key_lo, ext->cut_key_hi, sh};
  return SDPA_OK;
}

// Strides of a contiguous [B, H, L, D] tensor.
sdpa::Strides dense(int H, int L, int D) { return {(long long)H * L * D, (long long)L * D, D}; }

sdpa::AllStrides dense_all(const Shape& s) {
  const int Hkv = s.Hq / s.group;
  const sdpa::Strides q = dense(s.Hq, s.Lq, s.D), kv = dense(Hkv, s.Lk, s.D);
  return {q, kv, kv, q, q, q, kv, kv};
}

// Whether every tensor of a call is contiguous.
bool is_dense_call(const Shape& s, const sdpa::AllStrides& t) {
  const sdpa::AllStrides d = dense_all(s);
  return sdpa::same(t.q, d.q) && sdpa::same(t.k, d.k) && sdpa::same(t.v, d.v) && sdpa::same(t.o, d.o) &&
         sdpa::same(t.dO, d.dO) && sdpa::same(t.dq, d.dq) && sdpa::same(t.dk, d.dk) && sdpa::same(t.dv, d.dv);
}

// Caller strides (n tensors, in the AllStrides order q, k, v, o, dO, dq, dk, dv),
// or the contiguous layout when st is null. Every stride must be non-negative,
// a whole number of 16-byte units (so rows stay 16-byte aligned), and a row
// stride at least D and below 2^23 elements (tile offsets then fit 32 bits).
// K and V must share their row stride, and so must Q and dO.
int take_strides(const Shape& s, const sdpa_strides* st, int n, sdpa::AllStrides& out) {
  out = dense_all(s);
  if (st == nullptr) return SDPA_OK;
  sdpa::Strides* dst[] = {&out.q, &out.k, &out.v, &out.o, &out.dO, &out.dq, &out.dk, &out.dv};
  const long long unit = 16 / elem_bytes(s.dtype);
  for (int t = 0; t < n; t++) {
    const sdpa_strides& x = st[t];
    for (long long v : {(long long)x.b, (long long)x.h, (long long)x.l})
      if (v < 0 || v % unit != 0 || v > (1LL << 40)) return SDPA_ERR_INVALID_ARG;
    if (x.l < s.D || x.l >= (1LL << 23)) return SDPA_ERR_INVALID_ARG;
    *dst[t] = {(long long)x.b, (long long)x.h, (int)x.l};
  }
  // the tile loaders of the matrix-core kernels serve K and V (and Q and dO)
  // with one set of per-lane offsets
  if (out.k.l != out.v.l || (n > 4 && out.q.l != out.dO.l)) return SDPA_ERR_UNSUPPORTED;
  return SDPA_OK;
}

// Pointers of tensors that hold elements must be set and 16-byte aligned;
// those of empty tensors are not used.
bool ptr_ok(const void* p, bool used) { return !used || (p != nullptr && aligned16(p)); }

}  // namespace

extern "C" {

int sdpa_abi_version(void) { return 500; }

const char* sdpa_status_string(int status) {
  switch (status) {
    case SDPA_OK: return "ok";
    case SDPA_ERR_INVALID_ARG: return "invalid argument";
    case SDPA_ERR_UNSUPPORTED: return "unsupported combination (not built; no fallback)";
    case SDPA_ERR_WORKSPACE: return "workspace missing or too small";
    case SDPA_ERR_LAUNCH: return "kernel launch failed";
    case SDPA_ERR_SCRATCH_LIMIT:
      return "the allocation-free backward's fixed scratch is too small for this problem (use sdpa_bwd)";
    default: return "unknown status";
  }
}

size_t sdpa_bwd_workspace_bytes(int32_t B, int32_t Hq, int32_t Lq, int32_t D, int32_t dtype) {
  Shape s{B, Hq, 1, Lq, 0, D, dtype, SDPA_MASK_CAUSAL, 1, 1.f};
  if (check_shape(s) != SDPA_OK) return 0;
  return workspace_for(s);
}

size_t sdpa_bwd_workspace_bytes_ex(int32_t B, int32_t Hq, int32_t group, int32_t Lq, int32_t Lk, int32_t D,
                                   int32_t dtype, int32_t mask, int32_t window) {
  Shape s{B, Hq, group, Lq, Lk, D, dtype, mask, window, 1.f};
  if (check_shape(s) != SDPA_OK) return 0;
  const size_t base = workspace_for(s);
  if (base == 0 || s.no_keys()) return base;
  int dlo, dhi, nqb, nkb;
  s.band(dlo, dhi);
  const size_t band = wide_call(s, true) ? band_bytes(s, dlo, dhi, nqb, nkb) : 0;
  const size_t dq_split = band > 0 ? 0 : qsplit_bytes(s, qsplit_shares(s, true), false);
  return base + std::max(std::max(split_bytes(s, split_shares(s, true)), band), dq_split);
}

size_t sdpa_fwd_workspace_bytes(int32_t B, int32_t Hq, int32_t group, int32_t Lq, int32_t Lk, int32_t D,
                                int32_t dtype, int32_t mask, int32_t window) {
  Shape s{B, Hq, group, Lq, Lk, D, dtype, mask, window, 1.f};
  if (check_shape(s) != SDPA_OK) return 0;
  return qsplit_bytes(s, qsplit_shares(s, true), true);
}

}  // extern "C"

namespace {

int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
             size_t workspace_bytes, int32_t B, int32_t Hq, int32_t group, int32_t Lq, int32_t Lk, int32_t D,
             int32_t dtype, int32_t mask, int32_t window, float scale, const sdpa_ext* ext, hipStream_t stream) {
  const Shape s{B, Hq, group, Lq, Lk, D, dtype, mask, window, scale};
  int st = check_shape(s);
  if (st != SDPA_OK) return st;
  if (s.no_rows()) return SDPA_OK;
  const bool rows = true, keys = !s.no_keys();
  if (!ptr_ok(q, rows) || !ptr_ok(k, keys) || !ptr_ok(v, keys) || !ptr_ok(o, rows) || !ptr_ok(lse, rows))
    return SDPA_ERR_INVALID_ARG;
  const float* sinks = ext ? ext->sinks : nullptr;
  if (sinks != nullptr && !aligned16(sinks)) return SDPA_ERR_INVALID_ARG;
  sdpa::AllStrides str;
  if ((st = take_strides(s, ext ? ext->strides : nullptr, 4, str)) != SDPA_OK) return st;
  sdpa::Cut cut;
  if ((st = take_cut(s, ext, cut)) != SDPA_OK) return st;
  int dlo, dhi;
  s.band(dlo, dhi);
  if (workspace_bytes > 0 && (workspace == nullptr || !aligned16(workspace))) return SDPA_ERR_WORKSPACE;
  // the key-range split of a small dense call, when the workspace holds its partials
  const bool dense = is_dense_call(s, str) && cut.c0 == cut.c1;
  int qseg = qsplit_shares(s, dense);
  if (qseg > 1 && workspace_bytes < qsplit_bytes(s, qseg, true)) qseg = 1;
  float* part = qseg > 1 ? static_cast<float*>(workspace) : nullptr;
  switch (dtype * 1000 + D) {
#define SDPA_FWD_CASE(DT, E, DD)                                                                          \
  case DT * 1000 + DD:                                                                                    \
    return to_status(sdpa::launch_qs<DD, sdpa::QS_FWD, E>(q, k, v, nullptr, nullptr, lse, nullptr, o, sinks, \
                                                          B, Hq, group, Lq, Lk, dlo, dhi, cut, scale, str,    \
                                                          qseg, part, stream));
    SDPA_FWD_CASE(SDPA_BF16, bf16, 64)
    SDPA_FWD_CASE(SDPA_BF16, bf16, 128)
    SDPA_FWD_CASE(SDPA_BF16, bf16, 256)
    SDPA_FWD_CASE(SDPA_BF16, bf16, 512)
    SDPA_FWD_CASE(SDPA_F16, f16, 64)
    SDPA_FWD_CASE(SDPA_F16, f16, 128)
    SDPA_FWD_CASE(SDPA_F16, f16, 256)
    SDPA_FWD_CASE(SDPA_F16, f16, 512)
#undef SDPA_FWD_CASE
    case SDPA_F32 * 1000 + 64:
      return to_status(
          sdpa::launch_fwd_f32<64>(q, k, v, o, lse, B, Hq, sinks, group, Lq, Lk, dlo, dhi, cut, scale, str, stream));
    case SDPA_F32 * 1000 + 128:
      return to_status(
          sdpa::launch_fwd_f32<128>(q, k, v, o, lse, B, Hq, sinks, group, Lq, Lk, dlo, dhi, cut, scale, str, stream));
    case SDPA_F32 * 1000 + 256:
      return to_status(
          sdpa::launch_fwd_f32<256>(q, k, v, o, lse, B, Hq, sinks, group, Lq, Lk, dlo, dhi, cut, scale, str, stream));
    case SDPA_F32 * 1000 + 512:
      return to_status(
          sdpa::launch_fwd_f32<512>(q, k, v, o, lse, B, Hq, sinks, group, Lq, Lk, dlo, dhi, cut, scale, str, stream));
  }
  return SDPA_ERR_UNSUPPORTED;
}

}  // namespace

extern "C" {

int sdpa_fwd_lse_ex(const void* q, const void* k, const void* v, void* o, float* lse, int32_t B, int32_t Hq,
                    int32_t group, int32_t Lq, int32_t Lk, int32_t D, int32_t dtype, int32_t mask, int32_t window,
                    float scale, const sdpa_ext* ext, hipStream_t stream) {
  return fwd_impl(q, k, v, o, lse, nullptr, 0, B, Hq, group, Lq, Lk, D, dtype, mask, window, scale, ext, stream);
}

int sdpa_fwd_lse_ws(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                    size_t workspace_bytes, int32_t B, int32_t Hq, int32_t group, int32_t Lq, int32_t Lk, int32_t D,
                    int32_t dtype, int32_t mask, int32_t window, float scale, hipStream_t stream) {
  return fwd_impl(q, k, v, o, lse, workspace, workspace_bytes, B, Hq, group, Lq, Lk, D, dtype, mask, window, scale,
                  nullptr, stream);
}

int sdpa_fwd_lse(const void* q, const void* k, const void* v, void* o, float* lse, int32_t B, int32_t Hq,
                 int32_t group, int32_t Lq, int32_t Lk, int32_t D, int32_t dtype, int32_t mask, int32_t window,
                 float scale, hipStream_t stream) {
  return fwd_impl(q, k, v, o, lse, nullptr, 0, B, Hq, group, Lq, Lk, D, dtype, mask, window, scale, nullptr, stream);
}

}  // extern "C"

namespace {

int bwd_impl(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
             void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int32_t B, int32_t Hq,
             int32_t group, int32_t Lq, int32_t Lk, int32_t D, int32_t dtype, int32_t mask, int32_t window,
             float scale, const sdpa_ext* ext, hipStream_t stream, const hipEvent_t* events) {
  const Shape s{B, Hq, group, Lq, Lk, D, dtype, mask, window, scale};
  int st = check_shape(s);
  if (st != SDPA_OK) return st;
  const float* sinks = ext ? ext->sinks : nullptr;
  float* dsinks = ext ? ext->dsinks : nullptr;
  if ((sinks == nullptr) != (dsinks == nullptr)) return SDPA_ERR_INVALID_ARG;
  if (s.B == 0 || s.Hq == 0) return SDPA_OK;
  if (sinks != nullptr && (!aligned16(sinks) || !aligned16(dsinks))) return SDPA_ERR_INVALID_ARG;
  if (s.no_rows() && s.no_keys()) return sinks ? to_status(sdpa::launch_dsinks(nullptr, nullptr, sinks, dsinks, B,
                                                                               Hq, 0, stream))
                                               : SDPA_OK;
  const bool rows = !s.no_rows(), keys = !s.no_keys();
  if (!ptr_ok(q, rows) || !ptr_ok(o, rows) || !ptr_ok(dO, rows) || !ptr_ok(lse, rows) || !ptr_ok(dq, rows) ||
      !ptr_ok(k, keys) || !ptr_ok(v, keys) || !ptr_ok(dk, keys) || !ptr_ok(dv, keys))
    return SDPA_ERR_INVALID_ARG;
  sdpa::AllStrides str;
  if ((st = take_strides(s, ext ? ext->strides : nullptr, 8, str)) != SDPA_OK) return st;
  sdpa::Cut cut;
  if ((st = take_cut(s, ext, cut)) != SDPA_OK) return st;
  const size_t need = workspace_for(s);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)))
    return SDPA_ERR_WORKSPACE;
  float* delta = static_cast<float*>(workspace);
  int dlo, dhi;
  s.band(dlo, dhi);
  // the dK/dV split of a small dense call, or the dS band buffer of a bounded
  // band, when the workspace holds them (after the Delta rows)
  const bool dense = is_dense_call(s, str) && cut.c0 == cut.c1;
  char* extra = static_cast<char*>(workspace) + need;
  sdpa::BwdPlan plan{dense && split_shares(s, dense) == 1, nullptr, split_shares(s, dense), nullptr, 0, 0,
                     nullptr, qsplit_shares(s, dense)};
  if (plan.nseg > 1 && workspace_bytes < need + split_bytes(s, plan.nseg)) plan.nseg = 1;
  if (plan.nseg > 1) plan.part = reinterpret_cast<float*>(extra);
  if (wide_call(s, dense)) {
    int nqb, nkb;
    const size_t bb = band_bytes(s, dlo, dhi, nqb, nkb);
    if (bb > 0 && workspace_bytes >= need + bb) plan.band = extra, plan.nqb = nqb, plan.nkb = nkb;
  }
  // the dQ pass's key-range split (not with the band buffer, which forms dQ
  // without that pass); its partials share the memory after the Delta rows
  // with the dK/dV shares, which are written only after its combine
  if (plan.band != nullptr || workspace_bytes < need + qsplit_bytes(s, plan.qseg, false)) plan.qseg = 1;
  if (plan.qseg > 1) plan.qpart = reinterpret_cast<float*>(extra);
  hipError_t e;
  switch (dtype * 1000 + D) {
#define SDPA_BWD_CASE(DT, E, DD)                                                                              \
  case DT * 1000 + DD:                                                                                        \
    e = sdpa::launch_bwd_mfma<DD, E>(q, k, v, o, dO, lse, dq, dk, dv, delta, B, Hq, group, Lq, Lk, dlo, dhi,   \
                                     cut, scale, str, plan, stream, events);                                  \
    break;
    SDPA_BWD_CASE(SDPA_BF16, bf16, 64)
    SDPA_BWD_CASE(SDPA_BF16, bf16, 128)
    SDPA_BWD_CASE(SDPA_BF16, bf16, 256)
    SDPA_BWD_CASE(SDPA_BF16, bf16, 512)
    SDPA_BWD_CASE(SDPA_F16, f16, 64)
    SDPA_BWD_CASE(SDPA_F16, f16, 128)
    SDPA_BWD_CASE(SDPA_F16, f16, 256)
    SDPA_BWD_CASE(SDPA_F16, f16, 512)
#undef SDPA_BWD_CASE
    case SDPA_F32 * 1000 + 64:
      e = sdpa::launch_bwd_f32<64>(q, k, v, o, dO, lse, dq, dk, dv, delta, B, Hq, group, Lq, Lk, dlo, dhi, cut,
                                   scale, str, stream, events);
      break;
    case SDPA_F32 * 1000 + 128:
      e = sdpa::launch_bwd_f32<128>(q, k, v, o, dO, lse, dq, dk, dv, delta, B, Hq, group, Lq, Lk, dlo, dhi, cut,
                                    scale, str, stream, events);
      break;
    case SDPA_F32 * 1000 + 256:
      e = sdpa::launch_bwd_f32<256>(q, k, v, o, dO, lse, dq, dk, dv, delta, B, Hq, group, Lq, Lk, dlo, dhi, cut,
                                    scale, str, stream, events);
      break;
    case SDPA_F32 * 1000 + 512:
      e = sdpa::launch_bwd_f32<512>(q, k, v, o, dO, lse, dq, dk, dv, delta, B, Hq, group, Lq, Lk, dlo, dhi, cut,
                                    scale, str, stream, events);
      break;
    default:
      return SDPA_ERR_UNSUPPORTED;
  }
  if (e != hipSuccess) return SDPA_ERR_LAUNCH;
  // d sigma_h from lse and Delta (the dQ pass wrote Delta into the workspace)
  if (sinks != nullptr) e = sdpa::launch_dsinks(lse, delta, sinks, dsinks, B, Hq, Lq, stream);
  return to_status(e);
}

}  // namespace

extern "C" {

int sdpa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int32_t B, int32_t Hq,
                int32_t group, int32_t Lq, int32_t Lk, int32_t D, int32_t dtype, int32_t mask, int32_t window,
                float scale, const sdpa_ext* ext, hipStream_t stream) {
  return bwd_impl(q, k, v, o, dO, lse, dq, dk, dv, workspace, workspace_bytes, B, Hq, group, Lq, Lk, D, dtype,
                  mask, window, scale, ext, stream, nullptr);
}

int sdpa_bwd_timed(const void* q, const void* k, const void* v, const void* o, const void* dO,
                   const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                   int32_t B, int32_t Hq, int32_t group, int32_t Lq, int32_t Lk, int32_t D, int32_t dtype,
                   int32_t mask, int32_t window, float scale, hipStream_t stream, const hipEvent_t* events) {
  if (events != nullptr)
    for (int i = 0; i < 4; i++)
      if (events[i] == nullptr) return SDPA_ERR_INVALID_ARG;
  return bwd_impl(q, k, v, o, dO, lse, dq, dk, dv, workspace, workspace_bytes, B, Hq, group, Lq, Lk, D, dtype,
                  mask, window, scale, nullptr, stream, events);
}

int sdpa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
             void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int32_t B, int32_t Hq,
             int32_t group, int32_t Lq, int32_t Lk, int32_t D, int32_t dtype, int32_t mask, int32_t window,
             float scale, hipStream_t stream) {
  return bwd_impl(q, k, v, o, dO, lse, dq, dk, dv, workspace, workspace_bytes, B, Hq, group, Lq, Lk, D, dtype,
                  mask, window, scale, nullptr, stream, nullptr);
}

}  // extern "C"

// ---------------------------------------------------------------- allocation-free backward
namespace {

// The backward's scratch for sdpa_bwd_noalloc: one fixed array per GPU, held
// until the process ends. Host code must not use the array's name as a device
// address; each device's address comes from hipGetSymbolAddress (below).
constexpr size_t kScratchBytes = size_t(SDPA_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// This device's copy of `scratch` (looked up once per device, with that
// device current).
int current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SDPA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return SDPA_ERR_LAUNCH;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return SDPA_OK;
}

}  // namespace

extern "C" {

int sdpa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dO,
                     const float* lse, void* dq, void* dk, void* dv, int32_t B, int32_t Hq, int32_t group,
                     int32_t Lq, int32_t Lk, int32_t D, int32_t dtype, int32_t mask, int32_t window, float scale,
                     hipStream_t stream) {
  const Shape s{B, Hq, group, Lq, Lk, D, dtype, mask, window, scale};
  const int st = check_shape(s);
  if (st != SDPA_OK) return st;
  // the Delta rows must fit; the split shares or the dS band buffer are used
  // only when they fit as well (otherwise the plan without them runs)
  if (workspace_for(s) > kScratchBytes) return SDPA_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  if (workspace_for(s) > 0) {
    const int e = current_scratch(&ws);
    if (e != SDPA_OK) return e;
  }
  return bwd_impl(q, k, v, o, dO, lse, dq, dk, dv, ws, ws != nullptr ? kScratchBytes : 0, B, Hq, group, Lq, Lk, D,
                  dtype, mask, window, scale, nullptr, stream, nullptr);
}

}  // extern "C"
