// float32 attention forward (+lse) and backward on the vector ALUs.
//
// This path exists for float32 inputs, where the result must be computed in
// true fp32 (no reduced-precision matrix mode: page "Lab 028 lab detail: Off
// NVIDIA, you fix the platform yourself", section "Gradient parity", reports
// fp32 gradients that are noisy only when TF32-style math is on). It targets
// small problems: one group of D / 32 lanes per query row (forward, dQ) or per
// key (dK, dV), passes over the allowed keys, fp32 FMA throughout. D = 64, 128,
// 256 or 512.
#include <math.h>

#include "common.h"

namespace sdpa {

// Calls f(j) for every key j that row i sees: the band [i + dlo, i + dhi]
// within [0, Lk), except from the cut row on: the band from c1 on, and the
// band moved back by the cut's shift, clipped to the keys before c0.
template <typename F>
__device__ inline void for_row_keys(int i, int Lk, int dlo, int dhi, const Cut& cut, F&& f) {
  const int lo = max(0, i + dlo), hi = min(Lk - 1, i + dhi);
  if (i >= cut.r0 && cut.c0 < cut.c1) {
    for (int j = max(0, i + dlo - cut.sh), e = min(min(cut.c0 - 1, Lk - 1), i + dhi - cut.sh); j <= e; j++) f(j);
    for (int j = max(lo, cut.c1); j <= hi; j++) f(j);
  } else {
    for (int j = lo; j <= hi; j++) f(j);
  }
}

// Each query row (forward, dQ) or key (dK, dV) is spread over NT = D / 32
// consecutive lanes, each holding 32 of its D elements: dot products are
// summed over the group with lane shuffles, in a fixed order.
template <int D>
struct F32Cfg {
  static constexpr int NT = D / 32;     // lanes per row or key
  static constexpr int DT = D / NT;     // elements per lane (32)
  static constexpr int PER = 128 / NT;  // rows or keys per 128-thread block
  static_assert(D % 32 == 0 && NT >= 1 && NT <= 16, "head dimension");
};

// Sum of x over the NT lanes of this lane's group (butterfly: every lane of
// the group gets the same value).
template <int NT>
__device__ inline float group_sum(float x) {
#pragma unroll
  for (int o = NT / 2; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <int D>
__global__ void __launch_bounds__(128)
fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
               float* __restrict__ O, float* __restrict__ LSE, const float* __restrict__ Sinks, int Hq,
               int group, int Lq, int Lk, int dlo, int dhi, Cut cut, float scale, AllStrides st) {
  using C = F32Cfg<D>;
  constexpr int NT = C::NT, DT = C::DT;
  const int i = blockIdx.x * C::PER + threadIdx.x / NT, d0 = (threadIdx.x % NT) * DT;
  const int h = blockIdx.y, b = blockIdx.z;
  if (i >= Lq) return;  // (the whole group of row i)
  const int Hkv = Hq / group, g = h / group;
  const float* q = Q + b * st.q.b + h * st.q.h + (long long)i * st.q.l + d0;
  const float* Kg = K + b * st.k.b + g * st.k.h + d0;
  const float* Vg = V + b * st.v.b + g * st.v.h + d0;
  float qr[DT];
#pragma unroll
  for (int d = 0; d < DT; d++) qr[d] = q[d];
  // allowed keys of row i (empty: O = 0, lse = -inf)
  const float sink = Sinks != nullptr ? Sinks[h] : -INFINITY;  // one more score, with a zero value row
  auto score = [&](int j) {
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < DT; d++) s = fmaf(qr[d], Kg[(long long)j * st.k.l + d], s);
    return group_sum<NT>(s) * scale;
  };
  float m = sink;
  for_row_keys(i, Lk, dlo, dhi, cut, [&](int j) { m = fmaxf(m, score(j)); });
  float l = sink != -INFINITY ? expf(sink - m) : 0.f;
  for_row_keys(i, Lk, dlo, dhi, cut, [&](int j) { l += expf(score(j) - m); });
  const float lse = l > 0.f ? m + logf(l) : -INFINITY;
  float acc[DT];
#pragma unroll
  for (int d = 0; d < DT; d++) acc[d] = 0.f;
  for_row_keys(i, Lk, dlo, dhi, cut, [&](int j) {
    const float p = expf(score(j) - lse);
#pragma unroll
    for (int d = 0; d < DT; d++) acc[d] = fmaf(p, Vg[(long long)j * st.v.l + d], acc[d]);
  });
  float* o = O + b * st.o.b + h * st.o.h + (long long)i * st.o.l + d0;
#pragma unroll
  for (int d = 0; d < DT; d++) o[d] = acc[d];
  if (d0 == 0) LSE[((size_t)b * Hq + h) * Lq + i] = lse;
}

// dQ rows (and Delta_i = <dO_i, O_i>, kept for the key pass)
template <int D>
__global__ void __launch_bounds__(128)
bwd_dq_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
                  const float* __restrict__ O, const float* __restrict__ dO, const float* __restrict__ LSE,
                  float* __restrict__ dQ, float* __restrict__ Delta, int Hq, int group, int Lq, int Lk,
                  int dlo, int dhi, Cut cut, float scale, AllStrides st) {
  using C = F32Cfg<D>;
  constexpr int NT = C::NT, DT = C::DT;
  const int i = blockIdx.x * C::PER + threadIdx.x / NT, d0 = (threadIdx.x % NT) * DT;
  const int h = blockIdx.y, b = blockIdx.z;
  if (i >= Lq) return;  // (the whole group of row i)
  const int Hkv = Hq / group, g = h / group;
  const size_t row = ((size_t)b * Hq + h) * Lq + i;  // lse / Delta index
  const float* q = Q + b * st.q.b + h * st.q.h + (long long)i * st.q.l + d0;
  const float* o = O + b * st.o.b + h * st.o.h + (long long)i * st.o.l + d0;
  const float* dor = dO + b * st.dO.b + h * st.dO.h + (long long)i * st.dO.l + d0;
  const float* Kg = K + b * st.k.b + g * st.k.h + d0;
  const float* Vg = V + b * st.v.b + g * st.v.h + d0;
  float qr[DT], dr[DT], acc[DT];
  float delta = 0.f;
#pragma unroll
  for (int d = 0; d < DT; d++) {
    qr[d] = q[d];
    dr[d] = dor[d];
    delta = fmaf(dr[d], o[d], delta);
    acc[d] = 0.f;
  }
  delta = group_sum<NT>(delta);
  const float lse = LSE[row];
  for_row_keys(i, Lk, dlo, dhi, cut, [&](int j) {
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int d = 0; d < DT; d++) {
      s = fmaf(qr[d], Kg[(long long)j * st.k.l + d], s);
      dp = fmaf(dr[d], Vg[(long long)j * st.v.l + d], dp);
    }
    s = group_sum<NT>(s);
    dp = group_sum<NT>(dp);
    const float p = expf(s * scale - lse);
    const float ds = p * (dp - delta);
#pragma unroll
    for (int d = 0; d < DT; d++) acc[d] = fmaf(ds, Kg[(long long)j * st.k.l + d], acc[d]);
  });
  float* dq = dQ + b * st.dq.b + h * st.dq.h + (long long)i * st.dq.l + d0;
#pragma unroll
  for (int d = 0; d < DT; d++) dq[d] = acc[d] * scale;
  if (d0 == 0) Delta[row] = delta;
}

// dK, dV of one key, summed over the q-heads of its kv group
template <int D>
__global__ void __launch_bounds__(128)
bwd_dkv_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
                   const float* __restrict__ dO, const float* __restrict__ LSE,
                   const float* __restrict__ Delta, float* __restrict__ dK, float* __restrict__ dV, int Hq,
                   int group, int Lq, int Lk, int dlo, int dhi, Cut cut, float scale, AllStrides st) {
  using C = F32Cfg<D>;
  constexpr int NT = C::NT, DT = C::DT;
  const int j = blockIdx.x * C::PER + threadIdx.x / NT, d0 = (threadIdx.x % NT) * DT;
  const int g = blockIdx.y, b = blockIdx.z;
  if (j >= Lk) return;  // (the whole group of key j)
  const int Hkv = Hq / group;
  const float* kp = K + b * st.k.b + g * st.k.h + (long long)j * st.k.l + d0;
  const float* vp = V + b * st.v.b + g * st.v.h + (long long)j * st.v.l + d0;
  float kr[DT], vr[DT], dk[DT], dv[DT];
#pragma unroll
  for (int d = 0; d < DT; d++) {
    kr[d] = kp[d];
    vr[d] = vp[d];
    dk[d] = 0.f;
    dv[d] = 0.f;
  }
  // rows that see key j: dlo <= j - i <= dhi, 0 <= i < Lq; a cut key only
  // rows before r0; with a shift, a key before c0 rows before r0 through the
  // band and rows from r0 on through the band moved forward by the shift
  const bool cutk = cut.c0 < cut.c1;
  const bool kc = cutk && j >= cut.c0 && j < cut.c1, ks = cutk && j < cut.c0 && cut.sh > 0;
  const int ilo = max(0, j - dhi), ihi = min(kc || ks ? cut.r0 - 1 : Lq - 1, j - dlo);
  const int ilo2 = ks ? max(cut.r0, j + cut.sh - dhi) : 1, ihi2 = ks ? min(Lq - 1, j + cut.sh - dlo) : 0;
  for (int h = g * group; h < (g + 1) * group; h++) {
    const size_t hrow = ((size_t)b * Hq + h) * Lq;  // lse / Delta row block
    auto add_row = [&](int i) {
      const float* q = Q + b * st.q.b + h * st.q.h + (long long)i * st.q.l + d0;
      const float* dor = dO + b * st.dO.b + h * st.dO.h + (long long)i * st.dO.l + d0;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < DT; d++) {
        s = fmaf(q[d], kr[d], s);
        dp = fmaf(dor[d], vr[d], dp);
      }
      s = group_sum<NT>(s);
      dp = group_sum<NT>(dp);
      const float p = expf(s * scale - LSE[hrow + i]);
      const float ds = p * (dp - Delta[hrow + i]);
#pragma unroll
      for (int d = 0; d < DT; d++) {
        dk[d] = fmaf(ds, q[d], dk[d]);
        dv[d] = fmaf(p, dor[d], dv[d]);
      }
    };
    for (int i = ilo; i <= ihi; i++) add_row(i);
    for (int i = ilo2; i <= ihi2; i++) add_row(i);
  }
  float* dkp = dK + b * st.dk.b + g * st.dk.h + (long long)j * st.dk.l + d0;
  float* dvp = dV + b * st.dv.b + g * st.dv.h + (long long)j * st.dv.l + d0;
#pragma unroll
  for (int d = 0; d < DT; d++) {
    dkp[d] = dk[d] * scale;
    dvp[d] = dv[d];
  }
}

template <int D>
hipError_t launch_fwd_f32(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                          const float* sinks, int group, int Lq, int Lk, int dlo, int dhi, Cut cut, float scale,
                          const AllStrides& st, hipStream_t stream) {
  constexpr int PER = F32Cfg<D>::PER;
  dim3 grid((Lq + PER - 1) / PER, Hq, B);
  hipLaunchKernelGGL(fwd_f32_kernel<D>, grid, dim3(128), 0, stream, (const float*)q, (const float*)k,
                     (const float*)v, (float*)o, lse, sinks, Hq, group, Lq, Lk, dlo, dhi, cut, scale, st);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_f32(const void* q, const void* k, const void* v, const void* o, const void* dO,
                          const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int Hq,
                          int group, int Lq, int Lk, int dlo, int dhi, Cut cut, float scale, const AllStrides& st,
                          hipStream_t stream, const hipEvent_t* ev) {
  hipError_t e;
  if (ev != nullptr && (e = hipEventRecord(ev[0], stream)) != hipSuccess) return e;
  constexpr int PER = F32Cfg<D>::PER;
  if (Lq > 0) {
    dim3 grid((Lq + PER - 1) / PER, Hq, B);
    hipLaunchKernelGGL(bwd_dq_f32_kernel<D>, grid, dim3(128), 0, stream, (const float*)q, (const float*)k,
                       (const float*)v, (const float*)o, (const float*)dO, lse, (float*)dq, delta, Hq, group,
                       Lq, Lk, dlo, dhi, cut, scale, st);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (ev != nullptr && (e = hipEventRecord(ev[1], stream)) != hipSuccess) return e;
  if (Lk > 0) {
    dim3 grid2((Lk + PER - 1) / PER, Hq / group, B);
    hipLaunchKernelGGL(bwd_dkv_f32_kernel<D>, grid2, dim3(128), 0, stream, (const float*)q, (const float*)k,
                       (const float*)v, (const float*)dO, lse, (const float*)delta, (float*)dk, (float*)dv, Hq,
                       group, Lq, Lk, dlo, dhi, cut, scale, st);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  for (int i = 2; i < 4; i++)
    if (ev != nullptr && (e = hipEventRecord(ev[i], stream)) != hipSuccess) return e;
  return hipSuccess;
}

#define SDPA_INST_F32(D)                                                                                    \
  template hipError_t launch_fwd_f32<D>(const void*, const void*, const void*, void*, float*, int, int,      \
                                        const float*, int, int, int, int, int, Cut, float,                  \
                                        const AllStrides&, hipStream_t);                                    \
  template hipError_t launch_bwd_f32<D>(const void*, const void*, const void*, const void*, const void*,     \
                                        const float*, void*, void*, void*, float*, int, int, int, int, int,  \
                                        int, int, Cut, float, const AllStrides&, hipStream_t,                \
                                        const hipEvent_t*);
SDPA_INST_F32(64)
SDPA_INST_F32(128)
SDPA_INST_F32(256)
SDPA_INST_F32(512)

}  // namespace sdpa
