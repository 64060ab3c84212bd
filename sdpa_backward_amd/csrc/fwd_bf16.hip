// Attention forward with per-row logsumexp, bf16 inputs, fp32 accumulation
// and fp32 online-softmax state, for gfx950.
//
// The forward keeps the per-row softmax normaliser (logsumexp) so the
// backward can recompute P: page "Lab 028 lab detail: Off NVIDIA, you fix the
// platform yourself", section "What I changed, in plain terms", item 1.
// Tiles entirely outside the causal/window band are skipped (same page, items
// 3-4). The running max and sum stay in fp32: page "Training - design (ORPO,
// flash-CCE head, prefix sharing, segmented backward)", section 5.1, item 3,
// reports that a bf16 (m, d) recurrence breaks gradients.
//
// Work split. One workgroup = 4 waves = 128 query rows of one (b, h); each
// wave owns 32 query rows. The loop walks key tiles of BK keys:
//   S^T (BK x 32) = K_tile (LDS, direct) . Q_w^T (registers)      [MFMA]
// so the fp32 C tile puts one query per lane column and all of that query's
// keys in the lane (plus its partner lane l^32): row max and row sum need one
// cross-lane step. P^T is then reused in place as the B operand of
//   O^T (D x 32) += V_tile^T (LDS, transposed reads) . P^T       [MFMA]
// O^T stays in registers for the whole loop.
#include "common.h"

namespace sdpa {

template <int D>
struct FwdCfg {
  static constexpr int NW = 4;
  static constexpr int BQ = 32 * NW;           // query rows per workgroup
  static constexpr int BK = D <= 256 ? 64 : 32;  // keys per loop step
  static constexpr int LDK = D + 8;            // LDS row stride (elements); +16 B breaks bank aliasing
  static constexpr size_t LDS_BYTES = 2ull * BK * LDK * sizeof(bf16);
};

template <int D>
__global__ void __launch_bounds__(256, 1)
fwd_bf16_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
                bf16* __restrict__ O, float* __restrict__ LSE, int Hq, int group, int L, int w_eff,
                float scale_log2) {
  using C = FwdCfg<D>;
  constexpr int BK = C::BK, LDK = C::LDK, NDB = D / 32, NKS = D / 16, NMB = BK / 32;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  bf16* Ks = reinterpret_cast<bf16*>(smem_raw);
  bf16* Vs = Ks + BK * LDK;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int qt = gridDim.x - 1 - blockIdx.x;  // longest causal rows first
  const int h = blockIdx.y, b = blockIdx.z;
  const int Hkv = Hq / group, g = h / group;
  const bf16* Qh = Q + (size_t)(b * Hq + h) * L * D;
  const bf16* Kg = K + (size_t)(b * Hkv + g) * L * D;
  const bf16* Vg = V + (size_t)(b * Hkv + g) * L * D;

  const int i0 = qt * C::BQ;
  const int iw0 = i0 + 32 * w;        // first row of this wave
  const int hh = lane >> 5;           // lane half
  const int qi = iw0 + (lane & 31);   // this lane's query row

  // Q_w^T as B operands: lane holds row qi, d-slots 16*s + 8*hh + 0..7.
  bf16x8 qreg[NKS];
#pragma unroll
  for (int s = 0; s < NKS; s++)
    qreg[s] = qi < L ? *(const bf16x8*)(Qh + (size_t)qi * D + 16 * s + 8 * hh) : zero_bf16x8();

  f32x16 oacc[NDB];
#pragma unroll
  for (int d = 0; d < NDB; d++) oacc[d] = zero16();
  float m = -INFINITY, lsum = 0.f;

  const int i1 = min(i0 + C::BQ - 1, L - 1);
  const int klo = max(0, i0 - w_eff + 1);
  const int kt_lo = klo / BK, kt_hi = i1 / BK;
  const int wr0 = iw0, wr1 = min(iw0 + 31, L - 1);  // this wave's row range (wr1 < wr0: no rows)

  for (int kt = kt_lo; kt <= kt_hi; kt++) {
    const int j0 = kt * BK;
    __syncthreads();  // previous step is done reading the tiles
    load_tile<D, 256>(Ks, LDK, Kg + (size_t)j0 * D, BK, L - j0, tid);
    load_tile<D, 256>(Vs, LDK, Vg + (size_t)j0 * D, BK, L - j0, tid);
    __syncthreads();

    // wave-uniform tile classification
    const bool active = wr0 <= wr1 && j0 <= wr1 && j0 + BK - 1 > wr0 - w_eff;
    if (!active) continue;
    const bool full = j0 + BK - 1 <= wr0 && j0 > wr1 - w_eff && wr1 == iw0 + 31;

    f32x16 st[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; mb++) {
      st[mb] = zero16();
#pragma unroll
      for (int s = 0; s < NKS; s++) st[mb] = mfma(ld_op(Ks, LDK, 16 * s, 32 * mb, lane), qreg[s], st[mb]);
    }
    // scores in the log2 domain, masked to -inf outside the band
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < NMB; mb++)
#pragma unroll
      for (int i = 0; i < 16; i++) {
        float x = st[mb][i] * scale_log2;
        if (!full) {
          const int j = j0 + 32 * mb + c_row(i, hh);
          if (!allowed(qi, j, w_eff, L)) x = -INFINITY;
        }
        st[mb][i] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;  // rows with no key yet
    const float alpha = __builtin_amdgcn_exp2f(m - m_use);
    float rs = 0.f;
#pragma unroll
    for (int mb = 0; mb < NMB; mb++)
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const float p = __builtin_amdgcn_exp2f(st[mb][i] - m_use);
        st[mb][i] = p;
        rs += p;
      }
    rs += __shfl_xor(rs, 32);
    lsum = lsum * alpha + rs;
    m = m_new;
#pragma unroll
    for (int d = 0; d < NDB; d++)
#pragma unroll
      for (int i = 0; i < 16; i++) oacc[d][i] *= alpha;

    bf16x8 pb[2 * NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; mb++) {
      pb[2 * mb] = c_to_op(st[mb], 0);
      pb[2 * mb + 1] = c_to_op(st[mb], 1);
    }
#pragma unroll
    for (int d = 0; d < NDB; d++)
#pragma unroll
      for (int kk = 0; kk < 2 * NMB; kk++)
        oacc[d] = mfma(ld_op_tr(Vs, LDK, 16 * kk, 32 * d, lane), pb[kk], oacc[d]);
  }

  if (qi < L) {
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    bf16* orow = O + (size_t)(b * Hq + h) * L * D + (size_t)qi * D;
#pragma unroll
    for (int d = 0; d < NDB; d++)
#pragma unroll
      for (int blk = 0; blk < 4; blk++) {
        bf16x4 v;
#pragma unroll
        for (int r = 0; r < 4; r++) v[r] = (bf16)(oacc[d][4 * blk + r] * inv);
        *(bf16x4*)(orow + 32 * d + 8 * blk + 4 * hh) = v;
      }
    if (hh == 0) LSE[(size_t)(b * Hq + h) * L + qi] = lsum > 0.f ? (m + __log2f(lsum)) * kLn2 : -INFINITY;
  }
}

template <int D>
hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                           int Hq, int group, int L, int w_eff, float scale, hipStream_t stream) {
  using C = FwdCfg<D>;
  auto kern = fwd_bf16_kernel<D>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)C::LDS_BYTES);
  if (e != hipSuccess) return e;
  dim3 grid((L + C::BQ - 1) / C::BQ, Hq, B);
  hipLaunchKernelGGL(kern, grid, dim3(256), C::LDS_BYTES, stream, (const bf16*)q, (const bf16*)k,
                     (const bf16*)v, (bf16*)o, lse, Hq, group, L, w_eff, scale * kLog2e);
  return hipGetLastError();
}

template hipError_t launch_fwd_bf16<64>(const void*, const void*, const void*, void*, float*, int, int,
                                        int, int, int, float, hipStream_t);
template hipError_t launch_fwd_bf16<128>(const void*, const void*, const void*, void*, float*, int, int,
                                         int, int, int, float, hipStream_t);
template hipError_t launch_fwd_bf16<256>(const void*, const void*, const void*, void*, float*, int, int,
                                         int, int, int, float, hipStream_t);
template hipError_t launch_fwd_bf16<512>(const void*, const void*, const void*, void*, float*, int, int,
                                         int, int, int, float, hipStream_t);

}  // namespace sdpa
