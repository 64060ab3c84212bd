// Attention backward for gfx950, bf16 inputs, fp32 accumulation.
//
// Three launches on one stream:
//   1. bwd_pre:   Delta_i = <dO_i, O_i> (fp32) and zero the fp32 dQ accumulator
//   2. bwd_main:  KV-stationary tiles: recompute S and P = exp(S - lse), form
//                 dS = P * (dP - Delta), accumulate dK and dV in registers over
//                 every query tile and every q-head of the kv group (no atomics
//                 for the GQA sum), and add dQ tiles into the accumulator with
//                 fp32 atomics
//   3. dq_convert: dQ = scale * accumulator, rounded to bf16
//
// The per-element recompute of P and dS from S and the stored lse, and the
// whole-tile skips above the causal diagonal and behind the window, follow
// page "Lab 028 lab detail: Off NVIDIA, you fix the platform yourself",
// sections "2026-10-21" ("What the code says") and "What I changed, in plain
// terms" (items 3-5). dQ is accumulated from a zeroed buffer, so no query tile
// depends on a "first visit" (item 5a), and dK/dV are written for every key,
// attended or not (item 5b). S and dP stay in fp32 registers; only P and dS
// are rounded to bf16 as MFMA operands (section "fp32 score tiles": bf16
// score tiles were the source of the extra gradient error).
//
// Work split of bwd_main. One workgroup = 4 waves = one (b, kv head g) and a
// block of BKT keys. Wave w owns 32 keys (and, for D = 512, half of the head
// dimension: DS = 2 waves share a key block). Per query tile of 32 rows:
//   S  (32q x 32k) = Q_tile . K_w^T        A: Q (LDS, direct)   B: K (LDS, direct)
//   dP (32q x 32k) = dO_tile . V_w^T       A: dO (LDS, direct)  B: V_w (registers)
//   dV_w += P^T dO                          A: P^T (C tile reused) B: dO (LDS, transposed reads)
//   dK_w += dS^T Q                          A: dS^T (C tile)      B: Q  (LDS, transposed reads)
//   dS^T -> LDS (bf16); then every wave takes a slice of the head dimension:
//   dQ (32q x D/4) = dS . K                 A: dS (transposed reads) B: K (transposed reads)
#include "common.h"

namespace sdpa {

// ------------------------------------------------------------------ preprocess
template <int D>
__global__ void __launch_bounds__(256)
bwd_pre_kernel(const bf16* __restrict__ O, const bf16* __restrict__ dO, float* __restrict__ delta,
               float* __restrict__ dq_acc, long rows) {
  constexpr int TPR = D / 8;          // threads per row, 8 elements each
  constexpr int RPB = 256 / TPR;      // rows per block
  const int t = threadIdx.x;
  const long row = (long)blockIdx.x * RPB + t / TPR;
  const int c = (t % TPR) * 8;
  float s = 0.f;
  if (row < rows) {
    const bf16x8 a = *(const bf16x8*)(O + row * D + c);
    const bf16x8 bb = *(const bf16x8*)(dO + row * D + c);
#pragma unroll
    for (int j = 0; j < 8; j++) s += (float)a[j] * (float)bb[j];
    float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    *(float4*)(dq_acc + row * D + c) = z;
    *(float4*)(dq_acc + row * D + c + 4) = z;
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (row < rows && (t % TPR) == 0) delta[row] = s;
}

// ------------------------------------------------------------------ convert
__global__ void __launch_bounds__(256)
dq_convert_kernel(const float* __restrict__ acc, bf16* __restrict__ dq, float scale, long n8) {
  const long stride = (long)gridDim.x * blockDim.x;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += stride) {
    const float4 a = *(const float4*)(acc + 8 * i);
    const float4 c = *(const float4*)(acc + 8 * i + 4);
    bf16x8 r;
    r[0] = (bf16)(a.x * scale); r[1] = (bf16)(a.y * scale); r[2] = (bf16)(a.z * scale); r[3] = (bf16)(a.w * scale);
    r[4] = (bf16)(c.x * scale); r[5] = (bf16)(c.y * scale); r[6] = (bf16)(c.z * scale); r[7] = (bf16)(c.w * scale);
    *(bf16x8*)(dq + 8 * i) = r;
  }
}

// ------------------------------------------------------------------ main
template <int D>
struct BwdCfg {
  static constexpr int NW = 4;
  static constexpr int DS = D > 256 ? 2 : 1;     // waves sharing one key block (head-dim split)
  static constexpr int NWK = NW / DS;            // key blocks per workgroup
  static constexpr int BKT = 32 * NWK;           // keys per workgroup
  static constexpr int DW = D / DS;              // head-dim slice of one wave for dK/dV
  static constexpr int BQ = 32;                  // query rows per step
  static constexpr int LDK = D + 8;              // LDS row stride of K/Q/dO tiles
  static constexpr int LDS_T = BQ + 8;           // LDS row stride of the dS^T tile
  static constexpr int NDQ = D / 32;             // 32-wide dQ column blocks
  static constexpr int DQB = NDQ >= NW ? NDQ / NW : 1;   // dQ column blocks per wave
  static constexpr int KSPLIT = NDQ >= NW ? 1 : NW / NDQ;  // waves sharing one dQ block (split keys)
  static constexpr size_t K_OFF = 0;
  static constexpr size_t Q_OFF = K_OFF + (size_t)BKT * LDK * 2;
  static constexpr size_t DO_OFF = Q_OFF + (size_t)BQ * LDK * 2;
  static constexpr size_t DS_OFF = DO_OFF + (size_t)BQ * LDK * 2;
  static constexpr size_t X_OFF = DS_OFF + (size_t)BKT * LDS_T * 2;   // fp32 partial exchange (DS == 2)
  static constexpr size_t LDS_BYTES = X_OFF + (DS == 2 ? (size_t)NW * 16 * 64 * 4 : 0);
};

// Add the partner wave's partial C tile (DS == 2): both waves end with the same sum.
template <int NW>
SDPA_DEV void exchange_add(f32x16& c, float* xbuf, int w, int lane) {
#pragma unroll
  for (int i = 0; i < 16; i++) xbuf[(w * 16 + i) * 64 + lane] = c[i];
  __syncthreads();
  const int p = w ^ 1;
#pragma unroll
  for (int i = 0; i < 16; i++) c[i] += xbuf[(p * 16 + i) * 64 + lane];
  __syncthreads();
}

template <int D>
__global__ void __launch_bounds__(256, 1)
bwd_main_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
                const bf16* __restrict__ dO, const float* __restrict__ LSE,
                const float* __restrict__ Delta, float* __restrict__ dq_acc, bf16* __restrict__ dK,
                bf16* __restrict__ dV, int Hq, int group, int L, int w_eff, float scale,
                float scale_log2) {
  using C = BwdCfg<D>;
  constexpr int LDK = C::LDK, LDS_T = C::LDS_T, DW = C::DW, NDW = DW / 32, NKW = DW / 16;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  bf16* Ks = reinterpret_cast<bf16*>(smem_raw + C::K_OFF);
  bf16* Qs = reinterpret_cast<bf16*>(smem_raw + C::Q_OFF);
  bf16* dOs = reinterpret_cast<bf16*>(smem_raw + C::DO_OFF);
  bf16* dSt = reinterpret_cast<bf16*>(smem_raw + C::DS_OFF);
  float* xbuf = reinterpret_cast<float*>(smem_raw + C::X_OFF);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hh = lane >> 5;
  const int kwi = w / C::DS, dsi = w % C::DS;   // key block and head-dim slice of this wave
  const int dw0 = dsi * DW;
  const int kt = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int Hkv = Hq / group;
  const int k0 = kt * C::BKT;
  const int kb0 = k0 + 32 * kwi;                // first key of this wave's block
  const int kj = kb0 + (lane & 31);             // key held by this lane (C-tile column)
  const bf16* Kg = K + (size_t)(b * Hkv + g) * L * D;
  const bf16* Vg = V + (size_t)(b * Hkv + g) * L * D;

  load_tile<D, 256>(Ks, LDK, Kg + (size_t)k0 * D, C::BKT, L - k0, tid);
  // V_w^T as B operands of dP: lane holds key kj, d-slots dw0 + 16*s + 8*hh + 0..7
  bf16x8 vreg[NKW];
#pragma unroll
  for (int s = 0; s < NKW; s++)
    vreg[s] = kj < L ? *(const bf16x8*)(Vg + (size_t)kj * D + dw0 + 16 * s + 8 * hh) : zero_bf16x8();

  f32x16 dkacc[NDW], dvacc[NDW];
#pragma unroll
  for (int d = 0; d < NDW; d++) { dkacc[d] = zero16(); dvacc[d] = zero16(); }

  // query tiles that can see any key of this workgroup
  const int klast = min(k0 + C::BKT - 1, L - 1);
  const int qt_lo = k0 / C::BQ;
  const int qt_hi = min(L - 1, klast + w_eff - 1) / C::BQ;

  // dQ slice of this wave
  const int dq_blk0 = (w / C::KSPLIT) * C::DQB;           // first 32-wide dQ column block
  const int dq_ks = w % C::KSPLIT;                        // key split for D < 128
  constexpr int DQ_KEYS = C::BKT / C::KSPLIT;

  for (int hq = g * group; hq < (g + 1) * group; hq++) {
    const bf16* Qh = Q + (size_t)(b * Hq + hq) * L * D;
    const bf16* dOh = dO + (size_t)(b * Hq + hq) * L * D;
    const float* lse_h = LSE + (size_t)(b * Hq + hq) * L;
    const float* del_h = Delta + (size_t)(b * Hq + hq) * L;
    float* dqa_h = dq_acc + (size_t)(b * Hq + hq) * L * D;

    for (int qt = qt_lo; qt <= qt_hi; qt++) {
      const int q0 = qt * C::BQ;
      __syncthreads();  // previous step is done with Q/dO/dS^T
      load_tile<D, 256>(Qs, LDK, Qh + (size_t)q0 * D, C::BQ, L - q0, tid);
      load_tile<D, 256>(dOs, LDK, dOh + (size_t)q0 * D, C::BQ, L - q0, tid);

      // lse (log2 domain) and Delta for the 16 query rows this lane's C tile holds
      float lse2[16], del[16];
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const int qi = q0 + c_row(i, hh);
        lse2[i] = qi < L ? lse_h[qi] * kLog2e : 0.f;
        del[i] = qi < L ? del_h[qi] : 0.f;
      }
      // wave-uniform classification of (this query tile, this wave's key block)
      const int r0 = q0, r1 = min(q0 + 31, L - 1);
      const bool active = kb0 < L && kb0 <= r1 && kb0 + 31 > r0 - w_eff;
      const bool full = kb0 + 31 <= r0 && kb0 > q0 + 31 - w_eff && q0 + 31 < L;
      __syncthreads();

      f32x16 s_acc = zero16(), dp_acc = zero16();
      if (active) {
#pragma unroll
        for (int s = 0; s < NKW; s++) {
          const int d0 = dw0 + 16 * s;
          s_acc = mfma(ld_op(Qs, LDK, d0, 0, lane), ld_op(Ks, LDK, d0, 32 * kwi, lane), s_acc);
          dp_acc = mfma(ld_op(dOs, LDK, d0, 0, lane), vreg[s], dp_acc);
        }
      }
      if constexpr (C::DS == 2) {  // all waves take part in the exchange barriers
        exchange_add<C::NW>(s_acc, xbuf, w, lane);
        exchange_add<C::NW>(dp_acc, xbuf, w, lane);
      }
      if (active) {
        // P = exp(S - lse) (0 outside the band), dS = P * (dP - Delta)
#pragma unroll
        for (int i = 0; i < 16; i++) {
          float p = __builtin_amdgcn_exp2f(s_acc[i] * scale_log2 - lse2[i]);
          if (!full && !allowed(q0 + c_row(i, hh), kj, w_eff, L)) p = 0.f;
          s_acc[i] = p;
          dp_acc[i] = p * (dp_acc[i] - del[i]);
        }
        const bf16x8 pa0 = c_to_op(s_acc, 0), pa1 = c_to_op(s_acc, 1);
        const bf16x8 da0 = c_to_op(dp_acc, 0), da1 = c_to_op(dp_acc, 1);
#pragma unroll
        for (int d = 0; d < NDW; d++) {
          const int c0 = dw0 + 32 * d;
          dvacc[d] = mfma(pa0, ld_op_tr(dOs, LDK, 0, c0, lane), dvacc[d]);
          dvacc[d] = mfma(pa1, ld_op_tr(dOs, LDK, 16, c0, lane), dvacc[d]);
          dkacc[d] = mfma(da0, ld_op_tr(Qs, LDK, 0, c0, lane), dkacc[d]);
          dkacc[d] = mfma(da1, ld_op_tr(Qs, LDK, 16, c0, lane), dkacc[d]);
        }
      }
      // dS^T (bf16) -> LDS: row = key (lane column), 4 consecutive query rows per write
      if (dsi == 0) {
        bf16* drow = dSt + (32 * kwi + (lane & 31)) * LDS_T;
#pragma unroll
        for (int blk = 0; blk < 4; blk++) {
          bf16x4 v;
#pragma unroll
          for (int r = 0; r < 4; r++) v[r] = active ? (bf16)dp_acc[4 * blk + r] : (bf16)0.f;
          *(bf16x4*)(drow + 8 * blk + 4 * hh) = v;
        }
      }
      __syncthreads();

      // dQ slice: rows q0..q0+31, columns of blocks dq_blk0.., keys of split dq_ks
      f32x16 dq[C::DQB];
#pragma unroll
      for (int c = 0; c < C::DQB; c++) dq[c] = zero16();
      bool any = false;
#pragma unroll
      for (int kb = 0; kb < DQ_KEYS / 32; kb++) {
        const int kbl = dq_ks * DQ_KEYS + 32 * kb;   // key offset inside the workgroup tile
        const int kbg = k0 + kbl;
        const bool act = kbg < L && kbg <= r1 && kbg + 31 > r0 - w_eff;  // same test as the owner wave
        if (!act) continue;
        any = true;
#pragma unroll
        for (int kk = 0; kk < 2; kk++) {
          const bf16x8 a = ld_op_tr(dSt, LDS_T, kbl + 16 * kk, 0, lane);
#pragma unroll
          for (int c = 0; c < C::DQB; c++)
            dq[c] = mfma(a, ld_op_tr(Ks, LDK, kbl + 16 * kk, 32 * (dq_blk0 + c), lane), dq[c]);
        }
      }
      if (any) {
#pragma unroll
        for (int c = 0; c < C::DQB; c++) {
          const int col = 32 * (dq_blk0 + c) + (lane & 31);
#pragma unroll
          for (int i = 0; i < 16; i++) {
            const int qi = q0 + c_row(i, hh);
            if (qi < L) atomicAdd(dqa_h + (size_t)qi * D + col, dq[c][i]);
          }
        }
      }
    }
  }

  // dK = scale * dS^T Q, dV = P^T dO; C tile: column = head-dim index, rows = keys
  bf16* dKg = dK + (size_t)(b * Hkv + g) * L * D;
  bf16* dVg = dV + (size_t)(b * Hkv + g) * L * D;
#pragma unroll
  for (int d = 0; d < NDW; d++) {
    const int col = dw0 + 32 * d + (lane & 31);
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const int key = kb0 + c_row(i, hh);
      if (key < L) {
        dKg[(size_t)key * D + col] = (bf16)(dkacc[d][i] * scale);
        dVg[(size_t)key * D + col] = (bf16)dvacc[d][i];
      }
    }
  }
}

template <int D>
hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const void* dO,
                           const float* lse, void* dq, void* dk, void* dv, float* dq_acc, float* delta,
                           int B, int Hq, int group, int L, int w_eff, float scale, hipStream_t stream,
                           hipEvent_t main_begin, hipEvent_t main_end) {
  using C = BwdCfg<D>;
  const bool timed = main_begin != nullptr && main_end != nullptr;
  const long rows = (long)B * Hq * L;
  constexpr int RPB = 256 / (D / 8);
  hipLaunchKernelGGL(bwd_pre_kernel<D>, dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, stream,
                     (const bf16*)o, (const bf16*)dO, delta, dq_acc, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  auto kern = bwd_main_kernel<D>;
  e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS_BYTES);
  if (e != hipSuccess) return e;
  const int Hkv = Hq / group;
  dim3 grid((L + C::BKT - 1) / C::BKT, Hkv, B);
  if (timed && (e = hipEventRecord(main_begin, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL(kern, grid, dim3(256), C::LDS_BYTES, stream, (const bf16*)q, (const bf16*)k,
                     (const bf16*)v, (const bf16*)dO, lse, delta, dq_acc, (bf16*)dk, (bf16*)dv, Hq, group,
                     L, w_eff, scale, scale * kLog2e);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (timed && (e = hipEventRecord(main_end, stream)) != hipSuccess) return e;
  const long n8 = rows * D / 8;
  const long nblk = std::min<long>((n8 + 255) / 256, 256L * 64);
  hipLaunchKernelGGL(dq_convert_kernel, dim3((unsigned)nblk), dim3(256), 0, stream, dq_acc, (bf16*)dq,
                     scale, n8);
  return hipGetLastError();
}

#define SDPA_INST_BWD(D)                                                                              \
  template hipError_t launch_bwd_bf16<D>(const void*, const void*, const void*, const void*,         \
                                         const void*, const float*, void*, void*, void*, float*,     \
                                         float*, int, int, int, int, int, float, hipStream_t,      \
                                         hipEvent_t, hipEvent_t);
SDPA_INST_BWD(64)
SDPA_INST_BWD(128)
SDPA_INST_BWD(256)
SDPA_INST_BWD(512)

}  // namespace sdpa
