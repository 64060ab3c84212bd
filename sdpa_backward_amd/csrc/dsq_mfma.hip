// The two kernels around the key-stationary dK/dV pass when the backward keeps
// dS for a bounded band (sliding-window masks):
//
//   delta_kernel  Delta_i = <dO_i, O_i> over the head dimension, fp32, one
//                 value per query row (the row term of dS = P (dP - Delta);
//                 page "Lab 028 lab detail: Off NVIDIA, you fix the platform
//                 yourself", section "2026-10-21", "What the code says", where
//                 the backward forms P and dS per element).
//   dsq_kernel    dQ = scale * dS K from the dS^T tiles that the dK/dV pass
//                 wrote (the pages' backward likewise sums dQ over the key
//                 tiles of each query block, section "What I changed, in plain
//                 terms", item 5(a)); no score is recomputed here.
//
// The band buffer. For each (batch, q-head) and each block of kBandRows = 128
// query rows qb, the keys that some row of the block may see lie in the
// kBandKeys = 64-key tiles kt_lo(qb) .. kt_hi(qb), kt_lo = max(0, 128 qb + dlo)
// / 64; the host sizes every block for the widest range, nkb tiles. dS^T of
// tile kt of block qb is a row-major [64 keys][128 rows] 16-bit tile (16 KB) at
//   ((bh * nqb + qb) * nkb + (kt - kt_lo)) * 64 * 128   elements.
// The dK/dV pass writes the pairs it visits: every allowed pair, and zeros for
// the masked pairs of its edge tiles. Other entries of the rectangle are never
// written, so this kernel masks its edge tiles itself.
//
// dQ^T (D x 32 rows, per wave) += K^T (D x 16 keys) . dS^T (16 keys x 32 rows)
// on v_mfma_f32_32x32x16: A = K^T and B = dS^T both come from swizzled LDS
// tiles by transposed reads (rows of both tiles are the keys), so the
// key-major dS^T that the dK/dV lanes hold becomes the row-major operand the
// dQ product needs inside the read.
#include "common.h"

namespace sdpa {

// Delta_i = <dO_i, O_i> in fp32: D / 8 lanes per row, 8 elements (16 bytes) of
// each tensor per lane, then a butterfly sum over those lanes. Contiguous
// [rows][D] tensors.
template <int D, typename E>
__global__ void __launch_bounds__(256) delta_kernel(const E* __restrict__ O, const E* __restrict__ dO,
                                                    float* __restrict__ Delta, long long rows) {
  using ex8 = typename Vec<E>::x8;
  constexpr int LPR = D / 8;              // lanes per row
  constexpr int RPW = 256 / LPR;          // rows per workgroup
  const long long row = (long long)blockIdx.x * RPW + threadIdx.x / LPR;
  const int c = threadIdx.x % LPR;
  float s = 0.f;
  if (row < rows) {
    const ex8 a = *(const ex8*)(O + row * D + 8 * c);
    const ex8 b = *(const ex8*)(dO + row * D + 8 * c);
#pragma unroll
    for (int j = 0; j < 8; j++) s += (float)a[j] * (float)b[j];
  }
#pragma unroll
  for (int m = LPR / 2; m > 0; m >>= 1) s += __shfl_xor(s, m);
  if (row < rows && c == 0) Delta[row] = s;
}

// Two workgroups per CU: 32-key tiles keep a workgroup's three stages of K
// tiles and four of dS^T tiles at 80 KB of LDS (half the CU's) and its
// registers at 256 per lane. K tiles are loaded two steps ahead, the dS^T
// tiles (which stream from HBM once) three, and one workgroup's MFMAs run
// while the other waits.
template <int D, typename E>
__global__ void __launch_bounds__(256, 2)
dsq_kernel(const E* __restrict__ dST, const E* __restrict__ K, E* __restrict__ dQ, int Hq, int group, int Lq,
           int Lk, int dlo, int dhi, int nqb, int nkb, float scale) {
  using ex4 = typename Vec<E>::x4;
  using ex8 = typename Vec<E>::x8;
  constexpr int NW = 4, BQ = kBandRows, BK = 32, NDB = D / 32, NKS = BK / 16;
  constexpr int KT = BK * D, ST = BK * BQ;
  static_assert(kBandKeys % BK == 0, "a band tile holds whole key tiles of this kernel");
  // (separate arrays: the compiler then knows that loads into one buffer
  // cannot change another and keeps the LDS waits partial)
  __shared__ __attribute__((aligned(16))) E kb0[KT];
  __shared__ __attribute__((aligned(16))) E kb1[KT];
  __shared__ __attribute__((aligned(16))) E kb2[KT];
  __shared__ __attribute__((aligned(16))) E sb0[ST];
  __shared__ __attribute__((aligned(16))) E sb1[ST];
  __shared__ __attribute__((aligned(16))) E sb2[ST];
  __shared__ __attribute__((aligned(16))) E sb3[ST];

  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  LaneAddr<D> la;  // K tiles [BK][D]
  la.init(lane);
  // transposed reads of this wave's 32 rows (columns 32 w..) of a dS^T tile
  // [BK keys][128 rows]: the two 4-key halves of the paired k-slots, as in
  // LaneAddr<128> for column block w (computed here directly: an array
  // indexed by the wave index would live in scratch memory)
  uint32_t s_off[2];
  {
    const int G = lane >> 4, i = lane & 15, row = 4 * (G >> 1) + (i >> 2);
    const int c = 4 * w + 2 * (G & 1) + ((i & 3) >> 1);
#pragma unroll
    for (int h = 0; h < 2; h++)
      s_off[h] = (row + 8 * h) * BQ * 2 + (Tile<BQ>::slot(row + 8 * h, c) & 15) * 16 + (i & 1) * 8;
  }

  // the q-heads of a kv group innermost, then row blocks, so neighbouring
  // workgroups (one XCD's contiguous range) read the same K tiles
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int Hkv = Hq / group;
  const int hg = logical % group, qb = (logical / group) % nqb, bg = logical / (group * nqb);
  const int g = bg % Hkv, b = bg / Hkv, h = g * group + hg, bh = b * Hq + h;
  const E* Kg = K + ((size_t)b * Hkv + g) * Lk * D;

  const int i0 = qb * BQ, i1 = min(i0 + BQ - 1, Lq - 1);
  const int klo = max(0, i0 + dlo), khi = min(Lk - 1, i1 + dhi);
  const int kt_lo = klo / BK, nt = klo <= khi ? khi / BK - kt_lo + 1 : 0;
  // the block's band tiles start at key tile max(0, i0 + dlo) / kBandKeys
  const E* Sb = dST + (size_t)(bh * (long long)nqb + qb) * nkb * (kBandKeys * BQ) +
                (size_t)(kt_lo - klo / kBandKeys * (kBandKeys / BK)) * ST;
  const int wr0 = i0 + 32 * w, wr1 = min(wr0 + 31, Lq - 1);  // this wave's rows (wr1 < wr0: none)
  const int qi = wr0 + (lane & 31);
  // this row's keys: [jhi - span + 1, jhi] (span 0: none, or no such row)
  const int jhi = min(Lk - 1, qi + dhi), jlo = max(0, qi + dlo);
  const int span = qi < Lq && jhi >= jlo ? jhi - jlo + 1 : 0;

  TileLoader<D, BK, NW, true> ldk;
  ldk.init(w, lane, D);
  TileLoader<BQ, BK, NW, true> lds;
  lds.init(w, lane, BQ);
  using LK = decltype(ldk);
  using LS = decltype(lds);
  // every step issues the same number of loads per wave, K blocks first (past
  // the last tile they cover no rows), so "tile t + 1 landed" after step t
  // is: at most step t's loads and step t - 1's dS^T loads still outstanding
  // (they complete in order)
  constexpr int NLD = LK::NJ + LS::NJ;
  static_assert(LK::PER % NW == 0 && LS::PER % NW == 0, "every wave issues every step's loads");

  f32x16 acc[NDB];
#pragma unroll
  for (int d = 0; d < NDB; d++) acc[d] = zero16();

  // one key tile: first the loads of K tile t + 2 and dS^T tile t + 3 (into the
  // buffers tile t - 1 used), from every wave whether or not its rows meet
  // this tile. Issued ahead of the branch, they leave the compiler's tracking
  // of loads into LDS exact at the first operand read: after a branch that
  // issued them on one side only, it made that read wait for every load in
  // flight, the next tiles' included.
  auto step = [&](int t, const E* Kc, const E* Sc, E* Kn, E* Sn) {
    const int j0 = (kt_lo + t) * BK;
    const bool more = t + 2 < nt, more3 = t + 3 < nt;
    const int jn = more ? j0 + 2 * BK : 0;
    const auto krs = ldk.rsrc(Kg + (size_t)jn * D, more ? Lk - jn : 0);
    const auto srs = lds.rsrc(Sb + (size_t)(more3 ? t + 3 : 0) * ST, more3 ? BK : 0);
    auto load_one = [&, krs, srs](int j) {  // K blocks, then dS^T blocks
      if (j < LK::NJ) ldk.issue_one(Kn, krs, j, w);
      else lds.issue_one(Sn, srs, j - LK::NJ, w);
    };
    const bool active = wr0 <= wr1 && j0 <= wr1 + dhi && j0 + BK - 1 >= wr0 + dlo;
    const bool full = wr1 == wr0 + 31 && j0 >= wr1 + dlo && j0 + BK - 1 <= wr0 + dhi && j0 + BK <= Lk;
#pragma unroll
    for (int j = 0; j < NLD; j++) load_one(j);
    if (!active) return;
    // B operands: dS^T rows [16 s, 16 s + 16) (keys), column = this lane's row,
    // paired k-slots j <-> key 16 s + 8 (j / 4) + 4 hh + (j % 4); masked on edge tiles
    ex8 bop[NKS];
#pragma unroll
    for (int s = 0; s < NKS; s++) {
      const char* base = reinterpret_cast<const char*>(Sc) + 16 * s * BQ * 2;
      const ex4 lo = lds_tr4<E>(base + s_off[0]), hi = lds_tr4<E>(base + s_off[1]);
      bop[s] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      if (!full) {
        const int kb = jhi - (j0 + 16 * s + 4 * hh);
#pragma unroll
        for (int j = 0; j < 8; j++)
          if (!in_band(kb, 8 * (j >> 2) + (j & 3), span)) bop[s][j] = (E)0.f;
      }
    }
    constexpr int NM = NKS * NDB, AH = 4;
    ex8 ka[AH];
    auto rd = [&](int k) { ka[k % AH] = op_tr<D, E>(Kc, la, 16 * (k / NDB), 32 * (k % NDB)); };
#pragma unroll
    for (int k = 0; k < AH; k++) rd(k);
#pragma unroll
    for (int k = 0; k < NM; k++) {
      acc[k % NDB] = mfma(ka[k % AH], bop[k / NDB], acc[k % NDB]);
      if (k + AH < NM) rd(k + AH);
    }
  };

  constexpr int WAITN = NLD + LS::NJ;
  if (nt > 0) {
    zero_lds(kb0, KT, tid);
    zero_lds(kb1, KT, tid);
    zero_lds(kb2, KT, tid);
    lds_barrier();
    const int j1 = nt > 1 ? (kt_lo + 1) * BK : 0;
    ldk.issue(kb0, Kg + (size_t)kt_lo * BK * D, Lk - kt_lo * BK, w);
    lds.issue(sb0, Sb, BK, w);
    lds.issue(sb1, Sb + (nt > 1 ? ST : 0), nt > 1 ? BK : 0, w);
    ldk.issue(kb1, Kg + (size_t)j1 * D, nt > 1 ? Lk - j1 : 0, w);
    lds.issue(sb2, Sb + (nt > 2 ? 2 * ST : 0), nt > 2 ? BK : 0, w);
    wait_vm_and_barrier<WAITN>();
  }
  // 12 steps per loop iteration (K buffers rotate by 3, dS^T buffers by 4);
  // at the loop head the compiler still makes the first operand read wait for
  // the loads of the step before, once per 12 steps
#define DSQ_STEP(I)                                                                              \
  if (t + I >= nt) break;                                                                        \
  step(t + I, I % 3 == 0 ? kb0 : I % 3 == 1 ? kb1 : kb2,                                          \
       I % 4 == 0 ? sb0 : I % 4 == 1 ? sb1 : I % 4 == 2 ? sb2 : sb3,                               \
       (I + 2) % 3 == 0 ? kb0 : (I + 2) % 3 == 1 ? kb1 : kb2,                                      \
       (I + 3) % 4 == 0 ? sb0 : (I + 3) % 4 == 1 ? sb1 : (I + 3) % 4 == 2 ? sb2 : sb3);            \
  wait_vm_and_barrier<WAITN>();
  for (int t = 0; t < nt; t += 12) {
    DSQ_STEP(0) DSQ_STEP(1) DSQ_STEP(2) DSQ_STEP(3) DSQ_STEP(4) DSQ_STEP(5)
    DSQ_STEP(6) DSQ_STEP(7) DSQ_STEP(8) DSQ_STEP(9) DSQ_STEP(10) DSQ_STEP(11)
  }
#undef DSQ_STEP
  wait_all_and_barrier();  // (the last steps' no-op loads)

  // C tile = dQ^T: lane's column is its row, accumulator slot i holds head-dim
  // index 32 d + c_row(i, hh). The wave's 32 rows go out through LDS (no wave
  // reads the tile buffers any more): as global stores a lane's 4 consecutive
  // columns are 8-byte pieces of 32 rows each, staged each store writes 1 KB
  // of whole rows. Waves 0-2 stage in their K buffer (32 x D), wave 3 rows
  // 0-15 in sb0 and 16-31 in sb1 (16 x D each). Staging rows have a pitch of
  // D, their 16-byte chunks permuted (chunk c of row r at c ^ (r mod CPR)) so
  // that the 32 rows one store instruction writes fall in distinct banks.
  {
    constexpr int CPR = D / 8, NCH = 32 * CPR / 64;  // 16-byte chunks per row, per lane
    static_assert(KT == 32 * D && ST >= 16 * D, "a K buffer holds 32 staged rows, a dS^T buffer 16");
    E* const lo = w == 0 ? kb0 : w == 1 ? kb1 : w == 2 ? kb2 : sb0;  // rows 0-15
    E* const hi = w == 3 ? sb1 : lo + 16 * D;                        // rows 16-31
    auto stg = [&](int row) { return row < 16 ? lo + row * D : hi + (row - 16) * D; };
    const int r = lane & 31;
#pragma unroll
    for (int d = 0; d < NDB; d++)
#pragma unroll
      for (int blk = 0; blk < 4; blk++) {
        ex4 v;
#pragma unroll
        for (int i = 0; i < 4; i++) v[i] = (E)(acc[d][4 * blk + i] * scale);
        *(ex4*)(stg(r) + (((4 * d + blk) ^ (r % CPR)) * 8) + 4 * hh) = v;
      }
    wave_lds_sync();
    E* o0 = dQ + ((size_t)bh * Lq + wr0) * D;
#pragma unroll
    for (int k = 0; k < NCH; k++) {
      const int c = lane + 64 * k, row = c / CPR, j = c % CPR;
      const ex8 v = *(const ex8*)(stg(row) + ((j ^ (row % CPR)) * 8));
      if (wr0 + row < Lq) *(ex8*)(o0 + (size_t)row * D + 8 * j) = v;
    }
  }
}

template <int D, typename E>
hipError_t launch_delta(const void* o, const void* dO, float* delta, long long rows, hipStream_t stream) {
  constexpr int RPW = 256 / (D / 8);
  const long long nwg = (rows + RPW - 1) / RPW;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
  if (nwg == 0) return hipSuccess;
  hipLaunchKernelGGL((delta_kernel<D, E>), dim3((unsigned)nwg), dim3(256), 0, stream, (const E*)o, (const E*)dO,
                     delta, rows);
  return hipGetLastError();
}

template <int D, typename E>
hipError_t launch_dsq(const void* dst, const void* k, void* dq, int B, int Hq, int group, int Lq, int Lk, int dlo,
                      int dhi, int nqb, int nkb, float scale, hipStream_t stream) {
  const long nwg = (long)nqb * Hq * B;
  if (nwg > 0x7fffffffL) return hipErrorInvalidValue;
  if (nwg == 0) return hipSuccess;
  hipLaunchKernelGGL((dsq_kernel<D, E>), dim3((unsigned)nwg), dim3(256), 0, stream, (const E*)dst, (const E*)k,
                     (E*)dq, Hq, group, Lq, Lk, dlo, dhi, nqb, nkb, scale);
  return hipGetLastError();
}

#define SDPA_INST_DSQ(D, E)                                                                                 \
  template hipError_t launch_delta<D, E>(const void*, const void*, float*, long long, hipStream_t);          \
  template hipError_t launch_dsq<D, E>(const void*, const void*, void*, int, int, int, int, int, int, int, int, \
                                       int, float, hipStream_t);
SDPA_INST_DSQ(256, bf16)
SDPA_INST_DSQ(256, f16)

}  // namespace sdpa
