// Query-stationary attention kernels for gfx950 (bf16 or fp16 in, fp32 accumulate):
//
//   QS_FWD  forward: O and the per-row logsumexp (lse) that the backward reuses
//           (page "Lab 028 lab detail: Off NVIDIA, you fix the platform
//           yourself", section "What I changed, in plain terms", item 1)
//   QS_DQ   backward for dQ: recompute P = exp(S - lse) per key tile, form
//           dS = P * (dP - Delta) per element (same page, section "2026-10-21",
//           "What the code says") and accumulate dQ = scale * dS K; also
//           computes Delta_i = <dO_i, O_i> for its rows and stores it for the
//           key-stationary dK/dV kernel.
//
// One workgroup = 4 waves = BQ query rows of one (b, h). Each wave owns 32 rows
// (for D = 512 two waves share 32 rows and split the head dimension, adding
// their partial score tiles through LDS). The loop walks key tiles of BK keys
// in the mask's band only (tiles wholly outside it, above the diagonal, behind
// or ahead of a window, are never visited; a wave skips tiles outside its own
// rows' band, and applies the element mask only on edge tiles). K and V tiles stream into
// double-buffered LDS with asynchronous global->LDS loads.
//
// Per key tile, per wave (C tiles are 32x32 fp32, one query per lane column):
//   S^T  = K_tile . Q_w^T                  A: K (LDS, direct)  B: Q_w (registers)
//   FWD: online softmax in the log2 domain, fp32 state; the running max is only
//        raised when a tile exceeds it by more than 8 (2^8 headroom), so the
//        O rescale runs rarely; P^T feeds  O^T += V^T . P^T  (A: V, transposed reads)
//   DQ:  dP^T = V_tile . dO_w^T             A: V (LDS, direct)  B: dO_w (registers)
//        P^T = exp2(S^T c - lse2), dS^T = P^T (dP^T - Delta)
//        dQ^T += K^T . dS^T                 A: K (transposed reads) B: dS^T (C tile reused)
// S, P, dP stay fp32; only P and dS are rounded to the input type as MFMA operands
// (section "fp32 score tiles" of the Lab 028 page).
//
// Small grids (fewer workgroups than CUs): each query tile's key tiles are
// split into nseg consecutive ranges, one workgroup each. A workgroup then
// writes fp32 partial results instead of its outputs: the forward its
// unnormalised O rows with their used max m and row sum l, the dQ pass its
// unscaled dQ rows; a combine pass merges them (O = sum_s 2^(m_s - M) O_s /
// sum_s 2^(m_s - M) l_s with M = max_s m_s, and lse from M and that sum; dQ
// = scale sum_s dQ_s), the split-softmax merge of the online softmax.
#include <algorithm>
#include <type_traits>

#include "common.h"

namespace sdpa {

enum { QS_FWD = 0, QS_DQ = 1 };

// How many MFMAs ahead the LDS operand reads are issued (S / dP products, and
// the O / dQ products). Deeper look-ahead hides LDS latency at the cost of
// operand registers.
#ifndef QS_AHEAD_S
#define QS_AHEAD_S 4
#endif
#ifndef QS_AHEAD_O
#define QS_AHEAD_O 4
#endif

// Head dim 512 in the forward: each wave holds all of a row block's O (256
// accumulator registers) and its Q rows in VGPRs (QS_FWD512_FULL), or wave
// pairs split the head dim.
#ifndef QS_FWD512_FULL
#define QS_FWD512_FULL 1
#endif
template <int D, int MODE = 1>
struct QsCfg {
  static constexpr int NW = 4;
  static constexpr int DS = D > 256 && !(MODE == 0 && QS_FWD512_FULL) ? 2 : 1;  // waves sharing one 32-row block (head-dim split)
  static constexpr int NQW = NW / DS;           // 32-row blocks per workgroup
  static constexpr int BQ = 32 * NQW;           // query rows per workgroup
  static constexpr int DW = D / DS;             // head-dim slice of one wave
  static constexpr int BK = D > 256 ? 32 : 64;  // keys per tile
  static constexpr int NMB = BK / 32;           // 32-key blocks per tile
  static constexpr int TILE = BK * D;           // elements of one K (or V) tile
};

// Partial C tiles of the two waves that split the head dimension: each adds
// the partner's tiles (same lane layout), so both end with identical sums.
template <int N>
SDPA_DEV void exchange_add(f32x16 (&c)[N], float* xbuf, int w, int lane) {
#pragma unroll
  for (int t = 0; t < N; t++)
#pragma unroll
    for (int i = 0; i < 16; i++) xbuf[((w * N + t) * 16 + i) * 64 + lane] = c[t][i];
  lds_barrier();
  const int p = w ^ 1;
#pragma unroll
  for (int t = 0; t < N; t++)
#pragma unroll
    for (int i = 0; i < 16; i++) c[t][i] += xbuf[((p * N + t) * 16 + i) * 64 + lane];
}

template <int D, int MODE, typename E, bool DENSE>
__global__ void __launch_bounds__(256, 1)
qs_kernel(const E* __restrict__ Q, const E* __restrict__ K, const E* __restrict__ V,
          const E* __restrict__ O, const E* __restrict__ dO, float* __restrict__ LSE,
          float* __restrict__ Delta, E* __restrict__ Out, const float* __restrict__ Sinks, int Hq, int group,
          int Lq, int Lk, int dlo, int dhi, Cut cut_arg, float scale, float scale_log2, AllStrides st_arg,
          int nseg, float* __restrict__ part) {
  using C = QsCfg<D, MODE>;
  using ex8 = typename Vec<E>::x8;
  using ex4 = typename Vec<E>::x4;
  constexpr int BK = C::BK, NMB = C::NMB, DW = C::DW, NKS = DW / 16, NDB = DW / 32;
  constexpr int NX = MODE == QS_DQ ? 2 * NMB : NMB;  // C tiles exchanged when the head dim is split
  __shared__ __attribute__((aligned(16))) E kb0[C::TILE];
  __shared__ __attribute__((aligned(16))) E kb1[C::TILE];
  __shared__ __attribute__((aligned(16))) E vb0[C::TILE];
  __shared__ __attribute__((aligned(16))) E vb1[C::TILE];
  __shared__ __attribute__((aligned(16))) float xbuf[C::DS == 2 ? C::NW * NX * 1024 : 4];

  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform (SGPR)
  LaneAddr<D> la;  // per-lane LDS offsets of the operand read patterns
  la.init(lane);
  const AllStrides st = DENSE ? dense_strides<D>(Hq, Hq / group, Lq, Lk) : st_arg;
  const Cut cut = DENSE ? kNoCut : cut_arg;  // no cut in the dense instantiation
  // per-lane source offsets of the K and V tile loads (the two share their row
  // stride: the host checks it)
  TileLoader<D, C::BK, C::NW, DENSE> ldk;
  ldk.init(w, lane, st.k.l);
  const auto& ldv = ldk;
  const int qwi = w / C::DS, dsi = w % C::DS, dw0 = dsi * DW;
  const int nqt = (Lq + C::BQ - 1) / C::BQ;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int seg = logical % nseg, lw = logical / nseg;  // key range seg of query tile lw
  const int qt = nqt - 1 - lw % nqt;  // longest causal rows first within a head
  const int h = (lw / nqt) % Hq, b = lw / (nqt * Hq);
  const int Hkv = Hq / group, g = h / group;
  const size_t hrow = (size_t)b * Hq + h;  // lse / Delta row block
  const E* Kg = DENSE ? K + ((size_t)b * Hkv + g) * Lk * D : K + b * st.k.b + g * st.k.h;
  const E* Vg = DENSE ? V + ((size_t)b * Hkv + g) * Lk * D : V + b * st.v.b + g * st.v.h;

  const int i0 = qt * C::BQ, iw0 = i0 + 32 * qwi;
  const int qi = iw0 + (lane & 31);  // this lane's query row
  const bool qok = qi < Lq;
  // this row's keys: [jhi - span + 1, jhi] (span 0: none, or the row does not
  // exist), and from the cut row on a second range [jhi2 - span2 + 1, jhi2]:
  // the first is then the band from c1 on, the second the band moved back by
  // the cut's shift, clipped to the keys before c0 (the dense instantiation
  // has no cut: span2 = 0)
  int jhi = min(Lk - 1, qi + dhi), jlo = max(0, qi + dlo), jhi2 = 0, span2 = 0;
  if (!DENSE && qi >= cut.r0 && cut.c0 < cut.c1) {
    jlo = max(jlo, cut.c1);
    jhi2 = min(min(cut.c0 - 1, Lk - 1), qi + dhi - cut.sh);
    const int jlo2 = max(0, qi + dlo - cut.sh);
    span2 = qok && jhi2 >= jlo2 ? jhi2 - jlo2 + 1 : 0;
  }
  const int span = qok && jhi >= jlo ? jhi - jlo + 1 : 0;

  // this wave's rows as B operands: row qi, d-slots dw0 + 16*s + 8*hh + 0..7
  ex8 qreg[NKS];
  const E* qrow = Q + b * st.q.b + h * st.q.h + (long long)(qok ? qi : 0) * st.q.l;
#pragma unroll
  for (int s = 0; s < NKS; s++) qreg[s] = qok ? *(const ex8*)(qrow + dw0 + 16 * s + 8 * hh) : zero8<E>();

  ex8 dreg[MODE == QS_DQ ? NKS : 1];
  float lse2 = 0.f, dlt = 0.f;
  if constexpr (MODE == QS_DQ) {
    const E* drow = dO + b * st.dO.b + h * st.dO.h + (long long)(qok ? qi : 0) * st.dO.l;
    const E* orow = O + b * st.o.b + h * st.o.h + (long long)(qok ? qi : 0) * st.o.l;
#pragma unroll
    for (int s = 0; s < NKS; s++) dreg[s] = qok ? *(const ex8*)(drow + dw0 + 16 * s + 8 * hh) : zero8<E>();
    // Delta_i = <dO_i, O_i> over the whole head dimension, fp32
    float dot = 0.f;
    if (qok) {
#pragma unroll 4
      for (int s = 0; s < D / 16; s++) {
        const ex8 a = *(const ex8*)(drow + 16 * s + 8 * hh);
        const ex8 o = *(const ex8*)(orow + 16 * s + 8 * hh);
#pragma unroll
        for (int j = 0; j < 8; j++) dot += (float)a[j] * (float)o[j];
      }
    }
    dlt = dot + __shfl_xor(dot, 32);
    lse2 = qok ? LSE[hrow * Lq + qi] * kLog2e : 0.f;  // -inf for a row with no key (then every p is masked)
    if (qok && dsi == 0 && hh == 0 && seg == 0) Delta[hrow * Lq + qi] = dlt;
  }

  f32x16 acc[NDB];
#pragma unroll
  for (int d = 0; d < NDB; d++) acc[d] = zero16();
  float m = -INFINITY, lsum = 0.f;  // forward: running (used) max in log2 units and row sum
  if constexpr (MODE == QS_FWD) {
    // a sink logit joins the normalizer from the start: it becomes the used
    // max, contributing exp2(m - m) = 1 to the sum (and nothing to O)
    if (Sinks != nullptr && seg == 0) {
      const float sg = Sinks[h] * kLog2e;
      if (sg != -INFINITY) m = sg, lsum = 1.f;
    }
  }

  // key tiles that a row of this workgroup can see: the band's, and with a
  // shifted cut also the moved band's for the rows from r0 on (merged into
  // one range when the two touch); kt(t) is the t-th of the nt tiles
  const int i1 = min(i0 + C::BQ - 1, Lq - 1);
  const int klo = max(0, i0 + dlo), khi = min(Lk - 1, i1 + dhi);
  int kt_lo = klo / BK, kt_hi = klo <= khi ? khi / BK : kt_lo - 1;
  int kt2_lo = 0, nt2 = 0;  // the moved band's tiles, visited first
  if (!DENSE && cut.sh > 0 && cut.c0 < cut.c1 && i1 >= cut.r0) {
    const int lo2 = max(0, max(i0, cut.r0) + dlo - cut.sh), hi2 = min(min(cut.c0 - 1, Lk - 1), i1 + dhi - cut.sh);
    if (lo2 <= hi2) {
      const int a = lo2 / BK, z = hi2 / BK;
      if (kt_lo > kt_hi) kt_lo = a, kt_hi = z;
      else if (z + 1 >= kt_lo && a <= kt_hi + 1) kt_lo = min(kt_lo, a), kt_hi = max(kt_hi, z);
      else kt2_lo = a, nt2 = z - a + 1;
    }
  }
  const int nt = nt2 + max(0, kt_hi - kt_lo + 1);
  auto kt_of = [&](int t) { return t < nt2 ? kt2_lo + t : kt_lo + (t - nt2); };
  // this workgroup's tiles [t_b, t_e) of the nt (all of them without a split)
  const int t_b = (int)((long long)seg * nt / nseg), t_e = (int)((long long)(seg + 1) * nt / nseg);
  const int wr0 = iw0, wr1 = min(iw0 + 31, Lq - 1);  // this wave's rows (wr1 < wr0: none)
  // Rows [valid, BK) of a K and a V tile buffer (keys past Lk, in the last
  // key tile only): the loads do not fill them, and every operand read must
  // be finite (a masked score becomes -inf or p = 0, but 0 times a NaN bit
  // pattern left in LDS is NaN), so they are zeroed before the tile's loads.
  auto zero_tail = [&](E* Kb, E* Vb, int valid) {
    if (valid >= BK) return;
    const i32x4 z = {0, 0, 0, 0};
    for (int i = max(valid, 0) * D + tid * 8; i < C::TILE; i += C::NW * 64 * 8) {
      *(i32x4*)(Kb + i) = z;
      *(i32x4*)(Vb + i) = z;
    }
  };

  auto step = [&](int t, const E* Kc, const E* Vc, E* Kn, E* Vn) {
    const int kt = kt_of(t);
    // The next tile's loads (into the other buffers) are issued one at a time
    // between the score MFMAs below: issued back to back they stall the wave
    // until the CU's vector-memory path has taken the workgroup's whole tile.
    // Each load stays after the LDS reads that precede it in program order
    // (it writes LDS), so the operand reads are software-pipelined by hand and
    // the loads slot in between them. On the last tile the resources cover no
    // rows and the loads read nothing.
    const bool more = t + 1 < t_e;
    const int jn = more ? kt_of(t + 1) * BK : 0;
    if (more) zero_tail(Kn, Vn, Lk - jn);  // (no-op unless tile t + 1 runs past Lk)
    const auto krs = ldk.rsrc(Kg + (long long)jn * st.k.l, more ? Lk - jn : 0);
    const auto vrs = ldv.rsrc(Vg + (long long)jn * st.v.l, more ? Lk - jn : 0);
    using LD = decltype(ldk);
    constexpr int NJ = LD::NJ;
    auto load_one = [&, krs, vrs](int j) {  // j in [0, 2 NJ): K blocks, then V blocks
      if constexpr (LD::PER % C::NW != 0) {
        if ((j % NJ) * C::NW + w >= LD::PER) return;
      }
      if (j < NJ) ldk.issue_one(Kn, krs, j, w);
      else ldv.issue_one(Vn, vrs, j - NJ, w);
    };
#pragma unroll
    for (int s = 0; s < NKS; s++)
      if constexpr (4 * NKS + 16 * NDB <= 256) keep_in_agpr(qreg[s]);  // (at D = 512, Q stays in VGPRs)
#pragma unroll
    for (int d = 0; d < NDB; d++) keep_in_agpr(acc[d]);
    const int j0 = kt * BK;
    // some pair of the wave's rows and the tile's keys allowed / every pair allowed
    bool active, full;
    if constexpr (DENSE) {
      active = wr0 <= wr1 && j0 <= wr1 + dhi && j0 + BK - 1 >= wr0 + dlo;
      full = wr1 == wr0 + 31 && j0 >= wr1 + dlo && j0 + BK - 1 <= wr0 + dhi && j0 + BK <= Lk;
    } else {  // from the lanes' key ranges (the two ranges never touch: c0 < c1)
      const int j1 = j0 + BK - 1;
      auto meets = [&](int hi, int sp) { return sp > 0 && hi >= j0 && hi - sp + 1 <= j1; };
      auto covers = [&](int hi, int sp) { return sp > 0 && hi >= j1 && hi - sp + 1 <= j0; };
      active = __any(meets(jhi, span) || meets(jhi2, span2));
      full = __all(covers(jhi, span) || covers(jhi2, span2));
    }

    // Scores of every wave, also of waves whose rows miss this tile (they
    // would only wait at the tile barrier): no branch around the MFMAs.
    // Operand k (k < NM) is block mb = k / NKS, k-slice s = k % NKS; with
    // dP (dQ pass) every k has two reads and two MFMAs.
    f32x16 st[NX];  // [0, NMB): S^T blocks; [NMB, 2 NMB): dP^T blocks (DQ)
#pragma unroll
    for (int t = 0; t < NX; t++) st[t] = zero16();
    {
      constexpr int NM = NMB * NKS, AH = QS_AHEAD_S, NLD = 2 * NJ;
      constexpr int EVERY = NM / NLD > 0 ? NM / NLD : 1;  // MFMA steps between loads
      ex8 ka[AH], va[MODE == QS_DQ ? AH : 1];
      auto rd = [&](int k) {
        ka[k % AH] = op_direct<D, E>(Kc, la, dw0 + 16 * (k % NKS), 32 * (k / NKS));
        if constexpr (MODE == QS_DQ) va[k % AH] = op_direct<D, E>(Vc, la, dw0 + 16 * (k % NKS), 32 * (k / NKS));
      };
#pragma unroll
      for (int k = 0; k < AH; k++) rd(k);
#pragma unroll
      for (int k = 0; k < NM; k++) {
        const int mb = k / NKS, s = k % NKS;
        st[mb] = mfma(ka[k % AH], qreg[s], st[mb]);
        if constexpr (MODE == QS_DQ) st[NMB + mb] = mfma(va[k % AH], dreg[s], st[NMB + mb]);
        if (k + AH < NM) rd(k + AH);
        if (k % EVERY == EVERY - 1 && k / EVERY < NLD) load_one(k / EVERY);
      }
#pragma unroll
      for (int j = NM / EVERY; j < NLD; j++) load_one(j);  // (when there are more loads than MFMA steps)
    }
    if constexpr (C::DS == 2) exchange_add<NX>(st, xbuf, w, lane);
    if constexpr (MODE == QS_FWD) {
      // the softmax reads every score twice (max, then exp): move them to
      // VGPRs once here rather than out of the accumulator registers twice
#pragma unroll
      for (int t = 0; t < NX; t++) asm volatile("" : "+v"(st[t]));
    }
    if (!active) return;

    if constexpr (MODE == QS_FWD) {
      // The max is taken over raw scores (scale > 0 commutes with it); masked
      // entries become -inf first (edge tiles only).
      float mx = -INFINITY;
      auto scores = [&](auto masked) {
#pragma unroll
        for (int mb = 0; mb < NMB; mb++) {
          const int base = jhi - (j0 + 32 * mb + 4 * hh), base2 = jhi2 - (j0 + 32 * mb + 4 * hh);
#pragma unroll
          for (int i = 0; i < 16; i++) {
            const int r = 8 * (i >> 2) + (i & 3);
            if constexpr (decltype(masked)::value)
              st[mb][i] = in_band(base, r, span) || (!DENSE && in_band(base2, r, span2)) ? st[mb][i] : -INFINITY;
            mx = fmaxf(mx, st[mb][i]);
          }
        }
      };
      if (full) scores(std::false_type{});
      else scores(std::true_type{});
      mx = half_max(mx) * scale_log2;
      const bool need = mx > m + 8.f;  // raise the used max only beyond 2^8 headroom
      if (__any(need && m != -INFINITY)) {  // (the first tile of a row has nothing to rescale)
        const float alpha = need ? __builtin_amdgcn_exp2f(m - mx) : 1.f;
        lsum *= alpha;
        scale_in_agpr(acc, alpha);
      }
      if (need) m = mx;
      const float neg_m = m == -INFINITY ? 0.f : -m;
      float rs = 0.f;
#pragma unroll
      for (int mb = 0; mb < NMB; mb++)
#pragma unroll
        for (int i = 0; i < 16; i++) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(st[mb][i], scale_log2, neg_m));
          st[mb][i] = p;
          rs += p;
        }
      lsum += half_sum(rs);
#pragma unroll
      for (int mb = 0; mb < NMB; mb++) {
        const ex8 p0 = c_to_op<E>(st[mb], 0), p1 = c_to_op<E>(st[mb], 1);
#pragma unroll
        for (int d = 0; d < NDB; d++) {
          acc[d] = mfma(op_tr<D, E>(Vc, la, 32 * mb, dw0 + 32 * d), p0, acc[d]);
          acc[d] = mfma(op_tr<D, E>(Vc, la, 32 * mb + 16, dw0 + 32 * d), p1, acc[d]);
        }
      }
      // schedule: transposed reads run QS_AHEAD_O MFMAs ahead
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * QS_AHEAD_O, 1);
#pragma unroll
      for (int t = 0; t < NMB * NDB; t++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * QS_AHEAD_O, 1);
      }
    } else {
#pragma unroll
      for (int mb = 0; mb < NMB; mb++) {
        const int base = jhi - (j0 + 32 * mb + 4 * hh), base2 = jhi2 - (j0 + 32 * mb + 4 * hh);
        auto form = [&](auto masked) {  // dS^T = P^T (dP^T - Delta), masked on edge tiles
#pragma unroll
          for (int i = 0; i < 16; i++) {
            float p = __builtin_amdgcn_exp2f(__builtin_fmaf(st[mb][i], scale_log2, -lse2));
            const int r = 8 * (i >> 2) + (i & 3);
            if constexpr (decltype(masked)::value)
              p = in_band(base, r, span) || (!DENSE && in_band(base2, r, span2)) ? p : 0.f;
            st[NMB + mb][i] = p * (st[NMB + mb][i] - dlt);
          }
        };
        if (full) form(std::false_type{});
        else form(std::true_type{});
        const ex8 d0 = c_to_op<E>(st[NMB + mb], 0), d1 = c_to_op<E>(st[NMB + mb], 1);
#pragma unroll
        for (int d = 0; d < NDB; d++) {
          acc[d] = mfma(op_tr<D, E>(Kc, la, 32 * mb, dw0 + 32 * d), d0, acc[d]);
          acc[d] = mfma(op_tr<D, E>(Kc, la, 32 * mb + 16, dw0 + 32 * d), d1, acc[d]);
        }
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * QS_AHEAD_O, 1);
#pragma unroll
      for (int t = 0; t < NMB * NDB; t++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * QS_AHEAD_O, 1);
      }
    }
  };

  if (t_e > t_b) {  // first tile (uniform over the workgroup)
    const int j0 = kt_of(t_b) * BK;
    zero_tail(kb0, vb0, Lk - j0);
    ldk.issue(kb0, Kg + (long long)j0 * st.k.l, Lk - j0, w);
    ldv.issue(vb0, Vg + (long long)j0 * st.v.l, Lk - j0, w);
    wait_all_and_barrier();
  }
  for (int t = t_b; t < t_e; t += 2) {
    step(t, kb0, vb0, kb1, vb1);
    wait_all_and_barrier();
    if (t + 1 >= t_e) break;
    step(t + 1, kb1, vb1, kb0, vb0);
    wait_all_and_barrier();
  }

  if (nseg > 1) {  // fp32 partial rows (and the forward's m, l) for the combine pass
    if (!qok) return;
    const size_t rows = (size_t)(gridDim.x / nseg / nqt) * Lq;  // B * Hq * Lq: one partial's rows
    float* prow = part + ((size_t)seg * rows + hrow * Lq + qi) * D;
#pragma unroll
    for (int d = 0; d < NDB; d++)
#pragma unroll
      for (int blk = 0; blk < 4; blk++) {
        const f32x4 v = {acc[d][4 * blk], acc[d][4 * blk + 1], acc[d][4 * blk + 2], acc[d][4 * blk + 3]};
        *(f32x4*)(prow + dw0 + 32 * d + 8 * blk + 4 * hh) = v;
      }
    if (MODE == QS_FWD && dsi == 0 && hh == 0) {
      float* pml = part + (size_t)nseg * rows * D + ((size_t)seg * rows + hrow * Lq + qi) * 2;
      pml[0] = m;
      pml[1] = lsum;
    }
    return;
  }
  // The wave's 32 output rows (O / lsum, or scale dQ) go out through LDS: a
  // lane holds 4 consecutive columns of one row per C tile, which as global
  // stores are 8-byte pieces of 32 rows each; staged in the wave's own tile
  // buffer (the loop ended with a barrier, so no wave reads the buffers any
  // more; with no tile they were never used), each store writes 1 KB of whole
  // rows instead. Staging rows have a pitch of DW elements, their 16-byte
  // chunks permuted (chunk c of row r at c ^ (r mod CPR)) so that the 32 rows
  // one store instruction writes fall in distinct banks.
  {
    const float mul = MODE == QS_FWD ? (lsum > 0.f ? 1.f / lsum : 0.f) : scale;
    constexpr int CPR = DW / 8, NCH = 32 * CPR / 64;  // 16-byte chunks per row, per lane
    static_assert(32 * DW <= C::TILE, "the staging rows fit one tile buffer");
    E* stg = w == 0 ? kb0 : w == 1 ? kb1 : w == 2 ? vb0 : vb1;
    const int r = lane & 31;
#pragma unroll
    for (int d = 0; d < NDB; d++)
#pragma unroll
      for (int blk = 0; blk < 4; blk++) {
        ex4 v;
#pragma unroll
        for (int rr = 0; rr < 4; rr++) v[rr] = (E)(acc[d][4 * blk + rr] * mul);
        *(ex4*)(stg + r * DW + (((4 * d + blk) ^ (r % CPR)) * 8) + 4 * hh) = v;
      }
    wave_lds_sync();
    const Strides so = MODE == QS_FWD ? st.o : st.dq;
    E* o0 = Out + b * so.b + h * so.h + (long long)iw0 * so.l + dw0;
#pragma unroll
    for (int k = 0; k < NCH; k++) {
      const int c = lane + 64 * k, row = c / CPR, j = c % CPR;
      const ex8 v = *(const ex8*)(stg + row * DW + ((j ^ (row % CPR)) * 8));
      if (iw0 + row < Lq) *(ex8*)(o0 + (long long)row * so.l + 8 * j) = v;
    }
  }
  if (MODE == QS_FWD && qok && dsi == 0 && hh == 0)
    LSE[hrow * Lq + qi] = lsum > 0.f ? (m + __log2f(lsum)) * kLn2 : -INFINITY;
}

// Combine pass of a split call: one thread per 8 columns of a row (rows =
// B * Hq * Lq). Forward: O and lse from the nseg partial (O, m, l) of the row,
// as the online softmax would have reached them over all its key tiles; a row
// whose partials saw no key (and no sink) gets O = 0 and lse = -inf. dQ pass:
// scale times the sum of the partials, in segment order.
template <int D, int MODE, typename E>
__global__ void __launch_bounds__(256)
qs_combine_kernel(const float* __restrict__ part, E* __restrict__ Out, float* __restrict__ LSE, int nseg,
                  long long rows, int Hq, int Lq, Strides so, float scale) {
  using ex8 = typename Vec<E>::x8;
  constexpr int C8 = D / 8;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows * C8) return;
  const long long row = idx / C8;
  const int c = (int)(idx % C8) * 8;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float mul = scale, M = -INFINITY, L = 0.f;
  if constexpr (MODE == QS_FWD) {
    const float* pml = part + (size_t)nseg * rows * D;
    for (int sg = 0; sg < nseg; sg++) M = fmaxf(M, pml[((size_t)sg * rows + row) * 2]);
    for (int sg = 0; sg < nseg; sg++) {
      const float ms = pml[((size_t)sg * rows + row) * 2], ls = pml[((size_t)sg * rows + row) * 2 + 1];
      if (ls > 0.f) L += __builtin_amdgcn_exp2f(ms - M) * ls;
    }
    mul = L > 0.f ? 1.f / L : 0.f;
  }
  for (int sg = 0; sg < nseg; sg++) {
    float wgt = 1.f;
    if constexpr (MODE == QS_FWD) {
      const float ms = part[(size_t)nseg * rows * D + ((size_t)sg * rows + row) * 2];
      wgt = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - M);
    }
    const f32x4* p = (const f32x4*)(part + ((size_t)sg * rows + row) * D + c);
    const f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int j = 0; j < 4; j++) o[j] += wgt * a[j], o[4 + j] += wgt * b[j];
  }
  ex8 v;
#pragma unroll
  for (int j = 0; j < 8; j++) v[j] = (E)(o[j] * mul);
  const int bb = (int)(row / ((long long)Hq * Lq)), h = (int)(row / Lq % Hq), i = (int)(row % Lq);
  *(ex8*)(Out + bb * so.b + h * so.h + (long long)i * so.l + c) = v;
  if (MODE == QS_FWD && c == 0) LSE[row] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
}

// Key-range shares per query tile for a dense 16-bit call (1: no split): when
// the query tiles alone give at most half as many workgroups as the 256 CUs,
// the largest power of two up to 4 that keeps the grid within 256 workgroups
// and the longest query tile at two or more key tiles per share (counted with
// the dQ pass's tiles, which at D = 512 are half as tall as the forward's;
// both passes take the same shares).
template <int D>
int qs_split_shares(int B, int Hq, int Lq, int Lk, int dlo, int dhi, bool dense) {
  using C = QsCfg<D>;
  if (!dense || Lq <= 0 || Lk <= 0 || dlo > dhi) return 1;
  const long long nwg = (long long)((Lq + C::BQ - 1) / C::BQ) * Hq * B;
  const long long width = std::min<long long>(Lk, (long long)C::BQ - 1 + dhi - dlo + 1);  // keys of a query tile
  const long long ntmax = (width + C::BK - 1) / C::BK + 1;
  int n = 1;
  while (n < 4 && nwg * 2 * n <= 256 && ntmax >= 4 * n) n *= 2;
  return n;
}

template <int D, int MODE, typename E>
hipError_t launch_qs(const void* q, const void* k, const void* v, const void* o, const void* dO, float* lse,
                     float* delta, void* out, const float* sinks, int B, int Hq, int group, int Lq, int Lk,
                     int dlo, int dhi, Cut cut, float scale, const AllStrides& st, int nseg, float* part,
                     hipStream_t stream) {
  using C = QsCfg<D, MODE>;
  if (nseg < 1 || (nseg > 1 && part == nullptr)) return hipErrorInvalidValue;
  const long nwg = (long)((Lq + C::BQ - 1) / C::BQ) * Hq * B * nseg;
  if (nwg > 0x7fffffffL) return hipErrorInvalidValue;
  if (nwg == 0) return hipSuccess;
  auto kernel = is_dense<D>(st, Hq, Hq / group, Lq, Lk) && cut.c0 == cut.c1 ? qs_kernel<D, MODE, E, true> : qs_kernel<D, MODE, E, false>;
  hipLaunchKernelGGL(kernel, dim3((unsigned)nwg), dim3(256), 0, stream, (const E*)q, (const E*)k, (const E*)v,
                     (const E*)o, (const E*)dO, lse, delta, (E*)out, sinks, Hq, group, Lq, Lk, dlo, dhi, cut,
                     scale, scale * kLog2e, st, nseg, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nseg == 1) return e;
  const long long rows = (long long)B * Hq * Lq, threads = rows * (D / 8);
  if ((threads + 255) / 256 > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((qs_combine_kernel<D, MODE, E>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                     (const float*)part, (E*)out, lse, nseg, rows, Hq, Lq, MODE == QS_FWD ? st.o : st.dq, scale);
  return hipGetLastError();
}

#define SDPA_INST_QS(D, E)                                                                                  \
  template hipError_t launch_qs<D, QS_FWD, E>(const void*, const void*, const void*, const void*, const void*, \
                                              float*, float*, void*, const float*, int, int, int, int, int, int, \
                                              int, Cut, float, const AllStrides&, int, float*, hipStream_t);   \
  template hipError_t launch_qs<D, QS_DQ, E>(const void*, const void*, const void*, const void*, const void*,  \
                                             float*, float*, void*, const float*, int, int, int, int, int, int,  \
                                             int, Cut, float, const AllStrides&, int, float*, hipStream_t);
SDPA_INST_QS(64, bf16)
SDPA_INST_QS(128, bf16)
SDPA_INST_QS(256, bf16)
SDPA_INST_QS(512, bf16)
SDPA_INST_QS(64, f16)
SDPA_INST_QS(128, f16)
SDPA_INST_QS(256, f16)
SDPA_INST_QS(512, f16)
template int qs_split_shares<64>(int, int, int, int, int, int, bool);
template int qs_split_shares<128>(int, int, int, int, int, int, bool);
template int qs_split_shares<256>(int, int, int, int, int, int, bool);
template int qs_split_shares<512>(int, int, int, int, int, int, bool);

}  // namespace sdpa
