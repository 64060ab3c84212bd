// Key-stationary dK/dV kernel for gfx950 (bf16 or fp16 in, fp32 accumulate).
//
// One workgroup = 4 waves = one (b, kv head g) and a block of BKT keys. It
// walks every query tile of every q-head of the GQA group whose rows can see
// one of its keys (tiles wholly outside the mask's band are never visited), so
// dK and dV of the group are summed in registers without
// atomics, and every key gets its dK/dV written, attended or not (page "Lab
// 028 lab detail: Off NVIDIA, you fix the platform yourself", section "What I
// changed, in plain terms", items 3-5). P is recomputed from S and the stored
// lse and dS is formed per element (section "2026-10-21", "What the code
// says"); S and dP stay in fp32 registers, only P and dS are rounded to the
// input type as MFMA operands (section "fp32 score tiles").
//
// Per query tile of 32 rows, per wave (owning 32 keys):
//   S  (32q x 32k) = Q_tile . K_w^T   A: Q (LDS, direct)   B: K_w (LDS, direct)
//   dP (32q x 32k) = dO_tile . V_w^T  A: dO (LDS, direct)  B: V_w (registers)
//   P = exp2(S c - lse2), dS = P * (dP - Delta)      (Delta from the dQ pass)
//   dV_w += P^T . dO                  A: P^T (C tile reused)  B: dO (LDS, transposed reads)
//   dK_w += dS^T . Q                  A: dS^T (C tile)        B: Q  (LDS, transposed reads)
// Q/dO tiles stream into double-buffered LDS with asynchronous global->LDS
// loads. Head dims up to 256 (D = 512 runs the 16-key kernel of kv16_mfma.hip).
#include <type_traits>

#include "common.h"

namespace sdpa {

#ifndef KV_AHEAD
#define KV_AHEAD 3  // S / dP operand reads issued this many MFMAs ahead
#endif

template <int D>
struct KvCfg {
  static_assert(D <= 256, "the 32-key kernel serves head dims up to 256");
  static constexpr int NW = 4;
  static constexpr int BKT = 32 * NW;          // keys per workgroup
  static constexpr int BQ = 32;                // query rows per step
};

// SPLIT (dense, one pass): blockIdx also picks one of nseg equal shares of the
// key block's query tiles, and the workgroup writes fp32 partial dK (scaled)
// and dV for its keys into Part, share-major: [2][nseg][B][Hkv][Lk][D] (dK
// shares first); kv_reduce_kernel then sums the shares. Small problems whose
// key blocks alone would leave CUs idle get more workgroups this way.
template <int D, typename E, bool DENSE, bool SPLIT>
__global__ void __launch_bounds__(256, 1)
kv_kernel(const E* __restrict__ Q, const E* __restrict__ K, const E* __restrict__ V,
          const E* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Delta,
          E* __restrict__ dK, E* __restrict__ dV, int Hq, int group, int Lq, int Lk, int dlo, int dhi,
          Cut cut_arg, float scale, float scale_log2, AllStrides st_arg, float* __restrict__ Part, int nseg) {
  static_assert(!SPLIT || DENSE, "the split runs the dense kernel");
  using C = KvCfg<D>;
  using ex8 = typename Vec<E>::x8;
  constexpr int NKS = D / 16, NDB = D / 32, QT = C::BQ * D;
  __shared__ __attribute__((aligned(16))) E ks[C::BKT * D];
  __shared__ __attribute__((aligned(16))) E qb0[QT];
  __shared__ __attribute__((aligned(16))) E db0[QT];
  __shared__ __attribute__((aligned(16))) E qb1[QT];
  __shared__ __attribute__((aligned(16))) E db1[QT];
  __shared__ __attribute__((aligned(16))) float rv0[64];  // lse (rows 0..31) and Delta (rows 0..31) of a tile
  __shared__ __attribute__((aligned(16))) float rv1[64];

  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform (SGPR)
  LaneAddr<D> la;  // per-lane LDS offsets of the operand read patterns
  la.init(lane);
  const int Hkv = Hq / group;
  const AllStrides st = DENSE ? dense_strides<D>(Hq, Hkv, Lq, Lk) : st_arg;
  const Cut cut = DENSE ? kNoCut : cut_arg;  // no cut in the dense instantiation
  const int nkt = (Lk + C::BKT - 1) / C::BKT;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int seg = SPLIT ? logical % nseg : 0, kblk = SPLIT ? logical / nseg : logical;
  const int kt = kblk % nkt, g = (kblk / nkt) % Hkv, b = kblk / (nkt * Hkv);
  const int k0 = kt * C::BKT;
  const int kb0 = k0 + 32 * w;             // first key of this wave's block
  const int kj = kb0 + (lane & 31);        // key held by this lane (C-tile column)
  const E* Kg = K + b * st.k.b + g * st.k.h;
  const E* Vg = V + b * st.v.b + g * st.v.h;
  // this key's rows: [ihi - kspan + 1, ihi] (kspan 0: none, or the key does not exist);
  // a key inside the cut is seen only by rows before r0
  const bool kcut = kj >= cut.c0 && kj < cut.c1;
  // with a shifted cut, a key before c0 is seen by rows before r0 through the
  // band and by rows from r0 on through the band moved forward by the shift:
  // a second range [ihi2 - kspan2 + 1, ihi2] (the dense instantiation has no cut)
  const bool kshift = !DENSE && cut.sh > 0 && kj < cut.c0;
  const int ihi = min(kcut || kshift ? cut.r0 - 1 : Lq - 1, kj - dlo), ilo = max(0, kj - dhi);
  const int kspan = kj < Lk && ihi >= ilo ? ihi - ilo + 1 : 0;
  const int ihi2 = kshift ? min(Lq - 1, kj + cut.sh - dlo) : 0, ilo2 = max(cut.r0, kj + cut.sh - dhi);
  const int kspan2 = kshift && kj < Lk && ihi2 >= ilo2 ? ihi2 - ilo2 + 1 : 0;

  zero_lds(ks, C::BKT * D, tid);
  zero_lds(qb0, QT, tid);
  zero_lds(db0, QT, tid);
  zero_lds(qb1, QT, tid);
  zero_lds(db1, QT, tid);
  lds_barrier();
  {
    TileLoader<D, C::BKT, C::NW, DENSE> kld;
    kld.init(w, lane, st.k.l);
    kld.issue(ks, Kg + (long long)k0 * st.k.l, Lk - k0, w);
  }
  // per-lane source offsets of the Q and dO tile loads (the two share their row
  // stride: the host checks it)
  TileLoader<D, C::BQ, C::NW, DENSE> ldq;
  ldq.init(w, lane, st.q.l);
  const auto& ldd = ldq;
  using LD = decltype(ldq);
  // V_w^T as B operands of dP: lane holds key kj, d-slots 16*s + 8*hh + 0..7
  ex8 vreg[NKS];
  {
    const E* vrow = Vg + (long long)(kj < Lk ? kj : 0) * st.v.l;
#pragma unroll
    for (int s = 0; s < NKS; s++) vreg[s] = kj < Lk ? *(const ex8*)(vrow + 16 * s + 8 * hh) : zero8<E>();
  }

  f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int d = 0; d < NDB; d++) dkacc[d] = dvacc[d] = zero16();

  // query tiles that can see a key of this workgroup, for each q-head of the group
  // (none: total = 0, and the keys get zero gradients)
  const int klast = min(k0 + C::BKT - 1, Lk - 1);
  const bool all_cut = k0 >= cut.c0 && klast < cut.c1;  // every key of the workgroup inside the cut
  const bool all_shift = !DENSE && cut.sh > 0 && klast < cut.c0;  // every key seen from r0 on only when moved
  const int rlo = max(0, k0 - dhi), rhi = min(all_cut || all_shift ? cut.r0 - 1 : Lq - 1, klast - dlo);
  int qt_lo = rlo / C::BQ, nq = rlo <= rhi ? rhi / C::BQ - qt_lo + 1 : 0;
  // with a shifted cut, the rows from r0 on that see a key before c0 through
  // the moved band: their tiles come first, or merge with the band's range
  // when the two touch; q0_of(it) is the first row of the it-th tile
  int qt2_lo = 0, nq2 = 0;
  if (!DENSE && cut.sh > 0 && k0 < cut.c0) {
    const int lo2 = max(cut.r0, k0 + cut.sh - dhi), hi2 = min(Lq - 1, min(klast, cut.c0 - 1) + cut.sh - dlo);
    if (lo2 <= hi2) {
      const int a = lo2 / C::BQ, z = hi2 / C::BQ;
      if (nq == 0) qt_lo = a, nq = z - a + 1;
      else if (z + 1 >= qt_lo && a <= qt_lo + nq) {
        const int e = max(qt_lo + nq - 1, z);
        qt_lo = min(qt_lo, a);
        nq = e - qt_lo + 1;
      } else {
        qt2_lo = a, nq2 = z - a + 1;
      }
    }
  }
  nq += nq2;
  auto q0_of = [&](int it) {
    const int t = it % nq;
    return (t < nq2 ? qt2_lo + t : qt_lo + (t - nq2)) * C::BQ;
  };
  const int total = group * nq;
  // this workgroup's query tiles: [it_b, it_e) of the total (all of them without the split)
  const int it_b = SPLIT ? (int)((long long)seg * total / nseg) : 0;
  const int it_e = SPLIT ? (int)((long long)(seg + 1) * total / nseg) : total;
  const int kb1 = min(kb0 + 31, Lk - 1);  // this wave's last key (kb1 < kb0: none)
  const bool wcut = kb0 >= cut.c0 && kb1 < cut.c1;                 // all of the wave's keys inside the cut
  const int wrhi = wcut ? min(kb1 - dlo, cut.r0 - 1) : kb1 - dlo;  // last row that sees a key of the wave
  // some pair of the tile's rows [q0, q0 + 31] and the wave's keys allowed /
  // every pair allowed (general instantiation: from the lanes' row ranges,
  // which never touch)
  auto tile_tests = [&](int q0, bool& active, bool& full) {
    if constexpr (DENSE) {
      const int r1 = min(q0 + 31, Lq - 1);
      active = kb0 <= kb1 && q0 <= wrhi && r1 >= kb0 - dhi;
      full = kb0 + 32 <= Lk && q0 + 32 <= Lq && kb0 - q0 - 31 >= dlo && kb0 + 31 - q0 <= dhi;
    } else {
      const int q1 = q0 + 31;
      auto meets = [&](int hi, int sp) { return sp > 0 && hi >= q0 && hi - sp + 1 <= q1; };
      auto covers = [&](int hi, int sp) { return sp > 0 && hi >= q1 && hi - sp + 1 <= q0; };
      active = __any(meets(ihi, kspan) || meets(ihi2, kspan2));
      full = __all(covers(ihi, kspan) || covers(ihi2, kspan2));
    }
  };

  auto tile_src = [&](int it, const E*& qs, const E*& ds, int& q0) {
    const int hq = g * group + it / nq;
    q0 = q0_of(it);
    if constexpr (DENSE) {  // one offset for both (same layout), as few live scalars as possible
      const size_t off = (((size_t)b * Hq + hq) * Lq + q0) * D;
      qs = Q + off;
      ds = dO + off;
    } else {
      qs = Q + b * st.q.b + hq * st.q.h + (long long)q0 * st.q.l;
      ds = dO + b * st.dO.b + hq * st.dO.h + (long long)q0 * st.dO.l;
    }
  };
  // lanes 0..31: lse of the tile's rows, lanes 32..63: Delta of them (rows
  // clamped to Lq-1); one 4-byte buffer->LDS load per lane (wave 0 only). A
  // buffer load, not global_load_lds: while one of those is outstanding the
  // compiler waits for every earlier LDS read (lgkmcnt(0)) before each MFMA,
  // which undoes the operand look-ahead.
  auto load_rows = [&](int it, float* rv) {
    const int hq = g * group + it / nq;
    const int q0 = q0_of(it);
    const uint32_t off = (uint32_t)min(q0 + (lane & 31), Lq - 1) * 4;
    const size_t rb = ((size_t)b * Hq + hq) * Lq;
    auto* dst = (__attribute__((address_space(3))) void*)rv;
    if (lane < 32)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          __builtin_amdgcn_make_buffer_rsrc((void*)(LSE + rb), 0, (uint32_t)Lq * 4, 0x00020000), dst, 4, off, 0, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          __builtin_amdgcn_make_buffer_rsrc((void*)(Delta + rb), 0, (uint32_t)Lq * 4, 0x00020000), dst, 4, off, 0, 0, 0);
  };
  auto issue = [&](int it, E* qd, E* dd, float* rv) {
    const E *qs, *ds;
    int q0;
    tile_src(it, qs, ds, q0);
    ldq.issue(qd, qs, Lq - q0, w);
    ldd.issue(dd, ds, Lq - q0, w);
    if (w == 0) load_rows(it, rv);
  };

  // P = exp(S - lse), dS = P (dP - Delta) from the score tiles, then
  // dV += P^T dO and dK += dS^T Q for the query tile whose rows start at q0.
  auto form_and_update = [&](int q0, bool full, const float* rv, f32x16& s_acc, f32x16& dp_acc,
                             const E* Qc, const E* dOc) {
  // P = exp(S - lse) and dS = P (dP - Delta); the element mask only on edge
  // tiles, as a select (the wave-uniform test stays outside the element loop)
  // row q0 + c_row(i, hh) is allowed for this lane's key iff it lies in
  // [ihi - kspan + 1, ihi]: ihi - q0 - c_row = base - rr, one unsigned compare
  const int base = ihi - q0 - 4 * hh, base2 = ihi2 - q0 - 4 * hh;
  auto form = [&](auto masked) {
#pragma unroll
    for (int blk = 0; blk < 4; blk++) {
      const float4 l4 = *(const float4*)(rv + 8 * blk + 4 * hh);
      const float4 d4 = *(const float4*)(rv + 32 + 8 * blk + 4 * hh);
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int i = 4 * blk + r;
        const float lv = (&l4.x)[r] * kLog2e, dv = (&d4.x)[r];
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s_acc[i], scale_log2, -lv));
        if constexpr (decltype(masked)::value) {
          const int rr = 8 * blk + r;  // c_row(i, hh) - 4 hh
          p = in_band(base, rr, kspan) || (!DENSE && in_band(base2, rr, kspan2)) ? p : 0.f;
        }
        s_acc[i] = p;
        dp_acc[i] = p * (dp_acc[i] - dv);
      }
    }
  };
  if (full) form(std::false_type{});
  else form(std::true_type{});
  const ex8 pa0 = c_to_op<E>(s_acc, 0), pa1 = c_to_op<E>(s_acc, 1);
  const ex8 da0 = c_to_op<E>(dp_acc, 0), da1 = c_to_op<E>(dp_acc, 1);
  constexpr int MPB = 4;  // MFMAs per head-dim block
#pragma unroll
  for (int d = 0; d < NDB; d++) {
    const int c0 = 32 * d;
    dvacc[d] = mfma(pa0, op_tr<D, E>(dOc, la, 0, c0), dvacc[d]);
    dvacc[d] = mfma(pa1, op_tr<D, E>(dOc, la, 16, c0), dvacc[d]);
    dkacc[d] = mfma(da0, op_tr<D, E>(Qc, la, 0, c0), dkacc[d]);
    dkacc[d] = mfma(da1, op_tr<D, E>(Qc, la, 16, c0), dkacc[d]);
  }
  // schedule: transposed reads run one head-dim block ahead of their MFMAs
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * MPB, 1);
#pragma unroll
  for (int d = 0; d < NDB; d++) {
    __builtin_amdgcn_sched_group_barrier(0x008, MPB, 1);
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * MPB, 1);
  }
  };

  // One query tile. The next tile's Q, dO (and lse, Delta) loads into
  // (qn, dn, rvn) are issued one at a time between the S / dP MFMAs: in
  // one burst they stall the wave until the CU's vector-memory path has taken
  // them all. A load stays after the LDS reads that precede it in program
  // order (it writes LDS), so the operand reads are software-pipelined by hand
  // and the loads slot in between them. Past the last tile the resources cover
  // no rows (nothing is read).
  auto compute = [&](int it, const E* Qc, const E* dOc, const float* rv, E* qn, E* dn, float* rvn) {
    const int q0 = q0_of(it);
    bool active, full;
    tile_tests(q0, active, full);

    __amdgpu_buffer_rsrc_t qrs, drs;
    {
      const bool more = it + 1 < it_e;
      const E *qs, *ds;
      int q0n;
      tile_src(more ? it + 1 : it, qs, ds, q0n);
      qrs = ldq.rsrc(qs, more ? Lq - q0n : 0);
      drs = ldd.rsrc(ds, more ? Lq - q0n : 0);
      if (w == 0) load_rows(more ? it + 1 : it, rvn);
    }
    constexpr int NJ = LD::NJ;
    auto load_one = [&, qrs, drs](int j) {  // j in [0, 2 NJ): Q blocks, then dO blocks
      if constexpr (LD::PER % C::NW != 0) {
        if ((j % NJ) * C::NW + w >= LD::PER) return;
      }
      if (j < NJ) ldq.issue_one(qn, qrs, j, w);
      else ldd.issue_one(dn, drs, j - NJ, w);
    };

    // S (all of it first, so exp(S) can start while the dP MFMAs run), then
    // dP; computed by every wave (a wave whose keys miss this tile would only
    // wait at the tile barrier): no branch around the MFMAs. MFMA step k < NKS
    // is S with k-slice k, step NKS + k is dP with k-slice k.
    f32x16 s_acc = zero16(), dp_acc = zero16();
    {
      constexpr int NM = 2 * NKS, AH = KV_AHEAD, NLD = 2 * NJ;
      constexpr int EVERY = NM / NLD > 0 ? NM / NLD : 1;
      ex8 ra[AH], rb[AH];
      auto rd = [&](int k) {
        if (k < NKS) {
          ra[k % AH] = op_direct<D, E>(Qc, la, 16 * k, 0);
          rb[k % AH] = op_direct<D, E>(ks, la, 16 * k, 32 * w);
        } else {
          ra[k % AH] = op_direct<D, E>(dOc, la, 16 * (k - NKS), 0);
        }
      };
#pragma unroll
      for (int k = 0; k < AH; k++) rd(k);
#pragma unroll
      for (int k = 0; k < NM; k++) {
        if (k < NKS) s_acc = mfma(ra[k % AH], rb[k % AH], s_acc);
        else dp_acc = mfma(ra[k % AH], vreg[k - NKS], dp_acc);
        if (k + AH < NM) rd(k + AH);
        if (k % EVERY == EVERY - 1 && k / EVERY < NLD) load_one(k / EVERY);
      }
#pragma unroll
      for (int j = NM / EVERY; j < NLD; j++) load_one(j);
    }
    if (!active) return;
    form_and_update(q0, full, rv, s_acc, dp_acc, Qc, dOc);
  };

  if (it_b < it_e) {  // (none: no row sees these keys, or no tile falls to this share: zero gradients)
    issue(it_b, qb0, db0, rv0);
    wait_all_and_barrier();
    for (int it = it_b; it < it_e; it += 2) {
      compute(it, qb0, db0, rv0, qb1, db1, rv1);
      wait_all_and_barrier();
      if (it + 1 >= it_e) break;
      compute(it + 1, qb1, db1, rv1, qb0, db0, rv0);
      wait_all_and_barrier();
    }
  }

  // dK = scale * dS^T Q, dV = P^T dO; C tile: column = head-dim index, rows = keys
  if constexpr (SPLIT) {
    const size_t slice = (size_t)(gridDim.x / nseg / nkt) * Lk * D;  // B * Hkv * Lk * D
    float* pk = Part + (size_t)seg * slice + ((size_t)b * Hkv + g) * Lk * D;
    float* pv = pk + (size_t)nseg * slice;
#pragma unroll
    for (int d = 0; d < NDB; d++) {
      const int col = 32 * d + (lane & 31);
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const int key = kb0 + c_row(i, hh);
        if (key < Lk) {
          pk[(size_t)key * D + col] = dkacc[d][i] * scale;
          pv[(size_t)key * D + col] = dvacc[d][i];
        }
      }
    }
    return;
  }
  E* dKg = dK + b * st.dk.b + g * st.dk.h;
  E* dVg = dV + b * st.dv.b + g * st.dv.h;
#pragma unroll
  for (int d = 0; d < NDB; d++) {
    const int col = 32 * d + (lane & 31);
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const int key = kb0 + c_row(i, hh);
      if (key < Lk) {
        dKg[(long long)key * st.dk.l + col] = (E)(dkacc[d][i] * scale);
        dVg[(long long)key * st.dv.l + col] = (E)dvacc[d][i];
      }
    }
  }
}

// dK, dV = the sum of the nseg fp32 shares of Part ([2][nseg][n] with n =
// B * Hkv * Lk * D, contiguous outputs), summed in share order; 8 elements
// per thread, blockIdx.y = 0 for dK, 1 for dV.
template <typename E>
__global__ void __launch_bounds__(256) kv_reduce_kernel(const float* __restrict__ Part, E* __restrict__ dK,
                                                        E* __restrict__ dV, size_t n, int nseg) {
  using ex8 = typename Vec<E>::x8;
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= n) return;
  const float* p = Part + (size_t)blockIdx.y * nseg * n + i;
  float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < nseg; s++) {
    const float4 x = *(const float4*)(p + (size_t)s * n), y = *(const float4*)(p + (size_t)s * n + 4);
    a[0] += x.x, a[1] += x.y, a[2] += x.z, a[3] += x.w, a[4] += y.x, a[5] += y.y, a[6] += y.z, a[7] += y.w;
  }
  ex8 v;
#pragma unroll
  for (int j = 0; j < 8; j++) v[j] = (E)a[j];
  *(ex8*)((blockIdx.y == 0 ? dK : dV) + i) = v;
}

// Shares of the split for this shape, or 1 (no split): only for dense calls
// whose key blocks alone fill fewer than 256 workgroups.
template <int D>
int kv_split_shares(int B, int Hq, int group, int Lq, int Lk, bool dense) {
  if (!dense || Lq == 0) return 1;
  const long nwg = (long)((Lk + KvCfg<D>::BKT - 1) / KvCfg<D>::BKT) * (Hq / group) * B;
  int n = 1;
  while (n < 8 && nwg * n < 256) n *= 2;
  return n;
}

template <int D, typename E>
hipError_t launch_kv(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                     const float* delta, void* dk, void* dv, int B, int Hq, int group, int Lq, int Lk, int dlo,
                     int dhi, Cut cut, float scale, const AllStrides& st, float* part, int nseg,
                     hipStream_t stream) {
  using C = KvCfg<D>;
  const long nwg = (long)((Lk + C::BKT - 1) / C::BKT) * (Hq / group) * B;
  if (nwg * (nseg > 1 ? nseg : 1) > 0x7fffffffL) return hipErrorInvalidValue;
  if (nwg == 0) return hipSuccess;
  const bool dense = is_dense<D>(st, Hq, Hq / group, Lq, Lk) && cut.c0 == cut.c1;
  auto run = [&](auto dense_kernel, auto strided_kernel) {
    auto kernel = dense ? dense_kernel : strided_kernel;
    hipLaunchKernelGGL(kernel, dim3((unsigned)nwg), dim3(256), 0, stream,
                       (const E*)q, (const E*)k, (const E*)v, (const E*)dO, lse, delta, (E*)dk, (E*)dv, Hq, group,
                       Lq, Lk, dlo, dhi, cut, scale, scale * kLog2e, st, (float*)nullptr, 1);
    return hipGetLastError();
  };
  if (nseg <= 1 || part == nullptr || !dense) return run(kv_kernel<D, E, true, false>, kv_kernel<D, E, false, false>);
  hipLaunchKernelGGL((kv_kernel<D, E, true, true>), dim3((unsigned)(nwg * nseg)), dim3(256), 0, stream,
                     (const E*)q, (const E*)k, (const E*)v, (const E*)dO, lse, delta, (E*)dk, (E*)dv, Hq, group,
                     Lq, Lk, dlo, dhi, cut, scale, scale * kLog2e, st, part, nseg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t n = (size_t)B * (Hq / group) * Lk * D;
  hipLaunchKernelGGL(kv_reduce_kernel<E>, dim3((unsigned)((n / 8 + 255) / 256), 2), dim3(256), 0, stream,
                     (const float*)part, (E*)dk, (E*)dv, n, nseg);
  return hipGetLastError();
}

#define SDPA_INST_KV(D, E)                                                                                \
  template hipError_t launch_kv<D, E>(const void*, const void*, const void*, const void*, const float*,    \
                                      const float*, void*, void*, int, int, int, int, int, int, int, Cut,   \
                                      float, const AllStrides&, float*, int, hipStream_t);
SDPA_INST_KV(64, bf16)
SDPA_INST_KV(128, bf16)
SDPA_INST_KV(256, bf16)
SDPA_INST_KV(64, f16)
SDPA_INST_KV(128, f16)
SDPA_INST_KV(256, f16)
template int kv_split_shares<64>(int, int, int, int, int, bool);
template int kv_split_shares<128>(int, int, int, int, int, bool);
template int kv_split_shares<256>(int, int, int, int, int, bool);

}  // namespace sdpa
