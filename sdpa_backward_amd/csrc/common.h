// Device-side building blocks shared by the gfx950 attention kernels.
//
// MFMA used: v_mfma_f32_32x32x16_bf16 and its float16 twin
// v_mfma_f32_32x32x16_f16 (wave64), which share these lane layouts (checked
// on the hardware for bf16; the fp16 parity tests cover the other):
//   A (32x16, M x K): lane l holds row l%32, k-slots for half h = l/32
//   B (16x32, K x N): lane l holds col l%32, k-slots for half h = l/32
//   C (32x32 fp32):   lane l holds col l%32, rows 8*(i/4) + 4*h + (i%4), i = 0..15
// The contraction is a sum over k, so any slot->k assignment works as long
// as A and B use the same one. Two assignments are used here:
//   direct  slot j <-> k = 8*h + j                    (one 16-byte LDS read)
//   paired  slot j <-> k = 8*(j/4) + 4*h + (j%4)      (two 8-byte reads)
// "paired" is exactly what an fp32 C tile provides when it is reused as an
// operand (its rows become k), and what two ds_read_b64_tr_b16 reads give
// from a row-major tile whose rows are k.
//
// ds_read_b64_tr_b16 (checked on the hardware): within each 16-lane group,
// output lane j, element s comes from element j%4 of the 8 bytes addressed
// by lane 4*s + j/4 of the same group. If lane i addresses row r0 + i/4,
// column c0 + 4*(i%4) of a row-major tile, lane j receives column c0 + j,
// rows r0..r0+3: a 4x16 block arrives transposed.
//
// LDS tiles are row-major 16-bit [rows][D] with no padding; the 16-byte chunk c
// of row r sits at chunk slot c ^ swz(r). swz maps 16 consecutive rows to 16
// distinct slots (conflict-free 16-byte reads of one column chunk across rows)
// and 8 consecutive rows to 8 distinct chunk pairs (transposed reads).
//
// Tiles arrive by buffer_load_dwordx4 ... lds (checked on the hardware: the 16
// bytes a lane fetches land at LDS base + 16 * lane, one 1 KB block per wave
// instruction), so loads of the next tile run while the current one is used.
// The two buffers of a double-buffered tile are distinct __shared__ objects
// and the loop body is instantiated once per buffer parity: the compiler can
// then prove the prefetch target never aliases the tile being read and does
// not insert a wait on the prefetch before every LDS read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

#define SDPA_DEV __device__ __forceinline__

namespace sdpa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// The 16-bit input types (bfloat16, float16) share every kernel: the two MFMAs
// below have the same shape, lane layouts and fp32 accumulator; only the
// operand format and the rounding of P, dS and the outputs differ.
template <typename E>
struct Vec;
template <>
struct Vec<bf16> {
  typedef bf16x8 x8;
  typedef bf16x4 x4;
};
template <>
struct Vec<f16> {
  typedef f16x8 x8;
  typedef f16x4 x4;
};

SDPA_DEV f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
SDPA_DEV f32x16 mfma(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

SDPA_DEV f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; i++) z[i] = 0.f;
  return z;
}

template <typename E>
SDPA_DEV typename Vec<E>::x8 zero8() {
  typename Vec<E>::x8 z;
#pragma unroll
  for (int i = 0; i < 8; i++) z[i] = (E)0.f;
  return z;
}

// Row of the C tile held in accumulator slot i by a lane in half h.
SDPA_DEV int c_row(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

// fp32 C-tile values [8*op, 8*op+8) as a 16-bit "paired" operand (rows of the
// C tile become k: op 0 covers C rows 0..15, op 1 rows 16..31), rounded to
// nearest even.
template <typename E>
SDPA_DEV typename Vec<E>::x8 c_to_op(const f32x16& c, int op) {
  typename Vec<E>::x8 r;
#pragma unroll
  for (int j = 0; j < 8; j++) r[j] = (E)c[8 * op + j];
  return r;
}

// Max / sum of a value over the two 32-lane halves of the wave (lanes l and
// l ^ 32 hold the two halves of one C-tile column). v_permlane32_swap keeps the
// exchange in the VALU: no LDS round trip, no wait on outstanding LDS reads.
SDPA_DEV float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
SDPA_DEV float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Ask the register allocator to hold a value in AGPRs at this point (MFMAs read
// and write AGPRs directly; only VALU arithmetic needs VGPRs).
SDPA_DEV void keep_in_agpr(f32x16& x) { asm volatile("" : "+a"(x)); }
SDPA_DEV void keep_in_agpr(bf16x8& x) { asm volatile("" : "+a"(x)); }
SDPA_DEV void keep_in_agpr(f16x8& x) { asm volatile("" : "+a"(x)); }

// x[t] *= a for accumulator tiles that stay in AGPRs: each element is read
// into a VGPR, multiplied and written back inside one asm statement, so the
// register allocator never moves the tiles into VGPRs for this rare rescale
// (plain C++ makes it copy every tile out of and back into AGPRs on every
// iteration). The leading wait states cover an MFMA still writing a tile (a VALU
// read of an MFMA result needs them), the trailing ones a following MFMA that
// reads a tile as its accumulator input.
template <int N>
SDPA_DEV void scale_in_agpr(f32x16 (&x)[N], float a) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3");
#pragma unroll
  for (int t = 0; t < N; t++)
#pragma unroll
    for (int i = 0; i < 16; i++) {
      float e = x[t][i], tmp;
      asm volatile(
          "v_accvgpr_read_b32 %1, %0\n\t"
          "v_mul_f32_e32 %1, %2, %1\n\t"
          "v_accvgpr_write_b32 %0, %1"
          : "+a"(e), "=&v"(tmp)
          : "v"(a));
      x[t][i] = e;
    }
  asm volatile("s_nop 7");
}

// Allowed (query row i, key j) pairs, every mask as one band: with Lq query
// rows and Lk keys, the pair is allowed iff i < Lq, 0 <= j < Lk and
// dlo <= j - i <= dhi. The host derives dlo <= dhi from the mask, the window
// and the diagonal offset Lk - Lq (queries are the last Lq key positions):
//   no mask        [-(Lq-1), Lk-1]          (every pair)
//   causal         [-(Lq-1), off]
//   causal window  [off - W + 1, off]
//   window         [off - W + 1, off + W - 1]   (both sides of the diagonal)
// clamped to [-(Lq-1), Lk-1], so i + dhi and j - dlo never overflow.
// Row i's keys are [max(0, i + dlo), min(Lk - 1, i + dhi)] and key j's rows
// [max(0, j - dhi), min(Lq - 1, j - dlo)]: both ends rise with i (with j), so
// the rows of a tile see the union of their first and last row's ranges.
//
// A run of indices x0 + r is tested against a range [hi - span + 1, hi]
// (span = 0: empty) with one unsigned compare per element: x0 + r is inside
// iff (uint32)(hi - x0 - r) < span, so callers form base = hi - x0 once.
SDPA_DEV bool in_band(int base, int r, int span) { return (uint32_t)base - (uint32_t)r < (uint32_t)span; }

// ---------------------------------------------------------------- swizzled tiles
// Chunk c (16 bytes) of row r sits at chunk slot c ^ swz(r), swz(r) < 16:
//   bits 2-3 = r & 3, bit 1 = (r >> 2) & 1, bit 0 = (r >> 3) & 1   (D >= 128)
//   bits 2-3 = r & 3, bits 0-1 = (r >> 2) & 3, masked to 3 bits    (D = 64)
// 16 consecutive rows get 16 distinct slots (16-byte reads of one chunk
// across rows, serviced 16 lanes per cycle, hit 16 distinct 16-byte bank
// groups); rows r..r+3 (r a multiple of 4) get distinct 32-byte chunk pairs,
// and so do rows r+4..r+7 among themselves and against rows r..r+3
// (transposed reads, serviced 32 lanes per cycle: the 32x32x16 kernels read 4
// rows x 4 chunks, the 16x16x32 kernel 8 rows x 2 chunks at a time). The
// 32x32x16 patterns measured conflict-free on the hardware bank-conflict
// counter; the earlier D >= 128 form (bits 0-1 = (r >> 2) & 3) put rows r and
// r + 4 on one chunk pair and gave the 16x16x32 reads 2-way conflicts. Only
// the low 4 chunk bits are permuted, so higher chunk offsets stay additive and
// every read is a per-lane base plus an immediate offset.
template <int D>
struct Tile {
  static constexpr int CPR = D / 8;                         // 16-byte chunks per row
  static constexpr int SMASK = CPR >= 16 ? 15 : CPR - 1;   // swizzle bits available
  SDPA_DEV static int swz(int r) {
    if constexpr (CPR >= 16) return ((r & 3) << 2) | (((r >> 2) & 1) << 1) | ((r >> 3) & 1);
    else return (((r & 3) << 2) | ((r >> 2) & 3)) & SMASK;
  }
  SDPA_DEV static int slot(int r, int c) { return c ^ swz(r); }
};

// Per-lane LDS byte offsets for the two operand read patterns of a [rows][D]
// swizzled tile. 16 registers serve every tile with row length D.
//   dir[j]:  "direct" read, lane row l%32, chunk 2j + l/32 (j = 0..7)
//   trn[2q + h]: transposed read, chunk block q (columns 32q..), rows +0 (h=0) / +8 (h=1)
template <int D>
struct LaneAddr {
  uint32_t dir[8];
  uint32_t trn[8];
  SDPA_DEV void init(int lane) {
    const int r = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int j = 0; j < 8; j++) dir[j] = r * D * 2 + (Tile<D>::slot(r, 2 * j + hh) & 15) * 16;
    const int G = lane >> 4, i = lane & 15;
    const int row = 4 * (G >> 1) + (i >> 2);
    const int cl = 2 * (G & 1) + ((i & 3) >> 1), within = (i & 1) * 8;  // bytes inside the chunk
#pragma unroll
    for (int q = 0; q < 4; q++)
#pragma unroll
      for (int h = 0; h < 2; h++) {
        const int rr = row + 8 * h;
        trn[2 * q + h] = rr * D * 2 + (Tile<D>::slot(rr, 4 * q + cl) & 15) * 16 + within;
      }
  }
};

// 4 consecutive 16-bit elements of a row-major LDS tile, delivered transposed
// across each 16-lane group (see header comment).
template <typename E>
SDPA_DEV typename Vec<E>::x4 lds_tr4(const char* p) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(typename Vec<E>::x4, r);
}

// Operand from a swizzled tile T[k][mn] (rows are the contraction index):
// lane l gets column mn0 + l%32 with "paired" k-slots over rows [k0, k0+16).
// k0: multiple of 16; mn0: multiple of 32.
template <int D, typename E>
SDPA_DEV typename Vec<E>::x8 op_tr(const E* T, const LaneAddr<D>& a, int k0, int mn0) {
  const int q = mn0 / 32;  // 4 chunks per 32-column block
  const char* base = reinterpret_cast<const char*>(T) + k0 * D * 2 + (q >> 2) * 256;
  const typename Vec<E>::x4 lo = lds_tr4<E>(base + a.trn[2 * (q & 3)]);
  const typename Vec<E>::x4 hi = lds_tr4<E>(base + a.trn[2 * (q & 3) + 1]);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Operand from a swizzled tile T[mn][k] (columns are the contraction index):
// lane l gets row mn0 + l%32 with "direct" k-slots k0 + 8*(l/32) + j.
// k0: multiple of 16; mn0: multiple of 32.
template <int D, typename E>
SDPA_DEV typename Vec<E>::x8 op_direct(const E* T, const LaneAddr<D>& a, int k0, int mn0) {
  const int c = k0 / 8;  // even
  const char* p = reinterpret_cast<const char*>(T) + a.dir[(c & 15) >> 1] + (c >> 4) * 256 + mn0 * D * 2;
  return *(const typename Vec<E>::x8*)p;
}

// Element strides of a [B, H, L, D] tensor: batch, head and row (sequence
// position); the D elements of a row are contiguous.
struct Strides {
  long long b, h;
  int l;  // < 2^23 (checked by the host)
};

// Strides of every tensor of a forward / backward call (a kernel reads those
// of the tensors it touches). lse and Delta are always contiguous [B, Hq, Lq].
struct AllStrides {
  Strides q, k, v, o, dO, dq, dk, dv;
};

// Block-sparse cut on top of the mask: rows i >= r0 do not see keys
// c0 <= j < c1 (c0 == c1: no cut). With [prompt; chosen; rejected] and
// r0 = c1 = start of rejected, c0 = start of chosen, this is the
// prefix-sharing mask (page "Training - design (ORPO, flash-CCE head, prefix
// sharing, segmented backward)", section 5.4). sh is 0, or c1 - c0 for the
// window cut at logical positions (same section): rows from r0 on then see a
// key j < c0 through the band as if it sat at j + sh. So a row from r0 on
// sees two key ranges, [max(band lo, c1), band hi] and the band moved back by
// sh, clipped to [0, c0); a key before c0 is seen by two row ranges, rows
// before r0 through the band and rows from r0 on through the band moved
// forward by sh (one range when sh = 0).
struct Cut {
  int r0, c0, c1, sh;
};
// No cut (the rows that would be cut do not exist).
constexpr Cut kNoCut = {0x7fffffff, 0, 0, 0};

// The strides of contiguous [B, H, L, D] tensors. The kernels come in a dense
// instantiation that uses these and no cut (row stride D known at compile
// time, so tile offsets fold to constants, no stride occupies a register and
// the cut's tests vanish) and a general one that reads the caller's strides
// and cut.
template <int D>
__host__ __device__ inline AllStrides dense_strides(int Hq, int Hkv, int Lq, int Lk) {
  const Strides q{(long long)Hq * Lq * D, (long long)Lq * D, D}, kv{(long long)Hkv * Lk * D, (long long)Lk * D, D};
  return {q, kv, kv, q, q, q, kv, kv};
}

inline bool same(const Strides& a, const Strides& b) { return a.b == b.b && a.h == b.h && a.l == b.l; }

// Whether a call's tensors are all contiguous (the dense instantiation applies).
template <int D>
inline bool is_dense(const AllStrides& s, int Hq, int Hkv, int Lq, int Lk) {
  const AllStrides d = dense_strides<D>(Hq, Hkv, Lq, Lk);
  return same(s.q, d.q) && same(s.k, d.k) && same(s.v, d.v) && same(s.o, d.o) && same(s.dO, d.dO) &&
         same(s.dq, d.dq) && same(s.dk, d.dk) && same(s.dv, d.dv);
}

// Asynchronous global->LDS tile loads through a buffer resource. A wave
// issues whole 1 KB blocks (buffer_load_dwordx4 ... lds: lane l's 16 bytes land
// at the block's LDS base + 16 l). Block j of a tile covers RPB = 64 / CPR
// whole rows, so lane l of a wave's jj-th block reads row
// r = (jj NW + w) RPB + l / CPR at byte r * row_bytes + 16 slot(r, l % CPR).
// DENSE (row stride D, the contiguous layout): every offset is computed once
// and loads need no address arithmetic. Otherwise (any row stride) the
// swizzled slot depends on r only through r mod 16, which repeats every
// VP = 16 / gcd(16, NW RPB) blocks (1 for D <= 128, 2 for D = 256, 4 for
// D = 512): each lane keeps VP offsets and a load adds the uniform rest, a
// multiple of the row stride. The resource of each tile ends with its last
// valid row: lanes whose offset falls beyond it are range-checked by the
// hardware and read nothing from memory (rows past the end of the sequence are
// masked downstream; the buffers are zeroed once at kernel start, so such rows
// only ever hold zeros or finite data of an earlier tile).
template <int D, int R, int NW, bool DENSE>
struct TileLoader {
  static constexpr int CPR = D / 8;                // 16-byte chunks per row
  static constexpr int RPB = 64 / CPR;             // rows per 1 KB block
  static constexpr int PER = R * CPR / 64;         // 1 KB blocks per tile
  static constexpr int NJ = (PER + NW - 1) / NW;   // blocks issued by one wave
  static constexpr int G = (NW * RPB) % 16 == 0 ? 16 : (NW * RPB) % 8 == 0 ? 8 : (NW * RPB) % 4 == 0 ? 4 : 2;
  static constexpr int VP0 = 16 / G;               // period of the lane offsets in jj
  static constexpr int NOFF = DENSE ? NJ : (VP0 < NJ ? VP0 : NJ);
  static_assert(CPR <= 64 && (R * CPR) % 64 == 0, "tile must be a whole number of 1 KB blocks of whole rows");
  uint32_t lane_off[NOFF];
  uint32_t row_bytes;  // source row stride in bytes (uniform)
  // sl: the source's row stride in elements (D when DENSE; else >= D, bounded
  // by the host so every offset inside a tile fits 32 bits)
  SDPA_DEV void init(int w, int lane, long long sl) {
    row_bytes = DENSE ? D * 2 : (uint32_t)(sl * 2);
#pragma unroll
    for (int v = 0; v < NOFF; v++) {
      const int r = (v * NW + w) * RPB + lane / CPR;
      lane_off[v] = (uint32_t)r * row_bytes + (uint32_t)(Tile<D>::slot(r, lane % CPR) * 16);
    }
  }
  // Source offset of this lane in the wave's block jj.
  SDPA_DEV uint32_t voff(int jj) const {
    if constexpr (DENSE) return lane_off[jj];
    else return lane_off[jj % NOFF] + (uint32_t)((jj / NOFF) * NOFF * NW * RPB) * row_bytes;
  }
  // Resource covering rows [0, min(valid, R)) of the tile whose row 0 starts at
  // src; valid <= 0 gives an empty range (loads read nothing).
  SDPA_DEV __amdgpu_buffer_rsrc_t rsrc(const void* src, int valid) const {
    const int rows = __builtin_amdgcn_readfirstlane(valid < 0 ? 0 : valid < R ? valid : R);  // uniform
    uint32_t bytes;
    if constexpr (DENSE) bytes = rows * D * 2;
    else bytes = rows > 0 ? (uint32_t)(rows - 1) * row_bytes + D * 2 : 0;
    return __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, bytes, 0x00020000);
  }
  // This wave's block jj of a tile (jj < NJ, and jj * NW + w < PER).
  SDPA_DEV void issue_one(void* lds, __amdgpu_buffer_rsrc_t rs, int jj, int w) const {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs,
                                             (__attribute__((address_space(3))) void*)((char*)lds + (jj * NW + w) * 1024),
                                             16, (int)voff(jj), 0, 0, 0);
  }
  // Rows [0, min(valid, R)) of the tile whose row 0 starts at src.
  SDPA_DEV void issue(void* lds, const void* src, int valid, int w) const {
    __amdgpu_buffer_rsrc_t rs;
    if constexpr (DENSE) {  // valid is uniform and positive here
      const int rows = valid < R ? valid : R;
      rs = __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, rows * D * 2, 0x00020000);
    } else {
      rs = rsrc(src, valid);
    }
#pragma unroll
    for (int jj = 0; jj < NJ; jj++) {
      const int j = jj * NW + w;
      if (PER % NW != 0 && j >= PER) break;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)((char*)lds + j * 1024), 16,
                                               (int)voff(jj), 0, 0, 0);
    }
  }
};

// Zero n 16-bit elements of an LDS buffer with the workgroup's 256 threads
// (n a multiple of 8 * 256).
template <typename E>
SDPA_DEV void zero_lds(E* p, int n, int tid) {
  const i32x4 z = {0, 0, 0, 0};
  for (int i = tid * 8; i < n; i += 256 * 8) *(i32x4*)(p + i) = z;
}

// Wait for this wave's outstanding vector-memory loads and LDS operations,
// then a workgroup barrier with no cache fence: LDS tiles written by every
// wave are complete and every wave is done reading the previous buffer.
SDPA_DEV void wait_all_and_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) expcnt(7) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Wait until at most VM of this wave's vector-memory loads are outstanding
// (they complete in order, so the older ones have landed) and for its LDS
// operations, then a workgroup barrier.
template <int VM>
SDPA_DEV void wait_vm_and_barrier() {
  static_assert(VM >= 0 && VM < 64, "vmcnt field");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | ((VM >> 4) << 14));  // vmcnt(VM) expcnt(7) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Barrier for LDS-only hand-offs (no outstanding global loads are waited for).
SDPA_DEV void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// LDS hand-off between the lanes of one wave: this wave's LDS writes are
// complete, and the compiler moves no memory access across the call.
SDPA_DEV void wave_lds_sync() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Tiles of the dS band buffer that the dK/dV pass writes and the dQ pass
// reads (bounded bands): [kBandKeys keys][kBandRows query rows], key-major,
// one per (batch and q-head, block of kBandRows rows, key tile of the
// block's band).
constexpr int kBandRows = 128;
constexpr int kBandKeys = 64;

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2). Map dispatch order to a logical tile order in which each XCD receives a
// contiguous range, so neighbouring tiles (which share K/V or Q/dO bands)
// run on the same XCD. Bijection on [0, n).
SDPA_DEV int xcd_remap(int pid, int n) {
  constexpr int NX = 8;
  const int per = (n + NX - 1) / NX;
  const int tall = n % NX == 0 ? NX : n % NX;  // XCDs that get `per` tiles; the rest get per - 1
  const int x = pid % NX, local = pid / NX;
  return x < tall ? x * per + local : tall * per + (x - tall) * (per - 1) + local;
}

}  // namespace sdpa
