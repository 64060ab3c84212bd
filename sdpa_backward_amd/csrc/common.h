// Device-side building blocks shared by the gfx950 attention kernels.
//
// MFMA used: v_mfma_f32_32x32x16_bf16 (wave64). Lane layouts (checked on the
// hardware):
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
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

#define SDPA_DEV __device__ __forceinline__

namespace sdpa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

SDPA_DEV f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

SDPA_DEV f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; i++) z[i] = 0.f;
  return z;
}

SDPA_DEV bf16x8 zero_bf16x8() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; i++) z[i] = (bf16)0.f;
  return z;
}

// 4 consecutive bf16 of one row-major LDS tile, delivered transposed across
// each 16-lane group (see header comment).
SDPA_DEV bf16x4 lds_tr4(const bf16* p) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

// Operand from a row-major LDS tile T[k][mn] (rows are the contraction index):
// lane l gets column mn0 + l%32 with "paired" k-slots over rows [k0, k0+16).
SDPA_DEV bf16x8 ld_op_tr(const bf16* T, int ld, int k0, int mn0, int lane) {
  const int G = lane >> 4, i = lane & 15;
  const int row = k0 + 4 * (G >> 1) + (i >> 2);
  const int col = mn0 + 16 * (G & 1) + 4 * (i & 3);
  bf16x4 lo = lds_tr4(T + row * ld + col);
  bf16x4 hi = lds_tr4(T + (row + 8) * ld + col);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Operand from a row-major LDS tile T[mn][k] (columns are the contraction
// index): lane l gets row mn0 + l%32 with "direct" k-slots k0 + 8*(l/32) + j.
SDPA_DEV bf16x8 ld_op(const bf16* T, int ld, int k0, int mn0, int lane) {
  return *(const bf16x8*)(T + (mn0 + (lane & 31)) * ld + k0 + 8 * (lane >> 5));
}

// fp32 C-tile values [8*op, 8*op+8) as a bf16 "paired" operand (rows of the
// C tile become k: op 0 covers C rows 0..15, op 1 rows 16..31).
SDPA_DEV bf16x8 c_to_op(const f32x16& c, int op) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; j++) r[j] = (bf16)c[8 * op + j];
  return r;
}

// Row of the C tile held in accumulator slot i by a lane in half h.
SDPA_DEV int c_row(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

// Allowed (query i, key j) pair: causal diagonal, window (w_eff = min(window, L)
// or L for plain causal), both indices inside the sequence.
SDPA_DEV bool allowed(int i, int j, int w_eff, int L) {
  return j <= i && j > i - w_eff && i < L;  // j <= i < L implies j < L
}

// Copy a [rows x D] bf16 tile from global (row-major, stride D) into LDS with
// row stride ld, zero-filling rows >= valid_rows. 16-byte chunks, block-strided.
template <int D, int NTHREADS>
SDPA_DEV void load_tile(bf16* dst, int ld, const bf16* __restrict__ src, int rows, int valid_rows,
                        int tid) {
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  const int total = rows * CPR;
  for (int c = tid; c < total; c += NTHREADS) {
    const int r = c / CPR, k = (c % CPR) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < valid_rows) v = *(const uint4*)(src + (size_t)r * D + k);
    *(uint4*)(dst + r * ld + k) = v;
  }
}

}  // namespace sdpa
