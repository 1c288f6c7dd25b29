// wkv7_mfma.h -- bf16 matrix-core helpers for gfx950 (wave64).
//
// Operand layouts used throughout (lane l, g = l / 16, q = register index):
//   v_mfma_f32_16x16x16_bf16:  A[m][k]: m = l%16, k = 4g+q (q<4)
//                              B[k][n]: n = l%16, k = 4g+q
//   v_mfma_f32_16x16x32_bf16:  A[m][k]: m = l%16, k = 8g+q (q<8)
//                              B[k][n]: n = l%16, k = 8g+q
//   accumulator C/D[m][n]:     n = l%16, m = 4g+q (q<4)
// A D tile therefore feeds the next product directly as its B operand (its
// rows become the contraction index), so chains of left-multiplications stay
// in registers.  Any bijection of the contraction index applied to both A
// and B leaves the product unchanged; the kernels use this to feed two D
// tiles as one 32-deep B operand.
#pragma once

#include <hip/hip_runtime.h>

#include "wkv7_device.h"

namespace wkv7 {

typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// x[q] times what lane 4 JT + q of this lane's row holds in `f`: one DPP
// multiply each, so that 16 per-column factors spread over a row's lanes
// (one 4-byte LDS read per lane) reach an accumulator tile without a broadcast
// read of all 16 into every lane.
template <int JT>
__device__ __forceinline__ f32x4 mul_row_lanes4(float f, f32x4 x) {
    f32x4 o;
    o[0] = row16_bcast<4 * JT + 0>(f) * x[0];
    o[1] = row16_bcast<4 * JT + 1>(f) * x[1];
    o[2] = row16_bcast<4 * JT + 2>(f) * x[2];
    o[3] = row16_bcast<4 * JT + 3>(f) * x[3];
    return o;
}

// Accumulator chains never mix shapes.  On gfx950 a 16x16x16 MFMA whose
// accumulator input is the result of a 16x16x32 MFMA (or the reverse) reads
// stale accumulator registers unless 5 wait states separate the two, and the
// compiler does not insert them (same-shape chains forward correctly).  Partial
// sums of different shapes are therefore added with vector ALU instructions
// (add4); the compiler does protect a vector ALU read of an MFMA result.
__device__ __forceinline__ f32x4 add4(f32x4 a, f32x4 b) { return a + b; }

// An MFMA runs across the whole wave: with part of the EXEC mask off it does
// not compute the product of the full operands.  The compiler may sink an MFMA
// whose result only feeds a store under a divergent branch into that branch,
// so such results are pinned first (an empty asm that the branch cannot move).
__device__ __forceinline__ bf16x4 pin(bf16x4 x) {
    asm volatile("" : "+v"(x));
    return x;
}

__device__ __forceinline__ f32x4 zero4() {
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    return z;
}

// fp32 -> bf16, round to nearest even, two values per v_cvt_pk_bf16_f32.  The
// pairs travel as 32-bit words: converting a 4-vector directly makes the
// compiler convert one element at a time and repack with v_perm.
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ unsigned cvt2(float a, float b) {
    const f32x2 x = {a, b};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(x, bf16x2));
}
__device__ __forceinline__ bf16x4 cvt4(float a, float b, float c, float d) {
    const u32x2_t r = {cvt2(a, b), cvt2(c, d)};
    return __builtin_bit_cast(bf16x4, r);
}
__device__ __forceinline__ bf16x4 cvt4(f32x4 x) { return cvt4(x[0], x[1], x[2], x[3]); }
__device__ __forceinline__ bf16x8 cat8(bf16x4 lo, bf16x4 hi) {
    bf16x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}

// The 16x16 identity as a B operand: lane (g, l16) register q is [4g+q == l16].
__device__ __forceinline__ bf16x4 identity_b(int g, int l16) {
    return cvt4(4 * g + 0 == l16 ? 1.f : 0.f, 4 * g + 1 == l16 ? 1.f : 0.f,
                4 * g + 2 == l16 ? 1.f : 0.f, 4 * g + 3 == l16 ? 1.f : 0.f);
}
// Layout exchange of a 16x16 bf16 tile through the matrix core (exact: one
// non-zero product per output).  The row layout of X (lane (g, l16) holds
// X[l16][4g..4g+3], i.e. X as an A operand) and the accumulator layout of X
// (lane (g, l16) holds X[4g..4g+3][l16]) map to each other: X A-operand times
// I gives X's accumulator tile, and accumulator registers fed as an A operand
// stand for X^T, so X^T times I gives the row layout of X.
__device__ __forceinline__ bf16x4 swap_layout(bf16x4 x, bf16x4 ident) {
    return cvt4(mfma16(x, ident, zero4()));
}

// Transposed LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i receives element i % 4 of the 8-byte pieces that lanes i / 4 + 4 q
// (q = 0 .. 3) point at.  So for a row-major bf16 array X whose 16 x 16 tile
// starts at X[r0][c0], lane (g, j) passing &X[r0 + 4g + j/4][c0 + 4 (j%4)]
// receives X[r0 + 4g + q][c0 + j], q = 0 .. 3: the accumulator layout of the
// tile, i.e. the tile's transpose as an A operand (what swap_layout gives for
// the row-layout read, without the matrix core).
__device__ __forceinline__ const bf16_t* tr_addr(const bf16_t* tile, int row_stride, int g, int l16) {
    return tile + (4 * g + (l16 >> 2)) * row_stride + 4 * (l16 & 3);
}
__device__ __forceinline__ bf16x4 ld4_tr(const bf16_t* p) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4s*)(p));
    return __builtin_bit_cast(bf16x4, r);
}

// (I - A)^-1 for a strictly lower triangular 16x16 A (so A^16 = 0) as the
// doubling product (I + A)(I + A^2)(I + A^4)(I + A^8), all on bf16 MFMA with
// fp32 accumulation.  Inputs are the accumulator tiles of A and A^T; C-layout
// registers fed as an A operand stand for the transpose of their matrix, so
// the chain needs no data movement.  Returns T^T in C layout, i.e. lane
// (g, l16) register q holds T[l16][4g+q] -- exactly T's A-operand layout.
__device__ __forceinline__ f32x4 unit_lower_inverse_T(f32x4 A, f32x4 AT, int g, int l16) {
    const f32x4 z = zero4();
    const f32x4 A2 = mfma16(cvt4(AT), cvt4(A), z);     // A A
    const f32x4 A2T = mfma16(cvt4(A), cvt4(AT), z);    // A^T A^T
    const f32x4 A4 = mfma16(cvt4(A2T), cvt4(A2), z);
    const f32x4 A4T = mfma16(cvt4(A2), cvt4(A2T), z);
    const f32x4 A8 = mfma16(cvt4(A4T), cvt4(A4), z);
    f32x4 P = AT;                                      // (I + A)^T
#pragma unroll
    for (int q = 0; q < 4; ++q) P[q] += (4 * g + q == l16) ? 1.f : 0.f;
    P = mfma16(cvt4(A2), cvt4(P), P);                  // P^T += (A^2)^T P^T
    P = mfma16(cvt4(A4), cvt4(P), P);
    P = mfma16(cvt4(A8), cvt4(P), P);
    return P;
}

}  // namespace wkv7
