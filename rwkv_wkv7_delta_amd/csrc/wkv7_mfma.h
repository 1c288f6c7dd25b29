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

// Accumulator chains never mix shapes.  The CDNA3/CDNA4 ISA reference guides'
// table of required independent instructions between dependent matrix (XDL)
// operations lets an MFMA take the previous MFMA's result as its accumulator
// input (SrcC) back to back only when both are the same instruction; a SrcC
// written by an MFMA of another shape needs wait states that depend on the
// writer's pass count.  Rather than rely on those being inserted, partial sums
// of different shapes are added with vector ALU instructions (add4), whose read
// of an MFMA result the compiler does protect; tests/test_mfma_chains.py checks
// the built kernels for mixed-shape chains.
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

__device__ __forceinline__ f32x4 unpack4(bf16x4 x) {
    const u32x2_t u = __builtin_bit_cast(u32x2_t, x);
    f32x4 o;
    o[0] = __uint_as_float(u[0] << 16);
    o[1] = __uint_as_float(u[0] & 0xFFFF0000u);
    o[2] = __uint_as_float(u[1] << 16);
    o[3] = __uint_as_float(u[1] & 0xFFFF0000u);
    return o;
}

// An fp32 tile as two bf16 operands, hi = bf16(x) and lo = bf16(x - hi): a
// product summed as hi*hi' + hi*lo' + lo*hi' on the matrix core carries about
// 16 significant bits of each factor instead of 8.
struct Split4 {
    bf16x4 hi, lo;
};
__device__ __forceinline__ Split4 split4(f32x4 x) {
    Split4 s;
    s.hi = cvt4(x);
    s.lo = cvt4(x - unpack4(s.hi));
    return s;
}

// D + X Y from hi and lo bf16 parts of both factors (X as its A-operand image,
// Y as a B operand): hi*hi + hi*lo + lo*hi, the small terms first.
__device__ __forceinline__ f32x4 mul3(const Split4& x, const Split4& y, f32x4 d) {
    return mfma16(x.hi, y.hi, mfma16(x.hi, y.lo, mfma16(x.lo, y.hi, d)));
}

// Lane p of each group of four lanes (DPP quad_perm [p, p, p, p]).
template <int p>
__device__ __forceinline__ float quad_bcast(float x) {
    return __builtin_amdgcn_update_dpp(0.0f, x, p * 0x55, 0xF, 0xF, false);
}

// T = (I - A)^-1 for a strictly lower triangular 16x16 A, accurate to about
// 1e-5 relative to its largest entry, from four products on the matrix core:
//   Td = the inverses of the four 4x4 diagonal blocks of I - A, in fp32;
//   L  = A without its diagonal blocks;  N = Td L, strictly block-lower with
//        four block rows, so N^4 = 0 and
//   T  = (I - N)^-1 Td = (I + N)(I + N^2) Td.
// The direct doubling product (I + A)(I + A^2)(I + A^4)(I + A^8) is exact in
// exact arithmetic too, but its partial products hold binomial coefficients of
// up to C(15, 7) = 6435 when removal keys repeat or correlate inside a chunk
// (A[t][s] close to -1 for every s < t), and rounding those loses the O(1)
// result entirely.  Here the only large-sum cancellations are inside the
// 4x4 blocks, which are solved in fp32, and N's powers stay of order one; the
// products take hi and lo bf16 parts of both factors (mul3).
//
// In the accumulator layout (lane (g, l16) register q holds A[4g+q][l16]) the
// diagonal block of rows 4g.. sits in lanes l16 = 4g..4g+3 of row group g,
// one DPP quad, lane c holding its column c.  So every lane of that quad
// solves with the same six below-diagonal entries (quad broadcasts): lane c
// gets column c of the block's inverse (its accumulator registers, Td) and row
// c (the accumulator registers of Td^T).
//
// The work comes in two stages, which the kernels run in consecutive intervals
// on one wave: _begin forms Td, N and also the first product of the join (N N
// for the rows form, N^T N^T for the columns form), so that the two stages
// issue about as much work each; _end finishes T.
struct BlockInverse {
    f32x4 Td, NT, P;   // accumulator tiles of Td, N^T and the join's first product
};
template <bool kRows>
__device__ __forceinline__ BlockInverse unit_lower_inverse_begin(f32x4 A, int g, int l16) {
    const float a10 = quad_bcast<0>(A[1]), a20 = quad_bcast<0>(A[2]), a30 = quad_bcast<0>(A[3]);
    const float a21 = quad_bcast<1>(A[2]), a31 = quad_bcast<1>(A[3]);
    const float a32 = quad_bcast<2>(A[3]);
    const int c = l16 & 3;
    const float e0 = c == 0 ? 1.f : 0.f, e1 = c == 1 ? 1.f : 0.f;
    const float e2 = c == 2 ? 1.f : 0.f, e3 = c == 3 ? 1.f : 0.f;
    // column c of the block inverse: x_q = [q == c] + sum_{p<q} A[q][p] x_p
    const float x0 = e0;
    const float x1 = fmaf(a10, x0, e1);
    const float x2 = fmaf(a21, x1, fmaf(a20, x0, e2));
    const float x3 = fmaf(a32, x2, fmaf(a31, x1, fmaf(a30, x0, e3)));
    // row c: y_q = [q == c] + sum_{p>q} y_p A[p][q]
    const float y3 = e3;
    const float y2 = fmaf(y3, a32, e2);
    const float y1 = fmaf(y3, a31, fmaf(y2, a21, e1));
    const float y0 = fmaf(y3, a30, fmaf(y2, a20, fmaf(y1, a10, e0)));
    const bool diag = (l16 >> 2) == g;
    BlockInverse b;
    f32x4 TdT, L;
#pragma unroll
    for (int q = 0; q < 4; ++q) L[q] = diag ? 0.f : A[q];
    b.Td[0] = diag ? x0 : 0.f; b.Td[1] = diag ? x1 : 0.f; b.Td[2] = diag ? x2 : 0.f; b.Td[3] = diag ? x3 : 0.f;
    TdT[0] = diag ? y0 : 0.f; TdT[1] = diag ? y1 : 0.f; TdT[2] = diag ? y2 : 0.f; TdT[3] = diag ? y3 : 0.f;
    const Split4 sL = split4(L), sTdT = split4(TdT);
    const f32x4 N = mul3(sTdT, sL, zero4());   // Td L   (Td^T's registers are Td's A-operand image)
    b.NT = mul3(sL, sTdT, zero4());            // L^T Td^T
    const Split4 sN = split4(N), sNT = split4(b.NT);
    b.P = kRows ? mul3(sNT, sN, zero4())       // N N
                : mul3(sN, sNT, zero4());      // N^T N^T
    return b;
}
// The accumulator tile of T^T (= T's A-operand image: lane (g, l16) register q
// holds T[l16][4g+q]): T^T = Td^T (I + (N^T)^2)(I + N^T), from the rows form
// of _begin.
__device__ __forceinline__ f32x4 unit_lower_inverse_rows_end(const BlockInverse& b, int g, int l16) {
    f32x4 W1 = b.NT;                                      // I + N^T
#pragma unroll
    for (int q = 0; q < 4; ++q) W1[q] += (4 * g + q == l16) ? 1.f : 0.f;
    const f32x4 W2 = mul3(split4(b.P), split4(W1), W1);  // W1 + (N^T)^2 W1
    return mul3(split4(b.Td), split4(W2), zero4());      // Td^T W2
}
// The accumulator tile of T (= T^T's A-operand image: lane (g, l16) register q
// holds T[4g+q][l16]): T = (I + N)(I + N^2) Td, from the columns form of _begin.
__device__ __forceinline__ f32x4 unit_lower_inverse_cols_end(const BlockInverse& b) {
    const f32x4 V2 = mul3(split4(b.P), split4(b.Td), b.Td);   // Td + N^2 Td
    return mul3(split4(b.NT), split4(V2), V2);                // V2 + N V2
}

}  // namespace wkv7
