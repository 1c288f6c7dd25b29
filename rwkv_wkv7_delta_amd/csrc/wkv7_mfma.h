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

__device__ __forceinline__ f32x4 zero4() {
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    return z;
}

__device__ __forceinline__ bf16x4 cvt4(f32x4 x) {
    bf16x4 r;
    r[0] = (__bf16)x[0];
    r[1] = (__bf16)x[1];
    r[2] = (__bf16)x[2];
    r[3] = (__bf16)x[3];
    return r;
}
__device__ __forceinline__ bf16x4 cvt4(float a, float b, float c, float d) {
    bf16x4 r;
    r[0] = (__bf16)a;
    r[1] = (__bf16)b;
    r[2] = (__bf16)c;
    r[3] = (__bf16)d;
    return r;
}
__device__ __forceinline__ bf16x8 cat8(bf16x4 lo, bf16x4 hi) {
    bf16x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}

}  // namespace wkv7
