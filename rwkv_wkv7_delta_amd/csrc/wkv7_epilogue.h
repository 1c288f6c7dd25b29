// wkv7_epilogue.h -- the step after the read-out, on one (token, head) row.
//
// "Paper Review: RWKV-7 Goose", The approach: once the receptance has read the
// state, it also attends to the current token without storing it there, and the
// result is normalised per head and gated (the combination across heads, an
// output projection, is not part of this step).  The pages fix neither the
// current-token formula nor the normalisation nor their order; the library
// takes, with the learned parts as inputs:
//   s      = r_t . (u * k_t)                          (u: one vector per head)
//   norm x = gamma (x - mean x) rsqrt(var x + eps) + beta over the head's N
//            channels, var the mean squared deviation
//   mode 0: g_t (y_t + s v_t);  mode 1: g_t (norm(y_t) + s v_t);
//   mode 2: g_t norm(y_t + s v_t).
#pragma once

#include "wkv7_device.h"

namespace wkv7 {

// A row of N = C * P values lies in an aligned group of P lanes (P = 4, 8 or
// 16), C consecutive values per lane.  x: y in, the result out.  s: the row's
// r . (u * k) (used when `term`).  The moments are group sums over DPP, every
// lane of the group taking part with the same mode.
template <int C, int P>
__device__ __forceinline__ void epilogue_row(float (&x)[C], const float (&v)[C], float s, bool term,
                                             const float (&gam)[C], const float (&bet)[C],
                                             const float (&gate)[C], float eps, int mode) {
    constexpr float kInvN = 1.0f / (C * P);
    if (term && mode != 1) {
#pragma unroll
        for (int c = 0; c < C; ++c) x[c] = fmaf(s, v[c], x[c]);
    }
    if (mode != 0) {
        float m = 0.f;
#pragma unroll
        for (int c = 0; c < C; ++c) m += x[c];
        m = lanes_sum<P>(m) * kInvN;
        float q = 0.f;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            x[c] -= m;
            q = fmaf(x[c], x[c], q);
        }
        const float rs = rsqrtf(fmaf(lanes_sum<P>(q), kInvN, eps));
#pragma unroll
        for (int c = 0; c < C; ++c) x[c] = fmaf(x[c] * rs, gam[c], bet[c]);
        if (term && mode == 1) {
#pragma unroll
            for (int c = 0; c < C; ++c) x[c] = fmaf(s, v[c], x[c]);
        }
    }
#pragma unroll
    for (int c = 0; c < C; ++c) x[c] *= gate[c];
}

// C fp32 values (C a multiple of 4) from a 16-byte aligned address, or `fill`
// when p is null.
template <int C>
__device__ __forceinline__ void load_f32_or(const float* p, float fill, float (&x)[C]) {
    if (p) {
        load_cols<C>(p, x);
    } else {
#pragma unroll
        for (int c = 0; c < C; ++c) x[c] = fill;
    }
}

}  // namespace wkv7
