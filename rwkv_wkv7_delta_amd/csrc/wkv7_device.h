// wkv7_device.h -- device helpers shared by the WKV7 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wkv7 {

constexpr int kN = 64;           // head size: state is kN x kN

typedef uint16_t bf16_t;         // raw IEEE bfloat16 bits

// ---------------------------------------------------------------------------
// Element access for the two token dtypes.  bf16 -> fp32 is exact (a shift);
// fp32 -> bf16 rounds to nearest even via the gfx950 conversion instruction.
// ---------------------------------------------------------------------------
template <typename T> struct Elem;

template <> struct Elem<float> {
    // Four elements as loaded (raw4) and their fp32 values (cvt): a prefetch keeps
    // raw4 so that nothing uses the loaded registers before they are stashed.
    typedef float4 raw4;
    static __device__ __forceinline__ raw4 load_raw4(const float* p) {
        return *reinterpret_cast<const float4*>(p);
    }
    static __device__ __forceinline__ float4 cvt(raw4 x) { return x; }
    static __device__ __forceinline__ float4 load4(const float* p) {
        return *reinterpret_cast<const float4*>(p);
    }
    static __device__ __forceinline__ float2 load2(const float* p) {
        return *reinterpret_cast<const float2*>(p);
    }
    static __device__ __forceinline__ float load1(const float* p) { return *p; }
    static __device__ __forceinline__ void store1(float* p, float x) { *p = x; }
    static __device__ __forceinline__ void store4(float* p, float4 x) {
        *reinterpret_cast<float4*>(p) = x;
    }
};

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ bf16_t f2bf(float x) {
    __bf16 h = static_cast<__bf16>(x);
    return __builtin_bit_cast(bf16_t, h);
}
// Raw bits of a bf16 value (assigning __bf16 to an integer would convert the value).
__device__ __forceinline__ bf16_t bits(__bf16 h) { return __builtin_bit_cast(bf16_t, h); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}

template <> struct Elem<bf16_t> {
    typedef uint2 raw4;
    static __device__ __forceinline__ raw4 load_raw4(const bf16_t* p) {
        return *reinterpret_cast<const uint2*>(p);
    }
    static __device__ __forceinline__ float4 cvt(raw4 u) {
        return make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
    }
    static __device__ __forceinline__ float4 load4(const bf16_t* p) {
        const uint2 u = *reinterpret_cast<const uint2*>(p);
        return make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
    }
    static __device__ __forceinline__ float2 load2(const bf16_t* p) {
        const uint32_t u = *reinterpret_cast<const uint32_t*>(p);
        return make_float2(bf16_lo(u), bf16_hi(u));
    }
    static __device__ __forceinline__ float load1(const bf16_t* p) {
        return __uint_as_float((uint32_t)(*p) << 16);
    }
    static __device__ __forceinline__ void store1(bf16_t* p, float x) { *p = f2bf(x); }
    static __device__ __forceinline__ void store4(bf16_t* p, float4 x) {
        uint2 u;
        u.x = pack_bf16x2(x.x, x.y);
        u.y = pack_bf16x2(x.z, x.w);
        *reinterpret_cast<uint2*>(p) = u;
    }
};

// C consecutive elements (C = 2, 4 or 8) as fp32, and the fp32 store of C values.
template <int C, typename T>
__device__ __forceinline__ void load_cols(const T* p, float (&x)[C]) {
    static_assert(C == 2 || C % 4 == 0, "2, 4 or 8 columns per lane");
    if constexpr (C == 2) {
        const float2 f = Elem<T>::load2(p);
        x[0] = f.x; x[1] = f.y;
    } else {
#pragma unroll
        for (int i = 0; i < C; i += 4) {
            const float4 f = Elem<T>::load4(p + i);
            x[i] = f.x; x[i + 1] = f.y; x[i + 2] = f.z; x[i + 3] = f.w;
        }
    }
}
template <int C>
__device__ __forceinline__ void store_cols(float* p, const float (&x)[C]) {
    if constexpr (C == 2) {
        *reinterpret_cast<float2*>(p) = make_float2(x[0], x[1]);
    } else {
#pragma unroll
        for (int i = 0; i < C; i += 4)
            *reinterpret_cast<float4*>(p + i) = make_float4(x[i], x[i + 1], x[i + 2], x[i + 3]);
    }
}
// In-lane part of a dot product, accumulated in column order.
template <int C>
__device__ __forceinline__ float dot_cols(const float (&s)[C], const float (&q)[C]) {
    float acc = s[0] * q[0];
#pragma unroll
    for (int i = 1; i < C; ++i) acc = fmaf(s[i], q[i], acc);
    return acc;
}

// ---------------------------------------------------------------------------
// Sum over the 16 lanes of a DPP row; every lane of the row gets the total.
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float row16_sum(float x) {
    x += __builtin_amdgcn_update_dpp(0.0f, x, 0xB1, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0.0f, x, 0x4E, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0.0f, x, 0x141, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0.0f, x, 0x140, 0xF, 0xF, false);
    return x;
}

// Sum over each aligned group of P = 4, 8 or 16 lanes; every lane of the group
// gets the total (quad_perm [1,0,3,2], quad_perm [2,3,0,1], then for 8 lanes
// row_half_mirror, for 16 also row_mirror).
template <int P>
__device__ __forceinline__ float lanes_sum(float x) {
    static_assert(P == 4 || P == 8 || P == 16, "groups of 4, 8 or 16 lanes");
    x += __builtin_amdgcn_update_dpp(0.0f, x, 0xB1, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0.0f, x, 0x4E, 0xF, 0xF, false);
    if (P >= 8) x += __builtin_amdgcn_update_dpp(0.0f, x, 0x141, 0xF, 0xF, false);
    if (P >= 16) x += __builtin_amdgcn_update_dpp(0.0f, x, 0x140, 0xF, 0xF, false);
    return x;
}

// Inclusive running product over the 16 lanes of each DPP row, in lane order
// (row_shr 1, 2, 4, 8; lanes shifted in from outside the row contribute 1).
__device__ __forceinline__ float row16_cumprod(float x) {
    x *= __builtin_amdgcn_update_dpp(1.0f, x, 0x111, 0xF, 0xF, false);
    x *= __builtin_amdgcn_update_dpp(1.0f, x, 0x112, 0xF, 0xF, false);
    x *= __builtin_amdgcn_update_dpp(1.0f, x, 0x114, 0xF, 0xF, false);
    x *= __builtin_amdgcn_update_dpp(1.0f, x, 0x118, 0xF, 0xF, false);
    return x;
}
// The same running product for four independent values at once, one DPP
// multiply per step: with the bound control off, a lane whose source lies
// outside its row is left unwritten, i.e. keeps x (x times 1).  The leading
// s_nop gives the two wait states a DPP read needs after the VALU write of its
// operand; inside, each operand was written three instructions earlier.
__device__ __forceinline__ void row16_cumprod4(float& x0, float& x1, float& x2, float& x3) {
    asm volatile(
        "s_nop 1\n\t"
        "v_mul_f32_dpp %0, %0, %0 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %1, %1, %1 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %2, %2, %2 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %3, %3, %3 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %0, %0, %0 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %1, %1, %1 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %2, %2, %2 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %3, %3, %3 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %0, %0, %0 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %1, %1, %1 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %2, %2, %2 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %3, %3, %3 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %0, %0, %0 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %1, %1, %1 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %2, %2, %2 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %3, %3, %3 row_shr:8 row_mask:0xf bank_mask:0xf"
        : "+v"(x0), "+v"(x1), "+v"(x2), "+v"(x3));
}

// The value of the previous lane of the row (row_shr 1); the row's first lane gets `first`.
__device__ __forceinline__ float row16_prev(float x, float first) {
    return __builtin_amdgcn_update_dpp(first, x, 0x111, 0xF, 0xF, false);
}
// Lane 15 of each row broadcast to the whole row (row_newbcast 15).
__device__ __forceinline__ float row16_last(float x) {
    return __builtin_amdgcn_update_dpp(0.0f, x, 0x15F, 0xF, 0xF, false);
}

// Sum over the four 16-lane rows of a wave of the values at the same position
// in the row, in every lane: v_permlane32_swap of x with itself gives the rows
// (0, 1, 0, 1) and (2, 3, 2, 3); their sum s holds rows (0+2, 1+3, 0+2, 1+3);
// v_permlane16_swap of s with itself gives (0+2) and (1+3) in every row.
__device__ __forceinline__ float sum_rows4(float x) {
    const unsigned u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const unsigned s = __float_as_uint(__uint_as_float(a[0]) + __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(s, s, false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Lane n of each row broadcast to the whole row (row_newbcast n).
template <int n>
__device__ __forceinline__ float row16_bcast(float x) {
    return __builtin_amdgcn_update_dpp(0.0f, x, 0x150 + n, 0xF, 0xF, false);
}
__device__ __forceinline__ float dot4(float4 s, float4 q) {
    return fmaf(s.w, q.w, fmaf(s.z, q.z, fmaf(s.y, q.y, s.x * q.x)));
}

// 16-byte store of an output nothing in this kernel reads again (streamed past
// the caches: the non-temporal hint).
__device__ __forceinline__ void store_stream(void* dst, uint4 x) {
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(__builtin_bit_cast(u4, x), reinterpret_cast<u4*>(dst));
}

// Token tensor offset for [B][T][H][N].
template <int N = kN>
__device__ __forceinline__ size_t tok_off(int b, int t, int h, int T, int H) {
    return (((size_t)b * T + t) * H + h) * N;
}

// Work of one workgroup: a head over tokens [t_begin, t_end), started from the
// state rows at `init` (else the identity when `ident`, else zero), with v
// taken as zero when `vzero`; outputs (y, tape) only when `outs`; the final
// state to `fin` when not null.
struct Work {
    int bh, t_begin, t_end;
    const float* init;
    float* fin;
    bool ident, vzero, outs;
};

// The head that workgroup `blk` of `n` one-head workgroups takes.  The device
// hands workgroups to its eight XCDs in turn (workgroup u to XCD u mod 8), and
// heads whose index is the same mod 8 sit at the same place of every token row,
// which under the full round's memory traffic can make one such group slower
// than the rest (at H = 40 the heads = 3 mod 8 by about a fifth).  Rotating the
// heads of every group of eight workgroups by the group's index gives each XCD
// every residue, so no XCD holds all the slow heads and the work queued behind
// them (the next round, the split heads' runs) starts on time everywhere.
__device__ __forceinline__ int spread_heads(int blk, int n) {
    const int q = blk >> 3;
    return 8 * q + 8 > n ? blk : 8 * q + ((blk + q) & 7);
}

// blockIdx -> Work under a segment plan (FwdSplit): heads below split_from run
// whole in pass 0; every later head runs in nseg segments of seg_len tokens.
// Pass 0 also runs each split head's segment 0 (with outputs; its final state
// is the entry state of segment 1) and, for segments 1 .. nseg-2, the two runs
// whose final states give the segment's affine map S_out = S_in P + Hm: Hm from
// zero with the real v, P from the identity with v = 0 (the recurrence is
// affine in the state: S <- S M_t + v_t k_t^T).  Pass 1 re-runs segments
// 1 .. nseg-1 from their entry states (composed in between), with outputs.
// Per split head the workspace holds 3 nseg states: entry states (slot s),
// Hm (nseg + s) and P (2 nseg + s).
template <int N>
__device__ __forceinline__ Work work_of(int blk, int pass, int T, const float* s0, float* sT,
                                        int split_from, int nseg, int seg_len, float* states) {
    constexpr size_t NN = (size_t)N * N;
    Work wk{0, 0, T, nullptr, nullptr, false, false, true};
    if (pass == 0 && blk < split_from) {
        wk.bh = spread_heads(blk, split_from);
        wk.init = s0 ? s0 + (size_t)wk.bh * NN : nullptr;
        wk.fin = sT ? sT + (size_t)wk.bh * NN : nullptr;
        return wk;
    }
    const int j = pass == 0 ? blk - split_from : blk;
    const int per = pass == 0 ? 2 * nseg - 3 : nseg - 1;
    const int hs = j / per, rr = j % per;
    wk.bh = split_from + hs;
    float* const hst = states + (size_t)hs * 3 * nseg * NN;
    if (pass == 0 && rr == 0) {
        wk.t_end = seg_len;
        wk.init = s0 ? s0 + (size_t)wk.bh * NN : nullptr;
        wk.fin = hst + NN;
    } else if (pass == 0) {
        const int sg = 1 + (rr - 1) / 2;
        const bool pm = ((rr - 1) & 1) != 0;
        wk.t_begin = sg * seg_len;
        wk.t_end = wk.t_begin + seg_len;
        wk.ident = pm;
        wk.vzero = pm;
        wk.outs = false;
        wk.fin = hst + (size_t)((pm ? 2 : 1) * nseg + sg) * NN;
    } else {
        const int sg = 1 + rr;
        wk.t_begin = sg * seg_len;
        wk.t_end = sg == nseg - 1 ? T : wk.t_begin + seg_len;
        wk.init = hst + (size_t)sg * NN;
        wk.fin = (sg == nseg - 1 && sT) ? sT + (size_t)wk.bh * NN : nullptr;
    }
    return wk;
}

}  // namespace wkv7
