// wkv7_chunk128.hip -- chunked WKV7 forward at head size N = 128 on bf16 MFMA.
//
// The larger state is the expansion that "Millions of States: Designing a
// Scalable MoE Architecture with RWKV-7 Meta-learner" (Abstract) grows; the
// chunk algebra is the one of the N = 64 form (wkv7_chunk_fwd.hip), an exact
// rearrangement of the recurrence over a chunk of L = 16 tokens with entry
// state S0 (running decay G_t, At = a G_{t-1}, Rt = r G_t, Bh = b / G_t,
// Kh = k / G_t, Bb = Bh G_L, Kb = Kh G_L):
//   Aab = tril_-1(At Bh^T), Aak = tril_-1(At Kh^T), Arb = tril_0(Rt Bh^T),
//   Ark = tril_0(Rt Kh^T), Tm = (I - Aab)^-1,
//   Z = (Tm At) S0^T + (Tm Aak) V,   Y = Rt S0^T + Arb Z + Ark V,
//   S_L^T = diag(G_L) S0^T + Kb^T V + Bb^T Z.
// Given a chunk's factors, value row i of the state runs a chain of its own:
// row i of Z, Y and S_L reads only row i of S0 and column i of V.  So a head's
// 128 rows go to 8 / W workgroups of W waves, 16 rows per wave (the rows of
// S^T in eight 16 x 16 fp32 accumulator tiles, key blocks), and every
// workgroup forms the chunk's factors itself with all of its waves: no
// workspace, at the price of reading the head's token rows once per
// workgroup (the workgroups of one head go to one XCD, whose L2 then serves
// the later reads).  One chunk passes through five stages, a barrier after
// each:
//   (A) stash the chunk's raw rows (loaded one chunk ahead into registers),
//       store the previous chunk's read-outs, load the next chunk;
//   (B) E: decay products and scaled vectors, key groups of 16 over the waves;
//   (C) the L x L products over 128 keys: Aab and its inverse (wave 0), Aak
//       (wave 1), Arb (wave 2), Ark (wave 3);
//   (D) At' = Tm At (key tiles over the waves) and Aak' = Tm Aak (wave 0);
//   (E) each wave's state chain; its read-outs staged in LDS.
// Lane layouts of the matrix-core operands: wkv7_mfma.h.  Chunks are padded
// past T (w = 1, everything else 0: the identity on the state).

#include "wkv7.h"
#include "wkv7_device.h"
#include "wkv7_internal.h"
#include "wkv7_mfma.h"

namespace wkv7 {

namespace {

constexpr int kL = 16;
constexpr int kN128 = 128;
// LDS row stride in bf16 elements: 272 bytes, so that rows sit 4 banks apart
// and the 16 rows a DPP row of lanes reads in one access fall on different banks.
constexpr int kR128 = kN128 + 8;
constexpr int kJT = kN128 / 16;   // key tiles of 16
constexpr int kK2 = kN128 / 32;   // 32-deep contraction steps over the keys

enum { R_R = 0, R_W = 1, R_K = 2, R_A = 3, R_B = 4, R_V = 5 };
enum { T_AK = 0, T_RB = 1, T_RK = 2 };

template <int W>
struct __align__(16) Smem128 {
    bf16_t raw[6][kL][kR128];                  // r, w, k, a, b, v of the chunk (bf16 bits)
    bf16_t At[kL][kR128], Rt[kL][kR128];       // At is overwritten by At' = Tm At in (D)
    bf16_t Bh[kL][kR128], Kh[kL][kR128];
    bf16_t Bb[kL][kR128], Kb[kL][kR128];
    float gL[2 * 64];     // G_L of key 16 jt + 4 g + q at word 64 (jt / 4) + 16 g + 4 (jt % 4) + q
    uint2 tm_hi[64], tm_lo[64];   // hi and lo bf16 parts of Tm's A-operand image
    f32x4 aak[64];                // Aak in the accumulator layout [t][s], fp32
    uint2 tiles[3][64];           // A-operand images of Aak', Arb, Ark
    bf16_t Ys[kL][16 * W + 8];    // the read-outs of this workgroup's rows, [t][i]
};

__device__ __forceinline__ bf16x4 ld4(const bf16_t* p) {
    return __builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2*>(p));
}
__device__ __forceinline__ bf16x8 ld8(const bf16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ bf16x8 ld4x2(const bf16_t* p) { return cat8(ld4(p), ld4(p + 16)); }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// W waves per workgroup (4 or 8), 16 W value rows of one head; kAB = false:
// a = b = 0 (no removal terms: Y = Rt S0^T + Ark V, S_L^T = diag(G_L) S0^T +
// Kb^T V); kCk: also the fp32 state entering every chunk,
// [B][H][ceil(T/16)][N][N] (row = value channel).
template <int W, bool kAB, bool kCk>
__global__ __launch_bounds__(64 * W, 8 / W) void chunk128_fwd_kernel(
    int B, int T, int H, const bf16_t* __restrict__ r, const bf16_t* __restrict__ w,
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, const bf16_t* __restrict__ a,
    const bf16_t* __restrict__ b, const float* __restrict__ s0, bf16_t* __restrict__ y,
    float* __restrict__ sT, float* __restrict__ ckpt) {
    static_assert(W == 4 || W == 8, "four or eight waves");
    constexpr int kParts = 8 / W;               // workgroups per head
    constexpr int kRows = 16 * W;               // value rows per workgroup
    constexpr int kPieces = 24 / W;             // 16-byte raw pieces per thread and chunk
    constexpr size_t NN = (size_t)kN128 * kN128;
    __shared__ Smem128<W> sm;

    // Workgroups go to the eight XCDs in turn (u to XCD u mod 8).  Groups of 8
    // heads take 8 kParts consecutive workgroups, part-major, so that the parts
    // of a head share an XCD and run at about the same time.
    const int nbh = B * H;
    const int u = blockIdx.x;
    const int grp = u / (8 * kParts), within = u % (8 * kParts);
    const int m = min(8, nbh - 8 * grp);
    const int part = within / m;
    const int bh = 8 * grp + within % m;
    const int bb = bh / H, hh = bh % H;
    const int rb = part * kRows;                // first value row of this workgroup

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // The role branches of stages (C) and (D) test a scalar copy of the wave
    // index: scalar branches, so no matrix-core product runs with part of EXEC off.
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const int l16 = lane & 15, g = lane >> 4;
    const int col = rb + 16 * wave + l16;       // this lane's value row in the chain
    const int nch = (T + kL - 1) / kL;
    const bf16x4 ident = identity_b(g, l16);

    // ---- state: S^T tiles, lane holds S[col][16 jt + 4 g + q] ----------------
    f32x4 S[kJT];
#pragma unroll
    for (int jt = 0; jt < kJT; ++jt) S[jt] = zero4();
    if (s0) {
        const float* base = s0 + (size_t)bh * NN + (size_t)col * kN128;
#pragma unroll
        for (int jt = 0; jt < kJT; ++jt) {
            const float4 x = *reinterpret_cast<const float4*>(base + 16 * jt + 4 * g);
            S[jt][0] = x.x; S[jt][1] = x.y; S[jt][2] = x.z; S[jt][3] = x.w;
        }
        // settled here: left pending, every later use of S would wait on the
        // whole memory counter (and so on the chunks' stores)
        __builtin_amdgcn_s_waitcnt(0);
    }

    // ---- raw rows: 6 vectors x 16 tokens x 16 pieces of 16 bytes per chunk.
    // Piece p = tid + 64 W e: vector p / 256, token (p / 16) % 16, columns
    // 8 (p % 16) .. +7; a token row of a vector is 16 consecutive threads.
    const int ld_t = (tid >> 4) & 15, ld_c8 = tid & 15;
    // (vector of piece e: e at W = 4; 2 e or 2 e + 1 at W = 8, by wave half)
    const int vhi = W == 8 ? (tid >> 8) : 0;
    auto vec_of = [&](int e) __attribute__((always_inline)) { return W == 4 ? e : 2 * e + vhi; };
    auto src_of = [&](int e) __attribute__((always_inline)) -> const bf16_t* {
        const bf16_t* const src6[6] = {r, w, k, a, b, v};
        if constexpr (W == 4) return src6[e];
        else return vhi ? src6[2 * e + 1] : src6[2 * e];
    };
    auto load_raw = [&](int c, u32x4 (&o)[kPieces]) __attribute__((always_inline)) {
        const int t = min(c * kL + ld_t, T - 1);
        const size_t off = tok_off<kN128>(bb, t, hh, T, H) + 8 * ld_c8;
#pragma unroll
        for (int e = 0; e < kPieces; ++e) {
            const int vi = vec_of(e);
            if (kAB || (vi != R_A && vi != R_B)) {
                o[e] = *reinterpret_cast<const u32x4*>(src_of(e) + off);
            } else {
                const u32x4 z = {0u, 0u, 0u, 0u};
                o[e] = z;
            }
        }
    };
    auto stash_raw = [&](int c, const u32x4 (&o)[kPieces]) __attribute__((always_inline)) {
        const bool ok = c * kL + ld_t < T;
#pragma unroll
        for (int e = 0; e < kPieces; ++e) {
            const int vi = vec_of(e);
            const unsigned pad = vi == R_W ? 0x3F803F80u : 0u;   // padding: w = 1, the rest 0
            const u32x4 padv = {pad, pad, pad, pad};
            *reinterpret_cast<u32x4*>(&sm.raw[vi][ld_t][8 * ld_c8]) = ok ? o[e] : padv;
        }
    };

    // ---- (B) E: key group cg (16 keys); lane (g, l16) = token l16, keys j0 .. j0+3
    auto stage_E = [&](int cg) __attribute__((always_inline)) {
        const int j0 = 16 * cg + 4 * g;
        float X[6][4];
#pragma unroll
        for (int vi = 0; vi < 5; ++vi) {
            if (!kAB && (vi == R_A || vi == R_B)) continue;
            const uint2 q = *reinterpret_cast<const uint2*>(&sm.raw[vi][l16][j0]);
            X[vi][0] = bf16_lo(q.x); X[vi][1] = bf16_hi(q.x);
            X[vi][2] = bf16_lo(q.y); X[vi][3] = bf16_hi(q.y);
        }
        float G4[4] = {X[R_W][0], X[R_W][1], X[R_W][2], X[R_W][3]};
        row16_cumprod4(G4[0], G4[1], G4[2], G4[3]);
        f32x4 at, rt, bh4, kh4, bb4, kb4;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float Gt = G4[q];
            const float Gp = row16_prev(Gt, 1.f);
            const float GL = row16_last(Gt);
            const float inv = __builtin_amdgcn_rcpf(Gt);
            rt[q] = X[R_R][q] * Gt;
            kh4[q] = X[R_K][q] * inv;
            kb4[q] = kh4[q] * GL;
            if (kAB) {
                at[q] = X[R_A][q] * Gp;
                bh4[q] = X[R_B][q] * inv;
                bb4[q] = bh4[q] * GL;
            }
        }
        if (kAB) {
            *reinterpret_cast<bf16x4*>(&sm.At[l16][j0]) = cvt4(at);
            *reinterpret_cast<bf16x4*>(&sm.Bh[l16][j0]) = cvt4(bh4);
            *reinterpret_cast<bf16x4*>(&sm.Bb[l16][j0]) = cvt4(bb4);
        }
        *reinterpret_cast<bf16x4*>(&sm.Rt[l16][j0]) = cvt4(rt);
        *reinterpret_cast<bf16x4*>(&sm.Kh[l16][j0]) = cvt4(kh4);
        *reinterpret_cast<bf16x4*>(&sm.Kb[l16][j0]) = cvt4(kb4);
        if (l16 == kL - 1)
            *reinterpret_cast<float4*>(&sm.gL[64 * (cg >> 2) + 16 * g + 4 * (cg & 3)]) =
                make_float4(G4[0], G4[1], G4[2], G4[3]);
    };

    // ---- (C) a 16 x 16 product over the 128 keys: rows of X (A operand) and Y
    // (B operand), D[m][n] = X_m . Y_n in the accumulator layout.
    auto rows_product = [&](const bf16_t(*X)[kR128], const bf16_t(*Y)[kR128]) __attribute__((always_inline)) {
        bf16x8 xv[kK2], yv[kK2];
#pragma unroll
        for (int k2 = 0; k2 < kK2; ++k2) {
            xv[k2] = ld8(&X[l16][32 * k2 + 8 * g]);
            yv[k2] = ld8(&Y[l16][32 * k2 + 8 * g]);
        }
        f32x4 P = zero4();
#pragma unroll
        for (int k2 = 0; k2 < kK2; ++k2) P = mfma32(xv[k2], yv[k2], P);
        return P;
    };
    auto stage_products = [&]() __attribute__((always_inline)) {
        if (kAB && wave_s == 0) {
            f32x4 P = rows_product(sm.At, sm.Bh);   // [t][s] = Aab
#pragma unroll
            for (int q = 0; q < 4; ++q) P[q] = (l16 < 4 * g + q) ? P[q] : 0.f;
            const BlockInverse bi = unit_lower_inverse_begin<true>(P, g, l16);
            const Split4 tm = split4(unit_lower_inverse_rows_end(bi, g, l16));   // Tm's A image
            sm.tm_hi[lane] = __builtin_bit_cast(uint2, tm.hi);
            sm.tm_lo[lane] = __builtin_bit_cast(uint2, tm.lo);
        } else if (kAB && wave_s == 1) {
            f32x4 K = rows_product(sm.At, sm.Kh);   // [t][s] = Aak
#pragma unroll
            for (int q = 0; q < 4; ++q) K[q] = (l16 < 4 * g + q) ? K[q] : 0.f;
            sm.aak[lane] = K;
        } else if ((kAB && wave_s == 2) || wave_s == 3) {
            // [s][t] = Y_s . Rt_t, kept for s <= t: the accumulator registers
            // of Arb^T (Ark^T), i.e. the A-operand image of Arb (Ark)
            f32x4 PT = rows_product(wave_s == 2 ? sm.Bh : sm.Kh, sm.Rt);
#pragma unroll
            for (int q = 0; q < 4; ++q) PT[q] = (4 * g + q <= l16) ? PT[q] : 0.f;
            sm.tiles[wave_s == 2 ? T_RB : T_RK][lane] = __builtin_bit_cast(uint2, cvt4(PT));
        }
    };

    // ---- (D) At' = Tm At, key tile jt: At'^T tile = At^T[keys of jt] Tm^T,
    // whose accumulator registers hold At'[l16][16 jt + 4 g + q] (written over
    // the same columns of At, read first); Aak'^T = Aak^T Tm^T (wave 0).
    auto stage_apply = [&]() __attribute__((always_inline)) {
        Split4 tm;
        tm.hi = __builtin_bit_cast(bf16x4, sm.tm_hi[lane]);
        tm.lo = __builtin_bit_cast(bf16x4, sm.tm_lo[lane]);
#pragma unroll
        for (int e = 0; e < kJT / W; ++e) {
            const int jt = wave + W * e;
            const bf16x4 atT = ld4_tr(tr_addr(&sm.At[0][16 * jt], kR128, g, l16));
            const f32x4 d = mfma16(atT, tm.hi, mfma16(atT, tm.lo, zero4()));
            *reinterpret_cast<bf16x4*>(&sm.At[l16][16 * jt + 4 * g]) = cvt4(d);
        }
        if (wave_s == 0)
            sm.tiles[T_AK][lane] = __builtin_bit_cast(uint2, cvt4(mul3(split4(sm.aak[lane]), tm, zero4())));
    };

    // ---- (E) the state chain of value rows rb + 16 wave .. +15 ---------------
    auto stage_chain = [&](int c) __attribute__((always_inline)) {
        const bf16x4 V = ld4_tr(tr_addr(&sm.raw[R_V][0][rb + 16 * wave], kR128, g, l16));   // [t][i]
        const bf16x4 Ark = __builtin_bit_cast(bf16x4, sm.tiles[T_RK][lane]);
        bf16x4 Aak = {}, Arb = {};
        if (kAB) {
            Aak = __builtin_bit_cast(bf16x4, sm.tiles[T_AK][lane]);
            Arb = __builtin_bit_cast(bf16x4, sm.tiles[T_RB][lane]);
        }
        const float gl_lo = sm.gL[lane], gl_hi = sm.gL[64 + lane];
        bf16x4 Sb[kJT];
#pragma unroll
        for (int jt = 0; jt < kJT; ++jt) Sb[jt] = cvt4(S[jt]);
        if (kCk) {   // the entry state in fp32: row col, keys 16 jt + 4 g ..
            float* dst = ckpt + (((size_t)bh * nch + c) * kN128 + col) * kN128 + 4 * g;
#pragma unroll
            for (int jt = 0; jt < kJT; ++jt) store_stream(dst + 16 * jt, __builtin_bit_cast(uint4, S[jt]));
        }
        // Z = At' S0^T + Aak' V, Y = Rt S0^T + Arb Z + Ark V: the 32-deep
        // products over keys and the 16-deep ones over tokens accumulate
        // separately and meet on the vector ALU (add4).
        f32x4 Xs = zero4(), Ys = zero4();
#pragma unroll
        for (int k2 = 0; k2 < kK2; ++k2) {
            const bf16x8 bs = cat8(Sb[2 * k2], Sb[2 * k2 + 1]);
            if (kAB) Xs = mfma32(ld4x2(&sm.At[l16][32 * k2 + 4 * g]), bs, Xs);
            Ys = mfma32(ld4x2(&sm.Rt[l16][32 * k2 + 4 * g]), bs, Ys);
        }
        bf16x4 Zb = {};
        f32x4 Yt;
        if (kAB) {
            Zb = cvt4(add4(Xs, mfma16(Aak, V, zero4())));
            Yt = add4(Ys, mfma16(Ark, V, mfma16(Arb, Zb, zero4())));
        } else {
            Yt = add4(Ys, mfma16(Ark, V, zero4()));
        }
        // S_L^T = diag(G_L) S0^T + Kb^T V + Bb^T Z, key tile by key tile
        f32x4 dec[kJT];
        dec[0] = mul_row_lanes4<0>(gl_lo, S[0]);
        dec[1] = mul_row_lanes4<1>(gl_lo, S[1]);
        dec[2] = mul_row_lanes4<2>(gl_lo, S[2]);
        dec[3] = mul_row_lanes4<3>(gl_lo, S[3]);
        dec[4] = mul_row_lanes4<0>(gl_hi, S[4]);
        dec[5] = mul_row_lanes4<1>(gl_hi, S[5]);
        dec[6] = mul_row_lanes4<2>(gl_hi, S[6]);
        dec[7] = mul_row_lanes4<3>(gl_hi, S[7]);
#pragma unroll
        for (int jt = 0; jt < kJT; ++jt) {
            const bf16x4 kbt = ld4_tr(tr_addr(&sm.Kb[0][16 * jt], kR128, g, l16));   // Kb^T as an A operand
            const f32x4 acc = mfma16(kbt, V, dec[jt]);
            if (kAB) {
                const bf16x4 bbt = ld4_tr(tr_addr(&sm.Bb[0][16 * jt], kR128, g, l16));
                S[jt] = mfma16(bbt, Zb, acc);
            } else {
                S[jt] = acc;
            }
        }
        // read-outs in row layout (lane (g, l16): token l16, rows 4 g .. +3 of the wave's 16)
        *reinterpret_cast<bf16x4*>(&sm.Ys[l16][16 * wave + 4 * g]) = swap_layout(cvt4(Yt), ident);
    };

    // Staged read-outs of chunk c: 16 tokens x 16 W values, 2 W pieces of 16
    // bytes per token, from threads 0 .. 32 W - 1.
    auto store_y = [&](int c) __attribute__((always_inline)) {
        if (tid < 32 * W) {
            const int row = tid / (2 * W), piece = tid % (2 * W);
            const int tt = c * kL + row;
            if (tt < T)
                store_stream(y + tok_off<kN128>(bb, tt, hh, T, H) + rb + 8 * piece,
                             *reinterpret_cast<const uint4*>(&sm.Ys[row][8 * piece]));
        }
    };

    u32x4 ring[kPieces];
    load_raw(0, ring);
    for (int c = 0; c < nch; ++c) {
        stash_raw(c, ring);                        // (A)
        if (c > 0) store_y(c - 1);
        if (c + 1 < nch) load_raw(c + 1, ring);
        __syncthreads();
#pragma unroll
        for (int e = 0; e < kJT / W; ++e) stage_E(wave + W * e);   // (B)
        __syncthreads();
        stage_products();                          // (C)
        __syncthreads();
        if (kAB) {                                 // (D)
            stage_apply();
            __syncthreads();
        }
        stage_chain(c);                            // (E)
        __syncthreads();
    }
    if (nch > 0) store_y(nch - 1);
    if (sT) {
        float* dst = sT + (size_t)bh * NN + (size_t)col * kN128;
#pragma unroll
        for (int jt = 0; jt < kJT; ++jt)
            *reinterpret_cast<float4*>(dst + 16 * jt + 4 * g) = make_float4(S[jt][0], S[jt][1], S[jt][2], S[jt][3]);
    }
}

template <int W>
hipError_t launch_w(const FwdArgs& p, hipStream_t stream) {
    const int nbh = p.B * p.H;
    auto kern = p.a ? (p.ckpt ? chunk128_fwd_kernel<W, true, true> : chunk128_fwd_kernel<W, true, false>)
                    : (p.ckpt ? chunk128_fwd_kernel<W, false, true> : chunk128_fwd_kernel<W, false, false>);
    kern<<<dim3(nbh * (8 / W)), dim3(64 * W), 0, stream>>>(
        p.B, p.T, p.H, static_cast<const bf16_t*>(p.r), static_cast<const bf16_t*>(p.w),
        static_cast<const bf16_t*>(p.k), static_cast<const bf16_t*>(p.v),
        static_cast<const bf16_t*>(p.a), static_cast<const bf16_t*>(p.b), p.s0,
        static_cast<bf16_t*>(p.y), p.sT, p.ckpt);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_fwd128(const FwdArgs& p, int waves, hipStream_t stream) {
    if (!p.bf16 || p.N != kN128 || p.tape || p.T <= 0 || !p.y || (long long)p.B * p.H * 2 > INT32_MAX)
        return hipErrorInvalidValue;
    if ((p.a == nullptr) != (p.b == nullptr)) return hipErrorInvalidValue;
    if (p.B * p.H == 0) return hipSuccess;
    switch (waves) {
        case 4: return launch_w<4>(p, stream);
        case 8: return launch_w<8>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace wkv7
