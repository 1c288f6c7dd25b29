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
// 128 rows go to two workgroups of 64, and each workgroup forms the chunk's
// factors itself: no workspace, at the price of reading the head's token rows
// twice (the two workgroups of a head go to one XCD, whose L2 then serves the
// second read).  A workgroup has thirteen waves, split by role:
//   waves 0-3 (state chain): 16 value rows each, S^T in eight 16 x 16 fp32
//     accumulator tiles (key blocks); they apply Tm to At and Aak in
//     registers (At' = Tm At key tile by key tile: the accumulator registers
//     of At'^T = At^T Tm^T are the A operand of Z = At' S0^T, so At' never
//     passes through LDS), run the chain and store the read-outs;
//   waves 4-11 (producers): the raw token rows (loaded one chunk ahead into
//     registers, stashed in LDS), E -- decay products and scaled vectors of
//     one key group of 16 each -- and, on waves 9-11, one L x L product over
//     the 128 keys: Aak, Arb, Ark;
//   wave 12: Aab and the triangular inverse Tm = (I - Aab)^-1.
// Software pipeline, one barrier per interval: in interval i the producers
// stash chunk i+1, load chunk i+2 and run E(i) and the products of chunk i-1,
// the inverse wave chunk i-1's inverse, the state chain chunk i-2 and the
// stores of chunk i-3.  Each role runs a loop of its own over the same
// intervals, so the producers have only loads in flight and the state chain
// only stores: the compiler then waits for exactly the loads a stash needs
// instead of draining the memory counter (stores included) before it.  The
// roles share the SIMDs (two or three waves each), so one wave's latency
// hides behind the others' work (wave w runs on SIMD w mod 4: the products sit
// on the SIMDs that do not hold the inverse wave).  Chunk factors pass through three rotating
// LDS slots (Bh and Kh, read only in the interval after E, through two); the
// raw rows through two.  Lane layouts of the matrix-core operands:
// wkv7_mfma.h.  Chunks are padded past T (w = 1, everything else 0: the
// identity on the state), and the chunks before the first (-2, -1) are run as
// identities, so every loop body is the same in every interval.
//
// Each workgroup pair runs one item of the segment plan of the time split
// (work_of: a whole head, or one segment of it from its entry state, or one of
// a segment's two map runs, from the identity with v = 0 and from zero), as
// the N = 64 form's workgroups do; a map run's rows are the rows of the map.

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
constexpr int kSlots128 = 3;
// kParts workgroups per head (2, or 1 when two would not fit the device at
// once): 128 / kParts value rows each, 16 per state-chain wave; 8 producers of
// one key group each (two parts) or 4 of two (one part); either way 13 waves.
template <int kParts>
struct Shape128 {
    static_assert(kParts == 1 || kParts == 2, "one or two workgroups per head");
    static constexpr int kRows = kN128 / kParts;          // value rows per workgroup
    static constexpr int kCons = kRows / 16;              // state-chain waves
    static constexpr int kProd = kParts == 2 ? 8 : 4;     // producer waves
    static constexpr int kGroups = 8 / kProd;             // key groups of 16 per producer
    static constexpr int kPieces = 6 * kL * (kN128 / 8) / (64 * kProd);   // 16-byte raw pieces per producer thread
    // the producers that form Aak, Arb, Ark (the last three)
    static constexpr int P_AK = kProd - 3, P_RB = kProd - 2, P_RK = kProd - 1;
};
constexpr int kThreads128 = 64 * 13;
static_assert(64 * (Shape128<1>::kCons + Shape128<1>::kProd + 1) == kThreads128 &&
                  64 * (Shape128<2>::kCons + Shape128<2>::kProd + 1) == kThreads128,
              "thirteen waves either way");

enum { R_R = 0, R_W = 1, R_K = 2, R_A = 3, R_B = 4, R_V = 5 };
// (the products of a chunk in a slot: Aak, Arb, Ark; Aab stays in the inverse wave)

// What one chunk passes from E and the products to the state chain.
struct Slot128 {
    bf16_t At[kL][kR128], Rt[kL][kR128], Bb[kL][kR128], Kb[kL][kR128], V[kL][kR128];
    float gL[2 * 64];     // G_L of key 16 jt + 4 g + q at word 64 (jt / 4) + 16 g + 4 (jt % 4) + q
    uint2 tm_hi[64], tm_lo[64];   // hi and lo bf16 parts of Tm's A-operand image
    // The products in fp32, accumulator registers by lane: Aak as [t][s]
    // (strictly lower), Arb^T and Ark^T as [s][t] (s <= t), i.e. the A-operand
    // images of Arb and Ark.
    f32x4 prod[3][64];
};
struct BK128 {
    bf16_t Bh[kL][kR128], Kh[kL][kR128];
};
template <int kRows>
struct __align__(16) Smem128 {
    bf16_t raw[2][6][kL][kR128];    // r, w, k, a, b, v of two chunks (bf16 bits)
    Slot128 sl[kSlots128];
    BK128 bk[2];
    bf16_t Ys[2][kL][kRows + 8];    // read-outs of this workgroup's rows, [t][i]
};

__device__ __forceinline__ bf16x8 ld8(const bf16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ bf16x4 ld4(const bf16_t* p) {
    return __builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2*>(p));
}
__device__ __forceinline__ bf16x8 ld4x2(const bf16_t* p) { return cat8(ld4(p), ld4(p + 16)); }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// kAB = false: a = b = 0 (no removal terms: Y = Rt S0^T + Ark V, S_L^T =
// diag(G_L) S0^T + Kb^T V; the inverse wave idles); kCk: also the fp32 state
// entering every chunk, [B][H][ceil(T/16)][N][N] (row = value channel).
// nitems: the launch's items of the segment plan (two workgroups each).
template <int kParts, bool kAB, bool kCk>
__global__ __launch_bounds__(kThreads128, 1) void chunk128_fwd_kernel(
    int B, int T, int H, const bf16_t* __restrict__ r, const bf16_t* __restrict__ w,
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, const bf16_t* __restrict__ a,
    const bf16_t* __restrict__ b, const float* __restrict__ s0, bf16_t* __restrict__ y_all,
    float* __restrict__ sT, float* __restrict__ ckpt_all, int nitems, int pass, int split_from,
    int nseg, int seg_len, float* __restrict__ states) {
    using Sh = Shape128<kParts>;
    constexpr int kRows = Sh::kRows, kCons = Sh::kCons, kProd = Sh::kProd, kPieces = Sh::kPieces;
    constexpr int P_AK = Sh::P_AK, P_RB = Sh::P_RB, P_RK = Sh::P_RK;
    constexpr size_t NN = (size_t)kN128 * kN128;
    __shared__ Smem128<kRows> sm;

    // Workgroups go to the eight XCDs in turn (u to XCD u mod 8).  Groups of 8
    // items take 8 kParts consecutive workgroups, part-major, so that the parts
    // of an item share an XCD and run at about the same time.
    const int u = blockIdx.x;
    const int grp = u / (8 * kParts), within = u % (8 * kParts);
    const int m = min(8, nitems - 8 * grp);
    const int part = within / m;
    const Work wk = work_of<kN128>(8 * grp + within % m, pass, T, s0, sT, split_from, nseg, seg_len, states);
    const int bh = wk.bh;
    const int bb = bh / H, hh = bh % H;
    const int rb = part * kRows;                // first value row of this workgroup
    // Chunks c_begin .. c_begin + nch - 1 of the sequence; tokens from t_end on
    // are padding (t_begin is a multiple of 32).
    const int t_end = wk.t_end, c_begin = wk.t_begin / kL;
    const int nch = (t_end + kL - 1) / kL - c_begin;
    const int nch_all = (T + kL - 1) / kL;      // chunks of the checkpoints' layout
    bf16_t* const y = wk.outs ? y_all : nullptr;
    float* const ckpt = (kCk && wk.outs) ? ckpt_all : nullptr;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // A scalar copy of the wave index: the role branches are scalar (no
    // matrix-core product runs with part of EXEC off).
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const int l16 = lane & 15, g = lane >> 4;
    const int col = rb + 16 * (wave & (kCons - 1)) + l16;   // value row of this lane (state chain)
    const bf16x4 ident = identity_b(g, l16);

    // ---- raw rows (producers): 6 vectors x 16 tokens x 16 pieces of 16 bytes
    // per chunk; producer thread p takes pieces p + 64 kProd e: with 8
    // producers (e = 0 .. 2) vector 2 e + p / 256, with 4 (e = 0 .. 5) vector
    // e; token (p / 16) % 16, columns 8 (p % 16) .. +7 (a token row of a vector
    // is 16 consecutive threads).
    const int ptid = tid - 64 * kCons;
    const int ld_t = (ptid >> 4) & 15, ld_c8 = ptid & 15;
    const int vhi = kProd == 8 ? __builtin_amdgcn_readfirstlane(ptid >> 8) : 0;   // 0 or 1 for producers
    auto vec_of = [&](int e) __attribute__((always_inline)) { return kProd == 8 ? 2 * e + vhi : e; };
    auto src_of = [&](int e) __attribute__((always_inline)) -> const bf16_t* {
        const bf16_t* const src6[6] = {r, w, k, a, b, v};
        if constexpr (kProd == 8) return vhi ? src6[2 * e + 1] : src6[2 * e];
        else return src6[e];
    };
    auto load_raw = [&](int c, u32x4 (&o)[kPieces]) __attribute__((always_inline)) {
        const int t = min((c_begin + c) * kL + ld_t, t_end - 1);
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
        const bool ok = (c_begin + c) * kL + ld_t < t_end;
#pragma unroll
        for (int e = 0; e < kPieces; ++e) {
            const int vi = vec_of(e);
            const unsigned pad = vi == R_W ? 0x3F803F80u : 0u;   // padding: w = 1, the rest 0
            const u32x4 padv = {pad, pad, pad, pad};
            *reinterpret_cast<u32x4*>(&sm.raw[c & 1][vi][ld_t][8 * ld_c8]) = ok ? o[e] : padv;
        }
    };

    // ---- E(c) (producers): key group cg (16 keys); lane (g, l16) = token l16,
    // keys j0 .. j0+3
    auto stage_E = [&](int c, int cg) __attribute__((always_inline)) {
        const bf16_t(*Rr)[kL][kR128] = sm.raw[c & 1];
        Slot128& s = sm.sl[(c + 6) % kSlots128];
        BK128& bk = sm.bk[c & 1];
        const int j0 = 16 * cg + 4 * g;
        uint2 q6[6];
#pragma unroll
        for (int vi = 0; vi < 6; ++vi) {
            if (!kAB && (vi == R_A || vi == R_B)) continue;
            q6[vi] = *reinterpret_cast<const uint2*>(&Rr[vi][l16][j0]);
        }
        float X[5][4];
#pragma unroll
        for (int vi = 0; vi < 5; ++vi) {
            if (!kAB && (vi == R_A || vi == R_B)) continue;
            X[vi][0] = bf16_lo(q6[vi].x); X[vi][1] = bf16_hi(q6[vi].x);
            X[vi][2] = bf16_lo(q6[vi].y); X[vi][3] = bf16_hi(q6[vi].y);
        }
        float G4[4] = {X[R_W][0], X[R_W][1], X[R_W][2], X[R_W][3]};
        row16_cumprod4(G4[0], G4[1], G4[2], G4[3]);
        f32x4 at, rt, bh4, kh4, bb4, kb4, gl4;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float Gt = G4[q];
            const float Gp = row16_prev(Gt, 1.f);
            const float GL = row16_last(Gt);
            const float inv = __builtin_amdgcn_rcpf(Gt);
            gl4[q] = GL;
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
            *reinterpret_cast<bf16x4*>(&s.At[l16][j0]) = cvt4(at);
            *reinterpret_cast<bf16x4*>(&bk.Bh[l16][j0]) = cvt4(bh4);
            *reinterpret_cast<bf16x4*>(&s.Bb[l16][j0]) = cvt4(bb4);
        }
        *reinterpret_cast<bf16x4*>(&s.Rt[l16][j0]) = cvt4(rt);
        *reinterpret_cast<bf16x4*>(&bk.Kh[l16][j0]) = cvt4(kh4);
        *reinterpret_cast<bf16x4*>(&s.Kb[l16][j0]) = cvt4(kb4);
        *reinterpret_cast<uint2*>(&s.V[l16][j0]) = wk.vzero ? make_uint2(0u, 0u) : q6[R_V];
        // every lane of the row holds G_L of keys j0 .. j0+3 and writes it (the
        // same 16 bytes to the same place: no branch)
        *reinterpret_cast<f32x4*>(&s.gL[64 * (cg >> 2) + 16 * g + 4 * (cg & 3)]) = gl4;
    };


    // ---- L x L products over the 128 keys: rows of X (A operand) and Y (B
    // operand), D[m][n] = X_m . Y_n in the accumulator layout.
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
    // Producer pw = 5, 6, 7 forms Aak = At Kh^T ([t][s], strictly lower),
    // Arb^T = Bh Rt^T or Ark^T = Kh Rt^T ([s][t], s <= t); with a = b = 0 only Ark.
    auto stage_products = [&](int c, int pw) __attribute__((always_inline)) {
        Slot128& s = sm.sl[(c + 6) % kSlots128];
        const BK128& bk = sm.bk[c & 1];
        const bool strict = pw == P_AK;
        f32x4 P = pw == P_AK ? rows_product(s.At, bk.Kh)
                             : rows_product(pw == P_RB ? bk.Bh : bk.Kh, s.Rt);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const bool keep = strict ? (l16 < 4 * g + q) : (4 * g + q <= l16);
            P[q] = keep ? P[q] : 0.f;
        }
        s.prod[pw - P_AK][lane] = P;
    };
    // ---- the inverse wave: Aab = At Bh^T ([t][s], strictly lower), Tm = (I - Aab)^-1
    auto stage_inverse = [&](int c) __attribute__((always_inline)) {
        Slot128& s = sm.sl[(c + 6) % kSlots128];
        f32x4 P = rows_product(s.At, sm.bk[c & 1].Bh);
#pragma unroll
        for (int q = 0; q < 4; ++q) P[q] = (l16 < 4 * g + q) ? P[q] : 0.f;
        const BlockInverse bi = unit_lower_inverse_begin<true>(P, g, l16);
        const Split4 tm = split4(unit_lower_inverse_rows_end(bi, g, l16));   // Tm's A image
        s.tm_hi[lane] = __builtin_bit_cast(uint2, tm.hi);
        s.tm_lo[lane] = __builtin_bit_cast(uint2, tm.lo);
    };

    // ---- state chain (waves 0-3): value rows rb + 16 wave .. +15 --------------
    f32x4 S[kJT];
#pragma unroll
    for (int jt = 0; jt < kJT; ++jt) S[jt] = zero4();
    auto stage_chain = [&](int c) __attribute__((always_inline)) {
        const Slot128& s = sm.sl[(c + 6) % kSlots128];
        const bf16x4 V = ld4_tr(tr_addr(&s.V[0][rb + 16 * wave], kR128, g, l16));   // [t][i]
        const bf16x4 Ark = cvt4(s.prod[P_RK - P_AK][lane]);
        const float gl_lo = s.gL[lane], gl_hi = s.gL[64 + lane];
        // At' = Tm At: key tile jt of At'^T = At^T[keys of jt] Tm^T, whose
        // accumulator registers hold At'[l16][16 jt + 4 g + q]; two of them side
        // by side are the A operand of the 32-deep product over keys 32 k2 ..
        // (the same bijection of the contraction index as cat8(Sb[2 k2], Sb[2 k2 + 1])).
        bf16x4 Atp[kJT];
        bf16x4 Aak = {}, Arb = {};
        if (kAB) {
            Split4 tm;
            tm.hi = __builtin_bit_cast(bf16x4, s.tm_hi[lane]);
            tm.lo = __builtin_bit_cast(bf16x4, s.tm_lo[lane]);
#pragma unroll
            for (int jt = 0; jt < kJT; ++jt) {
                const bf16x4 atT = ld4_tr(tr_addr(&s.At[0][16 * jt], kR128, g, l16));
                Atp[jt] = cvt4(mfma16(atT, tm.hi, mfma16(atT, tm.lo, zero4())));
            }
            // Aak'^T = Aak^T Tm^T from Aak's accumulator layout: its registers are
            // the A-operand image of Aak' = Tm Aak
            Aak = cvt4(mul3(split4(s.prod[0][lane]), tm, zero4()));
            Arb = cvt4(s.prod[P_RB - P_AK][lane]);
        }
        bf16x4 Sb[kJT];
#pragma unroll
        for (int jt = 0; jt < kJT; ++jt) Sb[jt] = cvt4(S[jt]);
        if (kCk && ckpt && c >= 0) {   // the entry state in fp32: row col, keys 16 jt + 4 g ..
            float* dst = ckpt + (((size_t)bh * nch_all + c_begin + c) * kN128 + col) * kN128 + 4 * g;
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
            if (kAB) Xs = mfma32(cat8(Atp[2 * k2], Atp[2 * k2 + 1]), bs, Xs);
            Ys = mfma32(ld4x2(&s.Rt[l16][32 * k2 + 4 * g]), bs, Ys);
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
            const bf16x4 kbt = ld4_tr(tr_addr(&s.Kb[0][16 * jt], kR128, g, l16));   // Kb^T as an A operand
            const f32x4 acc = mfma16(kbt, V, dec[jt]);
            if (kAB) {
                const bf16x4 bbt = ld4_tr(tr_addr(&s.Bb[0][16 * jt], kR128, g, l16));
                S[jt] = mfma16(bbt, Zb, acc);
            } else {
                S[jt] = acc;
            }
        }
        // read-outs in row layout (lane (g, l16): token l16, rows 4 g .. +3 of the wave's 16)
        *reinterpret_cast<bf16x4*>(&sm.Ys[c & 1][l16][16 * wave + 4 * g]) = swap_layout(cvt4(Yt), ident);
    };


    // Staged read-outs of chunk c: 16 tokens x kRows values, kRows / 8 pieces
    // of 16 bytes per token, from the first 2 kRows threads of the state chain.
    auto store_y = [&](int c) __attribute__((always_inline)) {
        if (y && tid < 2 * kRows) {
            const int row = tid / (kRows / 8), piece = tid % (kRows / 8);
            const int tt = (c_begin + c) * kL + row;
            if (c >= 0 && tt < t_end)
                store_stream(y + tok_off<kN128>(bb, tt, hh, T, H) + rb + 8 * piece,
                             *reinterpret_cast<const uint4*>(&sm.Ys[c & 1][row][8 * piece]));
        }
    };

    // The slots of chunks -2 and -1 (slots 1 and 2) hold identity factors:
    // At = Rt = Bb = Kb = V = 0 and the products 0 (chunk -1's Bh and Kh too,
    // which its products read), G_L = 1; the chain of such a chunk leaves the
    // state as it is and stores nothing.
    {
        uint32_t* const z1 = reinterpret_cast<uint32_t*>(&sm.sl[1]);
        uint32_t* const z2 = reinterpret_cast<uint32_t*>(&sm.sl[2]);
        constexpr int nw = sizeof(Slot128) / 4;
        for (int x = tid; x < nw; x += kThreads128) {
            z1[x] = 0u;
            z2[x] = 0u;
        }
        uint32_t* const zb = reinterpret_cast<uint32_t*>(&sm.bk[1]);
        for (int x = tid; x < (int)(sizeof(BK128) / 4); x += kThreads128) zb[x] = 0u;
        __syncthreads();
        for (int x = tid; x < 2 * 64; x += kThreads128) {
            sm.sl[1].gL[x] = 1.f;
            sm.sl[2].gL[x] = 1.f;
        }
    }

    if (wave_s < kCons) {
        // ---- the state chain: chain(i-2) and the stores of chunk i-3 in interval i
        if (wk.init) {
            const float* base = wk.init + (size_t)col * kN128;
#pragma unroll
            for (int jt = 0; jt < kJT; ++jt) {
                const float4 x = *reinterpret_cast<const float4*>(base + 16 * jt + 4 * g);
                S[jt][0] = x.x; S[jt][1] = x.y; S[jt][2] = x.z; S[jt][3] = x.w;
            }
            // settled here: left pending, every later use of S would wait on
            // the whole memory counter (and so on the chunks' stores)
            __builtin_amdgcn_s_waitcnt(0);
        } else if (wk.ident) {
#pragma unroll
            for (int jt = 0; jt < kJT; ++jt)
#pragma unroll
                for (int q = 0; q < 4; ++q) S[jt][q] = col == 16 * jt + 4 * g + q ? 1.f : 0.f;
        }
        // the state chain and the inverse wave issue before the producers
        // when several waves of a SIMD are ready
        __builtin_amdgcn_s_setprio(3);
        __syncthreads();
        for (int i = 0; i < nch + 2; ++i) {
            store_y(i - 3);
            stage_chain(i - 2);
            __syncthreads();
        }
        store_y(nch - 1);
        if (wk.fin) {
            float* dst = wk.fin + (size_t)col * kN128;
#pragma unroll
            for (int jt = 0; jt < kJT; ++jt)
                *reinterpret_cast<float4*>(dst + 16 * jt + 4 * g) =
                    make_float4(S[jt][0], S[jt][1], S[jt][2], S[jt][3]);
        }
    } else if (wave_s < kCons + kProd) {
        // ---- producers: stash chunk i+1, load chunk i+2, E(i), products(i-1)
        const int pw = wave_s - kCons;
        u32x4 ring[kPieces];
        load_raw(0, ring);
        stash_raw(0, ring);
        load_raw(1, ring);
        __syncthreads();
        for (int i = 0; i < nch + 2; ++i) {
            stash_raw(i + 1, ring);
            load_raw(i + 2, ring);
#pragma unroll
            for (int e = 0; e < Sh::kGroups; ++e) stage_E(i, pw + kProd * e);
            if (kAB ? pw >= P_AK : pw == P_RK) stage_products(i - 1, pw);
            __syncthreads();
        }
    } else {
        // ---- the inverse wave: chunk i-1's inverse in interval i
        __builtin_amdgcn_s_setprio(3);
        __syncthreads();
        for (int i = 0; i < nch + 2; ++i) {
            if (kAB) stage_inverse(i - 1);
            __syncthreads();
        }
    }
}

template <int kParts, bool kAB, bool kCk>
hipError_t launch_k(const FwdArgs& p, int nitems, int pass, const FwdSplit& sp, hipStream_t stream) {
    if (nitems == 0) return hipSuccess;
    chunk128_fwd_kernel<kParts, kAB, kCk><<<dim3(kParts * nitems), dim3(kThreads128), 0, stream>>>(
        p.B, p.T, p.H, static_cast<const bf16_t*>(p.r), static_cast<const bf16_t*>(p.w),
        static_cast<const bf16_t*>(p.k), static_cast<const bf16_t*>(p.v),
        static_cast<const bf16_t*>(p.a), static_cast<const bf16_t*>(p.b), p.s0,
        static_cast<bf16_t*>(p.y), p.sT, p.ckpt, nitems, pass, sp.split_from, sp.nseg, sp.seg_len,
        sp.states);
    return hipGetLastError();
}

template <int kParts>
hipError_t launch_pass_p(const FwdArgs& p, int nitems, int pass, const FwdSplit& sp, hipStream_t stream) {
    if (p.a) return p.ckpt ? launch_k<kParts, true, true>(p, nitems, pass, sp, stream)
                           : launch_k<kParts, true, false>(p, nitems, pass, sp, stream);
    return p.ckpt ? launch_k<kParts, false, true>(p, nitems, pass, sp, stream)
                  : launch_k<kParts, false, false>(p, nitems, pass, sp, stream);
}
// Two workgroups per item while they fit the device in one round, else one.
hipError_t launch_pass(const FwdArgs& p, int nitems, int pass, const FwdSplit& sp, int ncu,
                       hipStream_t stream) {
    if (ncu > 0 && 2LL * nitems > ncu) return launch_pass_p<1>(p, nitems, pass, sp, stream);
    return launch_pass_p<2>(p, nitems, pass, sp, stream);
}

}  // namespace

hipError_t launch_chunk_fwd128(const FwdArgs& p, int ncu, hipStream_t stream) {
    return launch_chunk_fwd128_split(p, FwdSplit{p.B * p.H, 1, p.T, nullptr}, ncu, stream);
}

hipError_t launch_chunk_fwd128_split(const FwdArgs& p, const FwdSplit& sp, int ncu, hipStream_t stream) {
    if (!p.bf16 || p.N != kN128 || p.tape || p.T <= 0 || !p.y || (long long)p.B * p.H * 2 > INT32_MAX)
        return hipErrorInvalidValue;
    if ((p.a == nullptr) != (p.b == nullptr)) return hipErrorInvalidValue;
    const int nbh = p.B * p.H;
    const int nsplit = nbh - sp.split_from;
    if (nsplit < 0 || (nsplit > 0 && (sp.nseg < 2 || sp.seg_len % WKV7_TAPE_BLOCK != 0 || sp.seg_len <= 0 ||
                                       (long long)(sp.nseg - 1) * sp.seg_len >= p.T || !sp.states)))
        return hipErrorInvalidValue;
    if ((long long)2 * (sp.split_from + (long long)nsplit * (2 * sp.nseg - 3 > 0 ? 2 * sp.nseg - 3 : 0)) > INT32_MAX)
        return hipErrorInvalidValue;
    if (nbh == 0) return hipSuccess;
    // Pass 0: whole heads, each split head's segment 0 and its map runs; then
    // the entry states composed in fp32; pass 1: the segments from them.
    hipError_t e = launch_pass(p, sp.split_from + (nsplit > 0 ? nsplit * (2 * sp.nseg - 3) : 0), 0, sp, ncu, stream);
    if (e != hipSuccess || nsplit == 0) return e;
    if (sp.nseg > 2) {
        e = launch_seg_combine_n(kN128, nsplit, sp.nseg, sp.states, stream);
        if (e != hipSuccess) return e;
    }
    return launch_pass(p, nsplit * (sp.nseg - 1), 1, sp, ncu, stream);
}

}  // namespace wkv7
