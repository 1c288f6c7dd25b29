// wkv7_chunk_fwd.hip -- chunked (parallel-in-time) WKV7 forward on bf16 MFMA.
//
// The pages state that RWKV-7 keeps training parallelisable (Abstract; Elamur
// summary, Summary) without printing the parallel form.  The form used here
// is an exact rearrangement of the recurrence over a chunk of L = 16 tokens
// with entry state S0, pinned in fp64 against the sequential definition:
//
//   G_t[j] = prod_{u<=t} w_u[j]                        (running decay, fp32)
//   At = a G_{t-1},  Rt = r G_t,  Bh = b / G_t,  Kh = k / G_t,
//   Bb = b G_L / G_t,  Kb = k G_L / G_t
//   Aab = tril_-1(At Bh^T), Aak = tril_-1(At Kh^T),
//   Arb = tril_0(Rt Bh^T),  Ark = tril_0(Rt Kh^T)        (L x L)
//   Tm  = (I - Aab)^-1                                   (unit lower triangular)
//   W   = Tm At,   Q = Rt + Arb W                        (depend on r,w,k,a,b only)
//   U   = Tm Aak V,  Y0 = Arb U + Ark V,  H = Kb^T V     (add v, not the state)
//   Z   = W S0^T + U                 (row t of Z is z_t = S_{t-1} a_t)
//   Y   = Q S0^T + Y0                (row t of Y is y_t)
//   S_L^T = diag(G_L) S0^T + H + Bb^T Z
//
// Mapping to gfx950: one workgroup of 4 waves per (b, h).  Wave w owns value
// rows 16w..16w+15 of the state, held as S^T in four 16x16 fp32 accumulator
// tiles (key blocks); because an accumulator tile feeds the next product
// directly as its B operand (wkv7_mfma.h), every state-dependent product is a
// left multiplication that reads the state straight from registers.
//
// The per-chunk work is software-pipelined with ONE barrier per chunk.  In
// the barrier interval of iteration `it` every wave does, independently:
//   E(it)    decay products and scaled vectors of chunk it for its 16 key
//            columns (the running product over tokens is a prefix across
//            the wave's four lane groups, exchanged through wave-private LDS);
//   MW(it-1) the 16x16 products of chunk it-1, the triangular inverse, its
//            key block of W and Q, and U, Y0, H for its value rows -- each
//            wave recomputes the small L x L tiles itself instead of
//            exchanging them;
//   ST(it-2) the state chain of chunk it-2;
//   the coalesced y store of chunk it-3, the LDS stash of chunk it+1 and
//   the global loads of chunk it+4 (a three-deep register ring, so no load's
//   latency is ever waited on within the interval that issued it).
// Within the interval every LDS operand read is issued before any LDS write,
// since the compiler cannot prove the rotating slots disjoint.
// The four streams are independent within the interval, so their latencies
// overlap instead of adding up.  Chunks beyond T are all-padding (w = 1,
// everything else 0), for which every stage is the identity on the state.

#include "wkv7_device.h"
#include "wkv7_internal.h"
#include "wkv7_mfma.h"

namespace wkv7 {

namespace {

constexpr int kL = 16;
constexpr int kThreads = 256;
// LDS row strides (bf16 elements).  A 64-wide row would be exactly one sweep
// of the 32 four-byte banks, so the operand reads below (16 lanes on 16
// different rows, same columns) would all hit the same banks; 144-byte and
// 40-byte rows spread them.
constexpr int kRow = kN + 8;    // rows of 64 elements
constexpr int kRowT = kL + 4;   // rows of 16 elements

enum { RAW_R = 0, RAW_W = 1, RAW_K = 2, RAW_A = 3, RAW_B = 4, RAW_V = 5 };

// State-independent factors of one chunk, shared by the four waves.
struct Slot {
    bf16_t At[kL][kRow], Rt[kL][kRow], Bh[kL][kRow], Kh[kL][kRow];  // row-major [t][j]
    bf16_t BbT[kN][kRowT], KbT[kN][kRowT];                          // [j][t]
    float gL[kN];
};

struct __align__(16) FwdSmem {
    bf16_t raw[2][6][kL][kRow];   // r, w, k, a, b, v of two chunks (bf16 bits)
    Slot sl[3];
    bf16_t Wm[2][kL][kRow], Qm[2][kL][kRow];
    bf16_t Ys[2][kL][kRow];
    float red[4][4][16];          // wave-private prefix scratch
};

__device__ __forceinline__ float bf2f(bf16_t x) { return __uint_as_float((uint32_t)x << 16); }
__device__ __forceinline__ bf16x4 ld4(const bf16_t* p) {
    return __builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2*>(p));
}
__device__ __forceinline__ bf16x8 ld8(const bf16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ bf16x8 ld4x2(const bf16_t* p) { return cat8(ld4(p), ld4(p + 16)); }
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Outputs of E kept in registers for the same wave's MW one interval later.
struct ERegs {
    bf16x4 At;   // At[4g+q][16w+l16]: B operand of W = Tm At
    f32x4 Rt;    // Rt[4g+q][16w+l16]: accumulator init of Q
    bf16x4 V;    // v[4g+q][16w+l16]: B operand of the V products
};
// Outputs of MW kept for the same wave's ST one interval later.
struct MWRegs {
    f32x4 U, Y0;
    bf16x4 V;    // v of the chunk again, for H = Kb^T V inside ST
};

__global__ __launch_bounds__(kThreads, 2) void chunk_fwd_kernel(
    int T, int H, const bf16_t* __restrict__ r, const bf16_t* __restrict__ w,
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, const bf16_t* __restrict__ a,
    const bf16_t* __restrict__ b, const float* __restrict__ s0, bf16_t* __restrict__ y,
    float* __restrict__ sT, float* __restrict__ ckpt) {
    __shared__ FwdSmem sm;
    const int bh = blockIdx.x;
    const int bb = bh / H, hh = bh % H;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    const int col = 16 * wv + l16;            // key column (E) / value row (MW, ST) of this lane
    const int nck = (T + kCkptInterval - 1) / kCkptInterval;
    const int nch = (T + kL - 1) / kL;

    // ---- state: S^T tiles, lane holds S[col][16 jt + 4 g + q] ------------------
    f32x4 S[4];
    {
        const float* base = s0 ? s0 + ((size_t)bh * kN + col) * kN : nullptr;
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            if (base) {
                const float4 x = *reinterpret_cast<const float4*>(base + 16 * jt + 4 * g);
                S[jt][0] = x.x; S[jt][1] = x.y; S[jt][2] = x.z; S[jt][3] = x.w;
            } else {
                S[jt] = zero4();
            }
        }
        if (ckpt && T > 0) {
            float* dst = ckpt + ((size_t)bh * nck * kN + col) * kN;
#pragma unroll
            for (int jt = 0; jt < 4; ++jt)
                *reinterpret_cast<float4*>(dst + 16 * jt + 4 * g) =
                    make_float4(S[jt][0], S[jt][1], S[jt][2], S[jt][3]);
        }
    }

    // ---- raw token loads: 6 vectors x 16 tokens x 64 = 768 x 16 bytes.  Thread
    // tid loads vector 2p + (tid >= 128), token (tid >> 3) & 15, columns
    // 8 (tid & 7) .. +7, for p = 0, 1, 2.  Loads are branch-free (tokens past
    // T re-read token T-1; E replaces them by padding) and are issued three
    // intervals before E uses them, into a three-deep register ring; the
    // stash into LDS happens one interval before use, so it waits only on
    // loads that were issued two intervals earlier.
    const bool hi = tid >= 128;
    const bf16_t* const sp_p[3] = {hi ? w : r, hi ? a : k, hi ? v : b};
    const int ld_t = (tid >> 3) & 15, ld_c8 = tid & 7;
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));   // plain SSA vector
    struct Raw {
        u32x4 x[3];
    };
    auto load_raw = [&](int c, Raw& o) __attribute__((always_inline)) {
        const int t = min(c * kL + ld_t, T - 1);
        const size_t off = tok_off(bb, t, hh, T, H) + ld_c8 * 8;
#pragma unroll
        for (int p = 0; p < 3; ++p) o.x[p] = *reinterpret_cast<const u32x4*>(sp_p[p] + off);
    };
    // Padding tokens (past T) become w = 1 and zeros here, once, so that E's
    // reads need no conditions.
    auto stash_raw = [&](int c, const Raw& o) __attribute__((always_inline)) {
        const bool ok = c * kL + ld_t < T;
#pragma unroll
        for (int p = 0; p < 3; ++p) {
            const unsigned pad = (p == 0 && hi) ? 0x3F803F80u : 0u;
            const u32x4 padv = {pad, pad, pad, pad};
            *reinterpret_cast<u32x4*>(&sm.raw[c & 1][2 * p + (hi ? 1 : 0)][ld_t][ld_c8 * 8]) =
                ok ? o.x[p] : padv;
        }
    };

    // ---- E: decay products and scaled vectors of chunk c, key columns `col` ----
    auto stage_E = [&](int c) __attribute__((always_inline)) -> ERegs {
        Slot& s = sm.sl[c % 3];
        const bf16_t(*Rr)[kL][kRow] = sm.raw[c & 1];
        float R[6][4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int vi = 0; vi < 6; ++vi) R[vi][q] = bf2f(Rr[vi][4 * g + q][col]);
        float gp[4];
        float run = 1.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            run *= R[RAW_W][q];
            gp[q] = run;
        }
        sm.red[wv][g][l16] = run;
        wave_sync();
        const float g0 = sm.red[wv][0][l16], g1 = sm.red[wv][1][l16];
        const float g2 = sm.red[wv][2][l16], g3 = sm.red[wv][3][l16];
        const float before = g == 0 ? 1.f : g == 1 ? g0 : g == 2 ? g0 * g1 : (g0 * g1) * g2;
        const float GL = ((g0 * g1) * g2) * g3;
        ERegs e;
        float at[4], bb4[4], kb4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int t = 4 * g + q;
            const float Gt = before * gp[q];
            const float Gp = q == 0 ? before : before * gp[q - 1];
            const float inv = __builtin_amdgcn_rcpf(Gt);
            at[q] = R[RAW_A][q] * Gp;
            const float rt = R[RAW_R][q] * Gt;
            const float bh_ = R[RAW_B][q] * inv;
            const float kh_ = R[RAW_K][q] * inv;
            bb4[q] = bh_ * GL;
            kb4[q] = kh_ * GL;
            e.Rt[q] = rt;
            s.At[t][col] = f2bf(at[q]);
            s.Rt[t][col] = f2bf(rt);
            s.Bh[t][col] = f2bf(bh_);
            s.Kh[t][col] = f2bf(kh_);
        }
        *reinterpret_cast<bf16x4*>(&s.BbT[col][4 * g]) = cvt4(bb4[0], bb4[1], bb4[2], bb4[3]);
        *reinterpret_cast<bf16x4*>(&s.KbT[col][4 * g]) = cvt4(kb4[0], kb4[1], kb4[2], kb4[3]);
        if (g == 0) s.gL[col] = GL;
        e.At = cvt4(at[0], at[1], at[2], at[3]);
        e.V = cvt4(R[RAW_V][0], R[RAW_V][1], R[RAW_V][2], R[RAW_V][3]);
        return e;
    };

    // ---- MW: L x L tiles, inverse, W / Q key block, U / Y0 / H value block -----
    struct MWIn {
        bf16x8 av[2], rv[2], bv[2], kv[2];
    };
    auto read_MW = [&](int c) __attribute__((always_inline)) -> MWIn {
        const Slot& s = sm.sl[c % 3];
        MWIn in;
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            in.av[k2] = ld8(&s.At[l16][32 * k2 + 8 * g]);
            in.rv[k2] = ld8(&s.Rt[l16][32 * k2 + 8 * g]);
            in.bv[k2] = ld8(&s.Bh[l16][32 * k2 + 8 * g]);
            in.kv[k2] = ld8(&s.Kh[l16][32 * k2 + 8 * g]);
        }
        return in;
    };
    auto stage_MW = [&](int c, const MWIn& in, const ERegs& e) __attribute__((always_inline)) -> MWRegs {
        f32x4 ab = zero4(), abT = zero4(), akT = zero4(), rbT = zero4(), rkT = zero4();
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            ab = mfma32(in.av[k2], in.bv[k2], ab);     // [t][s] = At_t . Bh_s
            abT = mfma32(in.bv[k2], in.av[k2], abT);   // [s][t]
            akT = mfma32(in.kv[k2], in.av[k2], akT);   // [s][t] = At_t . Kh_s
            rbT = mfma32(in.bv[k2], in.rv[k2], rbT);   // [s][t] = Rt_t . Bh_s
            rkT = mfma32(in.kv[k2], in.rv[k2], rkT);   // [s][t] = Rt_t . Kh_s
        }
        // Masks in accumulator coordinates (row m = 4g+q, column n = l16).
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int m = 4 * g + q, n = l16;
            ab[q] = (n < m) ? ab[q] : 0.f;
            abT[q] = (m < n) ? abT[q] : 0.f;
            akT[q] = (m < n) ? akT[q] : 0.f;
            rbT[q] = (m <= n) ? rbT[q] : 0.f;
            rkT[q] = (m <= n) ? rkT[q] : 0.f;
        }
        // Tile registers of X^T fed as an A operand stand for X: Tm, Aak, Arb, Ark.
        const bf16x4 Tm = cvt4(unit_lower_inverse_T(ab, abT, g, l16));
        const bf16x4 Aak = cvt4(akT), Arb = cvt4(rbT), Ark = cvt4(rkT);
        const f32x4 Wt = mfma16(Tm, e.At, zero4());              // W[t][col]
        const f32x4 Qt = mfma16(Arb, cvt4(Wt), e.Rt);             // Q[t][col]
        bf16_t* Wd = &sm.Wm[c & 1][0][0];
        bf16_t* Qd = &sm.Qm[c & 1][0][0];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            Wd[(4 * g + q) * kRow + col] = f2bf(Wt[q]);
            Qd[(4 * g + q) * kRow + col] = f2bf(Qt[q]);
        }
        MWRegs m;
        const f32x4 AkV = mfma16(Aak, e.V, zero4());
        m.U = mfma16(Tm, cvt4(AkV), zero4());
        m.Y0 = mfma16(Ark, e.V, mfma16(Arb, cvt4(m.U), zero4()));
        m.V = e.V;
        return m;
    };

    // ---- ST: the state chain of chunk c -----------------------------------------
    struct STIn {
        bf16x8 wa[2], qa[2];
        bf16x4 bbt[4], kbt[4];
        float4 gl[4];
    };
    auto read_ST = [&](int c) __attribute__((always_inline)) -> STIn {
        const Slot& s = sm.sl[c % 3];
        const bf16_t* Wm = &sm.Wm[c & 1][0][0];
        const bf16_t* Qm = &sm.Qm[c & 1][0][0];
        STIn in;
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            in.wa[k2] = ld4x2(Wm + l16 * kRow + 32 * k2 + 4 * g);
            in.qa[k2] = ld4x2(Qm + l16 * kRow + 32 * k2 + 4 * g);
        }
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            in.bbt[jt] = ld4(&s.BbT[16 * jt + l16][4 * g]);
            in.kbt[jt] = ld4(&s.KbT[16 * jt + l16][4 * g]);
            in.gl[jt] = *reinterpret_cast<const float4*>(&s.gL[16 * jt + 4 * g]);
        }
        return in;
    };
    auto stage_ST = [&](int c, const STIn& in, const MWRegs& m) __attribute__((always_inline)) {
        bf16x4 Sb[4];
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) Sb[jt] = cvt4(S[jt]);
        f32x4 Z = m.U, Yt = m.Y0;
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            const bf16x8 bs = cat8(Sb[2 * k2], Sb[2 * k2 + 1]);
            Z = mfma32(in.wa[k2], bs, Z);
            Yt = mfma32(in.qa[k2], bs, Yt);
        }
        const bf16x4 Zb = cvt4(Z);
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            f32x4 acc;
            acc[0] = in.gl[jt].x * S[jt][0];
            acc[1] = in.gl[jt].y * S[jt][1];
            acc[2] = in.gl[jt].z * S[jt][2];
            acc[3] = in.gl[jt].w * S[jt][3];
            acc = mfma16(in.kbt[jt], m.V, acc);          // + H = Kb^T V
            S[jt] = mfma16(in.bbt[jt], Zb, acc);
        }
        bf16_t* Yd = &sm.Ys[c & 1][0][0];
#pragma unroll
        for (int q = 0; q < 4; ++q) Yd[(4 * g + q) * kRow + col] = f2bf(Yt[q]);
        const int done = (c + 1) * kL;
        if (ckpt && (done % kCkptInterval) == 0 && done < T) {
            float* dst = ckpt + (((size_t)bh * nck + done / kCkptInterval) * kN + col) * kN;
#pragma unroll
            for (int jt = 0; jt < 4; ++jt)
                *reinterpret_cast<float4*>(dst + 16 * jt + 4 * g) =
                    make_float4(S[jt][0], S[jt][1], S[jt][2], S[jt][3]);
        }
    };

    // y of chunk c: 16 tokens x 16 lanes x 8 B from the staged read-outs.
    const int yt = tid >> 4, yc4 = tid & 15;
    auto read_y = [&](int c) __attribute__((always_inline)) -> uint2 {
        return *reinterpret_cast<const uint2*>(&sm.Ys[c & 1][yt][yc4 * 4]);
    };
    auto store_y = [&](int c, uint2 val) __attribute__((always_inline)) {
        const int tt = c * kL + yt;
        if (y && tt < T)
            *reinterpret_cast<uint2*>(y + tok_off(bb, tt, hh, T, H) + yc4 * 4) = val;
    };

    if (T > 0) {
        // Register ring: the raw loads of chunk c live in ring slot c % 3 until
        // stashed.  Three named variables, not an array, so that the ring is
        // never promoted to LDS or scratch.
        Raw rb0, rb1, rb2;
        load_raw(0, rb0);
        load_raw(1, rb1);
        load_raw(2, rb2);
        stash_raw(0, rb0);
        load_raw(3, rb0);
        __syncthreads();
        // Prologue: E of chunks 0, 1 and MW of chunk 0.
        stash_raw(1, rb1);
        load_raw(4, rb1);
        ERegs e_prev = stage_E(0);
        __syncthreads();
        stash_raw(2, rb2);
        load_raw(5, rb2);
        MWRegs m_prev = stage_MW(0, read_MW(0), e_prev);
        e_prev = stage_E(1);
        __syncthreads();
        // One pipeline interval: E(it), MW(it-1), ST(it-2), y of chunk it-3;
        // chunk it+1 moves from the ring into LDS and chunk it+4 is loaded
        // into the freed ring slot.  (A macro rather than a lambda: the ring
        // variables must stay plain SSA values so they live in registers.)
#define WKV7_FWD_INTERVAL(IT, RING)                                   \
    {                                                                 \
        const int it_ = (IT);                                         \
        const MWIn mi = read_MW(it_ - 1);                             \
        const STIn si = read_ST(it_ - 2);                             \
        const uint2 yv = read_y(it_ - 3);                             \
        const ERegs e_cur = stage_E(it_);                             \
        stash_raw(it_ + 1, RING);                                     \
        load_raw(it_ + 4, RING);                                      \
        const MWRegs m_cur = stage_MW(it_ - 1, mi, e_prev);           \
        stage_ST(it_ - 2, si, m_prev);                                \
        if (it_ >= 3) store_y(it_ - 3, yv);                           \
        __syncthreads();                                              \
        e_prev = e_cur;                                               \
        m_prev = m_cur;                                               \
    }
        // Chunk it+1 sits in ring slot (it+1) % 3: it = 2, 3, 4 -> slots 0, 1, 2
        // (unrolled so the slot is a compile-time constant).
        for (int it = 2; it <= nch + 2; it += 3) {
            WKV7_FWD_INTERVAL(it, rb0);
            if (it + 1 > nch + 2) break;
            WKV7_FWD_INTERVAL(it + 1, rb1);
            if (it + 2 > nch + 2) break;
            WKV7_FWD_INTERVAL(it + 2, rb2);
        }
#undef WKV7_FWD_INTERVAL
    }

    if (sT) {
        float* dst = sT + ((size_t)bh * kN + col) * kN;
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
            *reinterpret_cast<float4*>(dst + 16 * jt + 4 * g) =
                make_float4(S[jt][0], S[jt][1], S[jt][2], S[jt][3]);
    }
}

}  // namespace

hipError_t launch_chunk_fwd(const FwdArgs& p, int chunk_len, hipStream_t stream) {
    if (chunk_len != kL || !p.bf16) return hipErrorInvalidValue;
    chunk_fwd_kernel<<<dim3(p.B * p.H), dim3(kThreads), 0, stream>>>(
        p.T, p.H, static_cast<const bf16_t*>(p.r), static_cast<const bf16_t*>(p.w),
        static_cast<const bf16_t*>(p.k), static_cast<const bf16_t*>(p.v),
        static_cast<const bf16_t*>(p.a), static_cast<const bf16_t*>(p.b), p.s0,
        static_cast<bf16_t*>(p.y), p.sT, p.ckpt);
    return hipGetLastError();
}

}  // namespace wkv7
