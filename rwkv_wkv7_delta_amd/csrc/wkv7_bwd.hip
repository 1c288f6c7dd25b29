// wkv7_bwd.hip -- chunked WKV7 backward on bf16 MFMA, gfx950.
//
// Gradient of L = sum_t <dy_t, y_t> + <dsT, S_T> through the chunk form of
// the recurrence (wkv7_chunk_fwd.hip).  Per chunk of L = 16 tokens with entry
// state S0, removal read-outs Z, read-out adjoint dY and the adjoint dS of
// the chunk's exit state:
//
//   dZ  = Arb^T dY + Bb dS^T            dX = Tm^T dZ = (Tm^T Bb) dS^T + (Arb Tm)^T dY
//   dV  = Aak^T dX + Ark^T dY + Kb dS^T
//   dS0 = dS diag(G_L) + dY^T Rt + dX^T At       (adjoint carried to the previous chunk)
//   dAab = tril_-1(dX Z^T)  dAak = tril_-1(dX V^T)
//   dArb = tril_0(dY Z^T)   dArk = tril_0(dY V^T)
//   dAt = dX S0 + dAab Bh + dAak Kh     dRt = dY S0 + dArb Bh + dArk Kh
//   dBh = dAab^T At + dArb^T Rt         dKh = dAak^T At + dArk^T Rt
//   dBb = Z dS                          dKb = V dS
// followed by the chain rule through the decay products: per token
// da = dAt G_{t-1}, dr = dRt G_t, db = (dBh + dBb G_L) / G_t,
// dk = (dKh + dKb G_L) / G_t, and d log w_u collects every factor that the
// running products G_t (t >= u) enter.
//
// Only the adjoint dS is sequential.  The backward therefore runs in two
// passes:
//   pass 1 (one workgroup per head, chunks last to first): the adjoint chain,
//     with the forward's producer/consumer structure -- producers rebuild the
//     chunk's decay products, scaled vectors and 16x16 tiles, two more waves
//     the triangular inverse (alternate chunks, each solve over two
//     intervals) and the state-independent factors Tm^T Bb (over Bb) and
//     (Arb Tm)^T; consumers own 16 value rows each of dS^T in accumulator
//     tiles and emit dv, dX and the chunk's incoming dS;
//   pass 2 (one independent wave per chunk and key block, no barriers): every
//     per-key gradient, from pass 1's dX and dS and the forward's tape (entry
//     states S0 and read-outs Z).

#include "wkv7.h"
#include "wkv7_device.h"
#include "wkv7_internal.h"
#include "wkv7_mfma.h"

namespace wkv7 {

namespace {

constexpr int kL = 16;
// Padded LDS rows (see wkv7_chunk_fwd.hip), for head size N = 32 or 64.
template <int N>
constexpr int kRowOf = N + 8;

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

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
struct Raw {
    u32x4 x[3];
};

// =============================================================================
// Pass 1: the adjoint chain.
// =============================================================================

// N/16 producer, N/16 consumer, 2 inverse waves (640 threads at N = 64; 384 at
// N = 32, two workgroups per compute unit).
template <int N>
constexpr int kP1Threads = 64 * (2 * (N / 16) + 2);
constexpr int kP1Slots = 4;
enum { P1_R = 0, P1_W = 1, P1_K = 2, P1_A = 3, P1_B = 4, P1_DY = 5 };
// Tile images in a slot: the A-operand image of (Arb Tm)^T, from INV; those of
// Aak^T, Ark^T, from MW.
enum { TILE_RB = 0, TILE_AK = 1, TILE_RK = 2 };

// Rows [t][j] (the chain reads At, Rt and dy transposed, which gives the
// matrix-core operand layouts directly) and images: register contents stored
// lane by lane (8 bytes per lane, read back by the same lane index).
template <int N>
struct P1Slot {
    static constexpr int kRow = kRowOf<N>;
    bf16_t At[kL][kRow], Rt[kL][kRow];                  // E -> MW, INV, chain
    bf16_t Bb[kL][kRow];                                // E -> INV; Tm^T Bb from INV -> chain
    bf16_t Kb[kL][kRow], dY[kL][kRow];                  // E -> chain
    float gL[64];         // G_L of key 16 jt + 4 g + q at word 16 g + 4 jt + q
    uint2 tiles[3][64];
};
// Bh and Kh, read only in the interval after E.
template <int N>
struct P1SlotBK {
    static constexpr int kRow = kRowOf<N>;
    bf16_t Bh[kL][kRow], Kh[kL][kRow];
};

template <int N>
struct __align__(16) P1Smem {
    static constexpr int kRow = kRowOf<N>;
    bf16_t raw[2][6][kL][kRow];   // r, w, k, a, b, dy of two chunks
    P1Slot<N> sl[kP1Slots];
    P1SlotBK<N> bk[2];
    bf16_t dXs[2][kL][kRow];      // [t][i]
    bf16_t dVs[2][kL][kRow];      // [t][i]
    bf16_t dSs[2][N][kRow];       // the adjoint leaving the chunk as [j][i] (kept per 32 tokens)
};

// Segments in time (nseg >= 2; every head split): the adjoint is affine in
// itself, dS_left = dS_right P + H over a segment (rows of dS evolve
// independently given the chunk factors), with P the run from the identity
// with dy = 0 and H the run from zero with the real dy.  Segments are numbered
// from the end (s' = nseg - 1 - s), so that the composition of the entry
// adjoints has the forward's form (seg_combine_kernel, the same layout of 3
// nseg states per head: entry adjoints at s', H at nseg + s', P at 2 nseg + s').
//   pass 0: the last segment from dsT with its outputs (its left-edge adjoint
//           to entry slot 1), and the two map runs of every middle segment;
//   pass 1: segments s' = 1 .. nseg-1 from their entry adjoints, with outputs
//           (the first segment's left-edge adjoint is ds0).
// nseg = 1: one workgroup per head over the whole sequence.
struct ChainWork {
    int bh, c_lo, c_hi;   // chunks [c_lo, c_hi), run from the last down
    const float* init;    // the adjoint at the right edge (else the identity when ident, else 0)
    float* fin;           // where the adjoint at the left edge goes (or null)
    bool ident, dyzero, outs;
};
__device__ __forceinline__ ChainWork chain_work(int blk, int nblk_grid, int nch, int pass, int nseg,
                                                int seg_chunks, const float* dsT, float* ds0,
                                                float* states, size_t NN) {
    ChainWork cw{0, 0, nch, nullptr, nullptr, false, false, true};
    if (nseg <= 1) {
        cw.bh = spread_heads(blk, nblk_grid);
        cw.init = dsT ? dsT + (size_t)cw.bh * NN : nullptr;
        cw.fin = ds0 ? ds0 + (size_t)cw.bh * NN : nullptr;
        return cw;
    }
    const int per = pass == 0 ? 2 * nseg - 3 : nseg - 1;
    const int hs = blk / per, rr = blk % per;
    float* const hst = states + (size_t)hs * 3 * nseg * NN;
    cw.bh = hs;
    if (pass == 0 && rr == 0) {   // the last segment, for real
        cw.c_lo = (nseg - 1) * seg_chunks;
        cw.init = dsT ? dsT + (size_t)hs * NN : nullptr;
        cw.fin = hst + NN;
        return cw;
    }
    const int sp = pass == 0 ? 1 + (rr - 1) / 2 : 1 + rr;   // s'
    const int sg = nseg - 1 - sp;                            // s
    cw.c_lo = sg * seg_chunks;
    cw.c_hi = cw.c_lo + seg_chunks;
    if (pass == 0) {
        const bool pm = ((rr - 1) & 1) != 0;   // the P run
        cw.ident = pm;
        cw.dyzero = pm;
        cw.outs = false;
        cw.fin = hst + (size_t)((pm ? 2 : 1) * nseg + sp) * NN;
    } else {
        cw.init = hst + (size_t)sp * NN;
        cw.fin = (sg == 0 && ds0) ? ds0 + (size_t)hs * NN : nullptr;
    }
    return cw;
}

// kAB = false: a = b = 0 (decay-only recurrence); a and b are not read and
// stand as zero rows, so the removal terms vanish from every product.
template <int N, bool kAB>
__global__ __launch_bounds__(kP1Threads<N>, N == 32 ? 2 : 1) void bwd_chain_kernel(
    int T, int H, const bf16_t* __restrict__ r, const bf16_t* __restrict__ w,
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ a, const bf16_t* __restrict__ b,
    const bf16_t* __restrict__ dy, const float* __restrict__ dsT, bf16_t* __restrict__ dv,
    float* __restrict__ ds0, bf16_t* __restrict__ wdX, bf16_t* __restrict__ wdS,
    int* __restrict__ counter, int pass, int nseg, int seg_chunks, float* __restrict__ states) {
    // (these hide the file-scope N = 64 constants in the body below)
    constexpr int kN = N, kRow = kRowOf<N>;
    constexpr int kP = N / 16;                  // producer (and consumer) waves
    constexpr int K2 = N / 32, JT = N / 16;     // 32-deep halves, 16-wide key tiles
    using P1Slot = wkv7::P1Slot<N>;
    using P1SlotBK = wkv7::P1SlotBK<N>;
    __shared__ P1Smem<N> sm;
    const int nch = (T + kL - 1) / kL;
    const ChainWork cw = chain_work(blockIdx.x, gridDim.x, nch, pass, nseg, seg_chunks, dsT, ds0,
                                    states, (size_t)kN * kN);
    const int bh = cw.bh;
    const int bb = bh / H, hh = bh % H;
    const int c_lo = cw.c_lo;
    const int tid = threadIdx.x;
    // Roles split by wave (the tests are uniform within a wave).  They are left
    // as per-lane conditions: branching on an SGPR copy of the wave index
    // measured several per cent slower.
    const int wave = tid >> 6;
    const bool producer = wave < kP;
    const bool consumer = wave >= kP && wave < 2 * kP;
    const bool inverter = wave >= 2 * kP;
    const int rtid = tid & (64 * kP - 1);
    const int lane = tid & 63, wp = (tid >> 6) & (kP - 1);
    const int l16 = lane & 15, g = lane >> 4;
    const int col = 16 * wp + l16;
    // wdX: [B][T][H][N]; wdS: [B][H][nblk][N][N]
    const int nblk = (nch + 1) / 2;
    // The adjoint leaving a 32-token block: after chunk c when c is odd or the last.
    auto keeps_dS = [&](int c) __attribute__((always_inline)) { return c >= c_lo && ((c & 1) || c == nch - 1); };
    // Interval it handles chunks from the last one of the range down; chunks
    // below c_lo (negative ones too) are all-padding, for which every stage is
    // the identity.
    auto chunk_of = [&](int it) __attribute__((always_inline)) { return cw.c_hi - 1 - it; };
    // (negative chunk indices in the padding intervals: two's complement & keeps
    // them in range)
    auto slot_of = [&](int c) __attribute__((always_inline)) { return c & (kP1Slots - 1); };

    // The per-key pass that follows takes its blocks from a queue: start it empty.
    if (blockIdx.x == 0 && tid == 0) {
        counter[0] = 0;
        counter[1] = 0;
    }

    // ---- consumer adjoint: dS^T tiles, lane holds dS[col][16 jt + 4 g + q] -------
    f32x4 dSt[JT];
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) dSt[jt] = zero4();
    if (consumer && cw.ident) {
#pragma unroll
        for (int jt = 0; jt < JT; ++jt)
#pragma unroll
            for (int q = 0; q < 4; ++q) dSt[jt][q] = col == 16 * jt + 4 * g + q ? 1.f : 0.f;
    } else if (consumer && cw.init) {
        const float* base = cw.init + (size_t)col * kN;
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
            const float4 x = *reinterpret_cast<const float4*>(base + 16 * jt + 4 * g);
            dSt[jt][0] = x.x; dSt[jt][1] = x.y; dSt[jt][2] = x.z; dSt[jt][3] = x.w;
        }
        // Settle the loads here: left pending into the loop, the compiler
        // guards every later use of dS with a wait on the whole memory counter,
        // which then also waits for the previous chunk's stores.
        __builtin_amdgcn_s_waitcnt(0);
    }

    // ---- producer raw loads (as in the forward; vector 5 is dy) -------------------
    const bool hi = rtid >= 2 * kN;
    const bf16_t* const sp_p[3] = {hi ? w : r, hi ? a : k, hi ? dy : b};
    const int ld_t = (rtid / (kN / 8)) & 15, ld_c8 = rtid & (kN / 8 - 1);
    auto load_raw = [&](int c, Raw& o) __attribute__((always_inline)) {
        const int t = max(0, min(c * kL + ld_t, T - 1));
        const size_t off = tok_off<N>(bb, t, hh, T, H) + ld_c8 * 8;
#pragma unroll
        for (int p = 0; p < 3; ++p) {
            if (kAB || !(p == 1 ? hi : p == 2 ? !hi : false)) {
                o.x[p] = *reinterpret_cast<const u32x4*>(sp_p[p] + off);
            } else {
                const u32x4 z = {0u, 0u, 0u, 0u};   // a (p = 1, hi) or b (p = 2, lo): zero
                o.x[p] = z;
            }
        }
    };
    auto stash_raw = [&](int c, const Raw& o) __attribute__((always_inline)) {
        if (c >= c_lo && (c + 1) * kL <= T) {   // a whole chunk (the common case: no selects)
#pragma unroll
            for (int p = 0; p < 3; ++p)
                *reinterpret_cast<u32x4*>(&sm.raw[c & 1][2 * p + (hi ? 1 : 0)][ld_t][ld_c8 * 8]) = o.x[p];
            return;
        }
        const int t = c * kL + ld_t;
        const bool ok = c >= c_lo && t < T;
#pragma unroll
        for (int p = 0; p < 3; ++p) {
            const unsigned pad = (p == 0 && hi) ? 0x3F803F80u : 0u;   // padding: w = 1
            const u32x4 padv = {pad, pad, pad, pad};
            *reinterpret_cast<u32x4*>(&sm.raw[c & 1][2 * p + (hi ? 1 : 0)][ld_t][ld_c8 * 8]) =
                ok ? o.x[p] : padv;
        }
    };

    // ---- E (producer): decay products, scaled vectors, dy images ------------------
    // Row layout: lane (g, l16) takes token t = l16 and key columns j0 .. j0+3,
    // j0 = 16p + 4g (8-byte LDS accesses; the running product over tokens is a
    // scan along the lanes of a DPP row).
    const int j0 = 16 * wp + 4 * g;
    const bf16x4 ident = identity_b(g, l16);
    struct ERaw {
        uint2 v[6];
    };
    auto read_E = [&](int c) __attribute__((always_inline)) -> ERaw {
        const bf16_t(*Rr)[kL][kRow] = sm.raw[c & 1];
        ERaw e;
#pragma unroll
        for (int vi = 0; vi < 6; ++vi) e.v[vi] = *reinterpret_cast<const uint2*>(&Rr[vi][l16][j0]);
        return e;
    };
    auto stage_E = [&](int c, const ERaw& er) __attribute__((always_inline)) {
        P1Slot& s = sm.sl[slot_of(c)];
        P1SlotBK& bk = sm.bk[c & 1];
        const uint2* raw6 = er.v;
        float X[6][4];
#pragma unroll
        for (int vi = 0; vi < 6; ++vi) {
            X[vi][0] = __uint_as_float(raw6[vi].x << 16);
            X[vi][1] = __uint_as_float(raw6[vi].x & 0xFFFF0000u);
            X[vi][2] = __uint_as_float(raw6[vi].y << 16);
            X[vi][3] = __uint_as_float(raw6[vi].y & 0xFFFF0000u);
        }
        f32x4 at, rt, bh4, kh4, bb4, kb4, gt;
        float G4[4] = {X[P1_W][0], X[P1_W][1], X[P1_W][2], X[P1_W][3]};
        row16_cumprod4(G4[0], G4[1], G4[2], G4[3]);
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            const float Gt = G4[cc];
            const float Gp = row16_prev(Gt, 1.f);
            const float GL = row16_last(Gt);
            const float inv = __builtin_amdgcn_rcpf(Gt);
            gt[cc] = Gt;
            at[cc] = X[P1_A][cc] * Gp;
            rt[cc] = X[P1_R][cc] * Gt;
            bh4[cc] = X[P1_B][cc] * inv;
            kh4[cc] = X[P1_K][cc] * inv;
            bb4[cc] = bh4[cc] * GL;
            kb4[cc] = kh4[cc] * GL;
        }
        const bf16x4 atb = cvt4(at), rtb = cvt4(rt);
        if (kAB) *reinterpret_cast<bf16x4*>(&s.At[l16][j0]) = atb;
        *reinterpret_cast<bf16x4*>(&s.Rt[l16][j0]) = rtb;
        if (kAB) *reinterpret_cast<bf16x4*>(&bk.Bh[l16][j0]) = cvt4(bh4);
        *reinterpret_cast<bf16x4*>(&bk.Kh[l16][j0]) = cvt4(kh4);
        if (kAB) *reinterpret_cast<bf16x4*>(&s.Bb[l16][j0]) = cvt4(bb4);
        *reinterpret_cast<bf16x4*>(&s.Kb[l16][j0]) = cvt4(kb4);
        *reinterpret_cast<uint2*>(&s.dY[l16][j0]) = cw.dyzero ? make_uint2(0u, 0u) : raw6[P1_DY];
        if (l16 == kL - 1) *reinterpret_cast<float4*>(&s.gL[16 * g + 4 * wp]) = make_float4(gt[0], gt[1], gt[2], gt[3]);
    };

    // ---- MW (producer): one 16x16 tile per wave ---------------------------------
    // The last two producer waves (2, 3 at N = 64; 0, 1 at N = 32) form Aak =
    // tril_-1(At Kh^T), Ark = tril_0(Rt Kh^T) as [t][s] = X_t . Y_s, whose
    // accumulator registers are the A-operand images of Aak^T, Ark^T; Aab, Arb
    // and the inverse come from the inverse waves.
    struct MWIn {
        bf16x8 xv[K2], yv[K2];
    };
    auto read_MW = [&](int c) __attribute__((always_inline)) -> MWIn {
        const P1Slot& s = sm.sl[slot_of(c)];
        const P1SlotBK& bk = sm.bk[c & 1];
        const bf16_t(*Xr)[kRow] = (wp & 1) ? s.Rt : s.At;
        const bf16_t(*Yr)[kRow] = bk.Kh;
        MWIn in;
#pragma unroll
        for (int k2 = 0; k2 < K2; ++k2) {
            in.xv[k2] = ld8(&Xr[l16][32 * k2 + 8 * g]);
            in.yv[k2] = ld8(&Yr[l16][32 * k2 + 8 * g]);
        }
        return in;
    };
    auto stage_MW = [&](int c, const MWIn& in) __attribute__((always_inline)) {
        P1Slot& s = sm.sl[slot_of(c)];
        f32x4 P = zero4();
#pragma unroll
        for (int k2 = 0; k2 < K2; ++k2) P = mfma32(in.xv[k2], in.yv[k2], P);   // [t][s] = X_t . Y_s
        const bool diag = (wp & 1) != 0;   // Ark keeps the diagonal
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int m = 4 * g + q, n = l16;
            P[q] = (n < m || (diag && n == m)) ? P[q] : 0.f;
        }
        // Accumulator registers of X fed as an A operand stand for X^T.
        s.tiles[(wp & 1) == 0 ? TILE_AK : TILE_RK][lane] = __builtin_bit_cast(uint2, cvt4(P));
    };
    // ---- INV (inverse waves): Aab, Tm = (I - Aab)^-1, Tm^T Bb, (Arb Tm)^T -------
    // In the interval after E(c) a wave forms Aab = tril_-1(At Bh^T) and Arb^T
    // (Arb = tril_0(Rt Bh^T), as [s][t]), the inverses of Aab's 4x4 diagonal
    // blocks, N = Td L and N^T N^T (wkv7_mfma.h); in the next it joins them into
    // Tm and applies Tm, as hi and lo bf16 parts, to the factors of
    // dX = (Tm^T Bb) dS^T + (Arb Tm)^T dY (the
    // transpose of the forward's Z = (Tm At) S0^T + (Tm Aak) V, with the same
    // cancellations kept inside these products):
    //   the accumulator tile of Bb^T[keys 16 jt ..] Tm holds (Tm^T Bb)[l16][16 jt
    //     + 4 g + q] -- its row layout, written over the same columns of Bb;
    //   Arb Tm from Arb's A-operand image (hi and lo), whose accumulator
    //     registers are the A-operand image of (Arb Tm)^T.
    struct InvState {
        BlockInverse bi;
        f32x4 ArbT;   // accumulator layout [s][t]: Arb's A-operand image
    };
    auto inv_begin = [&](int c) __attribute__((always_inline)) -> InvState {
        const P1Slot& s = sm.sl[slot_of(c)];
        const P1SlotBK& bk = sm.bk[c & 1];
        bf16x8 xv[K2], yv[K2], rv[K2];
#pragma unroll
        for (int k2 = 0; k2 < K2; ++k2) {
            xv[k2] = ld8(&s.At[l16][32 * k2 + 8 * g]);
            yv[k2] = ld8(&bk.Bh[l16][32 * k2 + 8 * g]);
            rv[k2] = ld8(&s.Rt[l16][32 * k2 + 8 * g]);
        }
        f32x4 P = zero4(), R = zero4();
#pragma unroll
        for (int k2 = 0; k2 < K2; ++k2) {
            P = mfma32(xv[k2], yv[k2], P);   // [t][s] = Aab[t][s]
            R = mfma32(yv[k2], rv[k2], R);   // [s][t] = Arb[t][s]
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            P[q] = (l16 < 4 * g + q) ? P[q] : 0.f;    // s < t
            R[q] = (4 * g + q <= l16) ? R[q] : 0.f;   // s <= t
        }
        return InvState{unit_lower_inverse_begin<false>(P, g, l16), R};
    };
    auto inv_end = [&](int c, const InvState& st) __attribute__((always_inline)) {
        P1Slot& s = sm.sl[slot_of(c)];
        bf16x4 bbT[JT];
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) bbT[jt] = ld4_tr(tr_addr(&s.Bb[0][16 * jt], kRow, g, l16));
        const Split4 tm = split4(unit_lower_inverse_cols_end(st.bi));
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
            const f32x4 d = mfma16(bbT[jt], tm.hi, mfma16(bbT[jt], tm.lo, zero4()));
            *reinterpret_cast<bf16x4*>(&s.Bb[l16][16 * jt + 4 * g]) = cvt4(d);
        }
        s.tiles[TILE_RB][lane] = __builtin_bit_cast(uint2, cvt4(mul3(split4(st.ArbT), tm, zero4())));
    };

    // ---- chain (consumer): value rows `col` of the adjoint ------------------------
    struct CIn {
        bf16x4 RbT, AakT, ArkT, dY;
        bf16x8 bb[K2], kb[K2];
        bf16x4 rtT[JT], atT[JT];
        float gl;   // G_L of key 16 jt + 4 g + q sits in lane 4 jt + q of row g
    };
    auto read_C = [&](int c) __attribute__((always_inline)) -> CIn {
        const P1Slot& s = sm.sl[slot_of(c)];
        CIn in;
        if (kAB) {
            in.RbT = __builtin_bit_cast(bf16x4, s.tiles[TILE_RB][lane]);   // (Arb Tm)^T
            in.AakT = __builtin_bit_cast(bf16x4, s.tiles[TILE_AK][lane]);
        }
        in.ArkT = __builtin_bit_cast(bf16x4, s.tiles[TILE_RK][lane]);
        in.dY = ld4_tr(tr_addr(&s.dY[0][16 * wp], kRow, g, l16));   // [t][i] as a B operand
#pragma unroll
        for (int k2 = 0; k2 < K2; ++k2) {
            if (kAB) in.bb[k2] = ld4x2(&s.Bb[l16][32 * k2 + 4 * g]);   // Tm^T Bb
            in.kb[k2] = ld4x2(&s.Kb[l16][32 * k2 + 4 * g]);
        }
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
            in.rtT[jt] = ld4_tr(tr_addr(&s.Rt[0][16 * jt], kRow, g, l16));   // Rt^T as an A operand
            if (kAB) in.atT[jt] = ld4_tr(tr_addr(&s.At[0][16 * jt], kRow, g, l16));
        }
        in.gl = s.gL[lane];
        return in;
    };
    auto stage_C = [&](int c, const CIn& in) __attribute__((always_inline)) {
        bf16x4 dSb[JT];
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) dSb[jt] = cvt4(dSt[jt]);
        // dX = Tm^T dZ = (Tm^T Bb) dS^T + (Arb Tm)^T dY with both factors from INV.
        // Partial sums of the two MFMA shapes meet on the vector ALU (add4).
        // (a = b = 0: Bb, Arb, Aak vanish, so dX = 0 and only the Kb and Ark
        // terms of dV remain.)
        f32x4 dXs = zero4(), dVk = zero4();
#pragma unroll
        for (int k2 = 0; k2 < K2; ++k2) {
            const bf16x8 ds8 = cat8(dSb[2 * k2], dSb[2 * k2 + 1]);
            if (kAB) dXs = mfma32(in.bb[k2], ds8, dXs);
            dVk = mfma32(in.kb[k2], ds8, dVk);
        }
        bf16x4 dXb = {};
        f32x4 dV = zero4();
        if (kAB) {
            dXb = cvt4(add4(dXs, mfma16(in.RbT, in.dY, zero4())));
            dV = mfma16(in.AakT, dXb, zero4());
        }
        dV = mfma16(in.ArkT, in.dY, dV);
        const bf16x4 dVb = cvt4(add4(dV, dVk));
        // Staged in row layout (swap_layout), 8 bytes per lane.
        const int sb = c & 1;
        const int i0 = 16 * wp + 4 * g;
        if (kAB) *reinterpret_cast<bf16x4*>(&sm.dXs[sb][l16][i0]) = swap_layout(dXb, ident);
        *reinterpret_cast<bf16x4*>(&sm.dVs[sb][l16][i0]) = swap_layout(dVb, ident);
        if (keeps_dS(c)) {
#pragma unroll
            for (int jt = 0; jt < JT; ++jt)   // as [j][i]: row layout of the dS^T tile of key block jt
                *reinterpret_cast<bf16x4*>(&sm.dSs[sb][16 * jt + l16][i0]) = swap_layout(dSb[jt], ident);
        }
        // dS0^T = G_L dS^T + Rt^T dY + At^T dX
        f32x4 dec[JT];
        dec[0] = mul_row_lanes4<0>(in.gl, dSt[0]);
        dec[1] = mul_row_lanes4<1>(in.gl, dSt[1]);
        if constexpr (JT > 2) {
            dec[2] = mul_row_lanes4<2>(in.gl, dSt[2]);
            dec[3] = mul_row_lanes4<3>(in.gl, dSt[3]);
        }
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
            const f32x4 acc = mfma16(in.rtT[jt], in.dY, dec[jt]);
            dSt[jt] = kAB ? mfma16(in.atT[jt], dXb, acc) : acc;
        }
    };

    // ---- outputs of chunk c (consumers): dv and dX rows, the chunk's exit adjoint --
    // N/8 consecutive threads write one row (128 bytes at N = 64) with 16-byte
    // stores: threads 0 .. 2N-1 dv, 2N .. 4N-1 dX.
    auto store_out = [&](int c) __attribute__((always_inline)) {
        if (c < c_lo || !cw.outs) return;
        const int sb = c & 1;
        const int row = (rtid / (kN / 8)) & 15, piece = rtid & (kN / 8 - 1);
        const int tt = c * kL + row;
        if (tt < T && (kAB || rtid < 2 * kN)) {   // a = b = 0: dX is zero, not stored
            bf16_t* base = rtid < 2 * kN ? dv : wdX;
            const bf16_t(*src)[kRow] = rtid < 2 * kN ? sm.dVs[sb] : sm.dXs[sb];
            store_stream(base + tok_off<N>(bb, tt, hh, T, H) + 8 * piece,
                         *reinterpret_cast<const uint4*>(&src[row][8 * piece]));
        }
        if (keeps_dS(c)) {
#pragma unroll
            for (int k2 = 0; k2 < K2; ++k2) {
                const int j = 32 * k2 + rtid / (kN / 8);   // 32 rows of the adjoint per pass
                store_stream(wdS + (((size_t)bh * nblk + (c >> 1)) * kN + j) * kN + 8 * piece,
                             *reinterpret_cast<const uint4*>(&sm.dSs[sb][j][8 * piece]));
            }
        }
    };

    {
        // Intervals 0 .. (c_hi - c_lo)+3 carry real work; the count is rounded up
        // to a multiple of three for the unrolled producer loop.  The extra
        // intervals see only all-padding chunks (identity, nothing stored).
        const int n_it = (cw.c_hi - c_lo + 6) / 3 * 3;
        // Each role runs its own loop over the same number of intervals (one
        // barrier each), so the compiler sees only loads on the producer side
        // and only stores on the consumer side; with both kinds in one loop it
        // must treat the memory counter as unordered and drain it completely.
        if (producer) {
            // The producers set each interval's length: they issue at the inverse
            // waves' priority (below the state chain), which measured about 2 %
            // faster than the default at the 2.9B shape.
            __builtin_amdgcn_s_setprio(2);
            Raw rb0, rb1, rb2;
            load_raw(chunk_of(0), rb0);
            load_raw(chunk_of(1), rb1);
            load_raw(chunk_of(2), rb2);
            stash_raw(chunk_of(0), rb0);
            load_raw(chunk_of(3), rb0);
            __syncthreads();
            // Interval it: E(chunk_of(it)) and MW(chunk_of(it-1)), stash
            // chunk_of(it+1) and load chunk_of(it+4).  (A macro, not a lambda, so
            // that the register ring stays plain SSA values.)  No early exit
            // inside the unrolled body: one makes the compiler drain the whole
            // counter before every stash.
#define WKV7_BWD_PRODUCE(IT, RING)                                             \
    {                                                                          \
        const int it_ = (IT);                                                  \
        const ERaw er = read_E(chunk_of(it_));                                 \
        MWIn mi;                                                               \
        if (it_ >= 1 && (kAB ? wp >= kP - 2 : wp == kP - 1)) mi = read_MW(chunk_of(it_ - 1)); \
        stage_E(chunk_of(it_), er);                                            \
        stash_raw(chunk_of(it_ + 1), RING);                                    \
        load_raw(chunk_of(it_ + 4), RING);                                     \
        if (it_ >= 1 && (kAB ? wp >= kP - 2 : wp == kP - 1)) stage_MW(chunk_of(it_ - 1), mi); \
        __syncthreads();                                                       \
    }
            for (int it = 0; it < n_it; it += 3) {
                WKV7_BWD_PRODUCE(it, rb1);
                WKV7_BWD_PRODUCE(it + 1, rb2);
                WKV7_BWD_PRODUCE(it + 2, rb0);
            }
#undef WKV7_BWD_PRODUCE
        } else if (inverter) {
            __builtin_amdgcn_s_setprio(2);
            __syncthreads();
            // chunk_of(j) belongs to wave 8 + (j & 1), which starts its inverse in
            // interval j + 1 (after E) and finishes it, with the dX factors, in
            // interval j + 2 (the chain reads them in interval j + 3): one half
            // per wave and interval, `st` carrying an inverse across one barrier.
            const int par = wave & 1;
            InvState st{{zero4(), zero4(), zero4()}, zero4()};
            for (int it = 0; it < n_it; ++it) {
                if (kAB && it >= 1) {
                    if (((it - 1) & 1) == par)
                        st = inv_begin(chunk_of(it - 1));
                    else if (it >= 2)
                        inv_end(chunk_of(it - 2), st);
                }
                __syncthreads();
            }
        } else {
            // The chain is the critical path: its waves issue first (then the
            // inverse waves, then the producers) when several are ready.
            __builtin_amdgcn_s_setprio(3);
            __syncthreads();
            // Interval it: the chain on chunk_of(it-3), the stores of chunk_of(it-4).
            for (int it = 0; it < n_it; ++it) {
                if (it >= 3) {
                    const CIn ci = read_C(chunk_of(it - 3));
                    stage_C(chunk_of(it - 3), ci);
                }
                if (it >= 4) store_out(chunk_of(it - 4));
                __syncthreads();
            }
        }
    }

    if (cw.fin && consumer) {
        float* dst = cw.fin + (size_t)col * kN;
#pragma unroll
        for (int jt = 0; jt < JT; ++jt)
            *reinterpret_cast<float4*>(dst + 16 * jt + 4 * g) =
                make_float4(dSt[jt][0], dSt[jt][1], dSt[jt][2], dSt[jt][3]);
    }
}

// =============================================================================
// Pass 2: per-key gradients, one workgroup per pair of chunks (32 tokens).
// =============================================================================
//
// The tape holds the state entering every 32-token block and the workspace the
// adjoint leaving it, which halves their traffic.  A workgroup takes the two
// chunks c0 = 2m, c1 = 2m + 1 of block m and first steps across the middle:
//   S0(c1)^T   = diag(G_L(c0)) S0(c0)^T + Kb(c0)^T V(c0) + Bb(c0)^T Z(c0)
//   dS(c0)^T   = diag(G_L(c1)) dS(c1)^T + Rt(c1)^T dY(c1) + At(c1)^T dX(c1)
// (the forward's state update and the chain's adjoint update of one chunk,
// contracted over the chunk's tokens), then computes every per-key gradient
// of c0 and of c1.  Wave p owns key columns 16p .. 16p+15 throughout, and
// reads and writes only its own rows of the [j][i] states.

// One wave per key block of 16 columns (256 threads at N = 64, 128 at N = 32).
template <int N>
constexpr int kP2Threads = 4 * N;
// Workgroups per launch: two per compute unit at N = 64, four at N = 32 (each
// looping over blocks).
template <int N>
constexpr int kP2Grid = N == 32 ? 1024 : 512;

// Rows of a chunk staged in LDS: the six token inputs the gradients need,
// then dX and Z; and the entry state and exit adjoint of both chunks as [j][i].
enum { P2_R = 0, P2_W = 1, P2_K = 2, P2_A = 3, P2_B = 4, P2_DY = 5, P2_V = 6, P2_DX = 7, P2_Z = 8 };
// The chunk's four L x L adjoints dAab, dAak, dArb, dArk (tile p from wave
// p mod N/16), bf16 in row layout; 20-element rows keep both the row reads and
// the transposed reads of a tile nearly free of bank conflicts.
constexpr int kTileRow = 20;
template <int N>
struct __align__(16) P2Smem {
    static constexpr int kRow = kRowOf<N>;
    bf16_t rows[2][9][kL][kRow];
    bf16_t st[2][2][N][kRow];    // [S0 | dS][chunk of the pair][j][i]
    bf16_t adj[4][kL][kTileRow];
};

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_v;

// Lane (g, l16) of wave p: key column col = 16p + l16, tokens 4g .. 4g+3.
struct KeyFactors {
    float R[5][4];                 // r, w, k, a, b
    float Gt[4], Gp[4], inv[4], GL;
    bf16x4 atI, rtI, bhI, khI, bbI, kbI;   // bf16 operand values of the forward
};

// The values that lanes (0, l16) .. (3, l16) of this wave hold (rows of 16
// lanes), in every lane: one 32-lane and two 16-lane swaps (v_permlane32_swap
// gives rows (0, 1, 0, 1) and (2, 3, 2, 3); v_permlane16_swap of each with
// itself spreads its even and its odd row).
__device__ __forceinline__ void rows_of(float x, float& x0, float& x1, float& x2, float& x3) {
    const unsigned u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const auto b = __builtin_amdgcn_permlane16_swap(a[0], a[0], false, false);
    const auto c = __builtin_amdgcn_permlane16_swap(a[1], a[1], false, false);
    x0 = __uint_as_float(b[0]);
    x1 = __uint_as_float(b[1]);
    x2 = __uint_as_float(c[0]);
    x3 = __uint_as_float(c[1]);
}

// kAB = false: a = b = 0; a, b and the removal read-outs Z are not read (they
// stand as zero rows) and da, db are not written.
template <int N, bool kAB>
__global__ __launch_bounds__(kP2Threads<N>) void bwd_keys_kernel(
    int T, int H, int nch, int nblk, int nblocks, const bf16_t* __restrict__ r,
    const bf16_t* __restrict__ w, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ a, const bf16_t* __restrict__ b, const bf16_t* __restrict__ dy,
    const bf16_t* __restrict__ tapeZ, const bf16_t* __restrict__ tapeS,
    const bf16_t* __restrict__ wdX, const bf16_t* __restrict__ wdS, bf16_t* __restrict__ dr,
    bf16_t* __restrict__ dw, bf16_t* __restrict__ dk, bf16_t* __restrict__ da,
    bf16_t* __restrict__ db, int* __restrict__ counter) {
    // (these hide the file-scope N = 64 constants in the body below)
    constexpr int kN = N, kRow = kRowOf<N>;
    constexpr int kP = N / 16;                  // waves: one per key block
    constexpr int K2 = N / 32, JT = N / 16;     // 32-deep halves, 16-wide blocks
    constexpr int SP = N / 32;                  // 16-byte pieces of a state per thread
    __shared__ P2Smem<N> sm;
    __shared__ int next_block;
    const int tid = threadIdx.x;
    // The wave index as a scalar (so that per-wave choices are uniform).
    const int lane = tid & 63, wp = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g = lane >> 4;
    const int col = 16 * wp + l16;     // key column j of this lane

    // ---- loads of one block: both chunks' rows as whole rows (N/8 threads per
    // row, 16 bytes each; threads 0..2N-1: r, k, b, v, Z, 2N..4N-1: w, a, dy,
    // dX), the block's entry state and exit adjoint (N/32 16-byte pieces each).
    // Both chunks are loaded even when the block has one (the second is then all
    // padding and never used).  They are issued one block ahead into registers
    // and stashed in LDS when the block comes up, tokens past T as padding
    // (w = 1, everything else 0). ------------------------------------------------
    const int ld_row = (tid / (kN / 8)) & 15, ld_piece = tid & (kN / 8 - 1);
    const bool lo = wp < kP / 2;   // threads 0..2N-1 (a wave-uniform choice)
    // With a = b = 0 the slots of a, b and dX load r instead (every thread issues
    // the same loads) and are stashed as zeros.
    const bf16_t* const src4[4] = {lo ? r : w, lo ? k : (kAB ? a : r), lo ? (kAB ? b : r) : dy,
                                   lo ? v : (kAB ? wdX : r)};
    struct P2Raw {
        uint4 x[2][5], s[2 * SP];
    };
    auto load_block = [&](int bi, P2Raw& o) __attribute__((always_inline)) {
        const int m = bi % nblk, bh = bi / nblk;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int t = min((2 * m + h) * kL + ld_row, T - 1);
            const size_t off = tok_off<N>(bh / H, t, bh % H, T, H) + 8 * ld_piece;
#pragma unroll
            for (int vi = 0; vi < 4; ++vi) o.x[h][vi] = *reinterpret_cast<const uint4*>(src4[vi] + off);
            // (threads 2N.. load the same Z pieces as ..2N-1 and drop them, so
            // that every thread issues the same loads)
            o.x[h][4] = kAB ? *reinterpret_cast<const uint4*>(tapeZ + off) : make_uint4(0u, 0u, 0u, 0u);
        }
        const size_t sbase = (size_t)bi * kN * kN;
#pragma unroll
        for (int h2 = 0; h2 < SP; ++h2) {
            const int j = tid / (kN / 8) + 32 * h2;
            o.s[h2] = *reinterpret_cast<const uint4*>(tapeS + sbase + j * kN + 8 * ld_piece);
            o.s[SP + h2] = *reinterpret_cast<const uint4*>(wdS + sbase + j * kN + 8 * ld_piece);
        }
    };
    auto stash_block = [&](int bi, int nh, const P2Raw& o) __attribute__((always_inline)) {
        const int m = bi % nblk;
        const int set_lo[5] = {P2_R, P2_K, P2_B, P2_V, P2_Z};
        const int set_hi[4] = {P2_W, P2_A, P2_DY, P2_DX};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const bool ok = (2 * m + h) * kL + ld_row < T;
#pragma unroll
            for (int vi = 0; vi < 4; ++vi) {
                const unsigned pad = (!lo && vi == 0) ? 0x3F803F80u : 0u;
                // a = b = 0: a (vi 1, threads 2N..), b (vi 2, threads ..2N-1), dX (vi 3, 2N..)
                const bool zero = !kAB && (vi == 1 ? !lo : vi == 2 ? lo : vi == 3 ? !lo : false);
                *reinterpret_cast<uint4*>(&sm.rows[h][lo ? set_lo[vi] : set_hi[vi]][ld_row][8 * ld_piece]) =
                    (ok && !zero) ? o.x[h][vi] : make_uint4(pad, pad, pad, pad);
            }
            if (lo)
                *reinterpret_cast<uint4*>(&sm.rows[h][P2_Z][ld_row][8 * ld_piece]) =
                    ok ? o.x[h][4] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int h2 = 0; h2 < SP; ++h2) {
            const int j = tid / (kN / 8) + 32 * h2;
            *reinterpret_cast<uint4*>(&sm.st[0][0][j][8 * ld_piece]) = o.s[h2];
            *reinterpret_cast<uint4*>(&sm.st[1][nh - 1][j][8 * ld_piece]) = o.s[SP + h2];
        }
    };

    // Blocks come from a queue (counter[0]), so workgroups that start late (the
    // compute units may still be busy with other work) simply take fewer; the
    // loads of the next block are in flight while the current one is computed,
    // and so is the queue's answer for the block after it (popped one block
    // early: waiting for an atomic's return right away costs a round trip per
    // block).  Every memory access in the loop is unconditional -- loads of a
    // block past the end re-read the last one, stores out of range fall outside
    // their buffer resource -- so the wait before a stash covers exactly the
    // loads it needs and the queue's answer, not the previous block's stores.
    if (tid == 0) next_block = atomicAdd(&counter[0], 1);
    __syncthreads();
    // (block indices as scalars: everything addressed from them is uniform)
    int bi = __builtin_amdgcn_readfirstlane(next_block);
    int q_ans = 0;   // the queue's answer in flight (thread 0)
    if (tid == 0) q_ans = atomicAdd(&counter[0], 1);
    P2Raw nxt;
    if (bi < nblocks) {
        load_block(bi, nxt);
        // As many stores (into a resource of no bytes: dropped) as a block
        // issues after its loads, after them (the scheduler may not hoist them),
        // so that the loop is entered with the same pending memory operations as
        // from its own end and the wait before the stash need not drain the
        // counter.
        __builtin_amdgcn_sched_barrier(0);
        const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc(nullptr, (short)0, 0, 0x00020000);
        typedef unsigned int su4 __attribute__((ext_vector_type(4)));
        const su4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int q = 0; q < 6; ++q) __builtin_amdgcn_raw_buffer_store_b128(zero, none, 16 * tid + 4096 * q, 0, 2);
    }
    while (bi < nblocks) {
    const int m = bi % nblk;
    const int bh = bi / nblk;
    const int bb = bh / H, hh = bh % H;
    const int c0 = 2 * m;
    const int nh = c0 + 1 < nch ? 2 : 1;   // chunks in this block
    stash_block(bi, nh, nxt);
    if (tid == 0) next_block = q_ans;
    __syncthreads();
    const int bn = __builtin_amdgcn_readfirstlane(next_block);
    if (tid == 0) q_ans = atomicAdd(&counter[0], 1);
    load_block(min(bn, nblocks - 1), nxt);

    // ---- decay products and scaled vectors of column `col` in chunk h ----------
    auto factors = [&](int h) __attribute__((always_inline)) -> KeyFactors {
        KeyFactors f;
        // Tokens 4g .. 4g+3 of column col, one transposed read per vector.
#pragma unroll
        for (int vi = 0; vi < 5; ++vi) {
            const uint2 u = __builtin_bit_cast(uint2, ld4_tr(tr_addr(&sm.rows[h][vi][0][16 * wp], kRow, g, l16)));
            f.R[vi][0] = __uint_as_float(u.x << 16);
            f.R[vi][1] = __uint_as_float(u.x & 0xFFFF0000u);
            f.R[vi][2] = __uint_as_float(u.y << 16);
            f.R[vi][3] = __uint_as_float(u.y & 0xFFFF0000u);
        }
        float gp[4];
        float run = 1.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            run *= f.R[P2_W][q];
            gp[q] = run;
        }
        float g0, g1, g2, g3;
        rows_of(run, g0, g1, g2, g3);
        const float before = ((g >= 1 ? g0 : 1.f) * (g >= 2 ? g1 : 1.f)) * (g >= 3 ? g2 : 1.f);
        f.GL = ((g0 * g1) * g2) * g3;
        float at[4], rt[4], bh_[4], kh_[4], bbar[4], kbar[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f.Gt[q] = before * gp[q];
            f.Gp[q] = q == 0 ? before : before * gp[q - 1];
            f.inv[q] = __builtin_amdgcn_rcpf(f.Gt[q]);
            at[q] = f.R[P2_A][q] * f.Gp[q];
            rt[q] = f.R[P2_R][q] * f.Gt[q];
            bh_[q] = f.R[P2_B][q] * f.inv[q];
            kh_[q] = f.R[P2_K][q] * f.inv[q];
            bbar[q] = bh_[q] * f.GL;
            kbar[q] = kh_[q] * f.GL;
        }
        // bf16 images: the forward's MFMA operand values, and the B operands (key
        // s = 4g+q, column col) of the products below.
        f.atI = cvt4(at[0], at[1], at[2], at[3]);
        f.rtI = cvt4(rt[0], rt[1], rt[2], rt[3]);
        f.bhI = cvt4(bh_[0], bh_[1], bh_[2], bh_[3]);
        f.khI = cvt4(kh_[0], kh_[1], kh_[2], kh_[3]);
        f.bbI = cvt4(bbar[0], bbar[1], bbar[2], bbar[3]);
        f.kbI = cvt4(kbar[0], kbar[1], kbar[2], kbar[3]);
        return f;
    };
    const bf16x4 ident = identity_b(g, l16);

    // ---- across the middle of the block: S0(c1) and dS(c0), rows `col` ---------
    if (nh == 2) {
        const KeyFactors f0 = factors(0), f1 = factors(1);
#pragma unroll
        for (int vb = 0; vb < JT; ++vb) {
            const int i0 = 16 * vb + 4 * g;
            // [t][i] tiles of value block vb in accumulator layout (lane holds
            // [4g+q][l16]); fed as A operands they stand for their transposes.
            const bf16x4 Vt = ld4_tr(tr_addr(&sm.rows[0][P2_V][0][16 * vb], kRow, g, l16));
            const bf16x4 dYt = ld4_tr(tr_addr(&sm.rows[1][P2_DY][0][16 * vb], kRow, g, l16));
            bf16x4 Zt = {}, dXt = {};
            if (kAB) {
                Zt = ld4_tr(tr_addr(&sm.rows[0][P2_Z][0][16 * vb], kRow, g, l16));
                dXt = ld4_tr(tr_addr(&sm.rows[1][P2_DX][0][16 * vb], kRow, g, l16));
            }
            const bf16x4 s0 = ld4(&sm.st[0][0][col][i0]);
            const bf16x4 ds1 = ld4(&sm.st[1][1][col][i0]);
            f32x4 sacc, dacc;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                sacc[q] = f0.GL * (float)s0[q];
                dacc[q] = f1.GL * (float)ds1[q];
            }
            sacc = mfma16(Vt, f0.kbI, sacc);                // + V^T Kb  ([i][j])
            if (kAB) sacc = mfma16(Zt, f0.bbI, sacc);       // + Z^T Bb
            dacc = mfma16(dYt, f1.rtI, dacc);               // + dY^T Rt
            if (kAB) dacc = mfma16(dXt, f1.atI, dacc);      // + dX^T At
            *reinterpret_cast<bf16x4*>(&sm.st[0][1][col][i0]) = cvt4(sacc);
            *reinterpret_cast<bf16x4*>(&sm.st[1][0][col][i0]) = cvt4(dacc);
        }
    }

    // Both chunks always (a block with one has an all-padding second chunk whose
    // stores fall out of range), unrolled: a fixed count of stores per block.
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int t0 = (c0 + h) * kL;
        const KeyFactors f = factors(h);
        // ---- the chunk's rows (row l16, 8 values at 32 k2 + 8 g) and column
        // `col` of S0 and dS ----------------------------------------------------------
        bf16x8 dXr[K2], Zr[K2], dYr[K2], Vr[K2], S0c[K2], dSc[K2];
#pragma unroll
        for (int k2 = 0; k2 < K2; ++k2) {
            const int i0 = 32 * k2 + 8 * g;
            if (kAB) {
                dXr[k2] = ld8(&sm.rows[h][P2_DX][l16][i0]);
                Zr[k2] = ld8(&sm.rows[h][P2_Z][l16][i0]);
            }
            dYr[k2] = ld8(&sm.rows[h][P2_DY][l16][i0]);
            Vr[k2] = ld8(&sm.rows[h][P2_V][l16][i0]);
            S0c[k2] = ld8(&sm.st[0][h][col][i0]);
            dSc[k2] = ld8(&sm.st[1][h][col][i0]);
        }

        // ---- the L x L adjoints: wave p forms tiles p, p + N/16, .. (one each at
        // N = 64, two at N = 32) of dAab = tril_-1(dX Z^T), dAak = tril_-1(dX V^T),
        // dArb = tril_0(dY Z^T), dArk = tril_0(dY V^T) ([t][s], contracted over
        // the value rows) and leaves them in row layout for the others -----------------
        // (a = b = 0: dX = Z = 0, so only dArk, tile 3, is formed.)
#pragma unroll
        for (int i = 0; i < 4 / kP; ++i) {
          const int tp = wp + kP * i;
          if (kAB || tp == 3) {
            const bool dyrow = (tp & 2) != 0, vcol = (tp & 1) != 0;
            f32x4 At_s = zero4();
#pragma unroll
            for (int k2 = 0; k2 < K2; ++k2)
                At_s = mfma32(dyrow ? dYr[k2] : dXr[k2], vcol ? Vr[k2] : Zr[k2], At_s);
            // bf16 bits of the four values, taken from the packed words with
            // integer shifts (a bit_cast of a single element of a bf16 vector
            // compiled to the low half of the first word for every element).
            const unsigned w01 = cvt2(At_s[0], At_s[1]), w23 = cvt2(At_s[2], At_s[3]);
            const unsigned bits[4] = {w01 & 0xFFFFu, w01 >> 16, w23 & 0xFFFFu, w23 >> 16};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int t = 4 * g + q, s_ = l16;   // accumulator layout: [t][s] = [4g+q][l16]
                const bool keep = dyrow ? s_ <= t : s_ < t;
                sm.adj[tp][t][s_] = (bf16_t)(keep ? bits[q] : 0u);
            }
          }
        }
        // ---- the contractions over value rows that involve this wave's columns ------
        f32x4 dAt = zero4(), dRt = zero4(), dBb = zero4(), dKb = zero4();
#pragma unroll
        for (int k2 = 0; k2 < K2; ++k2) {
            if (kAB) dAt = mfma32(dXr[k2], S0c[k2], dAt);     // dX S0
            dRt = mfma32(dYr[k2], S0c[k2], dRt);              // dY S0
            if (kAB) dBb = mfma32(Zr[k2], dSc[k2], dBb);      // Z dS
            dKb = mfma32(Vr[k2], dSc[k2], dKb);               // V dS
        }
        __syncthreads();   // the four adjoint tiles are in LDS
        // A tile read by rows is its A operand; read transposed, that of its
        // transpose.  The 16-deep partial sums join the 32-deep ones on the
        // vector ALU (add4).
        const bf16x4 Ark = ld4(&sm.adj[3][l16][4 * g]), ArkT = ld4_tr(tr_addr(&sm.adj[3][0][0], kTileRow, g, l16));
        f32x4 dBh = zero4(), dKh = zero4();
        if (kAB) {
            const bf16x4 Aab = ld4(&sm.adj[0][l16][4 * g]), AabT = ld4_tr(tr_addr(&sm.adj[0][0][0], kTileRow, g, l16));
            const bf16x4 Aak = ld4(&sm.adj[1][l16][4 * g]), AakT = ld4_tr(tr_addr(&sm.adj[1][0][0], kTileRow, g, l16));
            const bf16x4 Arb = ld4(&sm.adj[2][l16][4 * g]), ArbT = ld4_tr(tr_addr(&sm.adj[2][0][0], kTileRow, g, l16));
            dAt = add4(dAt, mfma16(Aak, f.khI, mfma16(Aab, f.bhI, zero4())));    // + dAab Bh + dAak Kh
            dRt = add4(dRt, mfma16(Ark, f.khI, mfma16(Arb, f.bhI, zero4())));    // + dArb Bh + dArk Kh
            dBh = mfma16(AabT, f.atI, zero4());                                   // dAab^T At
            dBh = mfma16(ArbT, f.rtI, dBh);                                       // + dArb^T Rt
            dKh = mfma16(AakT, f.atI, zero4());                                   // dAak^T At
        } else {
            dRt = add4(dRt, mfma16(Ark, f.khI, zero4()));                         // + dArk Kh
        }
        dKh = mfma16(ArkT, f.rtI, dKh);                                           // + dArk^T Rt

        // ---- sum_i dS[i][col] S0[i][col] over this lane's 16 value rows -----------
        float cs = 0.f;
#pragma unroll
        for (int k2 = 0; k2 < K2; ++k2) {
            const bf16x2_v* ds2 = reinterpret_cast<const bf16x2_v*>(&dSc[k2]);
            const bf16x2_v* s02 = reinterpret_cast<const bf16x2_v*>(&S0c[k2]);
#pragma unroll
            for (int q = 0; q < 4; ++q) cs = __builtin_amdgcn_fdot2_f32_bf16(ds2[q], s02[q], cs, false);
        }

        // ---- chain rule through the decay products (tokens t = 4g+q) --------------
        // d log w_u = sum_{t>=u} (dRt Rt - dBh Bh - dKh Kh)_t + sum_{t>=u+1} (dAt At)_t
        //           + sum_{t<u} (dBb Bb + dKb Kb)_t + G_L sum_i dS[i][j] S0[i][j];
        // the products use the bf16 operand values so that pair terms that cancel
        // exactly in the chunk algebra cancel to fp32 rounding.
        float base[4], e[4], bk[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            e[q] = kAB ? dAt[q] * (float)f.atI[q] : 0.f;
            bk[q] = kAB ? dBb[q] * (float)f.bbI[q] + dKb[q] * (float)f.kbI[q] : dKb[q] * (float)f.kbI[q];
            base[q] = kAB ? dRt[q] * (float)f.rtI[q] - dBh[q] * (float)f.bhI[q] - dKh[q] * (float)f.khI[q]
                          : dRt[q] * (float)f.rtI[q] - dKh[q] * (float)f.khI[q];
        }
        const float sum_base = base[0] + base[1] + base[2] + base[3];
        const float sum_e = e[0] + e[1] + e[2] + e[3];
        const float sum_bk = bk[0] + bk[1] + bk[2] + bk[3];
        float bs[4], es[4], ks[4], cg[4];
        rows_of(sum_base, bs[0], bs[1], bs[2], bs[3]);
        rows_of(sum_e, es[0], es[1], es[2], es[3]);
        rows_of(sum_bk, ks[0], ks[1], ks[2], ks[3]);
        rows_of(cs, cg[0], cg[1], cg[2], cg[3]);
        float base_after = 0.f, e_after = 0.f, bk_before = 0.f;
        const float cs_all = ((cg[0] + cg[1]) + cg[2]) + cg[3];
#pragma unroll
        for (int g2 = 0; g2 < 4; ++g2) {
            if (g2 > g) {
                base_after += bs[g2];
                e_after += es[g2];
            }
            if (g2 < g) bk_before += ks[g2];
        }
        const float csL = cs_all * f.GL;
        float pbk[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            pbk[q] = bk_before;
            bk_before += bk[q];
        }
        float dlw[4];
        {
            float sb = base_after, se = e_after;
#pragma unroll
            for (int q = 3; q >= 0; --q) {
                sb += base[q];
                dlw[q] = (sb + se) + (pbk[q] + csL);
                se += e[q];
            }
        }

        // ---- outputs: accumulator tiles [t][col] -> row layout (swap_layout) -> LDS
        // rows (over this chunk's r, w, k, a, b) -> whole-row stores -------------------
        f32x4 o_da, o_dr, o_db, o_dk, o_dw;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            o_da[q] = dAt[q] * f.Gp[q];
            o_dr[q] = dRt[q] * f.Gt[q];
            o_db[q] = (dBh[q] + dBb[q] * f.GL) * f.inv[q];
            o_dk[q] = (dKh[q] + dKb[q] * f.GL) * f.inv[q];
            o_dw[q] = dlw[q] * __builtin_amdgcn_rcpf(f.R[P2_W][q]);
        }
        __syncthreads();   // every wave is done reading this chunk's staged rows
        const int j0 = 16 * wp + 4 * g;
        *reinterpret_cast<bf16x4*>(&sm.rows[h][0][l16][j0]) = swap_layout(cvt4(o_dr), ident);
        *reinterpret_cast<bf16x4*>(&sm.rows[h][1][l16][j0]) = swap_layout(cvt4(o_dw), ident);
        *reinterpret_cast<bf16x4*>(&sm.rows[h][2][l16][j0]) = swap_layout(cvt4(o_dk), ident);
        *reinterpret_cast<bf16x4*>(&sm.rows[h][3][l16][j0]) = swap_layout(cvt4(o_da), ident);
        *reinterpret_cast<bf16x4*>(&sm.rows[h][4][l16][j0]) = swap_layout(cvt4(o_db), ident);
        __syncthreads();
        {
            // Three 16-byte stores per thread: the first half of the waves write
            // dr, dk, db and the second dw, da (and nothing), each through a
            // resource holding this chunk's rows of the head.
            const int row = (tid / (kN / 8)) & 15, piece = tid & (kN / 8 - 1);
            const bool lo_w = wp < kP / 2;
            // (a scalar: the clamp would otherwise land in a vector register, and
            // a resource built from one needs a loop over its distinct values)
            const int rows_in = __builtin_amdgcn_readfirstlane(max(0, min(kL, T - t0)));
            const size_t base = tok_off<N>(bb, t0, hh, T, H);
            const int voff = row * (H * kN * 2) + 16 * piece;
            typedef unsigned int su4 __attribute__((ext_vector_type(4)));
            // dst: never null (a stand-in where the output is absent); `on`: a
            // scalar condition, off = a resource of no bytes
            auto put = [&](bf16_t* dst, bool on, int set) __attribute__((always_inline)) {
                const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                    dst + base, (short)0, on ? rows_in * (H * kN * 2) : 0, 0x00020000);
                __builtin_amdgcn_raw_buffer_store_b128(
                    __builtin_bit_cast(su4, *reinterpret_cast<const uint4*>(&sm.rows[h][set][row][8 * piece])),
                    rs, voff, 0, 2);   // non-temporal
            };
            put(lo_w ? dr : dw, true, lo_w ? 0 : 1);
            put(lo_w ? dk : (kAB ? da : dk), lo_w || kAB, lo_w ? 2 : 3);
            put(kAB ? db : dr, lo_w && kAB, 4);
        }
    }
    __syncthreads();   // the output rows are read before the next stash overwrites them
    bi = bn;
    }
    // The last workgroup out empties the queue for the next launch.
    if (tid == 0 && atomicAdd(&counter[1], 1) == (int)gridDim.x - 1) {
        counter[0] = 0;
        counter[1] = 0;
    }
}

}  // namespace

namespace {

template <int N>
hipError_t launch_bwd_n(const BwdArgs& p, int stages, hipStream_t stream) {
    const bf16_t* r = static_cast<const bf16_t*>(p.r);
    const bf16_t* w = static_cast<const bf16_t*>(p.w);
    const bf16_t* k = static_cast<const bf16_t*>(p.k);
    const bf16_t* v = static_cast<const bf16_t*>(p.v);
    const bf16_t* a = static_cast<const bf16_t*>(p.a);
    const bf16_t* b = static_cast<const bf16_t*>(p.b);
    const bf16_t* dy = static_cast<const bf16_t*>(p.dy);
    if (stages & BWD_CHAIN) {
        auto chain = a ? bwd_chain_kernel<N, true> : bwd_chain_kernel<N, false>;
        const int nbh = p.B * p.H;
        auto run = [&](int pass, int grid) {
            chain<<<dim3(grid), dim3(kP1Threads<N>), 0, stream>>>(
                p.T, p.H, r, w, k, a, b, dy, p.dsT, static_cast<bf16_t*>(p.dv), p.ds0,
                static_cast<bf16_t*>(p.workX), static_cast<bf16_t*>(p.workS), p.counter, pass,
                p.nseg, p.seg_len / kL, p.states);
            return hipGetLastError();
        };
        if (p.nseg <= 1) {
            const hipError_t e = run(0, nbh);
            if (e != hipSuccess) return e;
        } else {
            hipError_t e = run(0, nbh * (2 * p.nseg - 3));
            if (e == hipSuccess && p.nseg > 2)
                e = N == 64 ? launch_seg_combine(nbh, p.nseg, p.states, stream)
                            : launch_seg_combine_n(N, nbh, p.nseg, p.states, stream);
            if (e == hipSuccess) e = run(1, nbh * (p.nseg - 1));
            if (e != hipSuccess) return e;
        }
    }
    if (!(stages & BWD_KEYS)) return hipSuccess;
    const int nch = (p.T + kL - 1) / kL;
    const int nblk = (nch + 1) / 2;
    const int nblocks = p.B * p.H * nblk;
    const int grid = nblocks < kP2Grid<N> ? nblocks : kP2Grid<N>;
    auto keys = a ? bwd_keys_kernel<N, true> : bwd_keys_kernel<N, false>;
    keys<<<dim3(grid), dim3(kP2Threads<N>), 0, stream>>>(
        p.T, p.H, nch, nblk, nblocks, r, w, k, v, a, b, dy, static_cast<const bf16_t*>(p.tapeZ),
        static_cast<const bf16_t*>(p.tapeS), static_cast<const bf16_t*>(p.workX),
        static_cast<const bf16_t*>(p.workS), static_cast<bf16_t*>(p.dr), static_cast<bf16_t*>(p.dw),
        static_cast<bf16_t*>(p.dk), static_cast<bf16_t*>(p.da), static_cast<bf16_t*>(p.db), p.counter);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& p, int chunk_len, int stages, hipStream_t stream) {
    if (chunk_len != kL || !p.bf16) return hipErrorInvalidValue;
    if (p.nseg > 1 && (p.seg_len <= 0 || p.seg_len % WKV7_TAPE_BLOCK != 0 || !p.states ||
                       (long long)(p.nseg - 1) * p.seg_len >= p.T ||
                       (long long)p.B * p.H * (2 * p.nseg - 3) > INT32_MAX))
        return hipErrorInvalidValue;
    switch (p.N) {
        case 32: return launch_bwd_n<32>(p, stages, stream);
        case 64: return launch_bwd_n<64>(p, stages, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace wkv7
