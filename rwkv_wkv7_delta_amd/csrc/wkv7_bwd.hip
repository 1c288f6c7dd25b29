// wkv7_bwd.hip -- chunked WKV7 backward (adjoint) on bf16 MFMA, gfx950.
//
// Gradient of L = sum_t <dy_t, y_t> + <dsT, S_T> through the chunk form of
// the recurrence (the forward's rearrangement, see wkv7_chunk_fwd.hip),
// visiting chunks of L = 16 tokens last to first and carrying the fp32
// adjoint dS of each chunk's exit state.  Per chunk, with entry state S0,
// Z the removal read-outs and dY the read-out adjoint:
//
//   dZ  = Arb^T dY + Bb dS^T            dX = Tm^T dZ
//   dV  = Aak^T dX + Ark^T dY + Kb dS^T
//   dAab = tril_-1(dX Z^T)  dAak = tril_-1(dX V^T)
//   dArb = tril_0(dY Z^T)   dArk = tril_0(dY V^T)
//   dAt = dX S0 + dAab Bh + dAak Kh     dRt = dY S0 + dArb Bh + dArk Kh
//   dBh = dAab^T At + dArb^T Rt         dKh = dAak^T At + dArk^T Rt
//   dBb = Z dS                          dKb = V dS
//   dS0 = dS diag(G_L) + dY^T Rt + dX^T At     (carried to the previous chunk)
// followed by the chain rule through the decay products: for each token,
// da = dAt G_{t-1}, dr = dRt G_t, db = dBh / G_t + dBb G_L / G_t,
// dk = dKh / G_t + dKb G_L / G_t, and d log G_t collects every factor that
// G_t enters; d log w_u = sum_{t >= u} d log G_t, dw = d log w / w.
//
// Entry states come from the forward's checkpoints (one every 64 tokens):
// for each 64-token block the kernel first re-runs the forward state chain
// over the block's chunks, keeping every chunk's entry state and removal
// read-outs Z in LDS (bf16), then walks the block's chunks backwards.
//
// Mapping: one workgroup of 4 waves per (b, h).  Wave w owns value rows
// 16w..16w+15 for the state-shaped work (dS^T is held in four 16x16 fp32
// accumulator tiles, exactly like the forward's state) and key columns
// 16w..16w+15 for the per-key gradients; contractions over value rows read
// the chunk's shared bf16 copies of S0, dS, Z and dX from LDS.

#include "wkv7_device.h"
#include "wkv7_internal.h"
#include "wkv7_mfma.h"

namespace wkv7 {

namespace {

constexpr int kL = 16;
constexpr int kThreads = 256;
constexpr int kChunksPerBlock = kCkptInterval / kL;   // 4
// LDS row strides (bf16 elements): 144-byte and 40-byte rows keep the MFMA
// operand reads (16 lanes on 16 different rows) off a single bank set.
constexpr int kRow = kN + 8;
constexpr int kRowT = kL + 4;

enum { RAW_R = 0, RAW_W = 1, RAW_K = 2, RAW_A = 3, RAW_B = 4, RAW_V = 5, RAW_DY = 6 };
enum { GS_DR = 0, GS_DW = 1, GS_DK = 2, GS_DV = 3, GS_DA = 4, GS_DB = 5 };

struct __align__(16) BwdSmem {
    bf16_t raw[7][kL][kRow];                   // r, w, k, a, b, v, dy (bf16 bits)
    float G[kL + 1][kN];                     // running decay products, G[0] = 1
    float gtot[4][kN];
    bf16_t At[kL][kRow], Rt[kL][kRow], Bh[kL][kRow], Kh[kL][kRow], Bb[kL][kRow], Kb[kL][kRow];
    bf16_t AtT[kN][kRowT], RtT[kN][kRowT], BhT[kN][kRowT], KhT[kN][kRowT], BbT[kN][kRowT],
        KbT[kN][kRowT];
    float Amat[4][kL][kL];                   // Aab, Aak, Arb, Ark
    float Tm[kL][kL];                        // (I - Aab)^-1
    bf16_t Wm[kL][kRow];                       // Tm At
    bf16_t Sblk[kChunksPerBlock][kN][kRow];    // entry states of the block's chunks, [j][i]
    bf16_t Zblk[kChunksPerBlock][kL][kRow];    // removal read-outs Z of the block's chunks, [t][i]
    bf16_t dXs[kL][kRow];                      // [t][i]
    bf16_t dSs[kN][kRow];                      // adjoint of the chunk's exit state, [j][i]
    float dAm[4][kL][kL];                    // dAab, dAak, dArb, dArk
    float colsum[4][kN];                     // per-wave partial sum_i dS[i][j] S0[i][j]
    float red[4][3][4][16];                  // per-wave scratch for token sums
    bf16_t gst[6][kL][kRow];                   // gradient staging for coalesced stores
};

__device__ __forceinline__ float bf2f(bf16_t x) { return __uint_as_float((uint32_t)x << 16); }
__device__ __forceinline__ bf16x4 ld4(const bf16_t* p) {
    return __builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2*>(p));
}
__device__ __forceinline__ bf16x8 ld8(const bf16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}
// 32-deep operand built from two 4-wide pieces at p and p + 16 (see wkv7_mfma.h).
__device__ __forceinline__ bf16x8 ld4x2(const bf16_t* p) { return cat8(ld4(p), ld4(p + 16)); }
__device__ __forceinline__ bf16x4 f4(const float* p0, int stride) {
    return cvt4(p0[0], p0[stride], p0[2 * stride], p0[3 * stride]);
}
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct Ctx {
    int T, H, bb, hh, tid, wv, lane, l16, g, irow;
    const bf16_t *r, *w, *k, *a, *b, *v, *dy;
};

// Raw loads of one chunk (nvec = 6 without dy, 7 with): 128 x 16 B per vector.
struct Prefetch {
    uint4 v[4];
};

__device__ __forceinline__ void load_raw(const Ctx& c, int t0, int nvec, Prefetch& pf) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int item = c.tid + p * kThreads;
        const int q = item >> 7, t = (item >> 3) & 15, c8 = item & 7;
        if (q >= nvec) continue;
        // vector q = 2p + (tid >= 128): r/w, k/a, b/v, dy
        const bool hi = c.tid >= 128;
        const bf16_t* sp = p == 0 ? (hi ? c.w : c.r) : p == 1 ? (hi ? c.a : c.k)
                         : p == 2 ? (hi ? c.v : c.b) : c.dy;
        if (t0 + t < c.T) {
            pf.v[p] = *reinterpret_cast<const uint4*>(sp + tok_off(c.bb, t0 + t, c.hh, c.T, c.H) + c8 * 8);
        } else {
            const uint32_t pad = (q == RAW_W) ? 0x3F803F80u : 0u;   // padding token: w = 1
            pf.v[p] = make_uint4(pad, pad, pad, pad);
        }
    }
}

__device__ __forceinline__ void stash_raw(const Ctx& c, BwdSmem& sm, int nvec, const Prefetch& pf) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int item = c.tid + p * kThreads;
        const int q = item >> 7, t = (item >> 3) & 15, c8 = item & 7;
        if (q < nvec) *reinterpret_cast<uint4*>(&sm.raw[q][t][c8 * 8]) = pf.v[p];
    }
}

// State-independent factors of the chunk whose raw inputs are in sm.raw.
// Ends with a barrier; Wm only when need_w.
__device__ void prep_chunk(const Ctx& c, BwdSmem& sm, bool need_w) {
    const int ej = c.tid & 63, eg = c.tid >> 6;
    float gp[4];
    {
        float run = 1.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            run *= bf2f(sm.raw[RAW_W][4 * eg + u][ej]);
            gp[u] = run;
        }
        sm.gtot[eg][ej] = run;
    }
    __syncthreads();
    {
        const float g0 = sm.gtot[0][ej], g1 = sm.gtot[1][ej], g2 = sm.gtot[2][ej], g3 = sm.gtot[3][ej];
        const float before = eg == 0 ? 1.f : eg == 1 ? g0 : eg == 2 ? g0 * g1 : (g0 * g1) * g2;
        const float GL = ((g0 * g1) * g2) * g3;
        float at4[4], rt4[4], bh4[4], kh4[4], bb4[4], kb4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int t = 4 * eg + u;
            const float Gt = before * gp[u];
            const float Gprev = u == 0 ? before : before * gp[u - 1];
            const float inv = __builtin_amdgcn_rcpf(Gt);
            at4[u] = bf2f(sm.raw[RAW_A][t][ej]) * Gprev;
            rt4[u] = bf2f(sm.raw[RAW_R][t][ej]) * Gt;
            bh4[u] = bf2f(sm.raw[RAW_B][t][ej]) * inv;
            kh4[u] = bf2f(sm.raw[RAW_K][t][ej]) * inv;
            bb4[u] = bh4[u] * GL;
            kb4[u] = kh4[u] * GL;
            sm.G[t + 1][ej] = Gt;
            sm.At[t][ej] = f2bf(at4[u]);
            sm.Rt[t][ej] = f2bf(rt4[u]);
            sm.Bh[t][ej] = f2bf(bh4[u]);
            sm.Kh[t][ej] = f2bf(kh4[u]);
            sm.Bb[t][ej] = f2bf(bb4[u]);
            sm.Kb[t][ej] = f2bf(kb4[u]);
        }
        if (eg == 0) sm.G[0][ej] = 1.f;
        *reinterpret_cast<bf16x4*>(&sm.AtT[ej][4 * eg]) = cvt4(at4[0], at4[1], at4[2], at4[3]);
        *reinterpret_cast<bf16x4*>(&sm.RtT[ej][4 * eg]) = cvt4(rt4[0], rt4[1], rt4[2], rt4[3]);
        *reinterpret_cast<bf16x4*>(&sm.BhT[ej][4 * eg]) = cvt4(bh4[0], bh4[1], bh4[2], bh4[3]);
        *reinterpret_cast<bf16x4*>(&sm.KhT[ej][4 * eg]) = cvt4(kh4[0], kh4[1], kh4[2], kh4[3]);
        *reinterpret_cast<bf16x4*>(&sm.BbT[ej][4 * eg]) = cvt4(bb4[0], bb4[1], bb4[2], bb4[3]);
        *reinterpret_cast<bf16x4*>(&sm.KbT[ej][4 * eg]) = cvt4(kb4[0], kb4[1], kb4[2], kb4[3]);
    }
    __syncthreads();
    {
        // L x L products: wave 0 Aab (+ transpose, then Tm = (I - Aab)^-1),
        // 1 Aak, 2 Arb, 3 Ark.
        const bf16_t* lrow = (c.wv < 2) ? &sm.At[c.l16][0] : &sm.Rt[c.l16][0];
        const bf16_t* rrow = (c.wv & 1) ? &sm.Kh[c.l16][0] : &sm.Bh[c.l16][0];
        f32x4 acc = zero4(), accT = zero4();
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            const bf16x8 av = ld8(lrow + 32 * k2 + 8 * c.g), bv = ld8(rrow + 32 * k2 + 8 * c.g);
            acc = mfma32(av, bv, acc);
            if (c.wv == 0) accT = mfma32(bv, av, accT);
        }
        const bool strict = c.wv < 2;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int t = 4 * c.g + q, s = c.l16;
            acc[q] = (strict ? (s < t) : (s <= t)) ? acc[q] : 0.f;
            accT[q] = (t < s) ? accT[q] : 0.f;
            sm.Amat[c.wv][t][s] = acc[q];
        }
        if (c.wv == 0) {
            const f32x4 TT = unit_lower_inverse_T(acc, accT, c.g, c.l16);
#pragma unroll
            for (int q = 0; q < 4; ++q) sm.Tm[c.l16][4 * c.g + q] = TT[q];
        }
    }
    __syncthreads();
    if (need_w) {
        const int j = 16 * c.wv + c.l16;
        const bf16x4 Trow = f4(&sm.Tm[c.l16][4 * c.g], 1);
        const bf16x4 Acol = cvt4(bf2f(sm.At[4 * c.g][j]), bf2f(sm.At[4 * c.g + 1][j]),
                                 bf2f(sm.At[4 * c.g + 2][j]), bf2f(sm.At[4 * c.g + 3][j]));
        const f32x4 Wt = mfma16(Trow, Acol, zero4());
#pragma unroll
        for (int q = 0; q < 4; ++q) sm.Wm[4 * c.g + q][j] = f2bf(Wt[q]);
        __syncthreads();
    }
}

__global__ __launch_bounds__(kThreads) void chunk_bwd_kernel(
    int T, int H, const bf16_t* __restrict__ r, const bf16_t* __restrict__ w,
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, const bf16_t* __restrict__ a,
    const bf16_t* __restrict__ b, const bf16_t* __restrict__ dy, const float* __restrict__ dsT,
    const float* __restrict__ ckpt, bf16_t* __restrict__ dr, bf16_t* __restrict__ dw,
    bf16_t* __restrict__ dk, bf16_t* __restrict__ dv, bf16_t* __restrict__ da,
    bf16_t* __restrict__ db, float* __restrict__ ds0) {
    __shared__ BwdSmem sm;
    Ctx c;
    c.T = T;
    c.H = H;
    const int bh = blockIdx.x;
    c.bb = bh / H;
    c.hh = bh % H;
    c.tid = threadIdx.x;
    c.lane = c.tid & 63;
    c.wv = c.tid >> 6;
    c.l16 = c.lane & 15;
    c.g = c.lane >> 4;
    c.irow = 16 * c.wv + c.l16;
    c.r = r; c.w = w; c.k = k; c.a = a; c.b = b; c.v = v; c.dy = dy;
    const int l16 = c.l16, g = c.g, wv = c.wv, irow = c.irow;
    const int nck = (T + kCkptInterval - 1) / kCkptInterval;

    // Adjoint of the current exit state, held as dS^T tiles like the forward's S^T.
    f32x4 dSt[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
        if (dsT) {
            const float4 x = *reinterpret_cast<const float4*>(dsT + ((size_t)bh * kN + irow) * kN + 16 * jt + 4 * g);
            dSt[jt][0] = x.x; dSt[jt][1] = x.y; dSt[jt][2] = x.z; dSt[jt][3] = x.w;
        } else {
            dSt[jt] = zero4();
        }
    }

    // Visiting order: for each block (last first) its chunks forwards (state
    // re-run), then backwards (adjoint).  step -> (chunk start, needs dy).
    auto step_chunk = [&](int blk, int nc, int s, int& t0, bool& back) {
        back = s >= nc;
        const int ci = back ? (2 * nc - 1 - s) : s;
        t0 = blk * kCkptInterval + ci * kL;
    };

    Prefetch pf;
    {
        const int blk = nck - 1;
        const int nc = (T - blk * kCkptInterval + kL - 1) / kL;
        int t0; bool back;
        step_chunk(blk, nc, 0, t0, back);
        load_raw(c, t0, back ? 7 : 6, pf);
    }

    for (int blk = nck - 1; blk >= 0; --blk) {
        const int tb0 = blk * kCkptInterval;
        const int nc = min(kChunksPerBlock, (T - tb0 + kL - 1) / kL);

        // Entry state of the block.
        f32x4 S[4];
        {
            const float* src = ckpt + (((size_t)bh * nck + blk) * kN + irow) * kN;
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) {
                const float4 x = *reinterpret_cast<const float4*>(src + 16 * jt + 4 * g);
                S[jt][0] = x.x; S[jt][1] = x.y; S[jt][2] = x.z; S[jt][3] = x.w;
            }
        }

        for (int s = 0; s < 2 * nc; ++s) {
            int t0; bool back;
            step_chunk(blk, nc, s, t0, back);
            const int ci = (t0 - tb0) / kL;
            const int nvec = back ? 7 : 6;
            __syncthreads();                 // previous users of sm.raw are done
            stash_raw(c, sm, nvec, pf);
            {
                // Prefetch the next step's raw inputs.
                int nblk = blk, ns = s + 1, nnc = nc;
                if (ns >= 2 * nc) {
                    nblk = blk - 1;
                    ns = 0;
                    nnc = nblk >= 0 ? min(kChunksPerBlock, (T - nblk * kCkptInterval + kL - 1) / kL) : 0;
                }
                if (nblk >= 0) {
                    int nt0; bool nback;
                    step_chunk(nblk, nnc, ns, nt0, nback);
                    load_raw(c, nt0, nback ? 7 : 6, pf);
                }
            }
            __syncthreads();
            prep_chunk(c, sm, !back);

            if (!back) {
                // ---- forward re-run: Z = W S0^T + Tm Aak V, next entry state ----
                const bf16x4 Vb = cvt4(bf2f(sm.raw[RAW_V][4 * g][irow]), bf2f(sm.raw[RAW_V][4 * g + 1][irow]),
                                       bf2f(sm.raw[RAW_V][4 * g + 2][irow]), bf2f(sm.raw[RAW_V][4 * g + 3][irow]));
                const f32x4 AkV = mfma16(f4(&sm.Amat[1][l16][4 * g], 1), Vb, zero4());
                f32x4 Z = mfma16(f4(&sm.Tm[l16][4 * g], 1), cvt4(AkV), zero4());
                bf16x4 Sb[4];
#pragma unroll
                for (int jt = 0; jt < 4; ++jt) Sb[jt] = cvt4(S[jt]);
#pragma unroll
                for (int k2 = 0; k2 < 2; ++k2)
                    Z = mfma32(ld4x2(&sm.Wm[l16][32 * k2 + 4 * g]), cat8(Sb[2 * k2], Sb[2 * k2 + 1]), Z);
#pragma unroll
                for (int jt = 0; jt < 4; ++jt)
#pragma unroll
                    for (int q = 0; q < 4; ++q) sm.Sblk[ci][16 * jt + 4 * g + q][irow] = bits(Sb[jt][q]);
#pragma unroll
                for (int q = 0; q < 4; ++q) sm.Zblk[ci][4 * g + q][irow] = f2bf(Z[q]);
                if (ci + 1 < nc) {
                    const bf16x4 Zb = cvt4(Z);
#pragma unroll
                    for (int jt = 0; jt < 4; ++jt) {
                        f32x4 acc = mfma16(ld4(&sm.KbT[16 * jt + l16][4 * g]), Vb, zero4());
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            acc[q] = fmaf(sm.G[kL][16 * jt + 4 * g + q], S[jt][q], acc[q]);
                        S[jt] = mfma16(ld4(&sm.BbT[16 * jt + l16][4 * g]), Zb, acc);
                    }
                }
                continue;
            }

            // ---- backward step for chunk ci of this block ------------------------
            const bf16_t* Ss = &sm.Sblk[ci][0][0];
            const bf16_t* Zs = &sm.Zblk[ci][0][0];
            const bf16x4 dYb = cvt4(bf2f(sm.raw[RAW_DY][4 * g][irow]), bf2f(sm.raw[RAW_DY][4 * g + 1][irow]),
                                    bf2f(sm.raw[RAW_DY][4 * g + 2][irow]), bf2f(sm.raw[RAW_DY][4 * g + 3][irow]));
            const bf16x4 Vb = cvt4(bf2f(sm.raw[RAW_V][4 * g][irow]), bf2f(sm.raw[RAW_V][4 * g + 1][irow]),
                                   bf2f(sm.raw[RAW_V][4 * g + 2][irow]), bf2f(sm.raw[RAW_V][4 * g + 3][irow]));
            bf16x4 dSb[4];
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) dSb[jt] = cvt4(dSt[jt]);
            // dZ = Arb^T dY + Bb dS^T ;  dX = Tm^T dZ
            f32x4 dZ = mfma16(f4(&sm.Amat[2][4 * g][l16], kL), dYb, zero4());
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2)
                dZ = mfma32(ld4x2(&sm.Bb[l16][32 * k2 + 4 * g]), cat8(dSb[2 * k2], dSb[2 * k2 + 1]), dZ);
            const f32x4 dX = mfma16(f4(&sm.Tm[4 * g][l16], kL), cvt4(dZ), zero4());
            const bf16x4 dXb = cvt4(dX);
            // dV = Aak^T dX + Ark^T dY + Kb dS^T
            f32x4 dV = mfma16(f4(&sm.Amat[1][4 * g][l16], kL), dXb, zero4());
            dV = mfma16(f4(&sm.Amat[3][4 * g][l16], kL), dYb, dV);
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2)
                dV = mfma32(ld4x2(&sm.Kb[l16][32 * k2 + 4 * g]), cat8(dSb[2 * k2], dSb[2 * k2 + 1]), dV);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                sm.dXs[4 * g + q][irow] = bits(dXb[q]);
                sm.gst[GS_DV][4 * g + q][irow] = f2bf(dV[q]);
            }
            // Share the incoming dS (bf16) and the partial sum_i dS * S0.
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int j = 16 * jt + 4 * g + q;
                    sm.dSs[j][irow] = bits(dSb[jt][q]);
                    const float p = row16_sum(dSt[jt][q] * bf2f(Ss[j * kRow + irow]));
                    if (l16 == 0) sm.colsum[wv][j] = p;
                }
            }
            // dS0 = dS diag(G_L) + dY^T Rt + dX^T At   (as transposed tiles)
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) {
                f32x4 acc;
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[q] = sm.G[kL][16 * jt + 4 * g + q] * dSt[jt][q];
                acc = mfma16(ld4(&sm.RtT[16 * jt + l16][4 * g]), dYb, acc);
                dSt[jt] = mfma16(ld4(&sm.AtT[16 * jt + l16][4 * g]), dXb, acc);
            }
            __syncthreads();

            // ---- L x L adjoints: wave 0 dAab, 1 dAak, 2 dArb, 3 dArk ---------------
            {
                const bf16_t* lrow = (wv < 2) ? &sm.dXs[l16][0] : &sm.raw[RAW_DY][l16][0];
                const bf16_t* rrow = (wv & 1) ? &sm.raw[RAW_V][l16][0] : Zs + l16 * kRow;
                f32x4 acc = zero4();
#pragma unroll
                for (int k2 = 0; k2 < 2; ++k2)
                    acc = mfma32(ld8(lrow + 32 * k2 + 8 * g), ld8(rrow + 32 * k2 + 8 * g), acc);
                const bool strict = wv < 2;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int t = 4 * g + q, s2 = l16;
                    sm.dAm[wv][t][s2] = (strict ? (s2 < t) : (s2 <= t)) ? acc[q] : 0.f;
                }
            }
            __syncthreads();

            // ---- per-key adjoints for key columns j = 16 wv + l16 -----------------
            const int jcol = 16 * wv + l16;
            f32x4 dAt = zero4(), dRt = zero4(), dBh, dKh, dBb = zero4(), dKb = zero4();
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                const bf16x8 s0v = ld8(Ss + jcol * kRow + 32 * k2 + 8 * g);
                const bf16x8 dsv = ld8(&sm.dSs[jcol][32 * k2 + 8 * g]);
                dAt = mfma32(ld8(&sm.dXs[l16][32 * k2 + 8 * g]), s0v, dAt);
                dRt = mfma32(ld8(&sm.raw[RAW_DY][l16][32 * k2 + 8 * g]), s0v, dRt);
                dBb = mfma32(ld8(Zs + l16 * kRow + 32 * k2 + 8 * g), dsv, dBb);
                dKb = mfma32(ld8(&sm.raw[RAW_V][l16][32 * k2 + 8 * g]), dsv, dKb);
            }
            {
                const bf16x4 bhT = ld4(&sm.BhT[jcol][4 * g]);
                const bf16x4 khT = ld4(&sm.KhT[jcol][4 * g]);
                const bf16x4 atT = ld4(&sm.AtT[jcol][4 * g]);
                const bf16x4 rtT = ld4(&sm.RtT[jcol][4 * g]);
                dAt = mfma16(f4(&sm.dAm[0][l16][4 * g], 1), bhT, dAt);
                dAt = mfma16(f4(&sm.dAm[1][l16][4 * g], 1), khT, dAt);
                dRt = mfma16(f4(&sm.dAm[2][l16][4 * g], 1), bhT, dRt);
                dRt = mfma16(f4(&sm.dAm[3][l16][4 * g], 1), khT, dRt);
                dBh = mfma16(f4(&sm.dAm[0][4 * g][l16], kL), atT, zero4());
                dBh = mfma16(f4(&sm.dAm[2][4 * g][l16], kL), rtT, dBh);
                dKh = mfma16(f4(&sm.dAm[1][4 * g][l16], kL), atT, zero4());
                dKh = mfma16(f4(&sm.dAm[3][4 * g][l16], kL), rtT, dKh);
            }

            // ---- chain rule through the decay products, tokens t = 4g+q ----------
            // d log w_u = sum_{t>=u} (dRt Rt - dBh Bh - dKh Kh)_t + sum_{t>=u+1} (dAt At)_t
            //           + sum_{t<u} (dBb Bb + dKb Kb)_t + G_L sum_i dS[i][j] S0[i][j].
            // The products use the same bf16 values as the MFMA operands, so the
            // pair terms that cancel exactly (both ends of an L x L factor on
            // the same side of u) cancel to fp32 rounding.
            {
                const float GL = sm.G[kL][jcol];
                float base[4], e[4], bk[4];
                float dav[4], drv[4], dbv[4], dkv[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int t = 4 * g + q;
                    const float Gt = sm.G[t + 1][jcol], Gp = sm.G[t][jcol];
                    const float inv = __builtin_amdgcn_rcpf(Gt);
                    dav[q] = dAt[q] * Gp;
                    drv[q] = dRt[q] * Gt;
                    dbv[q] = (dBh[q] + dBb[q] * GL) * inv;
                    dkv[q] = (dKh[q] + dKb[q] * GL) * inv;
                    e[q] = dAt[q] * bf2f(sm.At[t][jcol]);
                    bk[q] = dBb[q] * bf2f(sm.Bb[t][jcol]) + dKb[q] * bf2f(sm.Kb[t][jcol]);
                    base[q] = dRt[q] * bf2f(sm.Rt[t][jcol]) - dBh[q] * bf2f(sm.Bh[t][jcol]) -
                              dKh[q] * bf2f(sm.Kh[t][jcol]);
                }
                // Token sums across the four lane groups (tokens 4g..4g+3) of this wave.
                float* red = &sm.red[wv][0][0][0];
                red[(0 * 4 + g) * 16 + l16] = base[0] + base[1] + base[2] + base[3];
                red[(1 * 4 + g) * 16 + l16] = e[0] + e[1] + e[2] + e[3];
                red[(2 * 4 + g) * 16 + l16] = bk[0] + bk[1] + bk[2] + bk[3];
                wave_sync();
                float base_after = 0.f, e_after = 0.f, bk_before = 0.f;
#pragma unroll
                for (int g2 = 0; g2 < 4; ++g2) {
                    const float bs = red[(0 * 4 + g2) * 16 + l16];
                    const float es = red[(1 * 4 + g2) * 16 + l16];
                    const float ks = red[(2 * 4 + g2) * 16 + l16];
                    if (g2 > g) {
                        base_after += bs;
                        e_after += es;
                    }
                    if (g2 < g) bk_before += ks;
                }
                const float cs = (sm.colsum[0][jcol] + sm.colsum[1][jcol] + sm.colsum[2][jcol] +
                                  sm.colsum[3][jcol]) * GL;
                float pbk[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    pbk[q] = bk_before;
                    bk_before += bk[q];
                }
                float sb = base_after, se = e_after;
#pragma unroll
                for (int q = 3; q >= 0; --q) {
                    const int t = 4 * g + q;
                    sb += base[q];
                    const float dlw = (sb + se) + (pbk[q] + cs);
                    se += e[q];
                    const float wt = bf2f(sm.raw[RAW_W][t][jcol]);
                    sm.gst[GS_DW][t][jcol] = f2bf(dlw / wt);
                    sm.gst[GS_DA][t][jcol] = f2bf(dav[q]);
                    sm.gst[GS_DR][t][jcol] = f2bf(drv[q]);
                    sm.gst[GS_DB][t][jcol] = f2bf(dbv[q]);
                    sm.gst[GS_DK][t][jcol] = f2bf(dkv[q]);
                }
            }
            __syncthreads();
            // ---- coalesced gradient stores: 6 x 16 tokens x 128 B -----------------
#pragma unroll
            for (int p = 0; p < 3; ++p) {
                const int item = c.tid + p * kThreads;
                const int q = item >> 7, t = (item >> 3) & 15, c8 = item & 7;
                const bool hi = c.tid >= 128;   // q = 2p + hi: dr/dw, dk/dv, da/db
                bf16_t* gp = p == 0 ? (hi ? dw : dr) : p == 1 ? (hi ? dv : dk) : (hi ? db : da);
                if (t0 + t < T)
                    *reinterpret_cast<uint4*>(gp + tok_off(c.bb, t0 + t, c.hh, T, H) + c8 * 8) =
                        *reinterpret_cast<const uint4*>(&sm.gst[q][t][c8 * 8]);
            }
        }
    }

    if (ds0) {
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
            *reinterpret_cast<float4*>(ds0 + ((size_t)bh * kN + irow) * kN + 16 * jt + 4 * g) =
                make_float4(dSt[jt][0], dSt[jt][1], dSt[jt][2], dSt[jt][3]);
    }
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& p, int chunk_len, hipStream_t stream) {
    if (chunk_len != kL || !p.bf16) return hipErrorInvalidValue;
    chunk_bwd_kernel<<<dim3(p.B * p.H), dim3(kThreads), 0, stream>>>(
        p.T, p.H, static_cast<const bf16_t*>(p.r), static_cast<const bf16_t*>(p.w),
        static_cast<const bf16_t*>(p.k), static_cast<const bf16_t*>(p.v),
        static_cast<const bf16_t*>(p.a), static_cast<const bf16_t*>(p.b),
        static_cast<const bf16_t*>(p.dy), p.dsT, p.ckpt, static_cast<bf16_t*>(p.dr),
        static_cast<bf16_t*>(p.dw), static_cast<bf16_t*>(p.dk), static_cast<bf16_t*>(p.dv),
        static_cast<bf16_t*>(p.da), static_cast<bf16_t*>(p.db), p.ds0);
    return hipGetLastError();
}

}  // namespace wkv7
