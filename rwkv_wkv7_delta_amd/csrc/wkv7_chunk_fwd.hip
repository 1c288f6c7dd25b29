// wkv7_chunk_fwd.hip -- chunked (parallel-in-time) WKV7 forward on bf16 MFMA.
//
// The pages state that RWKV-7 keeps training parallelisable (Abstract; Elamur
// summary, Summary) without printing the parallel form.  The form used here
// is an exact rearrangement of the recurrence over a chunk of L = 16 tokens
// with entry state S0 (derivation written out in the project's design notes,
// pinned in fp64 against the sequential definition):
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
// Mapping to gfx950: one workgroup of 4 waves per (b, h), chunks in order.
// Wave w owns value rows 16w..16w+15 of the state, held as S^T in four 16x16
// fp32 accumulator tiles (key blocks); because of the D -> B operand identity
// (see wkv7_mfma.h) every state-dependent product is a left multiplication
// that reads the state straight from registers.  The state-independent
// factors (decay products, L x L products, the triangular inverse, W, Q) are
// shared through LDS.  All MFMA operands are bf16, accumulation and the
// carried state are fp32.

#include "wkv7_device.h"
#include "wkv7_internal.h"
#include "wkv7_mfma.h"

namespace wkv7 {

namespace {

constexpr int kL = 16;
constexpr int kThreads = 256;

struct __align__(16) ChunkSmem {
    bf16_t raw[6][kL][kN];        // r, w, k, a, b, v of the chunk (bf16 bits)
    bf16_t At[kL][kN], Rt[kL][kN], Bh[kL][kN], Kh[kL][kN];  // row-major [t][j]
    bf16_t BbT[kN][kL], KbT[kN][kL];                        // [j][t]
    float Rt32[kL][kN];
    float gtot[4][kN];
    float gL[kN];
    float Amat[4][kL][kL];        // Aab, Aak, Arb, Ark
    float Tm[kL][kL];
    bf16_t Wm[kL][kN], Qm[kL][kN];
    bf16_t Ys[kL][kN];
};

enum { RAW_R = 0, RAW_W = 1, RAW_K = 2, RAW_A = 3, RAW_B = 4, RAW_V = 5 };

__device__ __forceinline__ float bf2f(bf16_t x) { return __uint_as_float((uint32_t)x << 16); }

__device__ __forceinline__ bf16x4 ld_bf16x4(const bf16_t* p) {
    return __builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2*>(p));
}

__global__ __launch_bounds__(kThreads) void chunk_fwd_kernel(
    int T, int H, const bf16_t* __restrict__ r, const bf16_t* __restrict__ w,
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, const bf16_t* __restrict__ a,
    const bf16_t* __restrict__ b, const float* __restrict__ s0, bf16_t* __restrict__ y,
    float* __restrict__ sT, float* __restrict__ ckpt) {
    __shared__ ChunkSmem sm;
    const int bh = blockIdx.x;
    const int bb = bh / H, hh = bh % H;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    const bf16_t* src[6] = {r, w, k, a, b, v};
    const int nck = (T + kCkptInterval - 1) / kCkptInterval;

    // ---- state: S^T tiles, wave wv owns value rows i = 16 wv + l16 -------------
    const int irow = 16 * wv + l16;
    f32x4 S[4];
    {
        const float* base = s0 ? s0 + ((size_t)bh * kN + irow) * kN : nullptr;
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            if (base) {
                const float4 x = *reinterpret_cast<const float4*>(base + 16 * jt + 4 * g);
                S[jt][0] = x.x; S[jt][1] = x.y; S[jt][2] = x.z; S[jt][3] = x.w;
            } else {
                S[jt] = zero4();
            }
        }
    }

    // ---- raw token loads: 6 vectors x 16 tokens x 64 = 768 x 16 bytes ---------
    uint4 pre[3];
    auto load_chunk = [&](int t0) {
#pragma unroll
        for (int p = 0; p < 3; ++p) {
            const int item = tid + p * kThreads;
            const int q = item >> 7, t = (item >> 3) & 15, c8 = item & 7;
            const bf16_t* sp = (q & 1) ? src[2 * p + 1] : src[2 * p];   // q in {2p, 2p+1}
            if (t0 + t < T) {
                pre[p] = *reinterpret_cast<const uint4*>(sp + tok_off(bb, t0 + t, hh, T, H) + c8 * 8);
            } else {
                // Padding token: w = 1, everything else 0 -> no change of state.
                const uint32_t pad = (q == RAW_W) ? 0x3F803F80u : 0u;
                pre[p] = make_uint4(pad, pad, pad, pad);
            }
        }
    };
    auto stash_chunk = [&]() {
#pragma unroll
        for (int p = 0; p < 3; ++p) {
            const int item = tid + p * kThreads;
            const int q = item >> 7, t = (item >> 3) & 15, c8 = item & 7;
            *reinterpret_cast<uint4*>(&sm.raw[q][t][c8 * 8]) = pre[p];
        }
    };

    if (T > 0) {
        if (ckpt) {
            float* dst = ckpt + ((size_t)bh * nck * kN + irow) * kN;
#pragma unroll
            for (int jt = 0; jt < 4; ++jt)
                *reinterpret_cast<float4*>(dst + 16 * jt + 4 * g) =
                    make_float4(S[jt][0], S[jt][1], S[jt][2], S[jt][3]);
        }
        load_chunk(0);
        stash_chunk();
    }
    __syncthreads();

    const int ej = tid & 63;   // element phase: key column
    const int eg = tid >> 6;   // element phase: tokens 4 eg .. 4 eg + 3

    for (int t0 = 0; t0 < T; t0 += kL) {
        if (t0 + kL < T) load_chunk(t0 + kL);

        // ---- 1. running decay products and scaled vectors -------------------
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
            float g0 = sm.gtot[0][ej], g1 = sm.gtot[1][ej], g2 = sm.gtot[2][ej], g3 = sm.gtot[3][ej];
            const float before = eg == 0 ? 1.f : eg == 1 ? g0 : eg == 2 ? g0 * g1 : (g0 * g1) * g2;
            const float GL = ((g0 * g1) * g2) * g3;
            float bbar[4], kbar[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int t = 4 * eg + u;
                const float Gt = before * gp[u];
                const float Gprev = u == 0 ? before : before * gp[u - 1];
                const float inv = __builtin_amdgcn_rcpf(Gt);
                const float at = bf2f(sm.raw[RAW_A][t][ej]) * Gprev;
                const float rt = bf2f(sm.raw[RAW_R][t][ej]) * Gt;
                const float bhat = bf2f(sm.raw[RAW_B][t][ej]) * inv;
                const float khat = bf2f(sm.raw[RAW_K][t][ej]) * inv;
                sm.At[t][ej] = f2bf(at);
                sm.Rt[t][ej] = f2bf(rt);
                sm.Rt32[t][ej] = rt;
                sm.Bh[t][ej] = f2bf(bhat);
                sm.Kh[t][ej] = f2bf(khat);
                bbar[u] = bhat * GL;
                kbar[u] = khat * GL;
            }
            *reinterpret_cast<bf16x4*>(&sm.BbT[ej][4 * eg]) = cvt4(bbar[0], bbar[1], bbar[2], bbar[3]);
            *reinterpret_cast<bf16x4*>(&sm.KbT[ej][4 * eg]) = cvt4(kbar[0], kbar[1], kbar[2], kbar[3]);
            if (eg == 0) sm.gL[ej] = GL;
        }
        __syncthreads();

        // ---- 2. L x L products: wave 0 Aab, 1 Aak, 2 Arb, 3 Ark ---------------
        {
            const bf16_t* lrow = (wv < 2) ? &sm.At[l16][0] : &sm.Rt[l16][0];
            const bf16_t* rrow = (wv & 1) ? &sm.Kh[l16][0] : &sm.Bh[l16][0];
            f32x4 acc = zero4();
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const bf16x8 av = *reinterpret_cast<const bf16x8*>(lrow + 32 * c + 8 * g);
                const bf16x8 bv = *reinterpret_cast<const bf16x8*>(rrow + 32 * c + 8 * g);
                acc = mfma32(av, bv, acc);
            }
            const bool strict = wv < 2;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int t = 4 * g + q, s = l16;
                const bool keep = strict ? (s < t) : (s <= t);
                sm.Amat[wv][t][s] = keep ? acc[q] : 0.f;
            }
        }
        __syncthreads();

        // ---- 3. Tm = (I - Aab)^-1 by forward substitution (wave 0) -----------
        if (wv == 0) {
            float col[kL];
#pragma unroll
            for (int t = 0; t < kL; ++t) col[t] = (t == l16) ? 1.f : 0.f;
#pragma unroll
            for (int t = 1; t < kL; ++t) {
                float acc = col[t];
#pragma unroll
                for (int s = 0; s < t; ++s) acc = fmaf(sm.Amat[0][t][s], col[s], acc);
                col[t] = acc;
            }
            if (g == 0) {
#pragma unroll
                for (int t = 0; t < kL; ++t) sm.Tm[t][l16] = col[t];
            }
        }
        __syncthreads();

        // ---- 4. W = Tm At and Q = Rt + Arb W (wave wv: key block jt = wv) -----
        const bf16x4 Trow = cvt4(sm.Tm[l16][4 * g], sm.Tm[l16][4 * g + 1], sm.Tm[l16][4 * g + 2],
                                 sm.Tm[l16][4 * g + 3]);
        {
            const int j = 16 * wv + l16;
            const bf16x4 Acol = cvt4(bf2f(sm.At[4 * g][j]), bf2f(sm.At[4 * g + 1][j]),
                                     bf2f(sm.At[4 * g + 2][j]), bf2f(sm.At[4 * g + 3][j]));
            const f32x4 Wt = mfma16(Trow, Acol, zero4());
            f32x4 Qt;
#pragma unroll
            for (int q = 0; q < 4; ++q) Qt[q] = sm.Rt32[4 * g + q][j];
            const bf16x4 Arb_row = cvt4(sm.Amat[2][l16][4 * g], sm.Amat[2][l16][4 * g + 1],
                                        sm.Amat[2][l16][4 * g + 2], sm.Amat[2][l16][4 * g + 3]);
            Qt = mfma16(Arb_row, cvt4(Wt), Qt);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                sm.Wm[4 * g + q][j] = f2bf(Wt[q]);
                sm.Qm[4 * g + q][j] = f2bf(Qt[q]);
            }
        }

        // ---- 5. value-dependent, state-independent terms of this wave --------
        const bf16x4 Vb = cvt4(bf2f(sm.raw[RAW_V][4 * g][irow]), bf2f(sm.raw[RAW_V][4 * g + 1][irow]),
                               bf2f(sm.raw[RAW_V][4 * g + 2][irow]), bf2f(sm.raw[RAW_V][4 * g + 3][irow]));
        const bf16x4 Aak_row = cvt4(sm.Amat[1][l16][4 * g], sm.Amat[1][l16][4 * g + 1],
                                    sm.Amat[1][l16][4 * g + 2], sm.Amat[1][l16][4 * g + 3]);
        const bf16x4 Arb_row = cvt4(sm.Amat[2][l16][4 * g], sm.Amat[2][l16][4 * g + 1],
                                    sm.Amat[2][l16][4 * g + 2], sm.Amat[2][l16][4 * g + 3]);
        const bf16x4 Ark_row = cvt4(sm.Amat[3][l16][4 * g], sm.Amat[3][l16][4 * g + 1],
                                    sm.Amat[3][l16][4 * g + 2], sm.Amat[3][l16][4 * g + 3]);
        const f32x4 AkV = mfma16(Aak_row, Vb, zero4());
        const f32x4 U = mfma16(Trow, cvt4(AkV), zero4());
        f32x4 Y0 = mfma16(Arb_row, cvt4(U), zero4());
        Y0 = mfma16(Ark_row, Vb, Y0);
        f32x4 Hs[4];
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
            Hs[jt] = mfma16(ld_bf16x4(&sm.KbT[16 * jt + l16][4 * g]), Vb, zero4());
        __syncthreads();   // Wm, Qm complete

        // ---- 6. state-dependent chain ------------------------------------------
        bf16x4 Sb[4];
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) Sb[jt] = cvt4(S[jt]);
        f32x4 Z = U, Yt = Y0;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const bf16x8 bs = cat8(Sb[2 * c], Sb[2 * c + 1]);
            const bf16x8 wa = cat8(ld_bf16x4(&sm.Wm[l16][32 * c + 4 * g]),
                                   ld_bf16x4(&sm.Wm[l16][32 * c + 16 + 4 * g]));
            const bf16x8 qa = cat8(ld_bf16x4(&sm.Qm[l16][32 * c + 4 * g]),
                                   ld_bf16x4(&sm.Qm[l16][32 * c + 16 + 4 * g]));
            Z = mfma32(wa, bs, Z);
            Yt = mfma32(qa, bs, Yt);
        }
        const bf16x4 Zb = cvt4(Z);
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            f32x4 acc;
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[q] = fmaf(sm.gL[16 * jt + 4 * g + q], S[jt][q], Hs[jt][q]);
            S[jt] = mfma16(ld_bf16x4(&sm.BbT[16 * jt + l16][4 * g]), Zb, acc);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) sm.Ys[4 * g + q][irow] = f2bf(Yt[q]);

        const int done = t0 + kL;
        if (ckpt && (done % kCkptInterval) == 0 && done < T) {
            float* dst = ckpt + (((size_t)bh * nck + done / kCkptInterval) * kN + irow) * kN;
#pragma unroll
            for (int jt = 0; jt < 4; ++jt)
                *reinterpret_cast<float4*>(dst + 16 * jt + 4 * g) =
                    make_float4(S[jt][0], S[jt][1], S[jt][2], S[jt][3]);
        }
        __syncthreads();   // Ys complete; raw and factor buffers free

        // ---- 7. coalesced y store (16 tokens x 128 B) and next chunk's inputs -
        {
            const int t = tid >> 4, c4 = tid & 15;   // 16 tokens x 16 lanes x 8 B
            if (y && t0 + t < T)
                *reinterpret_cast<uint2*>(y + tok_off(bb, t0 + t, hh, T, H) + c4 * 4) =
                    *reinterpret_cast<const uint2*>(&sm.Ys[t][c4 * 4]);
        }
        if (t0 + kL < T) stash_chunk();
        __syncthreads();
    }

    if (sT) {
        float* dst = sT + ((size_t)bh * kN + irow) * kN;
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
