// wkv7_seq.hip -- sequential WKV7 scan and single-token decode step (gfx950).
//
// Per (batch b, head h) the N x N fp32 state evolves token by token as
//   z = S a_t;  S[i][j] = S[i][j] w_t[j] + z[i] b_t[j] + v_t[i] k_t[j];  y_t = S r_t
// (generalised delta rule with a diagonal-plus-rank-one transition and a
// read-out after the update: "Paper Review: RWKV-7 Goose", Architecture and
// The approach).
//
// Lane ownership: right-multiplication acts on each state row separately and
// row i only uses the scalar v_t[i], so value rows evolve independently.  A
// wave holds 4 rows; 16 lanes share one row, each owning 4 consecutive key
// columns as a float4 in VGPRs.  Row dot products (S a, S r) are a 4-term
// in-lane FMA chain followed by a 16-lane DPP butterfly.  A workgroup of
// WAVES waves owns 4*WAVES rows of one head; token vectors r,w,k,a,b (and the
// workgroup's slice of v) are loaded coalesced, converted to fp32 and staged
// through LDS 16 tokens at a time, with the next block prefetched into
// registers while the current one is consumed.

#include "wkv7_device.h"
#include "wkv7_internal.h"

namespace wkv7 {

namespace {

constexpr int kTB = 16;  // tokens per LDS stage
static_assert(kTB == 16, "the tape's removal read-outs and states follow 16-token chunks");

// kAB = false: a = b = 0 (decay-only recurrence S <- S diag(w) + v k^T); a and
// b are not read, z is not formed and the tape's Z part is not written.
template <typename Tin, int WAVES, bool kAB>
__global__ __launch_bounds__(64 * WAVES) void seq_fwd_kernel(
    int T, int H, const Tin* __restrict__ r, const Tin* __restrict__ w,
    const Tin* __restrict__ k, const Tin* __restrict__ v, const Tin* __restrict__ a,
    const Tin* __restrict__ b, const float* __restrict__ s0, Tin* __restrict__ y,
    float* __restrict__ sT, bf16_t* __restrict__ tape) {
    constexpr int R = 4 * WAVES;     // state rows per workgroup
    constexpr int NRB = kN / R;      // workgroups per head
    constexpr int NT = 64 * WAVES;   // threads
    constexpr int CH = kTB * 16;     // float4 chunks per token vector per stage
    constexpr int PER = (CH + NT - 1) / NT;

    __shared__ float4 sm[5][kTB][16];   // r, w, k, a, b as fp32
    __shared__ float sv[kTB][R];        // this workgroup's v slice
    __shared__ float sy[kTB][R];        // read-outs before the coalesced store
    __shared__ float sz[kTB][R];        // removal read-outs z = S a, for the tape

    const int rb = blockIdx.x % NRB;
    const int bh = blockIdx.x / NRB;
    const int bb = bh / H, hh = bh % H;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int rloc = wave * 4 + (lane >> 4);
    const int row = rb * R + rloc;
    const int cq = lane & 15;           // float4 column index
    const Tin* src[5] = {r, w, k, a, b};

    const size_t soff = ((size_t)bh * kN + row) * kN + cq * 4;
    float4 S = s0 ? *reinterpret_cast<const float4*>(s0 + soff) : make_float4(0.f, 0.f, 0.f, 0.f);
    // Tape for the backward: z as [B][T][H][N] bf16, then the state entering every
    // 32-token block as [B][H][nblk][N (key)][N (value)] bf16.
    const int nblk = (T + 31) / 32;
    bf16_t* const tapeZ = tape;
    bf16_t* const tapeS = tape ? tape + (size_t)(gridDim.x / NRB) / H * T * H * kN : nullptr;

    float4 pre[5][PER];
    float4 prev = make_float4(0.f, 0.f, 0.f, 0.f);
    constexpr int NQ = kAB ? 5 : 3;   // token vectors staged: r, w, k (, a, b)
    auto load_regs = [&](int t0) {
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int p = 0; p < PER; ++p) {
                const int idx = tid + p * NT;
                const int t = idx / 16, c = idx % 16;
                if (idx < CH && t0 + t < T)
                    pre[q][p] = Elem<Tin>::load4(src[q] + tok_off(bb, t0 + t, hh, T, H) + c * 4);
            }
        if (tid < kTB * (R / 4)) {
            const int t = tid / (R / 4), c = tid % (R / 4);
            if (t0 + t < T)
                prev = Elem<Tin>::load4(v + tok_off(bb, t0 + t, hh, T, H) + rb * R + c * 4);
        }
    };
    auto store_lds = [&]() {
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int p = 0; p < PER; ++p) {
                const int idx = tid + p * NT;
                if (idx < CH) sm[q][idx / 16][idx % 16] = pre[q][p];
            }
        if (tid < kTB * (R / 4)) {
            const int t = tid / (R / 4), c = tid % (R / 4);
            *reinterpret_cast<float4*>(&sv[t][c * 4]) = prev;
        }
    };

    if (T > 0) {
        load_regs(0);
        store_lds();
    }
    __syncthreads();
    for (int t0 = 0; t0 < T; t0 += kTB) {
        const int nt = min(kTB, T - t0);
        if (t0 + kTB < T) load_regs(t0 + kTB);
        if (tape && t0 % 32 == 0) {   // entry state of block t0 / 32
            bf16_t* dst = tapeS + ((size_t)bh * nblk + t0 / 32) * kN * kN + row;
            dst[(cq * 4 + 0) * kN] = f2bf(S.x);
            dst[(cq * 4 + 1) * kN] = f2bf(S.y);
            dst[(cq * 4 + 2) * kN] = f2bf(S.z);
            dst[(cq * 4 + 3) * kN] = f2bf(S.w);
        }
        for (int t = 0; t < nt; ++t) {
            const float4 W = sm[1][t][cq], K = sm[2][t][cq], Rr = sm[0][t][cq];
            const float vi = sv[t][rloc];
            if (kAB) {
                const float4 A = sm[3][t][cq], Bv = sm[4][t][cq];
                const float z = row16_sum(dot4(S, A));
                if (cq == 0) sz[t][rloc] = z;
                S.x = fmaf(vi, K.x, fmaf(z, Bv.x, S.x * W.x));
                S.y = fmaf(vi, K.y, fmaf(z, Bv.y, S.y * W.y));
                S.z = fmaf(vi, K.z, fmaf(z, Bv.z, S.z * W.z));
                S.w = fmaf(vi, K.w, fmaf(z, Bv.w, S.w * W.w));
            } else {
                S.x = fmaf(vi, K.x, S.x * W.x);
                S.y = fmaf(vi, K.y, S.y * W.y);
                S.z = fmaf(vi, K.z, S.z * W.z);
                S.w = fmaf(vi, K.w, S.w * W.w);
            }
            const float yy = row16_sum(dot4(S, Rr));
            if (cq == 0) sy[t][rloc] = yy;
        }
        __syncthreads();
        for (int idx = tid; y && idx < nt * R; idx += NT) {
            const int t = idx / R, i = idx % R;
            Elem<Tin>::store1(y + tok_off(bb, t0 + t, hh, T, H) + rb * R + i, sy[t][i]);
        }
        for (int idx = tid; kAB && tape && idx < nt * R; idx += NT) {
            const int t = idx / R, i = idx % R;
            tapeZ[tok_off(bb, t0 + t, hh, T, H) + rb * R + i] = f2bf(sz[t][i]);
        }
        if (t0 + kTB < T) store_lds();
        __syncthreads();
    }
    if (sT) *reinterpret_cast<float4*>(sT + soff) = S;
}

// One token on resident states.  One workgroup of 4 waves per (b, h); each
// wave updates 16 rows as 4 groups of 4 rows, every lane 4 consecutive
// columns, so each state row is one contiguous 256-byte segment per 16 lanes.
template <typename Tin, bool kAB>
__global__ __launch_bounds__(256) void decode_kernel(
    const Tin* __restrict__ r, const Tin* __restrict__ w, const Tin* __restrict__ k,
    const Tin* __restrict__ v, const Tin* __restrict__ a, const Tin* __restrict__ b,
    float* __restrict__ state, Tin* __restrict__ y) {
    const int bh = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int cq = lane & 15;
    const size_t io = (size_t)bh * kN;
    float* st = state + (size_t)bh * kN * kN;
    float4 S[4];
    float vv[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int row = wave * 16 + g * 4 + (lane >> 4);
        S[g] = *reinterpret_cast<const float4*>(st + row * kN + cq * 4);
        vv[g] = Elem<Tin>::load1(v + io + row);
    }
    // a = b = 0 (kAB false): nothing to load, z = 0.
    const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 A = kAB ? Elem<Tin>::load4(a + io + cq * 4) : zero;
    const float4 Bv = kAB ? Elem<Tin>::load4(b + io + cq * 4) : zero;
    const float4 W = Elem<Tin>::load4(w + io + cq * 4);
    const float4 K = Elem<Tin>::load4(k + io + cq * 4);
    const float4 Rr = Elem<Tin>::load4(r + io + cq * 4);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int row = wave * 16 + g * 4 + (lane >> 4);
        float4 s = S[g];
        const float z = kAB ? row16_sum(dot4(s, A)) : 0.f;
        s.x = fmaf(vv[g], K.x, fmaf(z, Bv.x, s.x * W.x));
        s.y = fmaf(vv[g], K.y, fmaf(z, Bv.y, s.y * W.y));
        s.z = fmaf(vv[g], K.z, fmaf(z, Bv.z, s.z * W.z));
        s.w = fmaf(vv[g], K.w, fmaf(z, Bv.w, s.w * W.w));
        const float yy = row16_sum(dot4(s, Rr));
        if (cq == 0) Elem<Tin>::store1(y + io + row, yy);
        *reinterpret_cast<float4*>(st + row * kN + cq * 4) = s;
    }
}

// Copies (or zero-fills, when src is null) B*H fp32 states of N x N.
__global__ __launch_bounds__(256) void state_copy_kernel(size_t n4, const float* __restrict__ src,
                                                         float* __restrict__ dst) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n4)
        reinterpret_cast<float4*>(dst)[i] =
            src ? reinterpret_cast<const float4*>(src)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
}

template <typename Tin>
hipError_t launch_seq_fwd_t(const FwdArgs& p, hipStream_t stream) {
    const int BH = p.B * p.H;
    const Tin* r = static_cast<const Tin*>(p.r);
    const Tin* w = static_cast<const Tin*>(p.w);
    const Tin* k = static_cast<const Tin*>(p.k);
    const Tin* v = static_cast<const Tin*>(p.v);
    const Tin* a = static_cast<const Tin*>(p.a);
    const Tin* b = static_cast<const Tin*>(p.b);
    Tin* y = static_cast<Tin*>(p.y);
    // Few heads: split each head's rows over 4 workgroups to occupy more CUs.
    if (BH < 512) {
        auto kern = a ? seq_fwd_kernel<Tin, 4, true> : seq_fwd_kernel<Tin, 4, false>;
        kern<<<dim3(BH * 4), dim3(256), 0, stream>>>(
            p.T, p.H, r, w, k, v, a, b, p.s0, y, p.sT, static_cast<bf16_t*>(p.tape));
    } else {
        auto kern = a ? seq_fwd_kernel<Tin, 16, true> : seq_fwd_kernel<Tin, 16, false>;
        kern<<<dim3(BH), dim3(1024), 0, stream>>>(
            p.T, p.H, r, w, k, v, a, b, p.s0, y, p.sT, static_cast<bf16_t*>(p.tape));
    }
    return hipGetLastError();
}

template <typename Tin>
hipError_t launch_decode_t(const DecodeArgs& p, hipStream_t stream) {
    auto kern = p.a ? decode_kernel<Tin, true> : decode_kernel<Tin, false>;
    kern<<<dim3(p.B * p.H), dim3(256), 0, stream>>>(
        static_cast<const Tin*>(p.r), static_cast<const Tin*>(p.w),
        static_cast<const Tin*>(p.k), static_cast<const Tin*>(p.v),
        static_cast<const Tin*>(p.a), static_cast<const Tin*>(p.b), p.state,
        static_cast<Tin*>(p.y));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_seq_fwd(const FwdArgs& p, hipStream_t stream) {
    return p.bf16 ? launch_seq_fwd_t<bf16_t>(p, stream) : launch_seq_fwd_t<float>(p, stream);
}

hipError_t launch_state_copy(int BH, const float* s0, float* sT, hipStream_t stream) {
    const size_t n4 = (size_t)BH * kN * kN / 4;
    state_copy_kernel<<<dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream>>>(n4, s0, sT);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& p, hipStream_t stream) {
    return p.bf16 ? launch_decode_t<bf16_t>(p, stream) : launch_decode_t<float>(p, stream);
}

}  // namespace wkv7
