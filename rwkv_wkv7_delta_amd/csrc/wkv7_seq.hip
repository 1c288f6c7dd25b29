// wkv7_seq.hip -- sequential WKV7 scan and single-token decode step (gfx950),
// for head sizes N = 32, 64 and 128.
//
// Per (batch b, head h) the N x N fp32 state evolves token by token as
//   z = S a_t;  S[i][j] = S[i][j] w_t[j] + z[i] b_t[j] + v_t[i] k_t[j];  y_t = S r_t
// (generalised delta rule with a diagonal-plus-rank-one transition and a
// read-out after the update: "Paper Review: RWKV-7 Goose", Architecture and
// The approach).  The head size is a template parameter: the state expansion
// of "Millions of States: Designing a Scalable MoE Architecture with RWKV-7
// Meta-learner" (Abstract) grows it.
//
// Lane ownership: right-multiplication acts on each state row separately and
// row i only uses the scalar v_t[i], so value rows evolve independently.  A
// wave holds 4 rows; 16 lanes share one row, each owning C = N/16 consecutive
// key columns in VGPRs.  Row dot products (S a, S r) are a C-term in-lane FMA
// chain followed by a 16-lane DPP butterfly.  A workgroup of WAVES waves owns
// 4*WAVES rows of one head; token vectors r,w,k,a,b (and the workgroup's
// slice of v) are loaded coalesced, converted to fp32 and staged through LDS
// 16 tokens at a time, with the next block prefetched into registers while the
// current one is consumed.

#include <type_traits>

#include "wkv7_device.h"
#include "wkv7_internal.h"

namespace wkv7 {

namespace {

constexpr int kTB = 16;  // tokens per LDS stage
static_assert(kTB == 16, "the tape's removal read-outs and states follow 16-token chunks");

// Token tensor offset for [B][T][H][N].
template <int N>
__device__ __forceinline__ size_t tok_off_n(int b, int t, int h, int T, int H) {
    return (((size_t)b * T + t) * H + h) * N;
}

// kAB = false: a = b = 0 (decay-only recurrence S <- S diag(w) + v k^T); a and
// b are not read, z is not formed and the tape's Z part is not written.
// P = lanes per state row (the lane-ownership knob): 16 keeps each token's
// dependent chain short (few heads: the latency of T serial tokens decides);
// 4 or 8 cut the per-row overhead of the row sums, selects and LDS reads
// (many heads: the vector-ALU issue rate decides).
// Under a segment plan (pass, split_from, nseg, seg_len, states: see work_of)
// a workgroup runs one segment, or one affine-map run, of its head.
template <typename Tin, int N, int WAVES, bool kAB, int P>
__global__ __launch_bounds__(64 * WAVES) void seq_fwd_kernel(
    int B, int T, int H, const Tin* __restrict__ r, const Tin* __restrict__ w,
    const Tin* __restrict__ k, const Tin* __restrict__ v, const Tin* __restrict__ a,
    const Tin* __restrict__ b, const float* __restrict__ s0, Tin* __restrict__ y,
    float* __restrict__ sT, bf16_t* __restrict__ tape, float* __restrict__ ckpt, int pass,
    int split_from, int nseg, int seg_len, float* __restrict__ states) {
    constexpr int C = N / P;         // key columns per lane
    constexpr int RW = 64 / P;       // state rows per wave
    constexpr int R = RW * WAVES;    // state rows per workgroup
    constexpr int NU = kTB / P;      // read-outs per lane and stage (token u P + lane in row)
    constexpr int NRB = N / R;       // workgroups per head
    constexpr int NT = 64 * WAVES;   // threads
    constexpr int G4 = N / 4;        // 4-element groups per token vector
    constexpr int CH = kTB * G4;     // ... per stage
    constexpr int PER = (CH + NT - 1) / NT;
    static_assert(NRB >= 1 && NRB * R == N, "rows per workgroup must divide N");

    __shared__ __align__(16) float sm[5][kTB][N];   // r, w, k, a, b as fp32
    __shared__ float sv[kTB][R];        // this workgroup's v slice
    __shared__ float sy[kTB][R];        // read-outs before the coalesced store
    __shared__ float sz[kTB][R];        // removal read-outs z = S a, for the tape

    const int rb = blockIdx.x % NRB;
    const Work wk = work_of<N>(blockIdx.x / NRB, pass, T, s0, sT, split_from, nseg, seg_len, states);
    const int bh = wk.bh;
    const int bb = bh / H, hh = bh % H;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int rloc = wave * RW + lane / P;
    const int row = rb * R + rloc;
    const int cq = lane % P;            // this lane's columns: C * cq .. C * cq + C - 1
    const Tin* src[5] = {r, w, k, a, b};

    const size_t roff = (size_t)row * N + cq * C;   // this lane's piece of a head's state
    float S[C];
    if (wk.init) {
        load_cols<C>(wk.init + roff, S);
        // Settle the load here: left pending on the path that skips the first
        // stage (T = 0), it would make the compiler wait for the whole memory
        // counter -- every stage's own prefetch -- before each use of S.
        __builtin_amdgcn_s_waitcnt(0);
    } else {
#pragma unroll
        for (int c = 0; c < C; ++c) S[c] = (wk.ident && cq * C + c == row) ? 1.f : 0.f;
    }
    // Tape for the backward: z as [B][T][H][N] bf16, then the state entering every
    // 32-token block as [B][H][nblk][N (key)][N (value)] bf16 (segment runs with
    // outputs write their own tokens and blocks; map runs write nothing).
    const int nblk = (T + 31) / 32;
    bf16_t* const tapeZ = wk.outs ? tape : nullptr;
    bf16_t* const tapeS = (tape && wk.outs) ? tape + (size_t)B * T * H * N : nullptr;
    Tin* const yo = wk.outs ? y : nullptr;
    float* const ck = wk.outs ? ckpt : nullptr;

    // Prefetched elements stay as loaded (bf16 words) until stashed: converting
    // them at the load would make the stage wait for its own prefetch.  Every
    // thread loads on every stage (indices clamped to the last token and the
    // last piece: the surplus loads repeat valid addresses), so no load sits on
    // a conditional path -- after such a path the compiler no longer knows
    // which loads are done and waits for the whole memory counter, stores
    // included, before reusing their registers.
    typedef typename Elem<Tin>::raw4 raw4;
    raw4 pre[5][PER];
    raw4 prev;
    constexpr int NQ = kAB ? 5 : 3;   // token vectors staged: r, w, k (, a, b)
    constexpr int VP = kTB * (R / 4); // 4-element pieces of this workgroup's v slice per stage
    auto load_regs = [&](int t0) {
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int p = 0; p < PER; ++p) {
                const int idx = min(tid + p * NT, CH - 1);
                const int t = min(t0 + idx / G4, T - 1), c = idx % G4;
                pre[q][p] = Elem<Tin>::load_raw4(src[q] + tok_off_n<N>(bb, t, hh, T, H) + c * 4);
            }
        const int vi = min(tid, VP - 1);
        const int t = min(t0 + vi / (R / 4), T - 1), c = vi % (R / 4);
        prev = Elem<Tin>::load_raw4(v + tok_off_n<N>(bb, t, hh, T, H) + rb * R + c * 4);
    };
    auto store_lds = [&]() {
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int p = 0; p < PER; ++p) {
                const int idx = tid + p * NT;
                if (idx < CH) *reinterpret_cast<float4*>(&sm[q][idx / G4][(idx % G4) * 4]) = Elem<Tin>::cvt(pre[q][p]);
            }
        if (tid < VP) {
            const int t = tid / (R / 4), c = tid % (R / 4);
            // the P run of an affine map takes v = 0
            *reinterpret_cast<float4*>(&sv[t][c * 4]) = wk.vzero ? make_float4(0.f, 0.f, 0.f, 0.f) : Elem<Tin>::cvt(prev);
        }
    };

    if (wk.t_begin < wk.t_end) {
        load_regs(wk.t_begin);
        store_lds();
    }
    __syncthreads();
    // Segments start on multiples of 32 tokens, so stages and tape blocks keep
    // their absolute positions.
    for (int t0 = wk.t_begin; t0 < wk.t_end; t0 += kTB) {
        const int nt = min(kTB, wk.t_end - t0);
        load_regs(t0 + kTB);   // the next stage (past the end: other tokens, unused)
        if (tapeS && t0 % 32 == 0) {   // entry state of block t0 / 32
            bf16_t* dst = tapeS + ((size_t)bh * nblk + t0 / 32) * N * N + row;
#pragma unroll
            for (int c = 0; c < C; ++c) dst[(cq * C + c) * N] = f2bf(S[c]);
        }
        if (ck)   // fp32 entry state of every stage, for the sequential reverse pass
            store_cols<C>(ck + (((size_t)bh * ((T + kTB - 1) / kTB) + t0 / kTB) * N + row) * N + cq * C, S);
        // One token of the recurrence on this lane's columns.  Whole stages are
        // unrolled so that the LDS reads of later tokens overlap the dependent
        // dot -> DPP sum -> update chain of the current one.  The read-outs of
        // token t stay in lane t mod P of the row, slot t / P (a select, not a
        // branched store, which would cut the stage into one basic block per
        // token) and are written to LDS once per stage.
        float y_l[NU], z_l[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) y_l[u] = z_l[u] = 0.f;
        auto step = [&](int t) __attribute__((always_inline)) {
            float W[C], K[C], Rr[C];
            load_cols<C>(&sm[1][t][cq * C], W);
            load_cols<C>(&sm[2][t][cq * C], K);
            load_cols<C>(&sm[0][t][cq * C], Rr);
            const float vi = sv[t][rloc];
            if (kAB) {
                float A[C], Bv[C];
                load_cols<C>(&sm[3][t][cq * C], A);
                load_cols<C>(&sm[4][t][cq * C], Bv);
                const float z = lanes_sum<P>(dot_cols(S, A));
#pragma unroll
                for (int u = 0; u < NU; ++u) z_l[u] = (cq == t - u * P) ? z : z_l[u];
#pragma unroll
                for (int c = 0; c < C; ++c) S[c] = fmaf(vi, K[c], fmaf(z, Bv[c], S[c] * W[c]));
            } else {
#pragma unroll
                for (int c = 0; c < C; ++c) S[c] = fmaf(vi, K[c], S[c] * W[c]);
            }
            const float yy = lanes_sum<P>(dot_cols(S, Rr));
#pragma unroll
            for (int u = 0; u < NU; ++u) y_l[u] = (cq == t - u * P) ? yy : y_l[u];
        };
        if (nt == kTB) {
#pragma unroll
            for (int t = 0; t < kTB; ++t) step(t);
        } else {
            for (int t = 0; t < nt; ++t) step(t);
        }
#pragma unroll
        for (int u = 0; u < NU; ++u) {   // rows t >= nt hold nothing and are not stored
            sy[u * P + cq][rloc] = y_l[u];
            if (kAB) sz[u * P + cq][rloc] = z_l[u];
        }
        __syncthreads();
        // The next stage's rows go to LDS before this stage's outputs leave, so
        // that the wait for the prefetch does not also wait for those stores.
        store_lds();
        static_assert(kTB * R % NT == 0, "whole read-outs per thread and stage");
#pragma unroll
        for (int u = 0; u < kTB * R / NT; ++u) {
            const int idx = tid + u * NT;
            if (idx < nt * R) {
                const int t = idx / R, i = idx % R;
                const size_t o = tok_off_n<N>(bb, t0 + t, hh, T, H) + rb * R + i;
                if (yo) Elem<Tin>::store1(yo + o, sy[t][i]);
                if (kAB && tapeZ) tapeZ[o] = f2bf(sz[t][i]);
            }
        }
        __syncthreads();
    }
    if (wk.fin) store_cols<C>(wk.fin + roff, S);
}

// One token on resident states.  A workgroup of 4 waves holds 4 / WPH heads,
// WPH waves per head (4, or 1 at N = 32, whose 4 KB state would leave a
// 4-wave workgroup with too little to move); each wave updates N / WPH rows as
// groups of 4 rows, every lane C = N/16 consecutive columns, so each state
// row is one contiguous segment per 16 lanes.
template <int N> struct DecodeShape {
    static constexpr int WPH = N == 32 ? 1 : 4;   // waves per head
    static constexpr int HPW = 4 / WPH;           // heads per workgroup
};
template <typename Tin, int N, bool kAB>
__global__ __launch_bounds__(256) void decode_kernel(
    int BH, const Tin* __restrict__ r, const Tin* __restrict__ w, const Tin* __restrict__ k,
    const Tin* __restrict__ v, const Tin* __restrict__ a, const Tin* __restrict__ b,
    float* __restrict__ state, Tin* __restrict__ y) {
    constexpr int WPH = DecodeShape<N>::WPH, HPW = DecodeShape<N>::HPW;
    constexpr int C = N / 16;          // columns per lane
    constexpr int G = N / (4 * WPH);   // groups of 4 rows per wave
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int bh = blockIdx.x * HPW + wv / WPH;
    const int wave = wv % WPH;         // wave within the head
    if (bh >= BH) return;              // the last workgroup's surplus waves (no barriers here)
    const int cq = lane & 15;
    const size_t io = (size_t)bh * N;
    float* st = state + (size_t)bh * N * N;
    float S[G][C];
    float vv[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int row = wave * (N / WPH) + g * 4 + (lane >> 4);
        load_cols<C>(st + row * N + cq * C, S[g]);
        vv[g] = Elem<Tin>::load1(v + io + row);
    }
    // a = b = 0 (kAB false): nothing to load, z = 0.
    float A[C], Bv[C], W[C], K[C], Rr[C];
    if (kAB) {
        load_cols<C>(a + io + cq * C, A);
        load_cols<C>(b + io + cq * C, Bv);
    }
    load_cols<C>(w + io + cq * C, W);
    load_cols<C>(k + io + cq * C, K);
    load_cols<C>(r + io + cq * C, Rr);
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int row = wave * (N / WPH) + g * 4 + (lane >> 4);
        if (kAB) {
            const float z = row16_sum(dot_cols(S[g], A));
#pragma unroll
            for (int c = 0; c < C; ++c) S[g][c] = fmaf(vv[g], K[c], fmaf(z, Bv[c], S[g][c] * W[c]));
        } else {
#pragma unroll
            for (int c = 0; c < C; ++c) S[g][c] = fmaf(vv[g], K[c], S[g][c] * W[c]);
        }
        const float yy = row16_sum(dot_cols(S[g], Rr));
        if (cq == 0) Elem<Tin>::store1(y + io + row, yy);
        store_cols<C>(st + row * N + cq * C, S[g]);
    }
}


// ---------------------------------------------------------------------------
// Sequential reverse pass: the adjoint recurrence token by token.  With the
// adjoint G = dL/dS_t (after token t's write), going backwards in time:
//   G += dy_t r_t^T;  dr_t = S_t^T dy_t;  dv_t = G k_t;  dk_t = G^T v_t;
//   dw_t[j] = sum_i G[i][j] S_{t-1}[i][j];  z = S_{t-1} a_t;  dz = G b_t;
//   db_t = G^T z;  da_t = S_{t-1}^T dz;  G <- G diag(w_t) + dz a_t^T
// and ds0 = G at the end (the transposed transition of the forward step S <-
// S (diag(w) + a b^T) + v k^T; "Paper Review: RWKV-7 Goose", The approach).
//
// One workgroup per head holds every row of G: rows are independent in the
// recurrence, as in the forward (16 lanes per row, C = N/16 columns per lane,
// four rows per 16-lane group).  The states S_t come from fp32 checkpoints at
// every 16th token, written by the forward scan: per 16-token stage the pass
// re-runs the forward from the checkpoint in sub-stages of KS tokens whose
// states stay in registers (earlier sub-stages re-run again for later ones),
// then steps G backwards over them.  The per-key gradients are sums over rows:
// within a wave by lane swaps, across waves through per-wave LDS slots summed
// once per sub-stage (atomics on shared addresses serialised across waves),
// and stored from there.
template <int N, int kSplit = 1> struct SeqBwdShape {
    // Four rows per 16-lane group: N/16 waves per head, over kSplit workgroups.
    static constexpr int RPL = 4;                 // rows per 16-lane group
    static constexpr int WAVES = N / (4 * RPL * kSplit);   // waves per workgroup
    static constexpr int C = N / 16;              // columns per lane
    // Tokens per sub-stage, whose states a lane keeps (RPL * C floats each):
    // 8 at N = 32 and 64, 2 at N = 128 (72, 144 and 96 floats per lane; at
    // N = 128 a fourth state spills past the 256 registers that two waves per
    // SIMD leave each wave, and at N = 32 one sub-stage of 16 tokens measured
    // slower than two of 8); 4 at N = 128 over two workgroups, whose four waves
    // have a SIMD each and twice the registers.  Each sub-stage re-runs the
    // stage's forward from its checkpoint, so a 16-token stage costs
    // 16 + KS (0 + 1 + .. + 16/KS - 1) forward steps: 24, 24 and 72 (40).
    static constexpr int KS = kSplit == 2 ? 4 : N == 128 ? 2 : 8;
};

// kSplit = 2: a head's rows over two workgroups (block 2 bh + half takes rows
// half N/2 ..); each adds its rows' share of the per-key sums to outputs that
// start at zero (fp32 atomics, or packed bf16 ones on pairs of columns), so
// every element receives exactly two additions onto 0, whose result does not
// depend on their order.  In bf16 each share is rounded before the addition.
template <typename Tin, int N, bool kAB, int kSplit = 1>
__global__ __launch_bounds__((64 * SeqBwdShape<N, kSplit>::WAVES)) void seq_bwd_kernel(
    int T, int H, const Tin* __restrict__ r, const Tin* __restrict__ w, const Tin* __restrict__ k,
    const Tin* __restrict__ v, const Tin* __restrict__ a, const Tin* __restrict__ b,
    const Tin* __restrict__ dy, const float* __restrict__ dsT, const float* __restrict__ ckpt,
    Tin* __restrict__ dr, Tin* __restrict__ dw, Tin* __restrict__ dk, Tin* __restrict__ dv,
    Tin* __restrict__ da, Tin* __restrict__ db, float* __restrict__ ds0) {
    using Sh = SeqBwdShape<N, kSplit>;
    static_assert(kSplit == 1 || kSplit == 2, "rows over one or two workgroups");
    constexpr int WAVES = Sh::WAVES, RPL = Sh::RPL, C = Sh::C, KS = Sh::KS;
    constexpr int NT = 64 * WAVES;
    constexpr int NG = kAB ? 5 : 3;   // per-key gradients: dr, dw, dk (, da, db)
    enum { VR, VW, VK, VV, VA, VB, VDY };
    __shared__ __align__(16) float sm[7][kTB][N];     // r, w, k, v, a, b, dy of the stage
    __shared__ __align__(16) float part[WAVES][KS][NG][N];   // per-wave sums of a sub-stage
    __shared__ float sdv[KS][N + 1];                  // column N: where surplus lanes write

    const int bh = blockIdx.x / kSplit, half = blockIdx.x % kSplit;
    const int bb = bh / H, hh = bh % H;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int grp = lane >> 4, cq = lane & 15;
    constexpr int NR = N / kSplit;                   // rows of this workgroup
    const int row0 = half * NR + (wave * 4 + grp) * RPL;   // rows row0 .. row0 + RPL - 1
    const int nstg = (T + kTB - 1) / kTB;
    auto off = [&](int t) { return (((size_t)bb * T + t) * H + hh) * N; };

    float G[RPL][C];
#pragma unroll
    for (int rr = 0; rr < RPL; ++rr) {
        if (dsT) {
            load_cols<C>(dsT + ((size_t)bh * N + row0 + rr) * N + cq * C, G[rr]);
        } else {
#pragma unroll
            for (int c = 0; c < C; ++c) G[rr][c] = 0.f;
        }
    }

    // One forward token on the state rows S (as in the scan).
    auto fwd = [&](int t, float (&S)[RPL][C]) __attribute__((always_inline)) {
        float W[C], K[C], A[C], Bv[C];
        load_cols<C>(&sm[VW][t][cq * C], W);
        load_cols<C>(&sm[VK][t][cq * C], K);
        if (kAB) {
            load_cols<C>(&sm[VA][t][cq * C], A);
            load_cols<C>(&sm[VB][t][cq * C], Bv);
        }
#pragma unroll
        for (int rr = 0; rr < RPL; ++rr) {
            const float vi = sm[VV][t][row0 + rr];
            if (kAB) {
                const float z = row16_sum(dot_cols(S[rr], A));
#pragma unroll
                for (int c = 0; c < C; ++c) S[rr][c] = fmaf(vi, K[c], fmaf(z, Bv[c], S[rr][c] * W[c]));
            } else {
#pragma unroll
                for (int c = 0; c < C; ++c) S[rr][c] = fmaf(vi, K[c], S[rr][c] * W[c]);
            }
        }
    };
    // Sums a per-lane partial over the wave's rows into its slot part[wave][kk][q]
    // (q: 0 dr, 1 dw, 2 dk, 3 da, 4 db).
    // Every group then holds every column's sum; group g writes columns c = g
    // (mod 4) of its lanes (a select, not a branch: no basic block ends here).
    auto add_rows = [&](int kk, int q, const float (&p)[C]) __attribute__((always_inline)) {
        float x[C];
#pragma unroll
        for (int c = 0; c < C; ++c) x[c] = sum_rows4(p[c]);
#pragma unroll
        for (int c0 = 0; c0 < C; c0 += 4) {
            const int c = c0 + (C >= 4 ? grp : grp & 1);
            float xs = x[c0];
#pragma unroll
            for (int u = 1; u < (C < 4 ? C : 4); ++u) xs = c == c0 + u ? x[c0 + u] : xs;
            part[wave][kk][q][cq * C + c] = xs;
        }
    };
    // One reverse token: St = S_t, Sp = S_{t-1}.  Each per-key sum is formed
    // and reduced on its own (one partial live at a time), the token's vectors
    // read from LDS where they are used.
    auto bwd = [&](int t, int kk, const float (&St)[RPL][C], const float (&Sp)[RPL][C])
        __attribute__((always_inline)) {
        float V[C], p[C];
        float dyi[RPL], vi[RPL];
#pragma unroll
        for (int rr = 0; rr < RPL; ++rr) {
            dyi[rr] = sm[VDY][t][row0 + rr];
            vi[rr] = sm[VV][t][row0 + rr];
        }
        load_cols<C>(&sm[VR][t][cq * C], V);
#pragma unroll
        for (int rr = 0; rr < RPL; ++rr)
#pragma unroll
            for (int c = 0; c < C; ++c) G[rr][c] = fmaf(dyi[rr], V[c], G[rr][c]);   // G = dL/dS_t
        // dr_t = S_t^T dy_t
#pragma unroll
        for (int c = 0; c < C; ++c) p[c] = 0.f;
#pragma unroll
        for (int rr = 0; rr < RPL; ++rr)
#pragma unroll
            for (int c = 0; c < C; ++c) p[c] = fmaf(St[rr][c], dyi[rr], p[c]);
        add_rows(kk, 0, p);
        // dk_t = G^T v_t
#pragma unroll
        for (int c = 0; c < C; ++c) p[c] = 0.f;
#pragma unroll
        for (int rr = 0; rr < RPL; ++rr)
#pragma unroll
            for (int c = 0; c < C; ++c) p[c] = fmaf(G[rr][c], vi[rr], p[c]);
        add_rows(kk, 2, p);
        // dw_t[j] = sum_i G[i][j] S_{t-1}[i][j]
#pragma unroll
        for (int c = 0; c < C; ++c) p[c] = 0.f;
#pragma unroll
        for (int rr = 0; rr < RPL; ++rr)
#pragma unroll
            for (int c = 0; c < C; ++c) p[c] = fmaf(G[rr][c], Sp[rr][c], p[c]);
        add_rows(kk, 1, p);
        // dv_t = G k_t: row i's value kept in lane rr of its group
        load_cols<C>(&sm[VK][t][cq * C], V);
        float dv_lane = 0.f;
#pragma unroll
        for (int rr = 0; rr < RPL; ++rr) {
            const float dvi = row16_sum(dot_cols(G[rr], V));
            dv_lane = cq == rr ? dvi : dv_lane;
        }
        sdv[kk][cq < RPL ? row0 + cq : N] = dv_lane;
        if (kAB) {
            // z = S_{t-1} a_t, dz = G b_t; db_t = G^T z, da_t = S_{t-1}^T dz
            float z[RPL], dz[RPL];
            load_cols<C>(&sm[VA][t][cq * C], V);
#pragma unroll
            for (int rr = 0; rr < RPL; ++rr) z[rr] = row16_sum(dot_cols(Sp[rr], V));
            load_cols<C>(&sm[VB][t][cq * C], V);
#pragma unroll
            for (int rr = 0; rr < RPL; ++rr) dz[rr] = row16_sum(dot_cols(G[rr], V));
#pragma unroll
            for (int c = 0; c < C; ++c) p[c] = 0.f;
#pragma unroll
            for (int rr = 0; rr < RPL; ++rr)
#pragma unroll
                for (int c = 0; c < C; ++c) p[c] = fmaf(G[rr][c], z[rr], p[c]);
            add_rows(kk, 4, p);
#pragma unroll
            for (int c = 0; c < C; ++c) p[c] = 0.f;
#pragma unroll
            for (int rr = 0; rr < RPL; ++rr)
#pragma unroll
                for (int c = 0; c < C; ++c) p[c] = fmaf(Sp[rr][c], dz[rr], p[c]);
            add_rows(kk, 3, p);
            // G <- G diag(w_t) + dz a_t^T
            float W[C];
            load_cols<C>(&sm[VW][t][cq * C], W);
            load_cols<C>(&sm[VA][t][cq * C], V);
#pragma unroll
            for (int rr = 0; rr < RPL; ++rr)
#pragma unroll
                for (int c = 0; c < C; ++c) G[rr][c] = fmaf(dz[rr], V[c], G[rr][c] * W[c]);
        } else {
            load_cols<C>(&sm[VW][t][cq * C], V);
#pragma unroll
            for (int rr = 0; rr < RPL; ++rr)
#pragma unroll
                for (int c = 0; c < C; ++c) G[rr][c] *= V[c];
        }
    };

    for (int stg = nstg - 1; stg >= 0; --stg) {
        const int t0 = stg * kTB, nt = min(kTB, T - t0);
        __syncthreads();   // the previous stage's rows and sums are consumed
        const Tin* src[7] = {r, w, k, v, a, b, dy};
        for (int idx = tid; idx < 7 * kTB * (N / 4); idx += NT) {
            const int q = idx / (kTB * (N / 4)), rem = idx % (kTB * (N / 4));
            const int t = rem / (N / 4), c = rem % (N / 4);
            float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
            if (t < nt && (kAB || (q != VA && q != VB)))
                x = Elem<Tin>::load4(src[q] + off(t0 + t) + c * 4);
            *reinterpret_cast<float4*>(&sm[q][t][c * 4]) = x;
        }
        __syncthreads();
        const float* cp = ckpt + ((size_t)bh * nstg + stg) * N * N;
        const int nsub = (nt + KS - 1) / KS;
        for (int sub = nsub - 1; sub >= 0; --sub) {
            float S[RPL][C];
#pragma unroll
            for (int rr = 0; rr < RPL; ++rr) load_cols<C>(cp + (size_t)(row0 + rr) * N + cq * C, S[rr]);
            for (int t = 0; t < sub * KS; ++t) fwd(t, S);
            float Ss[KS + 1][RPL][C];   // Ss[0]: the state before the sub-stage
#pragma unroll
            for (int rr = 0; rr < RPL; ++rr)
#pragma unroll
                for (int c = 0; c < C; ++c) Ss[0][rr][c] = S[rr][c];
            const int kend = min(KS, nt - sub * KS);
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                if (kk < kend) {
                    fwd(sub * KS + kk, S);
#pragma unroll
                    for (int rr = 0; rr < RPL; ++rr)
#pragma unroll
                        for (int c = 0; c < C; ++c) Ss[kk + 1][rr][c] = S[rr][c];
                }
            }
#pragma unroll
            for (int kk = KS - 1; kk >= 0; --kk)
                if (kk < kend) bwd(sub * KS + kk, kk, Ss[kk + 1], Ss[kk]);
            __syncthreads();   // every wave's sums and dv rows of the sub-stage are in LDS
            if constexpr (kSplit == 1) {
                for (int idx = tid; idx < kend * N; idx += NT) {
                    const int kk = idx / N, j = idx % N;
                    float x[NG];
#pragma unroll
                    for (int q = 0; q < NG; ++q) {
                        x[q] = part[0][kk][q][j];
#pragma unroll
                        for (int wv = 1; wv < WAVES; ++wv) x[q] += part[wv][kk][q][j];
                    }
                    const size_t o = off(t0 + sub * KS + kk) + j;
                    Elem<Tin>::store1(dr + o, x[0]);
                    Elem<Tin>::store1(dw + o, x[1]);
                    Elem<Tin>::store1(dk + o, x[2]);
                    Elem<Tin>::store1(dv + o, sdv[kk][j]);
                    if (kAB) {
                        Elem<Tin>::store1(da + o, x[NG > 3 ? 3 : 0]);
                        Elem<Tin>::store1(db + o, x[NG > 4 ? 4 : 0]);
                    }
                }
            } else {
                // this workgroup's share of the per-key sums, PW columns per atomic
                constexpr int PW = std::is_same<Tin, float>::value ? 1 : 2;
                for (int idx = tid; idx < kend * (N / PW); idx += NT) {
                    const int kk = idx / (N / PW), j = PW * (idx % (N / PW));
                    float x[NG][PW];
#pragma unroll
                    for (int q = 0; q < NG; ++q)
#pragma unroll
                        for (int e = 0; e < PW; ++e) {
                            x[q][e] = part[0][kk][q][j + e];
#pragma unroll
                            for (int wv = 1; wv < WAVES; ++wv) x[q][e] += part[wv][kk][q][j + e];
                        }
                    const size_t o = off(t0 + sub * KS + kk) + j;
                    auto add = [&](Tin* dst, const float (&xv)[PW]) __attribute__((always_inline)) {
                        if constexpr (PW == 1) {
                            unsafeAtomicAdd(dst, xv[0]);
                        } else {
                            typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
                            const bf16x2v pv = {(__bf16)xv[0], (__bf16)xv[1]};
                            __builtin_amdgcn_global_atomic_fadd_v2bf16(reinterpret_cast<bf16x2v*>(dst), pv);
                        }
                    };
                    add(dr + o, x[0]);
                    add(dw + o, x[1]);
                    add(dk + o, x[2]);
                    if (kAB) {
                        add(da + o, x[NG > 3 ? 3 : 0]);
                        add(db + o, x[NG > 4 ? 4 : 0]);
                    }
                }
                for (int idx = tid; idx < kend * NR; idx += NT) {   // dv: this workgroup's rows
                    const int kk = idx / NR, jr = half * NR + idx % NR;
                    Elem<Tin>::store1(dv + off(t0 + sub * KS + kk) + jr, sdv[kk][jr]);
                }
            }
            __syncthreads();   // the slots are read before the next sub-stage writes them
        }
    }
    if (ds0) {
#pragma unroll
        for (int rr = 0; rr < RPL; ++rr) store_cols<C>(ds0 + ((size_t)bh * N + row0 + rr) * N + cq * C, G[rr]);
    }
}

// Copies (or zero-fills, when src is null) n4 float4 values.
__global__ __launch_bounds__(256) void state_copy_kernel(size_t n4, const float* __restrict__ src,
                                                         float* __restrict__ dst) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n4)
        reinterpret_cast<float4*>(dst)[i] =
            src ? reinterpret_cast<const float4*>(src)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
}

// Entry states of the split segments at any N (N = 64 has its own kernel):
// S_in(s+1) = S_in(s) P(s) + Hm(s) for s = 1 .. nseg-2, in fp32, from
// S_in(1) = segment 0's final state.  Workgroup (head, q) takes rows
// 16 q .. 16 q + 15 of one split head through every step; thread t owns row
// 16 q + t / 16 and columns t % 16 + 16 e.  Each step stages P in LDS.
template <int N>
__global__ __launch_bounds__(256) void seg_combine_n_kernel(int nseg, float* __restrict__ states) {
    constexpr int NB = N / 16;   // workgroups per split head
    constexpr int E = N / 16;    // columns per thread
    constexpr size_t NN = (size_t)N * N;
    __shared__ float Pm[N][N];
    __shared__ float Sr[16][N];
    float* const hst = states + (size_t)(blockIdx.x / NB) * 3 * nseg * NN;
    const int t = threadIdx.x, li = t / 16, c = t % 16;
    const size_t ro = (size_t)((blockIdx.x % NB) * 16 + li) * N;   // this thread's row
#pragma unroll
    for (int e = 0; e < E; ++e) Sr[li][c + 16 * e] = hst[NN + ro + c + 16 * e];
    for (int sg = 1; sg + 1 < nseg; ++sg) {
        const float* P = hst + (size_t)(2 * nseg + sg) * NN;
        __syncthreads();   // the previous step's reads of Pm and writes of Sr are done
        for (int q = t; q < N * N; q += 256) Pm[q / N][q % N] = P[q];
        float acc[E];
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = hst[(size_t)(nseg + sg) * NN + ro + c + 16 * e];
        __syncthreads();
        for (int kk = 0; kk < N; ++kk) {
            const float sik = Sr[li][kk];
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] = fmaf(sik, Pm[kk][c + 16 * e], acc[e]);
        }
        __syncthreads();   // every row of Sr is read before it is replaced
#pragma unroll
        for (int e = 0; e < E; ++e) {
            hst[(size_t)(sg + 1) * NN + ro + c + 16 * e] = acc[e];
            Sr[li][c + 16 * e] = acc[e];
        }
    }
}

// One launch of `units` head runs (whole heads, segments or map runs of the
// pass, as work_of decodes them), blocks_per_head workgroups each.
template <typename Tin, int N, int WAVES, int P>
hipError_t launch_seq_fwd_w(const FwdArgs& p, int blocks_per_head, int units, int pass,
                            const FwdSplit& sp, hipStream_t stream) {
    const Tin* a = static_cast<const Tin*>(p.a);
    auto kern = a ? seq_fwd_kernel<Tin, N, WAVES, true, P> : seq_fwd_kernel<Tin, N, WAVES, false, P>;
    kern<<<dim3(units * blocks_per_head), dim3(64 * WAVES), 0, stream>>>(
        p.B, p.T, p.H, static_cast<const Tin*>(p.r), static_cast<const Tin*>(p.w),
        static_cast<const Tin*>(p.k), static_cast<const Tin*>(p.v), a,
        static_cast<const Tin*>(p.b), p.s0, static_cast<Tin*>(p.y), p.sT,
        static_cast<bf16_t*>(p.tape), p.ckpt, pass, sp.split_from, sp.nseg, sp.seg_len, sp.states);
    return hipGetLastError();
}

// Heads from which the scan switches to the many-heads layout: it needs
// several workgroups per compute unit to hide its longer per-token chain (at
// 256 and 320 heads it measured from 5 % faster to 35 % slower).
constexpr int kManyHeads = 512;

template <typename Tin, int N>
hipError_t launch_seq_fwd_pass(const FwdArgs& p, int units, int pass, const FwdSplit& sp,
                               hipStream_t stream) {
    // Few heads: 16 lanes per row, each head's rows over workgroups of 4 waves
    // (16 rows) to occupy more compute units.  Many heads: 4 lanes per row, one
    // workgroup of N/16 waves per head (1.3-1.5x the 16-lane form at 512 to
    // 1280 heads); N = 128 keeps 16 lanes per row in two workgroups of 16 waves
    // (8 lanes per row measured 2 % slower there).
    if (units < kManyHeads) return launch_seq_fwd_w<Tin, N, 4, 16>(p, N / 16, units, pass, sp, stream);
    if constexpr (N == 128) return launch_seq_fwd_w<Tin, N, 16, 16>(p, 2, units, pass, sp, stream);
    else return launch_seq_fwd_w<Tin, N, N / 16, 4>(p, 1, units, pass, sp, stream);
}

// The scan under a segment plan: pass 0 (whole heads, segment 0 and the map
// runs of every split head), the composition of the entry states, pass 1.
template <typename Tin, int N>
hipError_t launch_seq_fwd_n(const FwdArgs& p, const FwdSplit& sp, hipStream_t stream) {
    const int nbh = p.B * p.H;
    const int nsplit = nbh - sp.split_from;
    if (nsplit < 0 || (nsplit > 0 && (sp.nseg < 2 || sp.seg_len <= 0 ||
                                       sp.seg_len % 32 != 0 ||   // whole tape blocks
                                       (long long)(sp.nseg - 1) * sp.seg_len >= p.T || !sp.states)))
        return hipErrorInvalidValue;
    hipError_t e = launch_seq_fwd_pass<Tin, N>(
        p, sp.split_from + (nsplit > 0 ? nsplit * (2 * sp.nseg - 3) : 0), 0, sp, stream);
    if (e != hipSuccess || nsplit == 0) return e;
    if (sp.nseg > 2) {
        if constexpr (N == 64) {
            e = launch_seg_combine(nsplit, sp.nseg, sp.states, stream);
        } else {
            seg_combine_n_kernel<N><<<dim3(nsplit * (N / 16)), dim3(256), 0, stream>>>(sp.nseg, sp.states);
            e = hipGetLastError();
        }
        if (e != hipSuccess) return e;
    }
    return launch_seq_fwd_pass<Tin, N>(p, nsplit * (sp.nseg - 1), 1, sp, stream);
}

template <typename Tin>
hipError_t launch_seq_fwd_t(const FwdArgs& p, const FwdSplit& sp, hipStream_t stream) {
    switch (p.N) {
        case 32: return launch_seq_fwd_n<Tin, 32>(p, sp, stream);
        case 64: return launch_seq_fwd_n<Tin, 64>(p, sp, stream);
        case 128: return launch_seq_fwd_n<Tin, 128>(p, sp, stream);
        default: return hipErrorInvalidValue;
    }
}

template <typename Tin, int N>
hipError_t launch_decode_n(const DecodeArgs& p, hipStream_t stream) {
    auto kern = p.a ? decode_kernel<Tin, N, true> : decode_kernel<Tin, N, false>;
    constexpr int HPW = DecodeShape<N>::HPW;
    kern<<<dim3((p.B * p.H + HPW - 1) / HPW), dim3(256), 0, stream>>>(
        p.B * p.H, static_cast<const Tin*>(p.r), static_cast<const Tin*>(p.w),
        static_cast<const Tin*>(p.k), static_cast<const Tin*>(p.v),
        static_cast<const Tin*>(p.a), static_cast<const Tin*>(p.b), p.state,
        static_cast<Tin*>(p.y));
    return hipGetLastError();
}

template <typename Tin>
hipError_t launch_decode_t(const DecodeArgs& p, hipStream_t stream) {
    switch (p.N) {
        case 32: return launch_decode_n<Tin, 32>(p, stream);
        case 64: return launch_decode_n<Tin, 64>(p, stream);
        case 128: return launch_decode_n<Tin, 128>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

template <typename Tin, int N>
hipError_t launch_seq_bwd_n(const SeqBwdArgs& p, hipStream_t stream) {
    if (!p.ckpt_given) {
        FwdArgs f{p.B, p.T, p.H, N, p.bf16, p.r, p.w, p.k, p.v, p.a, p.b, p.s0, nullptr, nullptr, nullptr};
        f.ckpt = const_cast<float*>(p.ckpt);
        const hipError_t e = launch_seq_fwd_n<Tin, N>(f, FwdSplit{p.B * p.H, 1, p.T, nullptr}, stream);
        if (e != hipSuccess) return e;
    }
    if constexpr (N == 128) {
        if (p.split_rows) {
            // The per-key outputs start at zero (a fill kernel: no memset node
            // if the caller captures the stream).
            const size_t n16 = (size_t)p.B * p.T * p.H * N * sizeof(Tin) / 16;
            Tin* outs[5] = {static_cast<Tin*>(p.dr), static_cast<Tin*>(p.dw), static_cast<Tin*>(p.dk),
                            static_cast<Tin*>(p.da), static_cast<Tin*>(p.db)};
            for (int q = 0; q < (p.a ? 5 : 3); ++q) {
                state_copy_kernel<<<dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, stream>>>(
                    n16, nullptr, reinterpret_cast<float*>(outs[q]));
                const hipError_t e = hipGetLastError();
                if (e != hipSuccess) return e;
            }
            auto kern = p.a ? seq_bwd_kernel<Tin, N, true, 2> : seq_bwd_kernel<Tin, N, false, 2>;
            kern<<<dim3(2 * p.B * p.H), dim3(64 * SeqBwdShape<N, 2>::WAVES), 0, stream>>>(
                p.T, p.H, static_cast<const Tin*>(p.r), static_cast<const Tin*>(p.w),
                static_cast<const Tin*>(p.k), static_cast<const Tin*>(p.v),
                static_cast<const Tin*>(p.a), static_cast<const Tin*>(p.b),
                static_cast<const Tin*>(p.dy), p.dsT, p.ckpt, outs[0], outs[1], outs[2],
                static_cast<Tin*>(p.dv), outs[3], outs[4], p.ds0);
            return hipGetLastError();
        }
    }
    auto kern = p.a ? seq_bwd_kernel<Tin, N, true> : seq_bwd_kernel<Tin, N, false>;
    kern<<<dim3(p.B * p.H), dim3(64 * SeqBwdShape<N>::WAVES), 0, stream>>>(
        p.T, p.H, static_cast<const Tin*>(p.r), static_cast<const Tin*>(p.w),
        static_cast<const Tin*>(p.k), static_cast<const Tin*>(p.v), static_cast<const Tin*>(p.a),
        static_cast<const Tin*>(p.b), static_cast<const Tin*>(p.dy), p.dsT, p.ckpt,
        static_cast<Tin*>(p.dr), static_cast<Tin*>(p.dw), static_cast<Tin*>(p.dk),
        static_cast<Tin*>(p.dv), static_cast<Tin*>(p.da), static_cast<Tin*>(p.db), p.ds0);
    return hipGetLastError();
}

template <typename Tin>
hipError_t launch_seq_bwd_t(const SeqBwdArgs& p, hipStream_t stream) {
    switch (p.N) {
        case 32: return launch_seq_bwd_n<Tin, 32>(p, stream);
        case 64: return launch_seq_bwd_n<Tin, 64>(p, stream);
        case 128: return launch_seq_bwd_n<Tin, 128>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_seq_fwd(const FwdArgs& p, hipStream_t stream) {
    return launch_seq_fwd_split(p, FwdSplit{p.B * p.H, 1, p.T, nullptr}, stream);
}

hipError_t launch_seq_fwd_split(const FwdArgs& p, const FwdSplit& sp, hipStream_t stream) {
    return p.bf16 ? launch_seq_fwd_t<bf16_t>(p, sp, stream) : launch_seq_fwd_t<float>(p, sp, stream);
}

hipError_t launch_seg_combine_n(int N, int nsplit, int nseg, float* states, hipStream_t stream) {
    if (nsplit <= 0 || nseg < 3 || !states) return hipErrorInvalidValue;
    switch (N) {
        case 32:
            seg_combine_n_kernel<32><<<dim3(nsplit * 2), dim3(256), 0, stream>>>(nseg, states);
            break;
        case 128:
            seg_combine_n_kernel<128><<<dim3(nsplit * 8), dim3(256), 0, stream>>>(nseg, states);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_state_copy(int BH, int N, const float* s0, float* sT, hipStream_t stream) {
    const size_t n4 = (size_t)BH * N * N / 4;
    state_copy_kernel<<<dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream>>>(n4, s0, sT);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& p, hipStream_t stream) {
    return p.bf16 ? launch_decode_t<bf16_t>(p, stream) : launch_decode_t<float>(p, stream);
}

hipError_t launch_seq_bwd(const SeqBwdArgs& p, hipStream_t stream) {
    return p.bf16 ? launch_seq_bwd_t<bf16_t>(p, stream) : launch_seq_bwd_t<float>(p, stream);
}

}  // namespace wkv7
