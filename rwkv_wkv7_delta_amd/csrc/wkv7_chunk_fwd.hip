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
//   X   = At S0^T + Aak V
//   Z   = Tm X = (Tm At) S0^T + (Tm Aak) V   (row t of Z is z_t = S_{t-1} a_t)
//   Y   = Rt S0^T + Arb Z + Ark V    (row t of Y is y_t)
//   S_L^T = diag(G_L) S0^T + Kb^T V + Bb^T Z
//
// Mapping to gfx950: one workgroup of 10 waves per (b, h), split by role.
//   Producer waves p = 0..3 build each chunk's state-independent factors:
//     E   decay products and scaled vectors for key columns 16p..16p+15, in
//         row layout (a lane per token, four columns each: 8-byte LDS
//         accesses, the running product over tokens a DPP scan); the
//         consumers read Bb, Kb and v transposed (ds_read_b64_tr_b16), which
//         is the layout their matrix-core products take;
//     MW  one 16x16 tile each on waves 2, 3: Arb, Ark.
//   Two more waves form Aab, Aak and the triangular inverse Tm = (I - Aab)^-1
//   (4x4 diagonal blocks in fp32, joined on the matrix core: wkv7_mfma.h),
//   off the producers' path: wave 8 for even chunks, wave 9 for odd ones, each
//   inverse spread over two intervals.
//   The second interval also applies Tm to the state-independent factors of
//   Z: At' = Tm At (written over At) and Aak' = Tm Aak, from hi and lo bf16
//   parts of Tm and Aak (At is exact in bf16).  Applying Tm to the factors
//   instead of to X = At S0^T + Aak V keeps the cancellation that Tm X performs
//   (rows of X grow along a chunk whose removal keys repeat, while Z stays of
//   the order of v) inside those products, and the consumers' chain one
//   product shorter.
//   Consumer waves p = 0..3 own value rows 16p..16p+15 of the state, held as
//   S^T in four 16x16 fp32 accumulator tiles (key blocks); an accumulator
//   tile feeds the next product directly as its B operand (wkv7_mfma.h), so
//   every state-dependent product (Z, Y, the state update) is a left
//   multiplication that reads the state straight from registers.
// The work is software-pipelined with ONE barrier per chunk: in interval
// `it` the producers run E(it) and MW(it-1), the inverse waves the first half
// of chunk it-1's solve and the second half of chunk it-2's, and the
// consumers the state chain of chunk it-3, storing its y (and tape); chunk
// factors pass through four rotating LDS slots (Bh and Kh, read only in the
// interval after E, through two).  Each role needs few enough registers for
// two waves per SIMD, so a consumer's MFMA chain interleaves with a
// producer's VALU work.  Raw token loads run three intervals ahead in a
// register ring.  Chunks beyond T are all-padding (w = 1, everything else 0),
// for which every stage is the identity on the state.

#include "wkv7.h"
#include "wkv7_device.h"
#include "wkv7_epilogue.h"
#include "wkv7_internal.h"
#include "wkv7_mfma.h"

namespace wkv7 {

namespace {

constexpr int kL = 16;
// The kernel's shape for head size N = 32 or 64: N/16 producer and N/16
// consumer waves (16 key columns or value rows each) and two inverse waves
// (640 threads at N = 64, 384 at N = 32, where two workgroups share a compute
// unit).  With the step after the read-out fused (N = 64): 2 more waves for
// it.  Waves go to the four SIMDs in turn, so these take the two SIMDs that
// held only two waves; at three waves per SIMD either way, the register budget
// per wave is the same.
template <int N>
struct FwdShape {
    static_assert(N == 32 || N == 64, "head sizes of the chunked forward");
    static constexpr int P = N / 16;              // producer waves = consumer waves
    static constexpr int threads = 64 * (2 * P + 2);
    static constexpr int threads_epi = threads + 128;
    static constexpr int blocks_per_cu = N == 32 ? 2 : 1;
    // LDS row stride (bf16 elements).  A row of 64 would be exactly one sweep
    // of the four-byte banks, so the row reads below (16 lanes on 16 different
    // rows, same columns) would all hit the same banks; 8 more elements spread them.
    static constexpr int row = N + 8;
};
constexpr int kRow = FwdShape<64>::row;

enum { RAW_R = 0, RAW_W = 1, RAW_K = 2, RAW_A = 3, RAW_B = 4, RAW_V = 5 };
// Tile images in a slot: the A-operand images of Aak' = Tm Aak (from INV) and
// of Arb, Ark (from MW).
enum { TILE_AK = 0, TILE_RB = 1, TILE_RK = 2 };
constexpr int kSlots = 4;
static_assert((kSlots & (kSlots - 1)) == 0, "slot indices are taken with a mask");

// Everything one chunk passes from the producers to the consumers: rows
// [t][j] (the consumers read Bb, Kb and V transposed, which gives them the
// matrix-core operand layouts directly) and "images", register contents
// stored lane by lane (8 bytes per lane, read back by the same lane index).
template <int N>
struct Slot {
    static constexpr int kRow = FwdShape<N>::row;
    bf16_t At[kL][kRow];            // E -> MW, INV; At' = Tm At from INV -> ST
    bf16_t Rt[kL][kRow];            // E -> MW, ST
    bf16_t Bb[kL][kRow], Kb[kL][kRow], V[kL][kRow];   // E -> ST
    float gL[64];   // E -> ST: G_L of key 16 jt + 4 g + q at word 16 g + 4 jt + q
    uint2 tiles[3][64];
};
// Bh and Kh, read only in the interval after E.
template <int N>
struct SlotBK {
    static constexpr int kRow = FwdShape<N>::row;
    bf16_t Bh[kL][kRow], Kh[kL][kRow];
};

template <int N>
struct __align__(16) FwdSmem {
    static constexpr int kRow = FwdShape<N>::row;
    bf16_t raw[2][6][kL][kRow];   // r, w, k, a, b, v of two chunks (bf16 bits)
    Slot<N> sl[kSlots];
    SlotBK<N> bk[2];
    bf16_t Ys[2][kL][kRow];       // read-outs, staged in row layout
    bf16_t Zs[2][kL][kRow];       // removal read-outs, staged for the tape
    bf16_t S0s[2][N][kRow];       // chunk entry states as [j][i], staged for the tape
};
// With the step after the read-out fused (kEpi, N = 64: no tape), the
// read-outs are staged in fp32 over the space of Ys and Zs, and the tape's
// state staging S0s holds the step's own buffers (EpiSmem).
constexpr int kYfRow = kN + 4;
static_assert(offsetof(FwdSmem<64>, Zs) == offsetof(FwdSmem<64>, Ys) + sizeof(FwdSmem<64>::Ys) &&
                  offsetof(FwdSmem<64>, Ys) % 16 == 0 &&
                  2 * kL * kYfRow * sizeof(float) <= sizeof(FwdSmem<64>::Ys) + sizeof(FwdSmem<64>::Zs),
              "fp32 read-out staging fits over Ys and Zs");
struct EpiSmem {
    float ugb[3][kN];          // this head's u, gamma, beta
    float Es[8][kL];           // r . (u * k) per token of chunk c at [c % 8], from interval c to c+4
    bf16_t Vr[2][kL][kRow];    // v rows of chunk c at [c % 2], copied out of its slot in interval c+3
};
static_assert(sizeof(EpiSmem) <= sizeof(FwdSmem<64>::S0s) && offsetof(FwdSmem<64>, S0s) % 16 == 0,
              "the step's buffers fit over the tape's state staging");

__device__ __forceinline__ float bf2f(bf16_t x) { return __uint_as_float((uint32_t)x << 16); }
__device__ __forceinline__ bf16x4 ld4(const bf16_t* p) {
    return __builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2*>(p));
}
__device__ __forceinline__ bf16x8 ld8(const bf16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ bf16x8 ld4x2(const bf16_t* p) { return cat8(ld4(p), ld4(p + 16)); }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));   // plain SSA vector
struct Raw {
    u32x4 x[3];
};

// Sequential segments (kSeq): every head runs as nseg segments in order, one
// workgroup per segment, numbered segment-major: workgroup u runs segment
// u / (B*H) of head u % (B*H).  Its entry state is the final state that the
// head's previous segment (workgroup u - B*H) left in `states` (slot = head),
// announced by the head's flag sync[head] = segments done.  The scheme assumes
// that the device dispatches a grid's workgroups in order: the one waited for
// was dispatched earlier and finishes without waiting on any later one, so the
// wait ends.  It is bounded all the same (`spin_limit` polls, about a second by
// default), so that no fault elsewhere can turn it into a hang; a workgroup
// whose wait expires starts from a NaN state instead of the unpublished one,
// so its y, tape and final state -- and those of every later segment of the
// head, which start from them -- come out NaN rather than plausibly wrong.

// kAB = false: a_t = b_t = 0 (decay-only linear attention, the RWKV-6-style
// recurrence S <- S diag(w_t) + v_t k_t^T).  a and b are then not read; the
// removal read-outs Z, the triangular inverse and the tiles Aak, Arb vanish,
// leaving Y = Rt S0^T + Ark V and S_L^T = diag(G_L) S0^T + Kb^T V; the tape
// holds only the block entry states (its Z part is not written).
//
// kCk: also write the fp32 state entering every chunk (a template parameter, so
// that the kernel without it carries no trace of the stores).
//
// kEpi (N = 64): y_all receives the step after the read-out (wkv7_epilogue.h,
// settings `ep`) instead of y, computed from the fp32 read-outs by two more
// waves; no tape.
template <int N, bool kSeq, bool kAB, bool kCk, bool kEpi>
__global__ __launch_bounds__(kEpi ? FwdShape<N>::threads_epi : FwdShape<N>::threads,
                             FwdShape<N>::blocks_per_cu) void chunk_fwd_kernel(
    int B, int T, int H, const bf16_t* __restrict__ r, const bf16_t* __restrict__ w,
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, const bf16_t* __restrict__ a,
    const bf16_t* __restrict__ b, const float* __restrict__ s0, bf16_t* __restrict__ y_all,
    float* __restrict__ sT, bf16_t* __restrict__ tape_all, float* __restrict__ ckpt_all, int pass,
    int split_from, int nseg, int seg_len, float* __restrict__ states, int* __restrict__ sync,
    int spin_limit, EpiParams ep) {
    static_assert(!kEpi || N == 64, "the fused step is built for N = 64");
    // (these hide the file-scope N = 64 constants in the body below)
    constexpr int kN = N, kRow = FwdShape<N>::row;
    constexpr int kP = FwdShape<N>::P;          // producer (and consumer) waves
    constexpr int K2 = N / 32, JT = N / 16;     // 32-deep halves, 16-wide key tiles
    using Slot = wkv7::Slot<N>;
    using SlotBK = wkv7::SlotBK<N>;
    __shared__ FwdSmem<N> sm;
    float(*const Yf)[kL][kYfRow] = reinterpret_cast<float(*)[kL][kYfRow]>(&sm.Ys[0][0][0]);
    EpiSmem& es = *reinterpret_cast<EpiSmem*>(&sm.S0s[0][0][0]);
    __shared__ int entry_lost_sm;
    constexpr size_t NN = (size_t)kN * kN;
    Work wk;
    int seg = 0;
    bool entry_lost = false;
    if (kSeq) {
        const int nbh = B * H;
        seg = blockIdx.x / nbh;
        const int h = blockIdx.x % nbh;
        if (threadIdx.x == 0) {
            int lost = 0;
            if (seg > 0) {
                for (int spin = 0;
                     __hip_atomic_load(&sync[h], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < seg; ++spin) {
                    if (spin >= spin_limit) {
                        lost = 1;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                }
            }
            entry_lost_sm = lost;
        }
        __syncthreads();
        entry_lost = entry_lost_sm != 0;
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // the previous segment's state
        wk = Work{h, seg * seg_len, seg == nseg - 1 ? T : (seg + 1) * seg_len,
                  seg == 0 ? (s0 ? s0 + (size_t)h * NN : nullptr) : states + (size_t)h * NN,
                  seg == nseg - 1 ? (sT ? sT + (size_t)h * NN : nullptr) : states + (size_t)h * NN,
                  false, false, true};
    } else {
        wk = work_of<N>(blockIdx.x, pass, T, s0, sT, split_from, nseg, seg_len, states);
    }
    const int bh = wk.bh;
    const int bb = bh / H, hh = bh % H;
    const int t_end = wk.t_end;
    bf16_t* const y = wk.outs ? y_all : nullptr;
    bf16_t* const tape = wk.outs ? tape_all : nullptr;
    // fp32 state entering every chunk, [B][H][ceil(T/16)][N (value i)][N (key j)]
    float* const ckpt = (kCk && wk.outs) ? ckpt_all : nullptr;
    const int tid = threadIdx.x;
    // Roles split by wave (the tests are uniform within a wave).  They are left
    // as per-lane conditions: branching on an SGPR copy of the wave index
    // measured several per cent slower.
    const int wave = tid >> 6;
    const bool producer = wave < kP;
    const bool consumer = wave >= kP && wave < 2 * kP;
    const bool inverter = wave >= 2 * kP && wave < 2 * kP + 2;
    const bool epi_wave = kEpi && wave >= 2 * kP + 2;
    const int rtid = tid & (64 * kP - 1);     // index within the role
    const int lane = tid & 63, wp = (tid >> 6) & (kP - 1);
    const int l16 = lane & 15, g = lane >> 4;
    const int col = 16 * wp + l16;            // key column (producer) / value row (consumer)
    // Chunks [c_begin, c_end) of the sequence (t_begin is a multiple of 32).
    const int c_begin = wk.t_begin / kL, c_end = (t_end + kL - 1) / kL;
    // Tape for the backward: removal read-outs Z as [B][T][H][N] bf16, then the
    // state entering every 32-token block (even chunks) as
    // [B][H][nblk][N (key j)][N (value i)] bf16.
    const int nblk = ((T + kL - 1) / kL + 1) / 2;
    bf16_t* const tapeZ = tape;
    bf16_t* const tapeS = tape ? tape + (size_t)B * T * H * kN : nullptr;

    // ---- consumer state: S^T tiles, lane holds S[col][16 jt + 4 g + q] ----------
    f32x4 S[JT];
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) S[jt] = zero4();
    if (consumer) {
        if (kSeq && entry_lost) {
            const float nan = __builtin_nanf("");
#pragma unroll
            for (int jt = 0; jt < JT; ++jt) S[jt] = f32x4{nan, nan, nan, nan};
        } else if (wk.init) {
            const float* base = wk.init + (size_t)col * kN;
#pragma unroll
            for (int jt = 0; jt < JT; ++jt) {
                const float4 x = *reinterpret_cast<const float4*>(base + 16 * jt + 4 * g);
                S[jt][0] = x.x; S[jt][1] = x.y; S[jt][2] = x.z; S[jt][3] = x.w;
            }
            // Settle the loads here: left pending into the loop, the compiler
            // guards every later use of S with a wait on the whole memory
            // counter, which then also waits for the previous chunk's stores.
            __builtin_amdgcn_s_waitcnt(0);
        } else if (wk.ident) {
#pragma unroll
            for (int jt = 0; jt < JT; ++jt)
#pragma unroll
                for (int q = 0; q < 4; ++q) S[jt][q] = col == 16 * jt + 4 * g + q ? 1.f : 0.f;
        }
    }

    // ---- producer raw loads: 6 vectors x 16 tokens x N = 12 N pieces of 16 bytes
    // over 4 N threads.  Thread rtid loads vector 2p + (rtid >= 2N), token
    // (rtid / (N/8)) & 15, columns 8 (rtid % (N/8)) .. +7, for p = 0, 1, 2.
    // Loads are branch-free (tokens from
    // t_end on re-read token t_end-1 and become padding when stashed) and are
    // issued three intervals before use into a three-deep register ring; the
    // stash into LDS happens one interval before use.
    const bool hi = rtid >= 2 * kN;
    const bf16_t* const sp_p[3] = {hi ? w : r, hi ? a : k, hi ? v : b};
    const int ld_t = (rtid / (kN / 8)) & 15, ld_c8 = rtid & (kN / 8 - 1);
    auto load_raw = [&](int c, Raw& o) __attribute__((always_inline)) {
        const int t = min(c * kL + ld_t, t_end - 1);
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
        if ((c + 1) * kL <= t_end) {   // a whole chunk (the common case: no selects)
#pragma unroll
            for (int p = 0; p < 3; ++p)
                *reinterpret_cast<u32x4*>(&sm.raw[c & 1][2 * p + (hi ? 1 : 0)][ld_t][ld_c8 * 8]) = o.x[p];
            return;
        }
        const bool ok = c * kL + ld_t < t_end;
#pragma unroll
        for (int p = 0; p < 3; ++p) {
            const unsigned pad = (p == 0 && hi) ? 0x3F803F80u : 0u;   // padding: w = 1
            const u32x4 padv = {pad, pad, pad, pad};
            *reinterpret_cast<u32x4*>(&sm.raw[c & 1][2 * p + (hi ? 1 : 0)][ld_t][ld_c8 * 8]) =
                ok ? o.x[p] : padv;
        }
    };

    // ---- E (producer): decay products and scaled vectors --------------------------
    // Row layout: lane (g, l16) takes token t = l16 and key columns j0 .. j0+3,
    // j0 = 16p + 4g, so every LDS access is 8 bytes wide and the running product
    // over tokens is a scan along the lanes of a DPP row.
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
        Slot& s = sm.sl[c % kSlots];
        SlotBK& bk = sm.bk[c & 1];
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
        float G4[4] = {X[RAW_W][0], X[RAW_W][1], X[RAW_W][2], X[RAW_W][3]};
        row16_cumprod4(G4[0], G4[1], G4[2], G4[3]);
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            const float Gt = G4[cc];
            const float Gp = row16_prev(Gt, 1.f);
            const float GL = row16_last(Gt);
            const float inv = __builtin_amdgcn_rcpf(Gt);
            gt[cc] = Gt;
            at[cc] = X[RAW_A][cc] * Gp;
            rt[cc] = X[RAW_R][cc] * Gt;
            bh4[cc] = X[RAW_B][cc] * inv;
            kh4[cc] = X[RAW_K][cc] * inv;
            bb4[cc] = bh4[cc] * GL;
            kb4[cc] = kh4[cc] * GL;
        }
        if (kAB) {
            *reinterpret_cast<bf16x4*>(&s.At[l16][j0]) = cvt4(at);
            *reinterpret_cast<bf16x4*>(&bk.Bh[l16][j0]) = cvt4(bh4);
            *reinterpret_cast<bf16x4*>(&s.Bb[l16][j0]) = cvt4(bb4);
        }
        *reinterpret_cast<bf16x4*>(&s.Rt[l16][j0]) = cvt4(rt);
        *reinterpret_cast<bf16x4*>(&bk.Kh[l16][j0]) = cvt4(kh4);
        *reinterpret_cast<bf16x4*>(&s.Kb[l16][j0]) = cvt4(kb4);
        *reinterpret_cast<uint2*>(&s.V[l16][j0]) = wk.vzero ? make_uint2(0u, 0u) : raw6[RAW_V];
        if (l16 == kL - 1) *reinterpret_cast<float4*>(&s.gL[16 * g + 4 * wp]) = make_float4(gt[0], gt[1], gt[2], gt[3]);
    };

    // ---- MW (producer): one 16x16 tile per wave ---------------------------------
    // The last two producer waves (2, 3 at N = 64; 0, 1 at N = 32) form Arb =
    // tril_0(Rt Bh^T), Ark = tril_0(Rt Kh^T) as the transposed product [s][t] =
    // Rt_t . Y_s: accumulator registers of M^T fed as an A operand stand for M,
    // so these are the A-operand images.
    struct MWIn {
        bf16x8 xv[K2], yv[K2];
    };
    auto read_MW = [&](int c) __attribute__((always_inline)) -> MWIn {
        const Slot& s = sm.sl[c % kSlots];
        const SlotBK& bk = sm.bk[c & 1];
        const bf16_t(*Xr)[kRow] = s.Rt;
        const bf16_t(*Yr)[kRow] = (wp & 1) ? bk.Kh : bk.Bh;
        MWIn in;
#pragma unroll
        for (int k2 = 0; k2 < K2; ++k2) {
            in.xv[k2] = ld8(&Xr[l16][32 * k2 + 8 * g]);
            in.yv[k2] = ld8(&Yr[l16][32 * k2 + 8 * g]);
        }
        return in;
    };
    auto stage_MW = [&](int c, const MWIn& in) __attribute__((always_inline)) {
        Slot& s = sm.sl[c % kSlots];
        f32x4 PT = zero4();
#pragma unroll
        for (int k2 = 0; k2 < K2; ++k2) PT = mfma32(in.yv[k2], in.xv[k2], PT);   // [s][t]
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int m = 4 * g + q, n = l16;   // m = s, n = t; Arb, Ark keep the diagonal
            PT[q] = m <= n ? PT[q] : 0.f;
        }
        s.tiles[(wp & 1) == 0 ? TILE_RB : TILE_RK][lane] = __builtin_bit_cast(uint2, cvt4(PT));
    };
    // ---- INV (inverse waves): Aab, Aak, Tm = (I - Aab)^-1, At' and Aak' --------
    // In the interval after E(c) a wave forms Aab = tril_-1(At Bh^T) and Aak =
    // tril_-1(At Kh^T) (accumulator layout [t][s]), the inverses of Aab's 4x4
    // diagonal blocks, N = Td L and N N (wkv7_mfma.h); in the next it joins them
    // into Tm and applies Tm, as hi and lo bf16 images, to the factors of Z:
    //   At'^T tile jt = At^T[keys 16 jt ..] Tm^T, whose accumulator registers
    //     hold At'[l16][16 jt + 4 g + q] -- the row layout of At', written over
    //     the same columns of At (read first, by transposed reads);
    //   Aak'^T = Aak^T Tm^T from Aak's accumulator layout (hi and lo), whose
    //     accumulator registers are Aak''s A-operand image.
    struct InvState {
        BlockInverse bi;
        f32x4 Aak;   // accumulator layout [t][s]
    };
    auto inv_begin = [&](int c) __attribute__((always_inline)) -> InvState {
        const Slot& s = sm.sl[c % kSlots];
        const SlotBK& bk = sm.bk[c & 1];
        bf16x8 xv[K2], yv[K2], kv[K2];
#pragma unroll
        for (int k2 = 0; k2 < K2; ++k2) {
            xv[k2] = ld8(&s.At[l16][32 * k2 + 8 * g]);
            yv[k2] = ld8(&bk.Bh[l16][32 * k2 + 8 * g]);
            kv[k2] = ld8(&bk.Kh[l16][32 * k2 + 8 * g]);
        }
        f32x4 P = zero4(), K = zero4();
#pragma unroll
        for (int k2 = 0; k2 < K2; ++k2) {
            P = mfma32(xv[k2], yv[k2], P);   // [t][s] = Aab[t][s]
            K = mfma32(xv[k2], kv[k2], K);   // [t][s] = Aak[t][s]
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            P[q] = (l16 < 4 * g + q) ? P[q] : 0.f;
            K[q] = (l16 < 4 * g + q) ? K[q] : 0.f;
        }
        return InvState{unit_lower_inverse_begin<true>(P, g, l16), K};
    };
    auto inv_end = [&](int c, const InvState& st) __attribute__((always_inline)) {
        Slot& s = sm.sl[c % kSlots];
        bf16x4 atT[JT];
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) atT[jt] = ld4_tr(tr_addr(&s.At[0][16 * jt], kRow, g, l16));
        const Split4 tm = split4(unit_lower_inverse_rows_end(st.bi, g, l16));
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
            const f32x4 d = mfma16(atT[jt], tm.hi, mfma16(atT[jt], tm.lo, zero4()));
            *reinterpret_cast<bf16x4*>(&s.At[l16][16 * jt + 4 * g]) = cvt4(d);
        }
        s.tiles[TILE_AK][lane] = __builtin_bit_cast(uint2, cvt4(mul3(split4(st.Aak), tm, zero4())));
    };

    // ---- ST (consumer): value-row block `col` of the state chain of chunk c -----
    struct STIn {
        bf16x4 Aak, Arb, Ark, V;
        bf16x8 at[K2], rt[K2];
        bf16x4 bbt[JT], kbt[JT];
        float gl;   // G_L of key 16 jt + 4 g + q sits in lane 4 jt + q of row g
    };
    auto read_ST = [&](int c) __attribute__((always_inline)) -> STIn {
        const Slot& s = sm.sl[c % kSlots];
        STIn in;
        in.Ark = __builtin_bit_cast(bf16x4, s.tiles[TILE_RK][lane]);
        in.V = ld4_tr(tr_addr(&s.V[0][16 * wp], kRow, g, l16));   // [t][i] as a B operand
        if (kAB) {
            in.Aak = __builtin_bit_cast(bf16x4, s.tiles[TILE_AK][lane]);   // Aak' = Tm Aak
            in.Arb = __builtin_bit_cast(bf16x4, s.tiles[TILE_RB][lane]);
        }
#pragma unroll
        for (int k2 = 0; k2 < K2; ++k2) {
            if (kAB) in.at[k2] = ld4x2(&s.At[l16][32 * k2 + 4 * g]);   // At' = Tm At
            in.rt[k2] = ld4x2(&s.Rt[l16][32 * k2 + 4 * g]);
        }
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
            if (kAB) in.bbt[jt] = ld4_tr(tr_addr(&s.Bb[0][16 * jt], kRow, g, l16));   // Bb^T as an A operand
            in.kbt[jt] = ld4_tr(tr_addr(&s.Kb[0][16 * jt], kRow, g, l16));
        }
        in.gl = s.gL[lane];
        return in;
    };
    auto stage_ST = [&](int c, const STIn& in) __attribute__((always_inline)) {
        // Value block `col`: Z = At' S0^T + Aak' V with At' = Tm At, Aak' = Tm Aak
        // (from INV), Y = Rt S0^T + Arb Z + Ark V.  The 32-deep products (over
        // keys) and the 16-deep ones (over tokens) accumulate separately and meet
        // on the vector ALU (add4).
        bf16x4 Sb[JT];
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) Sb[jt] = cvt4(S[jt]);
        if (kCk && ckpt && c < c_end) {   // the entry state in fp32: row col, keys 16 jt + 4 g ..
            float* dst = ckpt + (((size_t)bh * ((T + kL - 1) / kL) + c) * kN + col) * kN + 4 * g;
#pragma unroll
            for (int jt = 0; jt < JT; ++jt)
                store_stream(dst + 16 * jt, __builtin_bit_cast(uint4, S[jt]));
        }
        f32x4 Xs = zero4(), Ys = zero4();
#pragma unroll
        for (int k2 = 0; k2 < K2; ++k2) {
            const bf16x8 bs = cat8(Sb[2 * k2], Sb[2 * k2 + 1]);
            if (kAB) Xs = mfma32(in.at[k2], bs, Xs);
            Ys = mfma32(in.rt[k2], bs, Ys);
        }
        bf16x4 Zb = {};
        f32x4 Yt;
        if (kAB) {
            Zb = cvt4(add4(Xs, mfma16(in.Aak, in.V, zero4())));
            Yt = add4(Ys, mfma16(in.Ark, in.V, mfma16(in.Arb, Zb, zero4())));
        } else {
            Yt = add4(Ys, mfma16(in.Ark, in.V, zero4()));
        }
        f32x4 dec[JT];
        dec[0] = mul_row_lanes4<0>(in.gl, S[0]);
        dec[1] = mul_row_lanes4<1>(in.gl, S[1]);
        if constexpr (JT > 2) {
            dec[2] = mul_row_lanes4<2>(in.gl, S[2]);
            dec[3] = mul_row_lanes4<3>(in.gl, S[3]);
        }
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
            const f32x4 acc = mfma16(in.kbt[jt], in.V, dec[jt]);   // G_L S^T + Kb^T V
            S[jt] = kAB ? mfma16(in.bbt[jt], Zb, acc) : acc;        // + Bb^T Z
        }
        // Outputs are staged in LDS in row layout (swap_layout: lane (g, l16)
        // holds 8 bytes of row l16) and leave next interval as whole 128-byte
        // rows (store_out), which HBM takes far better than 32-byte pieces.
        const int i0 = 16 * wp + 4 * g;
        if constexpr (kEpi) {
            // fp32, row layout: register q holds y of token 4 g + q, value row col
#pragma unroll
            for (int q = 0; q < 4; ++q) Yf[c & 1][4 * g + q][col] = Yt[q];
            return;
        }
        *reinterpret_cast<bf16x4*>(&sm.Ys[c & 1][l16][i0]) = swap_layout(cvt4(Yt), ident);
        if (tape) {
            if (kAB) *reinterpret_cast<bf16x4*>(&sm.Zs[c & 1][l16][i0]) = swap_layout(Zb, ident);
            if ((c & 1) == 0) {   // entry state of a 32-token block as [j][i]: row layout of S^T tile jt
#pragma unroll
                for (int jt = 0; jt < JT; ++jt)
                    *reinterpret_cast<bf16x4*>(&sm.S0s[(c >> 1) & 1][16 * jt + l16][i0]) =
                        swap_layout(Sb[jt], ident);
            }
        }
    };
    // Staged outputs of chunk c to global memory; N/8 consecutive threads write
    // one row (128 bytes at N = 64) with 16-byte stores: threads 0 .. 2N-1 the
    // read-outs, 2N .. 4N-1 the removal read-outs.
    auto store_out = [&](int c) __attribute__((always_inline)) {
        const int row = (rtid / (kN / 8)) & 15, piece = rtid & (kN / 8 - 1);
        const int tt = c * kL + row;
        if (tt < t_end) {
            bf16_t* base = rtid < 2 * kN ? y : (kAB ? tapeZ : nullptr);
            const bf16_t(*src)[kRow] = rtid < 2 * kN ? sm.Ys[c & 1] : sm.Zs[c & 1];
            if (base)
                store_stream(base + tok_off<N>(bb, tt, hh, T, H) + 8 * piece,
                             *reinterpret_cast<const uint4*>(&src[row][8 * piece]));
        }
        if (tape && c < c_end && (c & 1) == 0) {
#pragma unroll
            for (int k2 = 0; k2 < K2; ++k2) {
                const int j = 32 * k2 + rtid / (kN / 8);   // 32 rows of the state per pass
                store_stream(tapeS + (((size_t)bh * nblk + (c >> 1)) * kN + j) * kN + 8 * piece,
                             *reinterpret_cast<const uint4*>(&sm.S0s[(c >> 1) & 1][j][8 * piece]));
            }
        }
    };

    // ---- EPI (kEpi: waves 10, 11): the step after the read-out ----------------
    // Two waves take 8 tokens of a chunk each (wave 10: tokens 0-7, wave 11:
    // 8-15), a group of 8 lanes per token with 8 values per lane:
    //   interval c:   r . (u * k) from the chunk's raw r and k (in LDS for E);
    //   interval c+3: its v rows, copied out of the chunk's slot (E reuses the
    //                 slot in c+4), while the state chain stages its fp32 y;
    //   interval c+4: the step, and the store of the result.
    // g, the only input read from memory for it, is loaded three intervals
    // ahead, as the producers load theirs.  g and the result go through buffer
    // resources bounded to this head's tokens of its batch row (the launcher
    // keeps T * H * N * 2 bytes below 2^31), so rows past T, and the rows of the
    // chunks before the first that the steady-state loop also visits, are
    // dropped by the hardware's range check: every memory access of the loop is
    // unconditional, and the wait for a load three intervals old counts exactly.
    const int epi_row = 8 * (wave & 1) + (lane >> 3), epi_piece = lane & 7;   // waves 10, 11
    typedef unsigned int epi_u4 __attribute__((ext_vector_type(4)));
    const int epi_row_bytes = H * kN * 2;
    auto head_rsrc = [&](const void* base) __attribute__((always_inline)) {
        return __builtin_amdgcn_make_buffer_rsrc(
            base ? const_cast<bf16_t*>(static_cast<const bf16_t*>(base) + ((size_t)bb * T * H + hh) * kN)
                 : nullptr,
            (short)0, base ? T * epi_row_bytes : 0, 0x00020000);
    };
    // byte offset of this lane's piece of token c * 16 + epi_row (negative for
    // the chunks before the first: out of range as an unsigned offset)
    auto epi_off = [&](int c) __attribute__((always_inline)) {
        return (c * kL + epi_row) * epi_row_bytes + 16 * epi_piece;
    };
    auto epi_load_g = [&](const __amdgpu_buffer_rsrc_t& rs, int c) __attribute__((always_inline)) -> uint4 {
        return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, epi_off(c), 0, 0));
    };
    auto unpack8 = [](uint4 q, float (&x)[8]) __attribute__((always_inline)) {
        const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = bf16_lo(w4[i]);
            x[2 * i + 1] = bf16_hi(w4[i]);
        }
    };
    auto epi_coef = [&](int c) __attribute__((always_inline)) {
        const bf16_t(*Rr)[kL][kRow] = sm.raw[c & 1];
        float rr[8], kk[8], uu[8];
        unpack8(*reinterpret_cast<const uint4*>(&Rr[RAW_R][epi_row][8 * epi_piece]), rr);
        unpack8(*reinterpret_cast<const uint4*>(&Rr[RAW_K][epi_row][8 * epi_piece]), kk);
        load_cols<8>(&es.ugb[0][8 * epi_piece], uu);
        float sp = rr[0] * uu[0] * kk[0];
#pragma unroll
        for (int q = 1; q < 8; ++q) sp = fmaf(rr[q] * uu[q], kk[q], sp);
        sp = lanes_sum<8>(sp);
        if (epi_piece == 0) es.Es[c & 7][epi_row] = sp;
    };
    auto epi_copy = [&](int c) __attribute__((always_inline)) {
        *reinterpret_cast<uint4*>(&es.Vr[c & 1][epi_row][8 * epi_piece]) =
            *reinterpret_cast<const uint4*>(&sm.sl[c & (kSlots - 1)].V[epi_row][8 * epi_piece]);
    };
    auto epi_store = [&](const __amdgpu_buffer_rsrc_t& rs, int c, uint4 graw) __attribute__((always_inline)) {
        float x[8], vv[8], gt[8];
        const float4 y0 = *reinterpret_cast<const float4*>(&Yf[c & 1][epi_row][8 * epi_piece]);
        const float4 y1 = *reinterpret_cast<const float4*>(&Yf[c & 1][epi_row][8 * epi_piece + 4]);
        x[0] = y0.x; x[1] = y0.y; x[2] = y0.z; x[3] = y0.w;
        x[4] = y1.x; x[5] = y1.y; x[6] = y1.z; x[7] = y1.w;
        const bool term = ep.u != nullptr;
        float sc = 0.f;
        if (term) {
            unpack8(*reinterpret_cast<const uint4*>(&es.Vr[c & 1][epi_row][8 * epi_piece]), vv);
            sc = es.Es[c & 7][epi_row];
        } else {
#pragma unroll
            for (int q = 0; q < 8; ++q) vv[q] = 0.f;
        }
        if (ep.g) {
            unpack8(graw, gt);
        } else {
#pragma unroll
            for (int q = 0; q < 8; ++q) gt[q] = 1.f;
        }
        // the coefficient is already the whole row's: one lane's share of it is
        // a 1/8 part of a group sum; hand it over as that share
        float gm[8], bt[8];
        load_cols<8>(&es.ugb[1][8 * epi_piece], gm);
        load_cols<8>(&es.ugb[2][8 * epi_piece], bt);
        epilogue_row<8, 8>(x, vv, sc, term, gm, bt, gt, ep.eps, ep.mode);
        const epi_u4 o = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                          pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
        __builtin_amdgcn_raw_buffer_store_b128(o, rs, epi_off(c), 0, 2);   // non-temporal
    };

    if (t_end > wk.t_begin) {
        // Intervals 0 .. nch+3 carry real work (chunk c_begin + i enters in
        // interval i); the count is rounded up to a multiple of three for the
        // unrolled producer loop.  The extra intervals see only all-padding
        // chunks (identity on the state, nothing stored).
        const int nch = c_end - c_begin;
        const int cb = c_begin;
        if (kEpi && tid < 3 * kN / 4) {
            // u, gamma, beta of this head into LDS (absent: 0, 1, 0); every role
            // passes a barrier before its first use
            const int vec = tid / (kN / 4), q4 = tid % (kN / 4);
            const float* src = vec == 0 ? ep.u : vec == 1 ? ep.gamma : ep.beta;
            const float fill = vec == 1 ? 1.f : 0.f;
            *reinterpret_cast<float4*>(&es.ugb[vec][4 * q4]) =
                src ? *reinterpret_cast<const float4*>(src + (size_t)hh * kN + 4 * q4)
                    : make_float4(fill, fill, fill, fill);
        }
        const int n_it = (nch + 6) / 3 * 3;
        // Each role runs its own loop over the same number of intervals (one
        // barrier each), so the compiler sees only loads on the producer side
        // and only stores on the consumer side.  With both kinds in one loop it
        // must treat the memory counter as unordered and wait for it to drain
        // completely, which serialises the producers' read-ahead and makes the
        // consumers wait for their own previous stores.
        if (producer) {
            // The producers set each interval's length: they issue at the inverse
            // waves' priority (below the state chain), which measured about 2 %
            // faster than the default at the 2.9B shape.
            __builtin_amdgcn_s_setprio(2);
            // Register ring: the raw loads of chunk c live in ring slot c % 3
            // until stashed (three named variables, never an array, so that the
            // ring is neither promoted to LDS nor to scratch).
            Raw rb0, rb1, rb2;
            load_raw(cb, rb0);
            load_raw(cb + 1, rb1);
            load_raw(cb + 2, rb2);
            stash_raw(cb, rb0);
            load_raw(cb + 3, rb0);
            __syncthreads();
            // Interval it: E(it) and MW(it-1), stash chunk it+1 and load chunk
            // it+4 into the ring slot it frees.  (A macro, not a
            // lambda, so that the ring stays plain SSA values.)
#define WKV7_FWD_PRODUCE(IT, RING)                                          \
    {                                                                       \
        const int it_ = (IT);                                               \
        const int c_ = cb + it_;                                            \
        const ERaw er = read_E(c_);                                         \
        MWIn mi;                                                            \
        if (it_ >= 1 && (kAB ? wp >= kP - 2 : wp == kP - 1)) mi = read_MW(c_ - 1); \
        stage_E(c_, er);                                                    \
        stash_raw(c_ + 1, RING);                                            \
        load_raw(c_ + 4, RING);                                             \
        if (it_ >= 1 && (kAB ? wp >= kP - 2 : wp == kP - 1)) stage_MW(c_ - 1, mi); \
        __syncthreads();                                                    \
    }
            // Ring slot of interval it is (it + 1) % 3: it = 0, 1, 2 -> rb1, rb2, rb0.
            // No early exit inside the unrolled body: an exit there again makes
            // the compiler drain the whole counter before every stash.
            for (int it = 0; it < n_it; it += 3) {
                WKV7_FWD_PRODUCE(it, rb1);
                WKV7_FWD_PRODUCE(it + 1, rb2);
                WKV7_FWD_PRODUCE(it + 2, rb0);
            }
#undef WKV7_FWD_PRODUCE
        } else if (inverter) {
            __builtin_amdgcn_s_setprio(2);
            __syncthreads();
            // Chunk cb + j belongs to wave 8 + (j & 1), which starts its inverse in
            // interval j + 1 (after E) and finishes it, with At' and Aak', in
            // interval j + 2 (the consumers read them in interval j + 3); so each
            // of the two waves runs one half per interval, `st` carrying an
            // inverse across one barrier.
            const int par = wave & 1;
            InvState st{{zero4(), zero4(), zero4()}, zero4()};
            for (int it = 0; it < n_it; ++it) {
                if (kAB && it >= 1) {
                    if (((it - 1) & 1) == par)
                        st = inv_begin(cb + it - 1);
                    else if (it >= 2)
                        inv_end(cb + it - 2, st);
                }
                __syncthreads();
            }
        } else if (epi_wave) {
            const __amdgpu_buffer_rsrc_t out_rs = head_rsrc(y), g_rs = head_rsrc(ep.g);
            __syncthreads();
            // Interval it: the step for chunk it-4 (its g loaded in interval it-3
            // into ring register it % 3), v of chunk it-3, r . (u * k) of chunk
            // it, and the load of g for chunk it-1 into the register just freed.
            // Unrolled by three (a macro, three named registers) so that the ring
            // is never copied; every step runs from interval 0 on, on chunks
            // before the first whose stores fall out of range.
#define WKV7_EPI_STEP(IT, GREG)                                             \
    {                                                                       \
        const int it_ = (IT);                                               \
        epi_store(out_rs, cb + it_ - 4, GREG);                              \
        if (ep.u) {                                                         \
            epi_copy(cb + it_ - 3);                                         \
            epi_coef(cb + it_);                                             \
        }                                                                   \
        GREG = epi_load_g(g_rs, cb + it_ - 1);                              \
        __syncthreads();                                                    \
    }
            uint4 ga{}, gb{}, gc{};
            for (int it = 0; it < n_it; it += 3) {
                WKV7_EPI_STEP(it, ga);
                WKV7_EPI_STEP(it + 1, gb);
                WKV7_EPI_STEP(it + 2, gc);
            }
#undef WKV7_EPI_STEP
        } else {
            // The state chain is the critical path: its waves issue first (then
            // the inverse wave, then the producers) when several are ready, so
            // their LDS reads after each barrier are not queued behind the
            // producers' traffic.
            __builtin_amdgcn_s_setprio(3);
            __syncthreads();
            // Interval it: the state chain of chunk it-3 and the stores of chunk it-4.
            for (int it = 0; it < n_it; ++it) {
                if (it >= 3) {
                    const STIn si = read_ST(cb + it - 3);
                    stage_ST(cb + it - 3, si);
                    if (!kEpi && it >= 4) store_out(cb + it - 4);
                }
                __syncthreads();
            }
        }
    }

    if (wk.fin && consumer) {
        float* dst = wk.fin + (size_t)col * kN;
#pragma unroll
        for (int jt = 0; jt < JT; ++jt)
            *reinterpret_cast<float4*>(dst + 16 * jt + 4 * g) =
                make_float4(S[jt][0], S[jt][1], S[jt][2], S[jt][3]);
    }
    if (kSeq) {
        __syncthreads();   // every wave's share of the final state is stored
        if (tid == 0) {
            __threadfence();
            __hip_atomic_store(&sync[bh], seg + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// The per-head flags of the sequential segments start at zero.
__global__ void seg_sync_init_kernel(int* __restrict__ sync, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) sync[i] = 0;
}

// Entry states of the split segments: S_in(s+1) = S_in(s) P(s) + Hm(s) for
// s = 1 .. nseg-2, in fp32 (S_in(1) is segment 0's final state).  Rows are
// independent, so workgroup (head, q) takes rows 16 q .. 16 q + 15 of one split
// head through every step; thread t owns row 16 q + t / 16 and columns
// 4 (t % 16) .. +3.  The next step's P and Hm are loaded during the current one.
constexpr int kCombineRows = 16;
__global__ __launch_bounds__(256) void seg_combine_kernel(int nseg, float* __restrict__ states) {
    constexpr size_t NN = (size_t)kN * kN;
    __shared__ float4 Pm[2][kN][kN / 4];
    __shared__ float Sr[kCombineRows][kN + 4];
    float* const hst = states + (size_t)(blockIdx.x / (kN / kCombineRows)) * 3 * nseg * NN;
    const int t = threadIdx.x;
    const int i = (blockIdx.x % (kN / kCombineRows)) * kCombineRows + t / 16, li = t / 16;
    const int c4 = t % 16;
    // P (as 1024 float4, thread t taking t + 256 u) and this thread's piece of
    // Hm, for step sg: plain named registers.
    float4 pn0, pn1, pn2, pn3, hn;
#define WKV7_COMBINE_FETCH(SG)                                                                  \
    {                                                                                           \
        const float4* P_ = reinterpret_cast<const float4*>(hst + (size_t)(2 * nseg + (SG)) * NN); \
        pn0 = P_[t];                                                                            \
        pn1 = P_[t + 256];                                                                      \
        pn2 = P_[t + 512];                                                                      \
        pn3 = P_[t + 768];                                                                      \
        hn = reinterpret_cast<const float4*>(hst + (size_t)(nseg + (SG)) * NN + i * kN)[c4];      \
    }
    *reinterpret_cast<float4*>(&Sr[li][4 * c4]) = reinterpret_cast<const float4*>(hst + NN + i * kN)[c4];
    WKV7_COMBINE_FETCH(1)
    for (int sg = 1; sg + 1 < nseg; ++sg) {
        const int buf = sg & 1;
        Pm[buf][t / 16][t % 16] = pn0;
        Pm[buf][(t + 256) / 16][t % 16] = pn1;
        Pm[buf][(t + 512) / 16][t % 16] = pn2;
        Pm[buf][(t + 768) / 16][t % 16] = pn3;
        float4 acc = hn;
        if (sg + 2 < nseg) WKV7_COMBINE_FETCH(sg + 1)
        __syncthreads();
#pragma unroll 8
        for (int kk = 0; kk < kN; ++kk) {
            const float sik = Sr[li][kk];
            const float4 p = Pm[buf][kk][c4];
            acc.x = fmaf(sik, p.x, acc.x);
            acc.y = fmaf(sik, p.y, acc.y);
            acc.z = fmaf(sik, p.z, acc.z);
            acc.w = fmaf(sik, p.w, acc.w);
        }
        __syncthreads();   // every row of Sr is read before it is replaced
        reinterpret_cast<float4*>(hst + (size_t)(sg + 1) * NN + i * kN)[c4] = acc;
        *reinterpret_cast<float4*>(&Sr[li][4 * c4]) = acc;
    }
#undef WKV7_COMBINE_FETCH
}

}  // namespace

hipError_t launch_chunk_fwd(const FwdArgs& p, int chunk_len, hipStream_t stream) {
    return launch_chunk_fwd_split(p, chunk_len, FwdSplit{p.B * p.H, 1, p.T, nullptr}, stream);
}

namespace {

template <int N>
hipError_t launch_chunk_fwd_sequential_n(const FwdArgs& p, int nseg, int seg_len, float* states,
                                         int* sync, int spin_limit, hipStream_t stream) {
    const int nbh = p.B * p.H;
    seg_sync_init_kernel<<<dim3((nbh + 255) / 256), dim3(256), 0, stream>>>(sync, nbh);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    auto kern = p.a ? (p.ckpt ? chunk_fwd_kernel<N, true, true, true, false> : chunk_fwd_kernel<N, true, true, false, false>)
                    : (p.ckpt ? chunk_fwd_kernel<N, true, false, true, false> : chunk_fwd_kernel<N, true, false, false, false>);
    kern<<<dim3(nbh * nseg), dim3(FwdShape<N>::threads), 0, stream>>>(
        p.B, p.T, p.H, static_cast<const bf16_t*>(p.r), static_cast<const bf16_t*>(p.w),
        static_cast<const bf16_t*>(p.k), static_cast<const bf16_t*>(p.v),
        static_cast<const bf16_t*>(p.a), static_cast<const bf16_t*>(p.b), p.s0,
        static_cast<bf16_t*>(p.y), p.sT, static_cast<bf16_t*>(p.tape), p.ckpt, 2, 0, nseg, seg_len,
        states, sync, spin_limit < 0 ? 0 : spin_limit, EpiParams{});
    return hipGetLastError();
}

template <int N>
hipError_t launch_chunk_fwd_split_n(const FwdArgs& p, const FwdSplit& sp, hipStream_t stream) {
    const int nbh = p.B * p.H;
    const int nsplit = nbh - sp.split_from;
    auto run = [&](int pass, int grid) {
        auto kern = p.a ? (p.ckpt ? chunk_fwd_kernel<N, false, true, true, false> : chunk_fwd_kernel<N, false, true, false, false>)
                        : (p.ckpt ? chunk_fwd_kernel<N, false, false, true, false> : chunk_fwd_kernel<N, false, false, false, false>);
        kern<<<dim3(grid), dim3(FwdShape<N>::threads), 0, stream>>>(
            p.B, p.T, p.H, static_cast<const bf16_t*>(p.r), static_cast<const bf16_t*>(p.w),
            static_cast<const bf16_t*>(p.k), static_cast<const bf16_t*>(p.v),
            static_cast<const bf16_t*>(p.a), static_cast<const bf16_t*>(p.b), p.s0,
            static_cast<bf16_t*>(p.y), p.sT, static_cast<bf16_t*>(p.tape), p.ckpt, pass,
            sp.split_from, sp.nseg, sp.seg_len, sp.states, nullptr, 0, EpiParams{});
        return hipGetLastError();
    };
    hipError_t e = run(0, sp.split_from + (nsplit > 0 ? nsplit * (2 * sp.nseg - 3) : 0));
    if (e != hipSuccess || nsplit == 0) return e;
    if (sp.nseg > 2) {
        // (the scan's composition serves every head size; N = 64 has its own)
        e = N == 64 ? launch_seg_combine(nsplit, sp.nseg, sp.states, stream)
                    : launch_seg_combine_n(N, nsplit, sp.nseg, sp.states, stream);
        if (e != hipSuccess) return e;
    }
    return run(1, nsplit * (sp.nseg - 1));
}

}  // namespace

hipError_t launch_chunk_fwd_sequential(const FwdArgs& p, int chunk_len, int nseg, int seg_len,
                                       float* states, int* sync, int spin_limit, hipStream_t stream) {
    if (chunk_len != kL || !p.bf16) return hipErrorInvalidValue;
    const int nbh = p.B * p.H;
    if (nseg < 1 || seg_len <= 0 || seg_len % WKV7_TAPE_BLOCK != 0 ||
        (long long)(nseg - 1) * seg_len >= p.T || !states || !sync ||
        (long long)nbh * nseg > INT32_MAX)
        return hipErrorInvalidValue;
    switch (p.N) {
        case 32: return launch_chunk_fwd_sequential_n<32>(p, nseg, seg_len, states, sync, spin_limit, stream);
        case 64: return launch_chunk_fwd_sequential_n<64>(p, nseg, seg_len, states, sync, spin_limit, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_chunk_fwd_split(const FwdArgs& p, int chunk_len, const FwdSplit& sp,
                                  hipStream_t stream) {
    if (chunk_len != kL || !p.bf16) return hipErrorInvalidValue;
    const int nbh = p.B * p.H;
    const int nsplit = nbh - sp.split_from;
    if (nsplit < 0 || (nsplit > 0 && (sp.nseg < 2 || sp.seg_len % WKV7_TAPE_BLOCK != 0 || sp.seg_len <= 0 ||
                                       (long long)(sp.nseg - 1) * sp.seg_len >= p.T || !sp.states)))
        return hipErrorInvalidValue;
    switch (p.N) {
        case 32: return launch_chunk_fwd_split_n<32>(p, sp, stream);
        case 64: return launch_chunk_fwd_split_n<64>(p, sp, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_chunk_fwd_epilogue(const FwdArgs& p, const EpiParams& e, hipStream_t stream) {
    if (!p.bf16 || p.N != 64 || p.tape || p.ckpt || e.mode < 0 || e.mode > 2) return hipErrorInvalidValue;
    if (!chunk_fwd_epilogue_fits(p.T, p.H)) return hipErrorInvalidValue;   // 32-bit buffer offsets
    const int nbh = p.B * p.H;
    auto kern = p.a ? chunk_fwd_kernel<64, false, true, false, true> : chunk_fwd_kernel<64, false, false, false, true>;
    kern<<<dim3(nbh), dim3(FwdShape<64>::threads_epi), 0, stream>>>(
        p.B, p.T, p.H, static_cast<const bf16_t*>(p.r), static_cast<const bf16_t*>(p.w),
        static_cast<const bf16_t*>(p.k), static_cast<const bf16_t*>(p.v),
        static_cast<const bf16_t*>(p.a), static_cast<const bf16_t*>(p.b), p.s0,
        static_cast<bf16_t*>(p.y), p.sT, nullptr, nullptr, 0, nbh, 1, p.T, nullptr, nullptr, 0, e);
    return hipGetLastError();
}

hipError_t launch_seg_combine(int nsplit, int nseg, float* states, hipStream_t stream) {
    if (nsplit <= 0 || nseg < 3 || !states) return hipErrorInvalidValue;
    seg_combine_kernel<<<dim3(nsplit * (kN / kCombineRows)), dim3(256), 0, stream>>>(nseg, states);
    return hipGetLastError();
}

}  // namespace wkv7
