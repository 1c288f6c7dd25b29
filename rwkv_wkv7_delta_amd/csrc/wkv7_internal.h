// wkv7_internal.h -- launcher interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace wkv7 {

struct FwdArgs {
    int B, T, H, N;   // N: 32, 64 or 128 (the chunked form at 128: no tape)
    bool bf16;
    const void *r, *w, *k, *v, *a, *b;
    const float* s0;  // may be null
    void* y;          // may be null only when T == 0
    float* sT;        // may be null
    void* tape;       // may be null: bf16 Z [B][T][H][N] then entry states [B][H][nch][N][N]
    float* ckpt = nullptr;   // may be null: fp32 entry state of every 16 tokens
                             // [B][H][ceil(T/16)][N][N] (runs with outputs write theirs)
};

struct BwdArgs {
    int B, T, H;        // B: the batch rows of this call (a slice of the caller's)
    bool bf16;
    const void *r, *w, *k, *v, *a, *b;
    const float* s0;   // may be null
    const void* dy;
    const float* dsT;  // may be null
    const void* tapeZ; // removal read-outs [B][T][H][N] bf16, written by the forward
    const void* tapeS; // block entry states [B][H][nblk][N][N] bf16, written by the forward
    void *dr, *dw, *dk, *dv, *da, *db;
    float* ds0;        // may be null
    void* workX;       // dX [B][T][H][N] bf16
    void* workS;       // adjoint leaving every 32-token block [B][H][nblk][N][N] bf16
    int* counter;      // two ints: the per-key pass's block queue (reset by both passes)
    int N = 64;        // head size: 32 or 64
    // The adjoint chain in time segments (nseg >= 2, every head): segments of
    // seg_len tokens (a multiple of 32; the last takes the rest) composed by
    // maps; `states` holds 3 * nseg fp32 N x N states per head.  nseg = 1: none.
    int nseg = 1, seg_len = 0;
    float* states = nullptr;
};

// The sequential reverse pass: one workgroup per head over its fp32 checkpoints.
struct SeqBwdArgs {
    int B, T, H, N;
    bool bf16;
    const void *r, *w, *k, *v, *a, *b, *dy;   // a, b: both null for a = b = 0
    const float* s0;    // may be null
    const float* dsT;   // may be null
    void *dr, *dw, *dk, *dv, *da, *db;        // da, db: null when a = b = 0
    float* ds0;         // may be null
    float* ckpt;        // [B][H][ceil(T/16)][N][N] fp32: scratch the pass fills first, or
    bool ckpt_given;    // the caller's checkpoints (then no forward re-run)
    // N = 128: each head's rows over two workgroups (the caller's choice: when
    // twice B*H workgroups fit the device at once)
    bool split_rows = false;
};

struct DecodeArgs {
    int B, H, N;      // N: 32, 64 or 128
    bool bf16;
    const void *r, *w, *k, *v, *a, *b;
    float* state;
    void* y;
};

// The learned parts and settings of the step after the read-out (wkv7_epilogue.h).
struct EpiParams {
    const void* g = nullptr;        // gate [B][T][H][N] in the token dtype; null = 1
    const float* u = nullptr;       // [H][N]: current-token weights; null = no term
    const float* gamma = nullptr;   // [H][N]; null = 1
    const float* beta = nullptr;    // [H][N]; null = 0
    float eps = 0.f;
    int mode = 0;                   // 0: no norm; 1: norm, then term; 2: term, then norm
};

// The step after the read-out on its own: y -> out (out may be y).
struct EpiArgs {
    int B, T, H, N;   // N: 32, 64 or 128
    bool bf16;
    const void *y, *r, *k, *v;   // r, k, v are read only with the term (u)
    EpiParams e;
    void* out;
};

hipError_t launch_epilogue(const EpiArgs& p, hipStream_t stream);
// The chunked forward with the step after the read-out fused: p.y receives its
// result; no tape, no checkpoints, no split.  It addresses a head's tokens of one
// batch row with 32-bit byte offsets, so it takes T * H * 64 * 2 < 2^31 only.
hipError_t launch_chunk_fwd_epilogue(const FwdArgs& p, const EpiParams& e, hipStream_t stream);
inline bool chunk_fwd_epilogue_fits(int T, int H) { return (long long)T * H * 64 * 2 < (1LL << 31); }

hipError_t launch_seq_fwd(const FwdArgs& p, hipStream_t stream);
hipError_t launch_chunk_fwd(const FwdArgs& p, int chunk_len, hipStream_t stream);
// The chunked forward at N = 128 (wkv7_chunk128.hip): each head's value rows
// over two workgroups, or one when two would not fit the device's `ncu`
// compute units at once; y, sT and ckpt as in FwdArgs, no tape.
hipError_t launch_chunk_fwd128(const FwdArgs& p, int ncu, hipStream_t stream);
// The same under a segment plan (maps only; FwdSplit below).
struct FwdSplit;
hipError_t launch_chunk_fwd128_split(const FwdArgs& p, const FwdSplit& split, int ncu, hipStream_t stream);

// Segment plan of the chunked forward, split in time.  Heads [0, split_from)
// run whole; heads [split_from, B*H) run as nseg >= 2 segments of seg_len
// tokens (a multiple of 32; the last segment takes the rest, at least one
// token).  `states` holds 3 * nseg fp32 N x N states per split head.
struct FwdSplit {
    int split_from;
    int nseg;
    int seg_len;
    float* states;
};
hipError_t launch_chunk_fwd_split(const FwdArgs& p, int chunk_len, const FwdSplit& split,
                                  hipStream_t stream);
// The sequential scan under the same plan (N = 32, 64 or 128).
hipError_t launch_seq_fwd_split(const FwdArgs& p, const FwdSplit& split, hipStream_t stream);
// Entry states of segments 2 .. nseg-1 of nsplit split heads (N = 64), from
// segment 0's final state and the maps in `states` (the plan's layout).
hipError_t launch_seg_combine(int nsplit, int nseg, float* states, hipStream_t stream);
// The same composition for N = 32 or 128 (wkv7_seq.hip).
hipError_t launch_seg_combine_n(int N, int nsplit, int nseg, float* states, hipStream_t stream);
// Every head as nseg segments of seg_len tokens run in order (one workgroup
// per segment, segment-major); `states` holds one fp32 N x N state per head,
// `sync` B*H ints (cleared by the launch).  A segment polls its predecessor's
// flag at most spin_limit times, then starts from a NaN state.
hipError_t launch_chunk_fwd_sequential(const FwdArgs& p, int chunk_len, int nseg, int seg_len,
                                       float* states, int* sync, int spin_limit, hipStream_t stream);
// stages: bit 0 = the adjoint chain (dv, ds0, workspace), bit 1 = the per-key
// gradients (dr, dw, dk, da, db; reads the workspace the chain wrote).
enum { BWD_CHAIN = 1, BWD_KEYS = 2 };
hipError_t launch_bwd(const BwdArgs& p, int chunk_len, int stages, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& p, hipStream_t stream);
// Forward scan writing the checkpoints, then the reverse pass.
hipError_t launch_seq_bwd(const SeqBwdArgs& p, hipStream_t stream);
hipError_t launch_state_copy(int BH, int N, const float* s0, float* sT, hipStream_t stream);
// Device address of the current device's static scratch (WKV7_STATIC_SCRATCH_BYTES),
// looked up once per device.
hipError_t static_scratch(void** ptr);

}  // namespace wkv7
