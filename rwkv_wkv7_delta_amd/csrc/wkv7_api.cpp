// wkv7_api.cpp -- C ABI of the WKV7 library: validation, dispatch, status codes.
// Declarations and the contract of every entry point are in include/wkv7.h.

#include "wkv7.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdlib.h>

#include "wkv7_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Required pointer: non-null and 16-byte aligned.
bool req(const void* p) { return p != nullptr && aligned16(p); }
// Optional pointer: null, or 16-byte aligned.
bool opt(const void* p) { return p == nullptr || aligned16(p); }
// The removal pair: both given (aligned), or both null for a = b = 0.
bool pair(const void* a, const void* b) { return (a == nullptr && b == nullptr) || (req(a) && req(b)); }

int check_desc(const wkv7_desc* d) {
    if (!d) return WKV7_ERR_INVALID_ARG;
    if (d->B < 0 || d->T < 0 || d->H < 0 || d->N < 0) return WKV7_ERR_INVALID_ARG;
    if (d->N != 32 && d->N != 64 && d->N != 128) return WKV7_ERR_UNSUPPORTED;
    // Every form takes N = 32, 64 and 128, except the chunked backward (N = 32,
    // 64: run_backward) and the chunked forward's tape and time split at N = 128.
    if (d->dtype != WKV7_F32 && d->dtype != WKV7_BF16) return WKV7_ERR_UNSUPPORTED;
    if (d->chunk_len != 0 && d->chunk_len != 16) return WKV7_ERR_UNSUPPORTED;
    // The chunked form runs its products on bf16 matrix cores.
    if (d->chunk_len != 0 && d->dtype != WKV7_BF16) return WKV7_ERR_UNSUPPORTED;
    // Grid dimensions are B*H (times 4) workgroups.
    if ((int64_t)d->B * d->H > (int64_t)(1 << 28)) return WKV7_ERR_UNSUPPORTED;
    // Token and chunk indices are 32-bit in the kernels and their launchers.
    if (d->T > INT32_MAX - 64) return WKV7_ERR_UNSUPPORTED;
    return WKV7_OK;
}

// The chunked form at N = 128 writes no tape, has no chunked backward and no
// sequential segments (its heads split by value rows over two workgroups; it
// splits in time by maps).
bool no_tape(const wkv7_desc* d) { return d->chunk_len != 0 && d->N == 128; }

// Tape: bf16 removal read-outs [B][T][H][N], then the bf16 state entering every
// 32-token block [B][H][ceil(T/32)][N][N].  The backward's own scratch (dX, and
// the adjoint leaving every block) has the same shape.
size_t tape_bytes_unchecked(const wkv7_desc* d) {
    const size_t nblk = ((size_t)d->T + WKV7_TAPE_BLOCK - 1) / WKV7_TAPE_BLOCK;
    const size_t tok = (size_t)d->B * d->T * d->H * d->N;
    const size_t st = (size_t)d->B * d->H * nblk * d->N * d->N;
    return (tok + st) * 2;
}

// Workspace of the backward: its own scratch (dX per token, then the adjoint
// leaving every 32-token block: as large as the tape), the per-key pass's
// block queues (two groups of two ints, in 256 bytes), then -- when no tape is
// passed -- the tape of a forward re-run, then (from a 256-byte boundary) the
// states of the adjoint chain's time split, when there is one.
constexpr size_t kQueueBytes = 256;

// Workspace of the sequential reverse pass (chunk_len = 0): the fp32 state
// entering every 16 tokens, [B][H][ceil(T/16)][N][N].
size_t seq_ckpt_bytes(const wkv7_desc* d) {
    const size_t nstg = ((size_t)d->T + 15) / 16;
    return (size_t)d->B * d->H * nstg * d->N * d->N * sizeof(float);
}

int from_hip(hipError_t e) { return e == hipSuccess ? WKV7_OK : WKV7_ERR_LAUNCH; }

// Compute units of the current device (0 if the runtime cannot say).
int device_cus() {
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    return ncu;
}

// ---- segment plan of wkv7_forward_split --------------------------------------
// Two ways to split a head's sequence in time:
//   maps (mode 0): segment 0 and the two affine-map runs of segments 1 .. n-2
//     side by side, the entry states composed, then segments 1 .. n-1 again:
//     2n - 3 and then n - 1 workgroups of about T / n tokens each, the serial
//     chain falling from T to about 2T / n.  For few heads.
//   sequential (mode 1): the n segments of a head in order, one workgroup per
//     segment, segment-major, each handing its final state to the next: no
//     extra work, but the device takes the segments of every head as they come
//     instead of whole heads.  Only on request: at 320 heads on 256 compute
//     units it measured 476 us (n = 2) to 499 us (n = 4) for the 2.9B-shape
//     forward with tape, against 465 us for maps on the last, partial round of
//     heads and 456 us for no split once the heads were spread over the XCDs
//     (every segment pays the pipeline fill, and heads that no longer step
//     through the tokens together read their token rows at different times).
constexpr int kMaxSegments = 16;
constexpr int kMinSegmentTokens = 128;

// Polls of a sequential segment's wait for its predecessor (each a short sleep:
// about a second in all); WKV7_SEGMENT_SPIN_LIMIT, a non-negative integer,
// overrides it (a small value forces the wait to expire, for testing that an
// expired wait shows as NaN outputs).
int segment_spin_limit() {
    const char* e = getenv("WKV7_SEGMENT_SPIN_LIMIT");
    if (e && *e) {
        char* end = nullptr;
        const long v = strtol(e, &end, 10);
        if (end && *end == '\0' && v >= 0 && v <= (1L << 30)) return (int)v;
    }
    return 1 << 24;
}

struct SplitPlan {
    int split_from, nseg, seg_len, mode;
};

int segment_length(int T, int& nseg) {
    // Segments start at multiples of the tape's state block; the last one must
    // keep at least one token.  (64-bit arithmetic: T may be close to INT32_MAX.)
    while (nseg >= 2) {
        const int64_t per = ((int64_t)T + nseg - 1) / nseg;
        const int64_t len = (per + WKV7_TAPE_BLOCK - 1) / WKV7_TAPE_BLOCK * WKV7_TAPE_BLOCK;
        if ((nseg - 1) * len < T) return (int)len;
        --nseg;
    }
    return T;
}

SplitPlan plan_split(const wkv7_desc* d, int segments, int ncu) {
    const int nbh = d->B * d->H;
    const SplitPlan none{nbh, 1, d->T, 0};
    // The scan (chunk_len 0) splits by maps only.
    const bool scan = d->chunk_len == 0;
    if (nbh == 0 || d->T == 0 || segments == 1 || segments == -1 || ((scan || no_tape(d)) && segments < 0))
        return none;
    int from = 0, nseg = segments, mode = 0;
    if (segments < 0) {
        mode = 1;
        nseg = -segments;
    } else if (segments == 0) {
        // Automatic: split every head when the heads fill at most a third of
        // the device; else, with more heads than compute units, split the heads
        // of the last, partial round when they fill at most a fifth of it (both
        // by maps, with as many segments as the device holds).  On 256 compute
        // units (B = 8, T = 4096) the partial-round split took 0.341 against
        // 0.453 ms unsplit at 272 heads and 0.373 against 0.463 ms at 288, but
        // 0.462 against 0.456 ms at 320: there the second round's 64 heads start
        // as soon as the first round's faster heads finish.
        // The scan runs N/16 workgroups per head and no partial rounds: it
        // splits every head when those fill at most half of the device (at
        // 48 heads, 3/4 of it, segments measured no faster; at 320 heads
        // the chunked form's tail split made the scan 14 % slower).
        if (ncu <= 0) return none;
        // The chunked form at N = 32 runs two workgroups per compute unit; at
        // N = 128 two workgroups per head, each on a compute unit of its own,
        // while they fit at once (every head split when the pairs fill at most
        // a third of the device), else one per head: the heads of a last,
        // partial round are split when they fill at most a quarter of it
        // (B = 8, T = 4096: 264-288 heads 0.94 -> 0.77 ms, 320 heads 0.951 ->
        // 0.889 ms).
        if (!scan && d->N == 32) ncu *= 2;
        int part = nbh;
        if (scan) {
            if ((int64_t)nbh * (d->N / 16) * 2 > ncu) return none;
        } else if (no_tape(d) && 2 * nbh <= ncu) {
            ncu /= 2;   // two workgroups per head
        } else if (no_tape(d) && nbh <= ncu) {
            return none;   // one workgroup per head, one round
        } else if (nbh > ncu) {
            part = nbh % ncu;
            from = nbh - part;
            if ((no_tape(d) ? 4 : 5) * part > ncu) return none;
        }
        if (part == 0 || 3 * part > ncu) return none;
        nseg = (ncu / part + 3) / 2;
        // At N = 128 the map runs and the compositions cost more: with 4 or 12
        // heads 4 segments measured best for the scan (2.3x and 1.2x; 16
        // segments no faster than none) and about best for the chunked form
        // (B = 1: T = 2048, H = 4 0.170 -> 0.145 ms, 16 segments 0.340; T = 4096,
        // H = 12 0.337 -> 0.229 ms, 6 segments 0.219).
        if (d->N == 128 && nseg > 4) nseg = 4;
        if (nseg > d->T / kMinSegmentTokens) nseg = d->T / kMinSegmentTokens;
    }
    if (nseg > kMaxSegments) nseg = kMaxSegments;
    const int len = segment_length(d->T, nseg);
    if (nseg < 2) return none;
    return SplitPlan{from, nseg, len, mode};
}

size_t split_bytes(const wkv7_desc* d, const SplitPlan& p);

// The chunked backward splits its adjoint chain in time under the forward's
// automatic plan when that plan splits every head (few heads: the chain is one
// serial run per head, like the forward's); its states follow the rest of the
// workspace.
SplitPlan plan_bwd(const wkv7_desc* d) {
    const SplitPlan none{d->B * d->H, 1, d->T, 0};
    if (d->chunk_len == 0) return none;
    const SplitPlan p = plan_split(d, 0, device_cus());
    return p.nseg >= 2 && p.mode == 0 && p.split_from == 0 ? p : none;
}

// Offset of the split states in the backward's workspace, and its whole size.
size_t bwd_states_offset(const wkv7_desc* d, bool with_tape) {
    return (tape_bytes_unchecked(d) * (with_tape ? 1 : 2) + kQueueBytes + 255) / 256 * 256;
}
size_t bwd_workspace_bytes(const wkv7_desc* d, bool with_tape, const SplitPlan& bp);

size_t split_bytes(const wkv7_desc* d, const SplitPlan& p) {
    const size_t nbh = (size_t)d->B * d->H;
    const size_t st = (size_t)d->N * d->N * sizeof(float);
    if (p.nseg < 2) return 0;
    if (p.mode == 1) return nbh * st + (nbh * sizeof(int) + 255) / 256 * 256;
    const size_t nsplit = nbh - p.split_from;
    return nsplit == 0 ? 0 : nsplit * 3 * p.nseg * st;
}

size_t bwd_workspace_bytes(const wkv7_desc* d, bool with_tape, const SplitPlan& bp) {
    if (bp.nseg >= 2) return bwd_states_offset(d, with_tape) + split_bytes(d, bp);
    return tape_bytes_unchecked(d) * (with_tape ? 1 : 2) + kQueueBytes;
}

int run_forward(const wkv7_desc* d, const void* r, const void* w, const void* k, const void* v,
                const void* a, const void* b, const float* s0, void* y, float* sT,
                void* tape, hipStream_t stream, float* ckpt = nullptr) {
    if ((int64_t)d->B * d->H == 0) return WKV7_OK;
    if (d->T == 0) {
        if (sT) return from_hip(wkv7::launch_state_copy(d->B * d->H, d->N, s0, sT, stream));
        return WKV7_OK;
    }
    wkv7::FwdArgs p{d->B, d->T, d->H, d->N, d->dtype == WKV7_BF16, r, w, k, v, a, b, s0, y, sT, tape};
    p.ckpt = ckpt;
    if (d->chunk_len == 0) return from_hip(wkv7::launch_seq_fwd(p, stream));
    if (d->N == 128) {
        // No tape at N = 128 (the chunked backward takes N = 32 and 64).
        if (tape) return WKV7_ERR_UNSUPPORTED;
        return from_hip(wkv7::launch_chunk_fwd128(p, device_cus(), stream));
    }
    return from_hip(wkv7::launch_chunk_fwd(p, d->chunk_len, stream));
}

// The step after the read-out: settings valid and the per-head vectors aligned.
bool epi_params_ok(const wkv7_epilogue_params* e) {
    return e != nullptr && e->mode >= WKV7_EPI_PLAIN && e->mode <= WKV7_EPI_TERM_NORM &&
           isfinite(e->eps) && e->eps >= 0.f && opt(e->u) && opt(e->gamma) && opt(e->beta);
}

wkv7::EpiParams epi_params(const wkv7_epilogue_params* e, const void* g) {
    wkv7::EpiParams p;
    p.g = g;
    p.u = e->u;
    p.gamma = e->gamma;
    p.beta = e->beta;
    p.eps = e->eps;
    p.mode = e->mode;
    return p;
}

}  // namespace

extern "C" {

int wkv7_abi_version(void) { return WKV7_ABI_VERSION; }

const char* wkv7_status_string(int status) {
    switch (status) {
        case WKV7_OK: return "ok";
        case WKV7_ERR_INVALID_ARG: return "invalid argument (size, null or misaligned pointer)";
        case WKV7_ERR_UNSUPPORTED: return "unsupported configuration (head size, dtype or chunk length)";
        case WKV7_ERR_WORKSPACE: return "workspace too small";
        case WKV7_ERR_LAUNCH: return "kernel launch failed";
        case WKV7_ERR_STATIC_SCRATCH:
            return "the call needs more scratch than the library's static buffer holds "
                   "(WKV7_STATIC_SCRATCH_BYTES = 16 MiB); use wkv7_forward_split with a workspace";
        default: return "unknown status";
    }
}

size_t wkv7_tape_bytes(const wkv7_desc* desc) {
    if (check_desc(desc) != WKV7_OK || no_tape(desc)) return 0;
    return tape_bytes_unchecked(desc);
}

size_t wkv7_ckpt_bytes(const wkv7_desc* desc) {
    if (check_desc(desc) != WKV7_OK) return 0;
    return seq_ckpt_bytes(desc);
}

size_t wkv7_backward_workspace_bytes(const wkv7_desc* desc, int with_tape) {
    if (check_desc(desc) != WKV7_OK) return 0;
    if (desc->chunk_len == 0) return seq_ckpt_bytes(desc);
    if (desc->dtype != WKV7_BF16 || no_tape(desc)) return 0;
    return bwd_workspace_bytes(desc, with_tape != 0, plan_bwd(desc));
}

size_t wkv7_workspace_bytes(const wkv7_desc* desc) { return wkv7_backward_workspace_bytes(desc, 0); }

int wkv7_forward(const wkv7_desc* desc, const void* r, const void* w, const void* k,
                 const void* v, const void* a, const void* b, const float* s0, void* y,
                 float* sT, void* tape, void* stream) {
    const int st = check_desc(desc);
    if (st != WKV7_OK) return st;
    const bool has_tokens = (int64_t)desc->B * desc->T * desc->H > 0;
    if (has_tokens && !(req(r) && req(w) && req(k) && req(v) && pair(a, b) && req(y)))
        return WKV7_ERR_INVALID_ARG;
    if (!(opt(s0) && opt(sT) && opt(tape))) return WKV7_ERR_INVALID_ARG;
    return run_forward(desc, r, w, k, v, a, b, s0, y, sT, tape, static_cast<hipStream_t>(stream));
}

int wkv7_forward_ckpt(const wkv7_desc* desc, const void* r, const void* w, const void* k,
                      const void* v, const void* a, const void* b, const float* s0, void* y,
                      float* sT, float* ckpt, void* stream) {
    const int st = check_desc(desc);
    if (st != WKV7_OK) return st;
    const bool has_tokens = (int64_t)desc->B * desc->T * desc->H > 0;
    if (has_tokens && !(req(r) && req(w) && req(k) && req(v) && pair(a, b) && req(y)))
        return WKV7_ERR_INVALID_ARG;
    if (!(opt(s0) && opt(sT) && opt(ckpt))) return WKV7_ERR_INVALID_ARG;
    return run_forward(desc, r, w, k, v, a, b, s0, y, sT, nullptr, static_cast<hipStream_t>(stream),
                       ckpt);
}

size_t wkv7_forward_split_workspace_bytes(const wkv7_desc* desc, int32_t segments) {
    if (check_desc(desc) != WKV7_OK || segments < -kMaxSegments) return 0;
    return split_bytes(desc, plan_split(desc, segments, segments == 0 ? device_cus() : 0));
}

int wkv7_forward_split_plan(const wkv7_desc* desc, int32_t segments, wkv7_split_plan* plan) {
    const int st = check_desc(desc);
    if (st != WKV7_OK) return st;
    if (plan == nullptr || segments < -kMaxSegments) return WKV7_ERR_INVALID_ARG;
    if ((desc->chunk_len == 0 || no_tape(desc)) && segments < -1) return WKV7_ERR_UNSUPPORTED;
    const SplitPlan p = plan_split(desc, segments, segments == 0 ? device_cus() : 0);
    plan->kind = p.nseg < 2 ? WKV7_SPLIT_NONE : p.mode == 1 ? WKV7_SPLIT_SEQUENTIAL : WKV7_SPLIT_MAPS;
    plan->split_from = p.split_from;
    plan->nseg = p.nseg;
    plan->seg_len = p.seg_len;
    return WKV7_OK;
}

}  // extern "C"

namespace {

// wkv7_forward_split; `use_static` takes the scratch from the library's static
// buffer instead of `workspace`.
int run_forward_split(const wkv7_desc* desc, const void* r, const void* w, const void* k,
                      const void* v, const void* a, const void* b, const float* s0, void* y,
                      float* sT, void* tape, int32_t segments, void* workspace,
                      size_t workspace_bytes, void* stream, bool use_static) {
    const int st = check_desc(desc);
    if (st != WKV7_OK) return st;
    if (segments < -kMaxSegments) return WKV7_ERR_INVALID_ARG;
    if (desc->chunk_len == 0 || no_tape(desc) ? segments < -1
                                              : (segments > 1 || segments < -1) && desc->chunk_len != 16)
        return WKV7_ERR_UNSUPPORTED;
    if (no_tape(desc) && tape) return WKV7_ERR_UNSUPPORTED;
    const bool has_tokens = (int64_t)desc->B * desc->T * desc->H > 0;
    if (has_tokens && !(req(r) && req(w) && req(k) && req(v) && pair(a, b) && req(y)))
        return WKV7_ERR_INVALID_ARG;
    if (!(opt(s0) && opt(sT) && opt(tape) && opt(workspace))) return WKV7_ERR_INVALID_ARG;
    const SplitPlan plan = plan_split(desc, segments, segments == 0 ? device_cus() : 0);
    const size_t need = split_bytes(desc, plan);
    if (use_static && need > 0) {
        if (need > WKV7_STATIC_SCRATCH_BYTES) return WKV7_ERR_STATIC_SCRATCH;
        if (wkv7::static_scratch(&workspace) != hipSuccess) return WKV7_ERR_LAUNCH;
        workspace_bytes = WKV7_STATIC_SCRATCH_BYTES;
    }
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return WKV7_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (need == 0) return run_forward(desc, r, w, k, v, a, b, s0, y, sT, tape, s);
    const wkv7::FwdArgs p{desc->B, desc->T, desc->H, desc->N, desc->dtype == WKV7_BF16,
                          r, w, k, v, a, b, s0, y, sT, tape};
    const wkv7::FwdSplit sp{plan.split_from, plan.nseg, plan.seg_len, static_cast<float*>(workspace)};
    if (desc->chunk_len == 0) return from_hip(wkv7::launch_seq_fwd_split(p, sp, s));
    if (no_tape(desc)) return from_hip(wkv7::launch_chunk_fwd128_split(p, sp, device_cus(), s));
    if (plan.mode == 1) {
        float* states = static_cast<float*>(workspace);
        int* sync = reinterpret_cast<int*>(states + (size_t)desc->B * desc->H * desc->N * desc->N);
        return from_hip(wkv7::launch_chunk_fwd_sequential(p, 16, plan.nseg, plan.seg_len, states,
                                                          sync, segment_spin_limit(), s));
    }
    return from_hip(wkv7::launch_chunk_fwd_split(p, 16, sp, s));
}

}  // namespace

extern "C" {

int wkv7_forward_split(const wkv7_desc* desc, const void* r, const void* w, const void* k,
                       const void* v, const void* a, const void* b, const float* s0, void* y,
                       float* sT, void* tape, int32_t segments, void* workspace,
                       size_t workspace_bytes, void* stream) {
    return run_forward_split(desc, r, w, k, v, a, b, s0, y, sT, tape, segments, workspace,
                             workspace_bytes, stream, false);
}

int wkv7_forward_split_static(const wkv7_desc* desc, const void* r, const void* w,
                              const void* k, const void* v, const void* a, const void* b,
                              const float* s0, void* y, float* sT, void* tape, int32_t segments,
                              void* stream) {
    return run_forward_split(desc, r, w, k, v, a, b, s0, y, sT, tape, segments, nullptr, 0, stream,
                             true);
}

}  // extern "C"

namespace {

// The backward's arguments restricted to batch rows [b0, b0 + nb).
wkv7::BwdArgs slice(const wkv7_desc* d, int b0, int nb, const void* r, const void* w,
                    const void* k, const void* v, const void* a, const void* b, const float* s0,
                    const void* dy, const float* dsT, const void* tape, void* dr, void* dw,
                    void* dk, void* dv, void* da, void* db, float* ds0, void* workspace,
                    int group) {
    const size_t tok = (size_t)d->T * d->H * d->N;                 // elements per batch row
    const size_t nblk = ((size_t)d->T + WKV7_TAPE_BLOCK - 1) / WKV7_TAPE_BLOCK;
    const size_t st = (size_t)d->H * nblk * d->N * d->N;         // elements per batch row
    const size_t sst = (size_t)d->H * d->N * d->N;               // fp32 state elements per row
    const size_t ztot = (size_t)d->B * tok;
    auto tk = [&](const void* p) -> const void* {
        return p ? static_cast<const uint16_t*>(p) + (size_t)b0 * tok : nullptr;
    };
    auto tkm = [&](void* p) -> void* { return p ? static_cast<uint16_t*>(p) + (size_t)b0 * tok : nullptr; };
    auto sf = [&](const float* p) -> const float* { return p ? p + (size_t)b0 * sst : nullptr; };
    const uint16_t* tp = static_cast<const uint16_t*>(tape);
    uint16_t* wsp = static_cast<uint16_t*>(workspace);
    int* queue = reinterpret_cast<int*>(static_cast<char*>(workspace) + tape_bytes_unchecked(d)) + 2 * group;
    wkv7::BwdArgs p{nb, d->T, d->H, true, tk(r), tk(w), tk(k), tk(v), tk(a), tk(b), sf(s0),
                    tk(dy), sf(dsT), tp + (size_t)b0 * tok, tp + ztot + (size_t)b0 * st,
                    tkm(dr), tkm(dw), tkm(dk), tkm(dv), tkm(da), tkm(db),
                    ds0 ? ds0 + (size_t)b0 * sst : nullptr, wsp + (size_t)b0 * tok,
                    wsp + ztot + (size_t)b0 * st, queue};
    p.N = d->N;
    return p;
}

// Shared by every backward entry point.  stages: the passes to run; aux: a
// second stream (or null) that lets the per-key pass of the first batch rows
// overlap the adjoint chain of the remaining ones.
int run_backward(const wkv7_desc* desc, const void* r, const void* w, const void* k,
                 const void* v, const void* a, const void* b, const float* s0, const void* dy,
                 const float* dsT, const void* tape, void* dr, void* dw, void* dk, void* dv,
                 void* da, void* db, float* ds0, void* workspace, size_t workspace_bytes,
                 void* stream, int stages, void* aux, const float* ckpt = nullptr) {
    int st = check_desc(desc);
    if (st != WKV7_OK) return st;
    const bool seq = desc->chunk_len == 0;
    // The chunked adjoint runs on bf16 matrix cores at N = 32 and 64; the
    // sequential reverse pass (chunk_len = 0) takes either dtype and N = 32, 64,
    // 128, and has no separate stages.
    if (!seq && (desc->dtype != WKV7_BF16 || no_tape(desc))) return WKV7_ERR_UNSUPPORTED;
    if (seq && stages != (wkv7::BWD_CHAIN | wkv7::BWD_KEYS)) return WKV7_ERR_UNSUPPORTED;
    if ((int64_t)desc->B * desc->H * (((int64_t)desc->T + WKV7_TAPE_CHUNK - 1) / WKV7_TAPE_CHUNK) > INT32_MAX)
        return WKV7_ERR_UNSUPPORTED;
    const bool has_tokens = (int64_t)desc->B * desc->T * desc->H > 0;
    // With a = b = 0 (both null) da and db are not written and may be null.
    const bool ab = a != nullptr;
    if (has_tokens && !(req(r) && req(w) && req(k) && req(v) && pair(a, b) && req(dy) &&
                        req(dr) && req(dw) && req(dk) && req(dv) &&
                        (ab ? req(da) && req(db) : opt(da) && opt(db))))
        return WKV7_ERR_INVALID_ARG;
    if (!(opt(s0) && opt(dsT) && opt(tape) && opt(ds0) && opt(workspace)))
        return WKV7_ERR_INVALID_ARG;
    // A single stage needs the forward's tape: the workspace carries the
    // chain's results to the second stage, and a re-run would overwrite it.
    if (stages != (wkv7::BWD_CHAIN | wkv7::BWD_KEYS) && has_tokens && !tape)
        return WKV7_ERR_INVALID_ARG;
    // The sequential pass reads the caller's fp32 checkpoints (then it needs no
    // scratch), else it writes its own; it never reads the tape.
    const SplitPlan bp = seq ? SplitPlan{desc->B * desc->H, 1, desc->T, 0} : plan_bwd(desc);
    const size_t need = seq ? (ckpt ? 0 : seq_ckpt_bytes(desc))
                            : bwd_workspace_bytes(desc, tape != nullptr, bp);
    if (has_tokens && need > 0 && (workspace == nullptr || workspace_bytes < need))
        return WKV7_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((int64_t)desc->B * desc->H == 0) return WKV7_OK;
    if (desc->T == 0) {
        // L = <dsT, S_T> with S_T = s0: ds0 = dsT.
        if (ds0 && (stages & wkv7::BWD_CHAIN))
            return from_hip(wkv7::launch_state_copy(desc->B * desc->H, desc->N, dsT, ds0, s));
        return WKV7_OK;
    }
    char* ws = static_cast<char*>(workspace);
    if (seq) {
        // The sequential reverse pass reads fp32 checkpoints: the caller's or its
        // own, written into the workspace first (the tape is not used).
        wkv7::SeqBwdArgs p{desc->B, desc->T, desc->H, desc->N, desc->dtype == WKV7_BF16,
                           r, w, k, v, a, b, dy, s0, dsT, dr, dw, dk, dv, da, db, ds0,
                           ckpt ? const_cast<float*>(ckpt) : static_cast<float*>(workspace),
                           ckpt != nullptr};
        // N = 128 with few heads: each head's rows over two workgroups (0.19B
        // shape, B = 4, T = 1024, H = 12: fp32 5.65 -> 3.75 ms, bf16 5.6 -> 3.66).
        const int64_t nbh = (int64_t)desc->B * desc->H;
        p.split_rows = desc->N == 128 && 2 * nbh <= device_cus() &&
                       nbh * desc->T * desc->N / 1024 < INT32_MAX;
        return from_hip(wkv7::launch_seq_bwd(p, s));
    }
    const bool tape_given = tape != nullptr;
    if (!tape) {
        // Re-run the forward (without y) into the last part of the workspace.
        void* own = ws + tape_bytes_unchecked(desc) + kQueueBytes;
        st = run_forward(desc, r, w, k, v, a, b, s0, nullptr, nullptr, own, s);
        if (st != WKV7_OK) return st;
        tape = own;
    }
    // Two groups of batch rows when a second stream is given and the heads
    // exceed one per compute unit: the first group's chain fills the device
    // in one round, and its per-key pass runs beside the second group's chain.
    int b1 = desc->B;
    if (aux && desc->B > 1) {
        // (at N = 32 two chains share a compute unit)
        const int ncu = device_cus() * (desc->N == 32 ? 2 : 1);
        if (ncu > 0 && (int64_t)desc->B * desc->H > ncu) {
            b1 = ncu / desc->H;
            if (b1 < 1) b1 = 1;
            if (b1 > desc->B - 1) b1 = desc->B - 1;
        }
    }
    wkv7::BwdArgs g1 = slice(desc, 0, b1, r, w, k, v, a, b, s0, dy, dsT, tape, dr, dw, dk, dv,
                             da, db, ds0, ws, 0);
    if (bp.nseg >= 2 && b1 == desc->B) {   // the adjoint chain in time segments
        g1.nseg = bp.nseg;
        g1.seg_len = bp.seg_len;
        g1.states = reinterpret_cast<float*>(ws + bwd_states_offset(desc, tape_given));
    }
    if (b1 == desc->B) return from_hip(wkv7::launch_bwd(g1, 16, stages, s));
    const wkv7::BwdArgs g2 = slice(desc, b1, desc->B - b1, r, w, k, v, a, b, s0, dy, dsT, tape,
                                   dr, dw, dk, dv, da, db, ds0, ws, 1);
    hipStream_t s2 = static_cast<hipStream_t>(aux);
    hipEvent_t chained = nullptr, keyed = nullptr;
    if (hipEventCreateWithFlags(&chained, hipEventDisableTiming) != hipSuccess) return WKV7_ERR_LAUNCH;
    if (hipEventCreateWithFlags(&keyed, hipEventDisableTiming) != hipSuccess) {
        (void)hipEventDestroy(chained);
        return WKV7_ERR_LAUNCH;
    }
    hipError_t e = wkv7::launch_bwd(g1, 16, wkv7::BWD_CHAIN, s);
    if (e == hipSuccess) e = hipEventRecord(chained, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(s2, chained, 0);
    if (e == hipSuccess) e = wkv7::launch_bwd(g1, 16, wkv7::BWD_KEYS, s2);
    if (e == hipSuccess) e = hipEventRecord(keyed, s2);
    if (e == hipSuccess) e = wkv7::launch_bwd(g2, 16, wkv7::BWD_CHAIN | wkv7::BWD_KEYS, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, keyed, 0);
    (void)hipEventDestroy(chained);
    (void)hipEventDestroy(keyed);
    return from_hip(e);
}

}  // namespace

extern "C" {

int wkv7_backward(const wkv7_desc* desc, const void* r, const void* w, const void* k,
                  const void* v, const void* a, const void* b, const float* s0, const void* dy,
                  const float* dsT, const void* tape, void* dr, void* dw, void* dk, void* dv,
                  void* da, void* db, float* ds0, void* workspace, size_t workspace_bytes,
                  void* stream) {
    return run_backward(desc, r, w, k, v, a, b, s0, dy, dsT, tape, dr, dw, dk, dv, da, db, ds0,
                        workspace, workspace_bytes, stream, wkv7::BWD_CHAIN | wkv7::BWD_KEYS,
                        nullptr);
}

int wkv7_backward_ckpt(const wkv7_desc* desc, const void* r, const void* w, const void* k,
                       const void* v, const void* a, const void* b, const float* s0,
                       const void* dy, const float* dsT, const float* ckpt, void* dr, void* dw,
                       void* dk, void* dv, void* da, void* db, float* ds0, void* stream) {
    const int st = check_desc(desc);
    if (st != WKV7_OK) return st;
    if (desc->chunk_len != 0) return WKV7_ERR_UNSUPPORTED;
    if ((int64_t)desc->B * desc->T * desc->H > 0 && !req(ckpt)) return WKV7_ERR_INVALID_ARG;
    return run_backward(desc, r, w, k, v, a, b, s0, dy, dsT, nullptr, dr, dw, dk, dv, da, db, ds0,
                        nullptr, 0, stream, wkv7::BWD_CHAIN | wkv7::BWD_KEYS, nullptr, ckpt);
}

int wkv7_backward_overlapped(const wkv7_desc* desc, const void* r, const void* w, const void* k,
                             const void* v, const void* a, const void* b, const float* s0,
                             const void* dy, const float* dsT, const void* tape, void* dr, void* dw,
                             void* dk, void* dv, void* da, void* db, float* ds0, void* workspace,
                             size_t workspace_bytes, void* stream, void* aux_stream) {
    return run_backward(desc, r, w, k, v, a, b, s0, dy, dsT, tape, dr, dw, dk, dv, da, db, ds0,
                        workspace, workspace_bytes, stream, wkv7::BWD_CHAIN | wkv7::BWD_KEYS,
                        aux_stream);
}

int wkv7_backward_adjoint(const wkv7_desc* desc, const void* r, const void* w, const void* k,
                          const void* v, const void* a, const void* b, const float* s0,
                          const void* dy, const float* dsT, const void* tape, void* dr, void* dw,
                          void* dk, void* dv, void* da, void* db, float* ds0, void* workspace,
                          size_t workspace_bytes, void* stream) {
    return run_backward(desc, r, w, k, v, a, b, s0, dy, dsT, tape, dr, dw, dk, dv, da, db, ds0,
                        workspace, workspace_bytes, stream, wkv7::BWD_CHAIN, nullptr);
}

int wkv7_backward_gradients(const wkv7_desc* desc, const void* r, const void* w, const void* k,
                            const void* v, const void* a, const void* b, const float* s0,
                            const void* dy, const float* dsT, const void* tape, void* dr,
                            void* dw, void* dk, void* dv, void* da, void* db, float* ds0,
                            void* workspace, size_t workspace_bytes, void* stream) {
    return run_backward(desc, r, w, k, v, a, b, s0, dy, dsT, tape, dr, dw, dk, dv, da, db, ds0,
                        workspace, workspace_bytes, stream, wkv7::BWD_KEYS, nullptr);
}

int wkv7_decode_step(int32_t B, int32_t H, int32_t N, int32_t dtype, const void* r,
                     const void* w, const void* k, const void* v, const void* a, const void* b,
                     float* state, void* y, void* stream) {
    if (B < 0 || H < 0 || N < 0) return WKV7_ERR_INVALID_ARG;
    if (N != 32 && N != 64 && N != 128) return WKV7_ERR_UNSUPPORTED;
    if (dtype != WKV7_F32 && dtype != WKV7_BF16) return WKV7_ERR_UNSUPPORTED;
    if ((int64_t)B * H > (int64_t)(1 << 28)) return WKV7_ERR_UNSUPPORTED;
    if ((int64_t)B * H == 0) return WKV7_OK;
    if (!(req(r) && req(w) && req(k) && req(v) && pair(a, b) && req(state) && req(y)))
        return WKV7_ERR_INVALID_ARG;
    wkv7::DecodeArgs p{B, H, N, dtype == WKV7_BF16, r, w, k, v, a, b, state, y};
    return from_hip(wkv7::launch_decode(p, static_cast<hipStream_t>(stream)));
}

int wkv7_epilogue(const wkv7_desc* desc, const void* y, const void* r, const void* k,
                  const void* v, const void* g, const wkv7_epilogue_params* params, void* out,
                  void* stream) {
    if (!desc) return WKV7_ERR_INVALID_ARG;
    wkv7_desc d = *desc;
    d.chunk_len = 0;   // any form's read-out
    const int st = check_desc(&d);
    if (st != WKV7_OK) return st;
    if (!epi_params_ok(params)) return WKV7_ERR_INVALID_ARG;
    const bool has_tokens = (int64_t)d.B * d.T * d.H > 0;
    if (has_tokens && !(req(y) && req(out) && opt(g))) return WKV7_ERR_INVALID_ARG;
    if (has_tokens && params->u && !(req(r) && req(k) && req(v))) return WKV7_ERR_INVALID_ARG;
    if (!has_tokens) return WKV7_OK;
    const wkv7::EpiArgs p{d.B, d.T, d.H, d.N, d.dtype == WKV7_BF16, y, r, k, v, epi_params(params, g), out};
    return from_hip(wkv7::launch_epilogue(p, static_cast<hipStream_t>(stream)));
}

int wkv7_forward_epilogue(const wkv7_desc* desc, const void* r, const void* w, const void* k,
                          const void* v, const void* a, const void* b, const float* s0,
                          const void* g, const wkv7_epilogue_params* params, void* out,
                          float* sT, void* stream) {
    const int st = check_desc(desc);
    if (st != WKV7_OK) return st;
    if (!epi_params_ok(params)) return WKV7_ERR_INVALID_ARG;
    const bool has_tokens = (int64_t)desc->B * desc->T * desc->H > 0;
    if (has_tokens && !(req(r) && req(w) && req(k) && req(v) && pair(a, b) && req(out) && opt(g)))
        return WKV7_ERR_INVALID_ARG;
    if (!(opt(s0) && opt(sT))) return WKV7_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!has_tokens || desc->chunk_len == 0 || desc->N != WKV7_HEAD_SIZE ||
        !wkv7::chunk_fwd_epilogue_fits(desc->T, desc->H)) {
        // The forward writes y into out (nothing at all without tokens), then
        // the step runs on it in place: the scan, the chunked form at N = 32, and
        // chunked problems too large for the fused kernel's 32-bit offsets.
        const int fs = run_forward(desc, r, w, k, v, a, b, s0, out, sT, nullptr, s);
        if (fs != WKV7_OK || !has_tokens) return fs;
        return wkv7_epilogue(desc, out, r, k, v, g, params, out, stream);
    }
    wkv7::FwdArgs p{desc->B, desc->T, desc->H, desc->N, true, r, w, k, v, a, b, s0, out, sT, nullptr};
    return from_hip(wkv7::launch_chunk_fwd_epilogue(p, epi_params(params, g), s));
}

}  // extern "C"
