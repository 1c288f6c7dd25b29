// wkv7_api.cpp -- C ABI of the WKV7 library: validation, dispatch, status codes.
// Declarations and the contract of every entry point are in include/wkv7.h.

#include "wkv7.h"

#include <hip/hip_runtime.h>

#include "wkv7_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Required pointer: non-null and 16-byte aligned.
bool req(const void* p) { return p != nullptr && aligned16(p); }
// Optional pointer: null, or 16-byte aligned.
bool opt(const void* p) { return p == nullptr || aligned16(p); }

int check_desc(const wkv7_desc* d) {
    if (!d) return WKV7_ERR_INVALID_ARG;
    if (d->B < 0 || d->T < 0 || d->H < 0 || d->N < 0) return WKV7_ERR_INVALID_ARG;
    if (d->N != WKV7_HEAD_SIZE) return WKV7_ERR_UNSUPPORTED;
    if (d->dtype != WKV7_F32 && d->dtype != WKV7_BF16) return WKV7_ERR_UNSUPPORTED;
    if (d->chunk_len != 0 && d->chunk_len != 16) return WKV7_ERR_UNSUPPORTED;
    // The chunked form runs its products on bf16 matrix cores.
    if (d->chunk_len != 0 && d->dtype != WKV7_BF16) return WKV7_ERR_UNSUPPORTED;
    // Grid dimensions are B*H (times 4) workgroups.
    if ((int64_t)d->B * d->H > (int64_t)(1 << 28)) return WKV7_ERR_UNSUPPORTED;
    return WKV7_OK;
}

// Tape: bf16 removal read-outs [B][T][H][N], then the bf16 state entering every
// 32-token block [B][H][ceil(T/32)][N][N].  The backward's own scratch (dX, and
// the adjoint leaving every block) has the same shape.
size_t tape_bytes_unchecked(const wkv7_desc* d) {
    const size_t nblk = ((size_t)d->T + WKV7_TAPE_BLOCK - 1) / WKV7_TAPE_BLOCK;
    const size_t tok = (size_t)d->B * d->T * d->H * d->N;
    const size_t st = (size_t)d->B * d->H * nblk * d->N * d->N;
    return (tok + st) * 2;
}

int from_hip(hipError_t e) { return e == hipSuccess ? WKV7_OK : WKV7_ERR_LAUNCH; }

int run_forward(const wkv7_desc* d, const void* r, const void* w, const void* k, const void* v,
                const void* a, const void* b, const float* s0, void* y, float* sT,
                void* tape, hipStream_t stream) {
    if ((int64_t)d->B * d->H == 0) return WKV7_OK;
    if (d->T == 0) {
        if (sT) return from_hip(wkv7::launch_state_copy(d->B * d->H, s0, sT, stream));
        return WKV7_OK;
    }
    wkv7::FwdArgs p{d->B, d->T, d->H, d->dtype == WKV7_BF16, r, w, k, v, a, b, s0, y, sT, tape};
    if (d->chunk_len == 0) return from_hip(wkv7::launch_seq_fwd(p, stream));
    return from_hip(wkv7::launch_chunk_fwd(p, d->chunk_len, stream));
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
        default: return "unknown status";
    }
}

size_t wkv7_tape_bytes(const wkv7_desc* desc) {
    if (check_desc(desc) != WKV7_OK) return 0;
    return tape_bytes_unchecked(desc);
}

size_t wkv7_workspace_bytes(const wkv7_desc* desc, int with_tape) {
    if (check_desc(desc) != WKV7_OK) return 0;
    return tape_bytes_unchecked(desc) * (with_tape ? 1 : 2);
}

int wkv7_forward(const wkv7_desc* desc, const void* r, const void* w, const void* k,
                 const void* v, const void* a, const void* b, const float* s0, void* y,
                 float* sT, void* tape, void* stream) {
    const int st = check_desc(desc);
    if (st != WKV7_OK) return st;
    const bool has_tokens = (int64_t)desc->B * desc->T * desc->H > 0;
    if (has_tokens && !(req(r) && req(w) && req(k) && req(v) && req(a) && req(b) && req(y)))
        return WKV7_ERR_INVALID_ARG;
    if (!(opt(s0) && opt(sT) && opt(tape))) return WKV7_ERR_INVALID_ARG;
    return run_forward(desc, r, w, k, v, a, b, s0, y, sT, tape, static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

// Shared by wkv7_backward and its two stage entry points.
int run_backward(const wkv7_desc* desc, const void* r, const void* w, const void* k,
                 const void* v, const void* a, const void* b, const float* s0, const void* dy,
                 const float* dsT, const void* tape, void* dr, void* dw, void* dk, void* dv,
                 void* da, void* db, float* ds0, void* workspace, size_t workspace_bytes,
                 void* stream, int stages) {
    int st = check_desc(desc);
    if (st != WKV7_OK) return st;
    // The backward runs the chunked adjoint on bf16 matrix cores, one workgroup
    // per chunk and head in its second pass.
    if (desc->dtype != WKV7_BF16) return WKV7_ERR_UNSUPPORTED;
    if ((int64_t)desc->B * desc->H * ((desc->T + WKV7_TAPE_CHUNK - 1) / WKV7_TAPE_CHUNK) > INT32_MAX)
        return WKV7_ERR_UNSUPPORTED;
    const bool has_tokens = (int64_t)desc->B * desc->T * desc->H > 0;
    if (has_tokens && !(req(r) && req(w) && req(k) && req(v) && req(a) && req(b) && req(dy) &&
                        req(dr) && req(dw) && req(dk) && req(dv) && req(da) && req(db)))
        return WKV7_ERR_INVALID_ARG;
    if (!(opt(s0) && opt(dsT) && opt(tape) && opt(ds0) && opt(workspace)))
        return WKV7_ERR_INVALID_ARG;
    // A single stage needs the forward's tape: the workspace carries the
    // chain's results to the second stage, and a re-run would overwrite it.
    if (stages != (wkv7::BWD_CHAIN | wkv7::BWD_KEYS) && has_tokens && !tape)
        return WKV7_ERR_INVALID_ARG;
    const size_t need = tape_bytes_unchecked(desc) * (tape ? 1 : 2);
    if (has_tokens && (workspace == nullptr || workspace_bytes < need)) return WKV7_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((int64_t)desc->B * desc->H == 0) return WKV7_OK;
    if (desc->T == 0) {
        // L = <dsT, S_T> with S_T = s0: ds0 = dsT.
        if (ds0 && (stages & wkv7::BWD_CHAIN))
            return from_hip(wkv7::launch_state_copy(desc->B * desc->H, dsT, ds0, s));
        return WKV7_OK;
    }
    char* ws = static_cast<char*>(workspace);
    if (!tape) {
        // Re-run the forward (without y) into the second half of the workspace.
        void* own = ws + tape_bytes_unchecked(desc);
        st = run_forward(desc, r, w, k, v, a, b, s0, nullptr, nullptr, own, s);
        if (st != WKV7_OK) return st;
        tape = own;
    }
    wkv7::BwdArgs p{desc->B, desc->T, desc->H, true, r, w, k, v, a, b, s0, dy, dsT, tape,
                    dr, dw, dk, dv, da, db, ds0, ws};
    return from_hip(wkv7::launch_bwd(p, 16, stages, s));
}

}  // namespace

extern "C" {

int wkv7_backward(const wkv7_desc* desc, const void* r, const void* w, const void* k,
                  const void* v, const void* a, const void* b, const float* s0, const void* dy,
                  const float* dsT, const void* tape, void* dr, void* dw, void* dk, void* dv,
                  void* da, void* db, float* ds0, void* workspace, size_t workspace_bytes,
                  void* stream) {
    return run_backward(desc, r, w, k, v, a, b, s0, dy, dsT, tape, dr, dw, dk, dv, da, db, ds0,
                        workspace, workspace_bytes, stream, wkv7::BWD_CHAIN | wkv7::BWD_KEYS);
}

int wkv7_backward_adjoint(const wkv7_desc* desc, const void* r, const void* w, const void* k,
                          const void* v, const void* a, const void* b, const float* s0,
                          const void* dy, const float* dsT, const void* tape, void* dr, void* dw,
                          void* dk, void* dv, void* da, void* db, float* ds0, void* workspace,
                          size_t workspace_bytes, void* stream) {
    return run_backward(desc, r, w, k, v, a, b, s0, dy, dsT, tape, dr, dw, dk, dv, da, db, ds0,
                        workspace, workspace_bytes, stream, wkv7::BWD_CHAIN);
}

int wkv7_backward_gradients(const wkv7_desc* desc, const void* r, const void* w, const void* k,
                            const void* v, const void* a, const void* b, const float* s0,
                            const void* dy, const float* dsT, const void* tape, void* dr,
                            void* dw, void* dk, void* dv, void* da, void* db, float* ds0,
                            void* workspace, size_t workspace_bytes, void* stream) {
    return run_backward(desc, r, w, k, v, a, b, s0, dy, dsT, tape, dr, dw, dk, dv, da, db, ds0,
                        workspace, workspace_bytes, stream, wkv7::BWD_KEYS);
}

int wkv7_decode_step(int32_t B, int32_t H, int32_t N, int32_t dtype, const void* r,
                     const void* w, const void* k, const void* v, const void* a, const void* b,
                     float* state, void* y, void* stream) {
    if (B < 0 || H < 0 || N < 0) return WKV7_ERR_INVALID_ARG;
    if (N != WKV7_HEAD_SIZE) return WKV7_ERR_UNSUPPORTED;
    if (dtype != WKV7_F32 && dtype != WKV7_BF16) return WKV7_ERR_UNSUPPORTED;
    if ((int64_t)B * H > (int64_t)(1 << 28)) return WKV7_ERR_UNSUPPORTED;
    if ((int64_t)B * H == 0) return WKV7_OK;
    if (!(req(r) && req(w) && req(k) && req(v) && req(a) && req(b) && req(state) && req(y)))
        return WKV7_ERR_INVALID_ARG;
    wkv7::DecodeArgs p{B, H, dtype == WKV7_BF16, r, w, k, v, a, b, state, y};
    return from_hip(wkv7::launch_decode(p, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
