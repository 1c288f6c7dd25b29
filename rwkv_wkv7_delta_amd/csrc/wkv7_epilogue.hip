// wkv7_epilogue.hip -- the step after the read-out as a kernel of its own
// (formula and sources in wkv7_epilogue.h).
//
// Bound by HBM: per (token, head) row it reads y, v (and r, k with the
// current-token term, g with the gate) and writes the result.  An aligned
// group of N / 8 lanes takes a row, 8 consecutive values per lane (one 16-byte
// access per tensor in bf16), so a wave covers 512 contiguous bytes of every
// tensor; the row's sums are DPP reductions inside the group.  The per-head
// vectors u, gamma, beta (fp32, [H][N]) are small and stay in the caches.
// `out` may be `y` itself: every lane reads its values before it writes them.

#include "wkv7.h"
#include "wkv7_epilogue.h"
#include "wkv7_internal.h"

namespace wkv7 {

namespace {

constexpr int kEpiThreads = 256;
constexpr int kEpiC = 8;   // values per lane

template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&x)[kEpiC]);
template <>
__device__ __forceinline__ void store8<float>(float* p, const float (&x)[kEpiC]) {
    store_cols<kEpiC>(p, x);
}
template <>
__device__ __forceinline__ void store8<bf16_t>(bf16_t* p, const float (&x)[kEpiC]) {
    *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                              pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7]));
}

template <typename T, int N>
__global__ __launch_bounds__(kEpiThreads) void epilogue_kernel(
    long long rows, int H, const T* y, const T* __restrict__ r, const T* __restrict__ k,
    const T* __restrict__ v, const T* __restrict__ g, const float* __restrict__ u,
    const float* __restrict__ gamma, const float* __restrict__ beta, float eps, int mode, T* out) {
    constexpr int P = N / kEpiC, RPB = kEpiThreads / P;
    const int piece = threadIdx.x % P;
    const bool term = u != nullptr;
    for (long long row = (long long)blockIdx.x * RPB + threadIdx.x / P; row < rows;
         row += (long long)gridDim.x * RPB) {
        const size_t off = (size_t)row * N + piece * kEpiC;
        const size_t hoff = (size_t)(row % H) * N + piece * kEpiC;
        float x[kEpiC], vv[kEpiC], gt[kEpiC], gm[kEpiC], bt[kEpiC];
        load_cols<kEpiC>(y + off, x);
        float sp = 0.f;
        if (term) {
            float rr[kEpiC], kk[kEpiC], uu[kEpiC];
            load_cols<kEpiC>(r + off, rr);
            load_cols<kEpiC>(k + off, kk);
            load_cols<kEpiC>(v + off, vv);
            load_cols<kEpiC>(u + hoff, uu);
#pragma unroll
            for (int c = 0; c < kEpiC; ++c) sp = fmaf(rr[c] * uu[c], kk[c], sp);
        } else {
#pragma unroll
            for (int c = 0; c < kEpiC; ++c) vv[c] = 0.f;
        }
        if (g) {
            load_cols<kEpiC>(g + off, gt);
        } else {
#pragma unroll
            for (int c = 0; c < kEpiC; ++c) gt[c] = 1.f;
        }
        load_f32_or<kEpiC>(gamma ? gamma + hoff : nullptr, 1.f, gm);
        load_f32_or<kEpiC>(beta ? beta + hoff : nullptr, 0.f, bt);
        epilogue_row<kEpiC, P>(x, vv, term ? lanes_sum<P>(sp) : 0.f, term, gm, bt, gt, eps, mode);
        store8<T>(out + off, x);
    }
}

template <typename T, int N>
hipError_t launch_epilogue_n(const EpiArgs& p, hipStream_t stream) {
    constexpr int RPB = kEpiThreads / (N / kEpiC);
    const long long rows = (long long)p.B * p.T * p.H;
    if (rows == 0) return hipSuccess;
    // One workgroup per RPB rows, up to 2^20 of them (the loop strides over the
    // rest): at 1.3 M rows (B = 8, T = 4096, H = 40) one pass each measured
    // 0.188 ms against 0.204 ms with 8192 workgroups looping five times.
    const long long want = (rows + RPB - 1) / RPB;
    const unsigned grid = (unsigned)(want < (1LL << 20) ? want : (1LL << 20));
    epilogue_kernel<T, N><<<dim3(grid), dim3(kEpiThreads), 0, stream>>>(
        rows, p.H, static_cast<const T*>(p.y), static_cast<const T*>(p.r),
        static_cast<const T*>(p.k), static_cast<const T*>(p.v), static_cast<const T*>(p.e.g),
        p.e.u, p.e.gamma, p.e.beta, p.e.eps, p.e.mode, static_cast<T*>(p.out));
    return hipGetLastError();
}

template <typename T>
hipError_t launch_epilogue_t(const EpiArgs& p, hipStream_t stream) {
    switch (p.N) {
        case 32: return launch_epilogue_n<T, 32>(p, stream);
        case 64: return launch_epilogue_n<T, 64>(p, stream);
        case 128: return launch_epilogue_n<T, 128>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_epilogue(const EpiArgs& p, hipStream_t stream) {
    if (p.e.mode < 0 || p.e.mode > 2) return hipErrorInvalidValue;
    return p.bf16 ? launch_epilogue_t<bf16_t>(p, stream) : launch_epilogue_t<float>(p, stream);
}

}  // namespace wkv7
