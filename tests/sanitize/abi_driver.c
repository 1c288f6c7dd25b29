/* Host-only exercise of the C ABI's validation paths and size queries, built
 * with AddressSanitizer and UndefinedBehaviorSanitizer (no device involved:
 * every case fails validation or is empty, and the launchers are stubs that
 * would report WKV7_ERR_LAUNCH).  Exit status = number of failed checks. */
#include <stdint.h>
#include <stdio.h>

#include "wkv7.h"

static int failures = 0;
#define CHECK(cond)                                                      \
    do {                                                                 \
        if (!(cond)) {                                                   \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            ++failures;                                                  \
        }                                                                \
    } while (0)

static wkv7_desc D(int B, int T, int H, int N, int dt, int cl) {
    wkv7_desc d = {B, T, H, N, dt, cl};
    return d;
}

int main(void) {
    void* F = (void*)(uintptr_t)(1u << 20);      /* aligned, never dereferenced */
    void* M = (void*)(uintptr_t)((1u << 20) + 8); /* misaligned */
    const int sizes[][4] = {{1, 1, 1, 64}, {8, 4096, 40, 64}, {1, 0, 3, 32}, {0, 7, 0, 128},
                            {1 << 14, 1 << 20, 1 << 14, 64}, {2, 0x7fffffff, 2, 64},
                            {1, 0x7ffffff0, 1, 128}, {-1, 8, 1, 64}, {1, -8, 1, 64}, {1, 8, 1, 48}};
    const int nsz = (int)(sizeof(sizes) / sizeof(sizes[0]));
    const int chunk_lens[] = {-1, 0, 8, 16};
    for (int i = 0; i < nsz; ++i)
        for (int dt = -1; dt <= 2; ++dt)
            for (int ci = 0; ci < 4; ++ci) {
                wkv7_desc d = D(sizes[i][0], sizes[i][1], sizes[i][2], sizes[i][3], dt, chunk_lens[ci]);
                /* size queries never fail and never overflow silently */
                (void)wkv7_tape_bytes(&d);
                (void)wkv7_ckpt_bytes(&d);
                (void)wkv7_workspace_bytes(&d);
                (void)wkv7_backward_workspace_bytes(&d, 0);
                (void)wkv7_backward_workspace_bytes(&d, 1);
                for (int seg = -17; seg <= 17; seg += 3) (void)wkv7_forward_split_workspace_bytes(&d, seg);
                /* calls with a missing required pointer (y, r, workspace or ckpt)
                   fail validation: none may reach a launch */
                const int big = (int64_t)d.B * d.T * d.H > 0;
                int st = wkv7_forward(&d, F, F, F, F, F, F, NULL, NULL, NULL, NULL, NULL);
                CHECK(st != WKV7_ERR_LAUNCH || !big);
                st = wkv7_forward(&d, NULL, F, F, F, F, F, NULL, F, NULL, NULL, NULL);
                CHECK(st != WKV7_OK || !big);
                st = wkv7_backward(&d, F, F, F, F, F, F, NULL, F, NULL, NULL, F, F, F, F, F, F, NULL,
                                   NULL, 0, NULL);
                CHECK(st != WKV7_ERR_LAUNCH || !big);
                st = wkv7_backward_ckpt(&d, F, F, F, F, F, F, NULL, F, NULL, NULL, F, F, F, F, F, F,
                                        NULL, NULL);
                CHECK(st != WKV7_ERR_LAUNCH || !big);
                st = wkv7_forward_split(&d, F, F, F, F, F, F, NULL, NULL, NULL, NULL, 4, NULL, 0, NULL);
                CHECK(st != WKV7_ERR_LAUNCH || !big);
                wkv7_epilogue_params ep = {NULL, NULL, NULL, 1e-5f, ci % 3};
                st = wkv7_epilogue(&d, F, F, F, F, NULL, &ep, NULL, NULL);
                CHECK(st != WKV7_ERR_LAUNCH || !big);
                st = wkv7_forward_epilogue(&d, F, F, F, F, F, F, NULL, NULL, &ep, NULL, NULL, NULL);
                CHECK(st != WKV7_ERR_LAUNCH || !big);
            }
    /* explicit statuses */
    wkv7_desc d = D(1, 8, 1, 64, WKV7_BF16, 16);
    CHECK(wkv7_forward(NULL, F, F, F, F, F, F, NULL, F, NULL, NULL, NULL) == WKV7_ERR_INVALID_ARG);
    CHECK(wkv7_forward(&d, F, F, F, F, F, M, NULL, F, NULL, NULL, NULL) == WKV7_ERR_INVALID_ARG);
    CHECK(wkv7_forward(&d, F, F, F, F, F, NULL, NULL, F, NULL, NULL, NULL) == WKV7_ERR_INVALID_ARG);
    CHECK(wkv7_forward_ckpt(&d, F, F, F, F, F, F, NULL, F, NULL, M, NULL) == WKV7_ERR_INVALID_ARG);
    CHECK(wkv7_backward(&d, F, F, F, F, F, F, NULL, F, NULL, NULL, F, F, F, F, F, F, NULL, F, 16,
                        NULL) == WKV7_ERR_WORKSPACE);
    CHECK(wkv7_backward_ckpt(&d, F, F, F, F, F, F, NULL, F, NULL, F, F, F, F, F, F, F, NULL, NULL) ==
          WKV7_ERR_UNSUPPORTED);
    wkv7_desc e = D(0, 8, 4, 64, WKV7_BF16, 16);
    CHECK(wkv7_forward(&e, F, F, F, F, F, F, NULL, F, NULL, NULL, NULL) == WKV7_OK);
    CHECK(wkv7_decode_step(1, 1, 48, WKV7_BF16, F, F, F, F, F, F, F, F, NULL) == WKV7_ERR_UNSUPPORTED);
    CHECK(wkv7_decode_step(-1, 1, 64, WKV7_BF16, F, F, F, F, F, F, F, F, NULL) == WKV7_ERR_INVALID_ARG);
    CHECK(wkv7_decode_step(0, 1, 64, WKV7_BF16, F, F, F, F, F, F, F, F, NULL) == WKV7_OK);
    CHECK(wkv7_decode_step(1, 1, 64, WKV7_F32, F, F, F, F, F, M, F, F, NULL) == WKV7_ERR_INVALID_ARG);
    wkv7_epilogue_params bad = {NULL, NULL, NULL, -1.0f, 1};
    CHECK(wkv7_epilogue(&d, F, F, F, F, NULL, &bad, F, NULL) == WKV7_ERR_INVALID_ARG);
    CHECK(wkv7_epilogue(&d, F, F, F, F, NULL, NULL, F, NULL) == WKV7_ERR_INVALID_ARG);
    /* sizes: exact values */
    d = D(8, 4096, 40, 64, WKV7_BF16, 16);
    CHECK(wkv7_ckpt_bytes(&d) == (size_t)8 * 40 * 256 * 64 * 64 * 4);
    CHECK(wkv7_workspace_bytes(&d) == 2 * wkv7_tape_bytes(&d) + 256);
    CHECK(wkv7_abi_version() == WKV7_ABI_VERSION);
    for (int s = -3; s < 8; ++s) CHECK(wkv7_status_string(s) != NULL);
    printf("abi driver: %d failed checks\n", failures);
    return failures;
}
