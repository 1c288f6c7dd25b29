/* The fp64 oracle under AddressSanitizer and UndefinedBehaviorSanitizer: every
 * entry point on small ragged shapes (one thread), with two of its own
 * identities as a sanity check -- T decode steps equal the sequence forward,
 * and the chunked rearrangement equals the sequential recurrence -- plus the
 * step after the read-out in its three modes.  Exit status
 * = number of failed checks. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

void wkv7_oracle_forward(int B, int T, int H, int N, const double *r, const double *w,
                         const double *k, const double *v, const double *a, const double *b,
                         const double *s0, double *y, double *sT, int nthreads);
void wkv7_oracle_decode_step(int B, int H, int N, const double *r, const double *w,
                             const double *k, const double *v, const double *a,
                             const double *b, double *state, double *y, int nthreads);
void wkv7_oracle_backward(int B, int T, int H, int N, const double *r, const double *w,
                          const double *k, const double *v, const double *a, const double *b,
                          const double *s0, const double *dy, const double *dsT, double *dr,
                          double *dw, double *dk, double *dv, double *da, double *db,
                          double *ds0, int nthreads);
void wkv7_oracle_forward_chunked(int B, int T, int H, int N, int L, const double *r,
                                 const double *w, const double *k, const double *v,
                                 const double *a, const double *b, const double *s0, double *y,
                                 double *sT, int nthreads);
void wkv7_oracle_backward_chunked(int B, int T, int H, int N, int L, const double *r,
                                  const double *w, const double *k, const double *v,
                                  const double *a, const double *b, const double *s0,
                                  const double *dy, const double *dsT, double *dr, double *dw,
                                  double *dk, double *dv, double *da, double *db, double *ds0,
                                  int nthreads);
void wkv7_oracle_epilogue(int B, int T, int H, int N, const double *y, const double *r,
                          const double *k, const double *v, const double *g, const double *u,
                          const double *gamma, const double *beta, double eps, int mode,
                          double *out, int nthreads);

static unsigned long long rng = 88172645463325252ull;
static double uni(void) {   /* xorshift64, uniform in (-1, 1) */
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    return (double)(rng >> 11) / 4503599627370496.0 - 1.0;
}
static double *fill(size_t n, double lo, double hi) {
    double *p = malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * 0.5 * (uni() + 1.0);
    return p;
}
static double maxdiff(const double *x, const double *y, size_t n) {
    double m = 0;
    for (size_t i = 0; i < n; ++i) m = fmax(m, fabs(x[i] - y[i]));
    return m;
}

int main(void) {
    int failures = 0;
    const int B = 2, T = 37, H = 3, N = 8;
    const size_t nt = (size_t)B * T * H * N, ns = (size_t)B * H * N * N;
    double *r = fill(nt, -1, 1), *k = fill(nt, -1, 1), *v = fill(nt, -1, 1);
    double *w = fill(nt, 0.6, 1.0), *a = fill(nt, -0.3, 0.3), *b = fill(nt, -0.3, 0.3);
    double *s0 = fill(ns, -0.1, 0.1), *dy = fill(nt, -1, 1), *dsT = fill(ns, -0.1, 0.1);
    double *y = calloc(nt, sizeof(double)), *y2 = calloc(nt, sizeof(double));
    double *sT = calloc(ns, sizeof(double)), *sT2 = calloc(ns, sizeof(double));
    wkv7_oracle_forward(B, T, H, N, r, w, k, v, a, b, s0, y, sT, 1);
    /* decode, token by token, on a copy of s0 */
    double *st = malloc(ns * sizeof(double));
    for (size_t i = 0; i < ns; ++i) st[i] = s0[i];
    const size_t nh = (size_t)B * H * N;
    double *tok[6], *yt = malloc(nh * sizeof(double));
    for (int q = 0; q < 6; ++q) tok[q] = malloc(nh * sizeof(double));
    const double *src[6] = {r, w, k, v, a, b};
    double dec = 0;
    for (int t = 0; t < T; ++t) {
        for (int q = 0; q < 6; ++q)
            for (int bb = 0; bb < B; ++bb)
                for (int hh = 0; hh < H; ++hh)
                    for (int j = 0; j < N; ++j)
                        tok[q][((size_t)bb * H + hh) * N + j] = src[q][(((size_t)bb * T + t) * H + hh) * N + j];
        wkv7_oracle_decode_step(B, H, N, tok[0], tok[1], tok[2], tok[3], tok[4], tok[5], st, yt, 1);
        for (int bb = 0; bb < B; ++bb)
            for (int hh = 0; hh < H; ++hh)
                for (int j = 0; j < N; ++j)
                    dec = fmax(dec, fabs(yt[((size_t)bb * H + hh) * N + j] -
                                         y[(((size_t)bb * T + t) * H + hh) * N + j]));
    }
    if (dec > 1e-12 || maxdiff(st, sT, ns) > 1e-12) { fprintf(stderr, "decode != forward\n"); ++failures; }
    for (int L = 1; L <= 16; L *= 4) {
        wkv7_oracle_forward_chunked(B, T, H, N, L, r, w, k, v, a, b, s0, y2, sT2, 1);
        if (maxdiff(y, y2, nt) > 1e-10 || maxdiff(sT, sT2, ns) > 1e-10) {
            fprintf(stderr, "chunked (L=%d) != sequential\n", L);
            ++failures;
        }
    }
    double *g1[7], *g2[7];
    for (int q = 0; q < 6; ++q) { g1[q] = calloc(nt, sizeof(double)); g2[q] = calloc(nt, sizeof(double)); }
    g1[6] = calloc(ns, sizeof(double)); g2[6] = calloc(ns, sizeof(double));
    wkv7_oracle_backward(B, T, H, N, r, w, k, v, a, b, s0, dy, dsT, g1[0], g1[1], g1[2], g1[3], g1[4],
                         g1[5], g1[6], 1);
    wkv7_oracle_backward_chunked(B, T, H, N, 16, r, w, k, v, a, b, s0, dy, dsT, g2[0], g2[1], g2[2],
                                 g2[3], g2[4], g2[5], g2[6], 1);
    for (int q = 0; q < 7; ++q)
        if (maxdiff(g1[q], g2[q], q < 6 ? nt : ns) > 1e-9) { fprintf(stderr, "gradient %d\n", q); ++failures; }
    /* empty and NULL-state calls */
    wkv7_oracle_forward(B, 0, H, N, r, w, k, v, a, b, NULL, y, sT, 1);
    wkv7_oracle_forward(0, T, H, N, r, w, k, v, a, b, NULL, y, sT, 1);
    wkv7_oracle_backward(B, T, H, N, r, w, k, v, a, b, NULL, dy, NULL, g1[0], g1[1], g1[2], g1[3],
                         g1[4], g1[5], g1[6], 1);
    /* the step after the read-out: every mode, with and without the optional
       inputs; mode 0 without term and gate is the identity */
    double *u = fill((size_t)H * N, -1, 1), *gam = fill((size_t)H * N, 0.5, 1.5);
    double *bet = fill((size_t)H * N, -0.2, 0.2);
    for (int mode = 0; mode < 3; ++mode) {
        wkv7_oracle_epilogue(B, T, H, N, y, r, k, v, dy, u, gam, bet, 1e-5, mode, y2, 1);
        wkv7_oracle_epilogue(B, T, H, N, y, r, k, v, NULL, NULL, NULL, NULL, 1e-5, mode, y2, 1);
    }
    wkv7_oracle_epilogue(B, T, H, N, y, r, k, v, NULL, NULL, NULL, NULL, 0.0, 0, y2, 1);
    if (maxdiff(y, y2, nt) != 0.0) { fprintf(stderr, "epilogue identity\n"); ++failures; }
    wkv7_oracle_epilogue(B, 0, H, N, y, r, k, v, NULL, NULL, NULL, NULL, 0.0, 1, y2, 1);
    free(u); free(gam); free(bet);
    for (int q = 0; q < 7; ++q) { free(g1[q]); free(g2[q]); }
    for (int q = 0; q < 6; ++q) free(tok[q]);
    free(yt); free(st); free(r); free(k); free(v); free(w); free(a); free(b); free(s0); free(dy);
    free(dsT); free(y); free(y2); free(sT); free(sT2);
    printf("oracle driver: %d failed checks\n", failures);
    return failures;
}
