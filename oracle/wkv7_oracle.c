/*
 * wkv7_oracle.c -- plain fp64 CPU oracle for the WKV7 state recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or constant with the HIP library and must never serve as a
 * fallback for it.
 *
 * What it computes (per batch b and head h, independently):
 *
 *   The state S is an N x N matrix, row i = value channel, column j = key
 *   channel.  For each token t, in order,
 *       z      = S a_t                              (removal read-out)
 *       S[i][j] = S[i][j] w_t[j] + z[i] b_t[j] + v_t[i] k_t[j]
 *       y_t    = S r_t                              (receptance read-out)
 *   i.e. S <- S (diag(w_t) + a_t b_t^T) + v_t k_t^T, then y_t = S r_t.
 *
 * Sources on the RWKV-7 "Goose" pages:
 *   - the transition is a diagonal-plus-rank-one generalisation of the delta
 *     rule with a vector-valued, data-dependent decay and separate removal and
 *     replacement keys ("Paper Review: RWKV-7 Goose", section Architecture;
 *     "RWKV-7 Goose with Expressive Dynamic State Evolution", Abstract;
 *     Elamur summary page, Summary);
 *   - the state is updated per head with decay, selective forgetting and
 *     insertion of the new value, and the receptance reads the state once it
 *     has been updated ("Paper Review", section The approach);
 *   - constant memory and constant time per token at inference (Abstract):
 *     the decode step is one iteration of the same loop on a resident state;
 *   - after the read-out, the receptance also attends to the current token and
 *     the result is normalised per head and gated ("Paper Review", The
 *     approach): wkv7_oracle_epilogue, its reading stated there.
 *
 * Readings taken where the pages are silent: z uses the undecayed previous
 * state (sum form, not (S diag(w)) a); y is read after the update; w is the
 * multiplicative decay itself.
 *
 * Layouts (row-major, last index fastest):
 *   token tensors r,w,k,v,a,b,y,dy and gradients  [B][T][H][N]
 *   states s0, sT, dsT, ds0                        [B][H][N][N]
 * All arrays are double.  s0 / dsT may be NULL (= zeros).
 *
 * Parity pins: every function here is checked in the CPU test suite against
 * closed forms, exact rational arithmetic, brute-force matrix products and
 * finite differences, never against the GPU.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

typedef struct {
    int B, T, H, N;
} shape_t;

static size_t tok(const shape_t *s, int b, int t, int h) {
    return (((size_t)b * s->T + t) * s->H + h) * (size_t)s->N;
}
static size_t st(const shape_t *s, int b, int h) {
    return ((size_t)b * s->H + h) * (size_t)s->N * s->N;
}

static int pick_threads(int nthreads) {
    return nthreads > 0 ? nthreads : omp_get_max_threads();
}

int wkv7_oracle_max_threads(void) { return omp_get_max_threads(); }

/* One token of the recurrence on state S (N x N, row-major), in place.
   Writes z (length N) and, if y != NULL, the read-out y = S r. */
static void step(int N, double *S, const double *r, const double *w, const double *k,
                 const double *v, const double *a, const double *b, double *z, double *y) {
    for (int i = 0; i < N; ++i) {
        double acc = 0.0;
        for (int j = 0; j < N; ++j) acc += S[i * N + j] * a[j];
        z[i] = acc;
    }
    for (int i = 0; i < N; ++i)
        for (int j = 0; j < N; ++j)
            S[i * N + j] = S[i * N + j] * w[j] + z[i] * b[j] + v[i] * k[j];
    if (y) {
        for (int i = 0; i < N; ++i) {
            double acc = 0.0;
            for (int j = 0; j < N; ++j) acc += S[i * N + j] * r[j];
            y[i] = acc;
        }
    }
}

/* Sequential forward: y [B][T][H][N]; sT [B][H][N][N] (may be NULL). */
void wkv7_oracle_forward(int B, int T, int H, int N, const double *r, const double *w,
                         const double *k, const double *v, const double *a, const double *b,
                         const double *s0, double *y, double *sT, int nthreads) {
    shape_t sh = {B, T, H, N};
    const int BH = B * H;
#pragma omp parallel for schedule(dynamic, 1) num_threads(pick_threads(nthreads))
    for (int bh = 0; bh < BH; ++bh) {
        const int bb = bh / H, hh = bh % H;
        double *S = (double *)malloc(sizeof(double) * N * N);
        double *z = (double *)malloc(sizeof(double) * N);
        if (s0) memcpy(S, s0 + st(&sh, bb, hh), sizeof(double) * N * N);
        else memset(S, 0, sizeof(double) * N * N);
        for (int t = 0; t < T; ++t) {
            const size_t o = tok(&sh, bb, t, hh);
            step(N, S, r + o, w + o, k + o, v + o, a + o, b + o, z, y + o);
        }
        if (sT) memcpy(sT + st(&sh, bb, hh), S, sizeof(double) * N * N);
        free(S);
        free(z);
    }
}

/* Single-token decode step on resident states, in place.
   r..b and y are [B][H][N]; state is [B][H][N][N]. */
void wkv7_oracle_decode_step(int B, int H, int N, const double *r, const double *w,
                             const double *k, const double *v, const double *a,
                             const double *b, double *state, double *y, int nthreads) {
    const int BH = B * H;
#pragma omp parallel for schedule(static) num_threads(pick_threads(nthreads))
    for (int bh = 0; bh < BH; ++bh) {
        double *z = (double *)malloc(sizeof(double) * N);
        const size_t o = (size_t)bh * N;
        step(N, state + (size_t)bh * N * N, r + o, w + o, k + o, v + o, a + o, b + o, z, y + o);
        free(z);
    }
}

/*
 * Reverse-mode gradient of the scalar
 *     L = sum_t <dy_t, y_t> + <dsT, S_T>
 * with respect to r, w, k, v, a, b and s0.  Keeps every state of one head
 * (T+1 matrices) and walks time backwards with the adjoint G = dL/dS_t:
 *     G     += dy_t r_t^T
 *     dr_t   = S_t^T dy_t
 *     dv_t   = G k_t,          dk_t = G^T v_t
 *     z      = S_{t-1} a_t,    dz   = G b_t
 *     db_t   = G^T z,          da_t = S_{t-1}^T dz
 *     dw_t[j] = sum_i G[i][j] S_{t-1}[i][j]
 *     G      = G diag(w_t) + dz a_t^T
 * and ds0 = G after the first token.  dsT and s0 may be NULL (zeros).
 */
void wkv7_oracle_backward(int B, int T, int H, int N, const double *r, const double *w,
                          const double *k, const double *v, const double *a, const double *b,
                          const double *s0, const double *dy, const double *dsT, double *dr,
                          double *dw, double *dk, double *dv, double *da, double *db,
                          double *ds0, int nthreads) {
    shape_t sh = {B, T, H, N};
    const int BH = B * H;
    const size_t NN = (size_t)N * N;
#pragma omp parallel for schedule(dynamic, 1) num_threads(pick_threads(nthreads))
    for (int bh = 0; bh < BH; ++bh) {
        const int bb = bh / H, hh = bh % H;
        /* hist[t] = state before token t (t = 0..T); hist[0] = s0. */
        double *hist = (double *)malloc(sizeof(double) * NN * ((size_t)T + 1));
        double *G = (double *)malloc(sizeof(double) * NN);
        double *z = (double *)malloc(sizeof(double) * N);
        double *dz = (double *)malloc(sizeof(double) * N);
        if (s0) memcpy(hist, s0 + st(&sh, bb, hh), sizeof(double) * NN);
        else memset(hist, 0, sizeof(double) * NN);
        for (int t = 0; t < T; ++t) {
            const size_t o = tok(&sh, bb, t, hh);
            memcpy(hist + NN * (t + 1), hist + NN * t, sizeof(double) * NN);
            step(N, hist + NN * (t + 1), r + o, w + o, k + o, v + o, a + o, b + o, z, NULL);
        }
        if (dsT) memcpy(G, dsT + st(&sh, bb, hh), sizeof(double) * NN);
        else memset(G, 0, sizeof(double) * NN);
        for (int t = T - 1; t >= 0; --t) {
            const size_t o = tok(&sh, bb, t, hh);
            const double *Sprev = hist + NN * t;       /* S_{t-1} */
            const double *Scur = hist + NN * (t + 1);  /* S_t     */
            const double *rt = r + o, *wt = w + o, *kt = k + o, *vt = v + o, *at = a + o,
                         *bt = b + o, *dyt = dy + o;
            for (int i = 0; i < N; ++i)
                for (int j = 0; j < N; ++j) G[i * N + j] += dyt[i] * rt[j];
            for (int j = 0; j < N; ++j) {
                double acc = 0.0;
                for (int i = 0; i < N; ++i) acc += Scur[i * N + j] * dyt[i];
                dr[o + j] = acc;
            }
            for (int i = 0; i < N; ++i) {
                double acc = 0.0, acc2 = 0.0, acc3 = 0.0;
                for (int j = 0; j < N; ++j) {
                    acc += G[i * N + j] * kt[j];
                    acc2 += Sprev[i * N + j] * at[j];
                    acc3 += G[i * N + j] * bt[j];
                }
                dv[o + i] = acc;
                z[i] = acc2;
                dz[i] = acc3;
            }
            for (int j = 0; j < N; ++j) {
                double sk = 0.0, sb = 0.0, sa = 0.0, sw = 0.0;
                for (int i = 0; i < N; ++i) {
                    sk += G[i * N + j] * vt[i];
                    sb += G[i * N + j] * z[i];
                    sa += Sprev[i * N + j] * dz[i];
                    sw += G[i * N + j] * Sprev[i * N + j];
                }
                dk[o + j] = sk;
                db[o + j] = sb;
                da[o + j] = sa;
                dw[o + j] = sw;
            }
            for (int i = 0; i < N; ++i)
                for (int j = 0; j < N; ++j)
                    G[i * N + j] = G[i * N + j] * wt[j] + dz[i] * at[j];
        }
        if (ds0) memcpy(ds0 + st(&sh, bb, hh), G, sizeof(double) * NN);
        free(hist);
        free(G);
        free(z);
        free(dz);
    }
}

/* ------------------------------------------------------------------------
 * Chunked (parallel-in-time) rearrangement, fp64.  Kept only to pin the
 * chunk algebra against the sequential definition above; the pages state the
 * model stays parallelisable in training (Abstract; Elamur Summary) without
 * printing the form, so this is a derivation, written out plainly.
 *
 * For a chunk of length L with entry state S0 and local times t = 1..L:
 *   G_t[j] = prod_{u<=t} w_u[j],  G_0 = 1
 *   At_t = a_t G_{t-1},  Rt_t = r_t G_t,  Bh_t = b_t / G_t,  Kh_t = k_t / G_t,
 *   Bb_t = b_t G_L / G_t, Kb_t = k_t G_L / G_t
 *   Aab[t][s] = At_t . Bh_s (s < t),   Aak[t][s] = At_t . Kh_s (s < t)
 *   Arb[t][s] = Rt_t . Bh_s (s <= t),  Ark[t][s] = Rt_t . Kh_s (s <= t)
 *   (I - Aab) Z = At S0^T + Aak V        (row t of Z is z_t = S_{t-1} a_t)
 *   Y = Rt S0^T + Arb Z + Ark V
 *   S_L = S0 diag(G_L) + Z^T Bb + V^T Kb
 * ---------------------------------------------------------------------- */

typedef struct {
    int L, N;
    double *G;                           /* (L+1) x N, G[0] = 1 */
    double *At, *Rt, *Bh, *Kh, *Bb, *Kb; /* L x N */
    double *Aab, *Aak, *Arb, *Ark;       /* L x L */
    double *Tinv;                        /* L x L, (I - Aab)^{-1} */
} chunk_t;

static void chunk_alloc(chunk_t *c, int L, int N) {
    c->L = L;
    c->N = N;
    c->G = (double *)calloc((size_t)(L + 1) * N, sizeof(double));
    double **vecs[] = {&c->At, &c->Rt, &c->Bh, &c->Kh, &c->Bb, &c->Kb};
    for (int q = 0; q < 6; ++q) *vecs[q] = (double *)calloc((size_t)L * N, sizeof(double));
    double **mats[] = {&c->Aab, &c->Aak, &c->Arb, &c->Ark, &c->Tinv};
    for (int q = 0; q < 5; ++q) *mats[q] = (double *)calloc((size_t)L * L, sizeof(double));
}
static void chunk_free(chunk_t *c) {
    free(c->G);
    free(c->At); free(c->Rt); free(c->Bh); free(c->Kh); free(c->Bb); free(c->Kb);
    free(c->Aab); free(c->Aak); free(c->Arb); free(c->Ark); free(c->Tinv);
}

/* Fill the chunk's decay products, scaled vectors, L x L factors and
   Tinv = (I - Aab)^{-1} for tokens t0 .. t0+L-1 of head (bb, hh). */
static void chunk_prepare(chunk_t *c, const shape_t *sh, int bb, int hh, int t0,
                          const double *r, const double *w, const double *k,
                          const double *a, const double *b) {
    const int L = c->L, N = c->N;
    for (int j = 0; j < N; ++j) c->G[j] = 1.0;
    for (int t = 1; t <= L; ++t) {
        const size_t o = tok(sh, bb, t0 + t - 1, hh);
        for (int j = 0; j < N; ++j) c->G[t * N + j] = c->G[(t - 1) * N + j] * w[o + j];
    }
    const double *GL = c->G + (size_t)L * N;
    for (int t = 1; t <= L; ++t) {
        const size_t o = tok(sh, bb, t0 + t - 1, hh);
        const double *Gt = c->G + (size_t)t * N, *Gp = c->G + (size_t)(t - 1) * N;
        const int q = (t - 1) * N;
        for (int j = 0; j < N; ++j) {
            c->At[q + j] = a[o + j] * Gp[j];
            c->Rt[q + j] = r[o + j] * Gt[j];
            c->Bh[q + j] = b[o + j] / Gt[j];
            c->Kh[q + j] = k[o + j] / Gt[j];
            c->Bb[q + j] = b[o + j] * (GL[j] / Gt[j]);
            c->Kb[q + j] = k[o + j] * (GL[j] / Gt[j]);
        }
    }
    for (int t = 0; t < L; ++t)
        for (int s = 0; s < L; ++s) {
            double ab = 0, ak = 0, rb = 0, rk = 0;
            for (int j = 0; j < N; ++j) {
                ab += c->At[t * N + j] * c->Bh[s * N + j];
                ak += c->At[t * N + j] * c->Kh[s * N + j];
                rb += c->Rt[t * N + j] * c->Bh[s * N + j];
                rk += c->Rt[t * N + j] * c->Kh[s * N + j];
            }
            c->Aab[t * L + s] = s < t ? ab : 0.0;
            c->Aak[t * L + s] = s < t ? ak : 0.0;
            c->Arb[t * L + s] = s <= t ? rb : 0.0;
            c->Ark[t * L + s] = s <= t ? rk : 0.0;
        }
    /* Tinv by forward substitution: row t = e_t + sum_{s<t} Aab[t][s] Tinv[s]. */
    for (int t = 0; t < L; ++t)
        for (int c2 = 0; c2 < L; ++c2) {
            double acc = (t == c2) ? 1.0 : 0.0;
            for (int s = 0; s < t; ++s) acc += c->Aab[t * L + s] * c->Tinv[s * L + c2];
            c->Tinv[t * L + c2] = acc;
        }
}

/* Chunk forward given S0 (N x N): fills Z, Y (L x N, [t][i]) and S_L. */
static void chunk_forward(const chunk_t *c, const double *S0, const double *V, double *X,
                          double *Z, double *Y, double *SL) {
    const int L = c->L, N = c->N;
    for (int t = 0; t < L; ++t)
        for (int i = 0; i < N; ++i) {
            double acc = 0;
            for (int j = 0; j < N; ++j) acc += c->At[t * N + j] * S0[i * N + j];
            for (int s = 0; s < L; ++s) acc += c->Aak[t * L + s] * V[s * N + i];
            X[t * N + i] = acc;
        }
    for (int t = 0; t < L; ++t)
        for (int i = 0; i < N; ++i) {
            double acc = 0;
            for (int s = 0; s < L; ++s) acc += c->Tinv[t * L + s] * X[s * N + i];
            Z[t * N + i] = acc;
        }
    if (Y) {
        for (int t = 0; t < L; ++t)
            for (int i = 0; i < N; ++i) {
                double acc = 0;
                for (int j = 0; j < N; ++j) acc += c->Rt[t * N + j] * S0[i * N + j];
                for (int s = 0; s < L; ++s)
                    acc += c->Arb[t * L + s] * Z[s * N + i] + c->Ark[t * L + s] * V[s * N + i];
                Y[t * N + i] = acc;
            }
    }
    const double *GL = c->G + (size_t)L * N;
    for (int i = 0; i < N; ++i)
        for (int j = 0; j < N; ++j) {
            double acc = S0[i * N + j] * GL[j];
            for (int t = 0; t < L; ++t)
                acc += Z[t * N + i] * c->Bb[t * N + j] + V[t * N + i] * c->Kb[t * N + j];
            SL[i * N + j] = acc;
        }
}

static void gather_v(const shape_t *sh, int bb, int hh, int t0, int L, const double *src,
                     double *dst) {
    for (int t = 0; t < L; ++t)
        memcpy(dst + (size_t)t * sh->N, src + tok(sh, bb, t0 + t, hh), sizeof(double) * sh->N);
}

/* Chunked forward, chunk length L (last chunk may be shorter). */
void wkv7_oracle_forward_chunked(int B, int T, int H, int N, int L, const double *r,
                                 const double *w, const double *k, const double *v,
                                 const double *a, const double *b, const double *s0, double *y,
                                 double *sT, int nthreads) {
    shape_t sh = {B, T, H, N};
    const int BH = B * H;
    const size_t NN = (size_t)N * N;
#pragma omp parallel for schedule(dynamic, 1) num_threads(pick_threads(nthreads))
    for (int bh = 0; bh < BH; ++bh) {
        const int bb = bh / H, hh = bh % H;
        double *S = (double *)calloc(NN, sizeof(double));
        double *SL = (double *)calloc(NN, sizeof(double));
        double *V = (double *)calloc((size_t)L * N, sizeof(double));
        double *X = (double *)calloc((size_t)L * N, sizeof(double));
        double *Z = (double *)calloc((size_t)L * N, sizeof(double));
        double *Y = (double *)calloc((size_t)L * N, sizeof(double));
        if (s0) memcpy(S, s0 + st(&sh, bb, hh), sizeof(double) * NN);
        for (int t0 = 0; t0 < T; t0 += L) {
            const int Lc = (T - t0) < L ? (T - t0) : L;
            chunk_t c;
            chunk_alloc(&c, Lc, N);
            chunk_prepare(&c, &sh, bb, hh, t0, r, w, k, a, b);
            gather_v(&sh, bb, hh, t0, Lc, v, V);
            chunk_forward(&c, S, V, X, Z, Y, SL);
            for (int t = 0; t < Lc; ++t)
                memcpy(y + tok(&sh, bb, t0 + t, hh), Y + (size_t)t * N, sizeof(double) * N);
            memcpy(S, SL, sizeof(double) * NN);
            chunk_free(&c);
        }
        if (sT) memcpy(sT + st(&sh, bb, hh), S, sizeof(double) * NN);
        free(S); free(SL); free(V); free(X); free(Z); free(Y);
    }
}

/*
 * Chunked backward (reverse-mode through the chunk form above), fp64.
 * Chunks are visited last to first with the incoming adjoint dSL of the
 * chunk's exit state; each chunk's entry state is recomputed by a forward
 * sweep kept in memory.  Per chunk, with dY the read-out adjoint:
 *   dZ = Arb^T dY + Bb dSL^T,      dX = Tinv^T dZ
 *   dAab = tril_-1(dX Z^T), dAak = tril_-1(dX V^T),
 *   dArb = tril_0(dY Z^T),  dArk = tril_0(dY V^T)
 *   dV  = Aak^T dX + Ark^T dY + Kb dSL^T
 *   dAt = dX S0 + dAab Bh + dAak Kh,   dRt = dY S0 + dArb Bh + dArk Kh
 *   dBh = dAab^T At + dArb^T Rt,       dKh = dAak^T At + dArk^T Rt
 *   dBb = Z dSL,                        dKb = V dSL
 *   dS0 = dSL diag(G_L) + dY^T Rt + dX^T At
 * then the chain rule through the scaled vectors and the log of the decay
 * products (d log G_t collects every factor that G_t enters).
 */
void wkv7_oracle_backward_chunked(int B, int T, int H, int N, int L, const double *r,
                                  const double *w, const double *k, const double *v,
                                  const double *a, const double *b, const double *s0,
                                  const double *dy, const double *dsT, double *dr, double *dw,
                                  double *dk, double *dv, double *da, double *db, double *ds0,
                                  int nthreads) {
    shape_t sh = {B, T, H, N};
    const int BH = B * H;
    const size_t NN = (size_t)N * N;
    const int nchunks = (T + L - 1) / L;
#pragma omp parallel for schedule(dynamic, 1) num_threads(pick_threads(nthreads))
    for (int bh = 0; bh < BH; ++bh) {
        const int bb = bh / H, hh = bh % H;
        double *entry = (double *)calloc(NN * (size_t)nchunks, sizeof(double));
        double *dS = (double *)calloc(NN, sizeof(double));
        double *dSn = (double *)calloc(NN, sizeof(double));
        double *SL = (double *)calloc(NN, sizeof(double));
        const size_t LN = (size_t)L * N, LL = (size_t)L * L;
        double *V = calloc(LN, sizeof(double)), *X = calloc(LN, sizeof(double));
        double *Z = calloc(LN, sizeof(double)), *dY = calloc(LN, sizeof(double));
        double *dZ = calloc(LN, sizeof(double)), *dX = calloc(LN, sizeof(double));
        double *dV = calloc(LN, sizeof(double)), *dAt = calloc(LN, sizeof(double));
        double *dRt = calloc(LN, sizeof(double)), *dBh = calloc(LN, sizeof(double));
        double *dKh = calloc(LN, sizeof(double)), *dBb = calloc(LN, sizeof(double));
        double *dKb = calloc(LN, sizeof(double)), *dlg = calloc(LN, sizeof(double));
        double *dAab = calloc(LL, sizeof(double)), *dAak = calloc(LL, sizeof(double));
        double *dArb = calloc(LL, sizeof(double)), *dArk = calloc(LL, sizeof(double));
        double *dlgL = calloc((size_t)N, sizeof(double));

        if (s0) memcpy(entry, s0 + st(&sh, bb, hh), sizeof(double) * NN);
        for (int c = 0; c < nchunks; ++c) {
            const int t0 = c * L, Lc = (T - t0) < L ? (T - t0) : L;
            chunk_t ch;
            chunk_alloc(&ch, Lc, N);
            chunk_prepare(&ch, &sh, bb, hh, t0, r, w, k, a, b);
            gather_v(&sh, bb, hh, t0, Lc, v, V);
            chunk_forward(&ch, entry + NN * c, V, X, Z, NULL, SL);
            if (c + 1 < nchunks) memcpy(entry + NN * (c + 1), SL, sizeof(double) * NN);
            chunk_free(&ch);
        }
        if (dsT) memcpy(dS, dsT + st(&sh, bb, hh), sizeof(double) * NN);

        for (int c = nchunks - 1; c >= 0; --c) {
            const int t0 = c * L, Lc = (T - t0) < L ? (T - t0) : L;
            const double *S0 = entry + NN * c;
            chunk_t ch;
            chunk_alloc(&ch, Lc, N);
            chunk_prepare(&ch, &sh, bb, hh, t0, r, w, k, a, b);
            gather_v(&sh, bb, hh, t0, Lc, v, V);
            gather_v(&sh, bb, hh, t0, Lc, dy, dY);
            chunk_forward(&ch, S0, V, X, Z, NULL, SL);
            const double *GL = ch.G + (size_t)Lc * N;
            /* dZ = Arb^T dY + Bb dS^T */
            for (int t = 0; t < Lc; ++t)
                for (int i = 0; i < N; ++i) {
                    double acc = 0;
                    for (int s = 0; s < Lc; ++s) acc += ch.Arb[s * Lc + t] * dY[s * N + i];
                    for (int j = 0; j < N; ++j) acc += ch.Bb[t * N + j] * dS[i * N + j];
                    dZ[t * N + i] = acc;
                }
            /* dX = Tinv^T dZ */
            for (int t = 0; t < Lc; ++t)
                for (int i = 0; i < N; ++i) {
                    double acc = 0;
                    for (int s = 0; s < Lc; ++s) acc += ch.Tinv[s * Lc + t] * dZ[s * N + i];
                    dX[t * N + i] = acc;
                }
            /* L x L adjoints (lower-triangular masks as in the forward). */
            for (int t = 0; t < Lc; ++t)
                for (int s = 0; s < Lc; ++s) {
                    double xz = 0, xv = 0, yz = 0, yv = 0;
                    for (int i = 0; i < N; ++i) {
                        xz += dX[t * N + i] * Z[s * N + i];
                        xv += dX[t * N + i] * V[s * N + i];
                        yz += dY[t * N + i] * Z[s * N + i];
                        yv += dY[t * N + i] * V[s * N + i];
                    }
                    dAab[t * Lc + s] = s < t ? xz : 0.0;
                    dAak[t * Lc + s] = s < t ? xv : 0.0;
                    dArb[t * Lc + s] = s <= t ? yz : 0.0;
                    dArk[t * Lc + s] = s <= t ? yv : 0.0;
                }
            /* dV = Aak^T dX + Ark^T dY + Kb dS^T */
            for (int t = 0; t < Lc; ++t)
                for (int i = 0; i < N; ++i) {
                    double acc = 0;
                    for (int s = 0; s < Lc; ++s)
                        acc += ch.Aak[s * Lc + t] * dX[s * N + i] +
                               ch.Ark[s * Lc + t] * dY[s * N + i];
                    for (int j = 0; j < N; ++j) acc += ch.Kb[t * N + j] * dS[i * N + j];
                    dV[t * N + i] = acc;
                }
            /* [t][j]-shaped adjoints of the scaled vectors. */
            for (int t = 0; t < Lc; ++t)
                for (int j = 0; j < N; ++j) {
                    double at_ = 0, rt_ = 0, bh_ = 0, kh_ = 0, bb_ = 0, kb_ = 0;
                    for (int i = 0; i < N; ++i) {
                        at_ += dX[t * N + i] * S0[i * N + j];
                        rt_ += dY[t * N + i] * S0[i * N + j];
                        bb_ += Z[t * N + i] * dS[i * N + j];
                        kb_ += V[t * N + i] * dS[i * N + j];
                    }
                    for (int s = 0; s < Lc; ++s) {
                        at_ += dAab[t * Lc + s] * ch.Bh[s * N + j] +
                               dAak[t * Lc + s] * ch.Kh[s * N + j];
                        rt_ += dArb[t * Lc + s] * ch.Bh[s * N + j] +
                               dArk[t * Lc + s] * ch.Kh[s * N + j];
                        bh_ += dAab[s * Lc + t] * ch.At[s * N + j] +
                               dArb[s * Lc + t] * ch.Rt[s * N + j];
                        kh_ += dAak[s * Lc + t] * ch.At[s * N + j] +
                               dArk[s * Lc + t] * ch.Rt[s * N + j];
                    }
                    dAt[t * N + j] = at_;
                    dRt[t * N + j] = rt_;
                    dBh[t * N + j] = bh_;
                    dKh[t * N + j] = kh_;
                    dBb[t * N + j] = bb_;
                    dKb[t * N + j] = kb_;
                }
            /* Gradients of the raw inputs and of log G_t. */
            for (int j = 0; j < N; ++j) {
                double acc = 0;
                for (int i = 0; i < N; ++i) acc += dS[i * N + j] * S0[i * N + j];
                dlgL[j] = acc * GL[j];
            }
            for (int t = 0; t < Lc; ++t) {
                const size_t o = tok(&sh, bb, t0 + t, hh);
                const double *Gt = ch.G + (size_t)(t + 1) * N, *Gp = ch.G + (size_t)t * N;
                for (int j = 0; j < N; ++j) {
                    const int q = t * N + j;
                    da[o + j] = dAt[q] * Gp[j];
                    dr[o + j] = dRt[q] * Gt[j];
                    db[o + j] = dBh[q] / Gt[j] + dBb[q] * (GL[j] / Gt[j]);
                    dk[o + j] = dKh[q] / Gt[j] + dKb[q] * (GL[j] / Gt[j]);
                    dv[o + j] = dV[q];
                    double g = dRt[q] * ch.Rt[q] - dBh[q] * ch.Bh[q] - dKh[q] * ch.Kh[q] -
                               dBb[q] * ch.Bb[q] - dKb[q] * ch.Kb[q];
                    if (t + 1 < Lc) g += dAt[q + N] * ch.At[q + N];
                    dlg[q] = g;
                    dlgL[j] += dBb[q] * ch.Bb[q] + dKb[q] * ch.Kb[q];
                }
            }
            for (int j = 0; j < N; ++j) dlg[(Lc - 1) * N + j] += dlgL[j];
            /* log G_t = sum_{u<=t} log w_u  =>  d log w_u = sum_{t>=u} dlg_t. */
            for (int j = 0; j < N; ++j) {
                double acc = 0;
                for (int t = Lc - 1; t >= 0; --t) {
                    const size_t o = tok(&sh, bb, t0 + t, hh);
                    acc += dlg[t * N + j];
                    dw[o + j] = acc / w[o + j];
                }
            }
            /* dS0 = dS diag(G_L) + dY^T Rt + dX^T At */
            for (int i = 0; i < N; ++i)
                for (int j = 0; j < N; ++j) {
                    double acc = dS[i * N + j] * GL[j];
                    for (int t = 0; t < Lc; ++t)
                        acc += dY[t * N + i] * ch.Rt[t * N + j] + dX[t * N + i] * ch.At[t * N + j];
                    dSn[i * N + j] = acc;
                }
            memcpy(dS, dSn, sizeof(double) * NN);
            chunk_free(&ch);
        }
        if (ds0) memcpy(ds0 + st(&sh, bb, hh), dS, sizeof(double) * NN);
        free(entry); free(dS); free(dSn); free(SL);
        free(V); free(X); free(Z); free(dY); free(dZ); free(dX); free(dV);
        free(dAt); free(dRt); free(dBh); free(dKh); free(dBb); free(dKb); free(dlg);
        free(dAab); free(dAak); free(dArb); free(dArk); free(dlgL);
    }
}

/*
 * The step after the read-out, per token and head (fp64).  "Paper Review:
 * RWKV-7 Goose", The approach: the receptance also attends to the current token
 * without storing it in the state, and the result is normalised, combined
 * across heads and gated (the combination, an output projection, lies outside
 * this step).  The pages fix neither the current-token formula nor the
 * normalisation, nor the order of the two; the reading taken, with the learned
 * parts as inputs:
 *   s      = sum_j r_t[j] u[j] k_t[j]                    (u: one vector per head)
 *   norm x = gamma (x - mean x) / sqrt(var x + eps) + beta over the head's N
 *            channels, var the mean squared deviation
 *   mode 0: out = g_t (y_t + s v_t)                       (no normalisation)
 *   mode 1: out = g_t (norm(y_t) + s v_t)
 *   mode 2: out = g_t norm(y_t + s v_t)
 * Layouts: y, r, k, v, g, out [B][T][H][N]; u, gamma, beta [H][N].  NULL
 * means g = 1, u = 0, gamma = 1, beta = 0.
 */
void wkv7_oracle_epilogue(int B, int T, int H, int N, const double *y, const double *r,
                          const double *k, const double *v, const double *g, const double *u,
                          const double *gamma, const double *beta, double eps, int mode,
                          double *out, int nthreads) {
    shape_t sh = {B, T, H, N};
    const long rows = (long)B * T * H;
#pragma omp parallel for schedule(static) num_threads(pick_threads(nthreads))
    for (long row = 0; row < rows; ++row) {
        const int h = (int)(row % H);
        const long t = row / H;
        const int b = (int)(t / T), tt = (int)(t % T);
        const size_t o = tok(&sh, b, tt, h);
        double *x = malloc(sizeof(double) * (size_t)N);
        double s = 0.0;
        if (u)
            for (int j = 0; j < N; ++j) s += r[o + j] * u[(size_t)h * N + j] * k[o + j];
        /* x = what is normalised (mode 1, 2) or the result before the gate (mode 0) */
        for (int i = 0; i < N; ++i) x[i] = (mode == 1) ? y[o + i] : y[o + i] + s * v[o + i];
        if (mode != 0) {
            double mean = 0.0, var = 0.0;
            for (int i = 0; i < N; ++i) mean += x[i];
            mean /= N;
            for (int i = 0; i < N; ++i) var += (x[i] - mean) * (x[i] - mean);
            var /= N;
            const double inv_sd = 1.0 / sqrt(var + eps);
            for (int i = 0; i < N; ++i) {
                double n = (x[i] - mean) * inv_sd;
                if (gamma) n *= gamma[(size_t)h * N + i];
                if (beta) n += beta[(size_t)h * N + i];
                x[i] = (mode == 1) ? n + s * v[o + i] : n;
            }
        }
        for (int i = 0; i < N; ++i) out[o + i] = (g ? g[o + i] : 1.0) * x[i];
        free(x);
    }
}
