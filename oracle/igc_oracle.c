/*
 * igc_oracle.c -- plain, slow, obviously-correct CPU reference for the GEMM and
 * the NHWC convolution that the HIP library computes.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, calls or
 * includes this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header or constant with the HIP path.
 *
 * What it computes (the definitions, written out):
 *
 *   GEMM   C[i][j] = sum_{k<K} a(i,k) * b(k,j)
 *          a(i,k) = A[i*lda + k] (row-major) or A[k*lda + i] (column-major),
 *          b(k,j) = B[k*ldb + j] (row-major) or B[j*ldb + k] (column-major).
 *          This is the product whose tiled, software-pipelined evaluation the
 *          "B200 TMA Pipeline Designer" page describes (its "Executable steps":
 *          the stage ring feeding the MMA, and its validation list of small
 *          asymmetric matrices, boundary tiles and varied K_TILES).
 *
 *   CONV   y[n][p][q][k] = sum_{r<R, s<S, c<C} x[n][h][w][c] * wt[k][r][s][c],
 *          h = p*sh - ph + r*dh,  w = q*sw - pw + s*dw,
 *          terms whose (h, w) lies outside the H x W image are omitted (zero
 *          padding).  x is NHWC, wt is KRSC, y is NPQK with
 *          P = (H + 2ph - dh(R-1) - 1)/sh + 1 and Q likewise.  This is the
 *          convolution that the "two free pipeline stages" note runs as an
 *          implicit GEMM with IM2COL loads (section "The atom changes the
 *          fragment"); cross-correlation, forward only.
 *
 *   DGRAD  dx[n][h][w][c] = sum over (r, s, k) of dy[n][p][q][k] * wt[k][r][s][c],
 *          over the filter taps at which the forward convolution reads
 *          x[n][h][w]: p*sh - ph + r*dh = h and q*sw - pw + s*dw = w for
 *          integers 0 <= p < P, 0 <= q < Q.  This is the derivative of
 *          sum(y * dy) with respect to x, i.e. the adjoint of the forward
 *          convolution in x.  dy is NPQK, dx is NHWC.
 *
 *   WGRAD  dw[k][r][s][c] = sum over (n, p, q) of dy[n][p][q][k] * x[n][h][w][c],
 *          h = p*sh - ph + r*dh, w = q*sw - pw + s*dw, terms outside the
 *          image omitted: the derivative of sum(y * dy) with respect to the
 *          filter, the adjoint of the forward convolution in wt.  dw is KRSC.
 *          Both gradients run on the same implicit-GEMM mainloop as the
 *          forward pass (the "two free pipeline stages" note runs the forward
 *          convolution through it; the data and filter gradients are the two
 *          other convolutions of a training step).
 *
 *   Each output also gets its absolute-product sum S = sum |a*b| (same index
 *   set), which scales the error bound |y - C| <= 1e-4*S + 1e-6.
 *
 * How: every stored 16-bit input is decoded exactly to double, every product
 * of two bf16 or two fp16 values is exact in double, and each output's sum is
 * taken sequentially in increasing k (GEMM) or in (r, s, c) order (conv) in
 * double (dgrad in (r, s, k) order, wgrad in (n, p, q) order).  Threads split
 * the OUTPUT elements only, so the result does not depend
 * on the thread count.  No fast-math.
 *
 * dtype: 0 = bfloat16 bits, 1 = IEEE binary16 bits.
 * Return value: number of threads used (>= 1), or a negative error code.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define OR_EINVAL (-1)
#define OR_ENOMEM (-2)

/* bfloat16: the upper 16 bits of an IEEE binary32. */
static double dec_bf16(uint16_t bits) {
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double dec_fp16(uint16_t bits) {
    int sign = (bits >> 15) & 1;
    int e = (bits >> 10) & 0x1f;
    int m = bits & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
    } else if (e == 31) {
        v = m ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

static double dec(uint16_t bits, int dtype) { return dtype ? dec_fp16(bits) : dec_bf16(bits); }

double oracle_decode(uint16_t bits, int dtype) { return dec(bits, dtype); }

static int pick_threads(int want, int64_t work_rows) {
    int n = want;
    if (n <= 0) {
        long c = sysconf(_SC_NPROCESSORS_ONLN);
        n = c > 0 ? (int)c : 1;
    }
    if (n > 256) n = 256;
    if ((int64_t)n > work_rows) n = work_rows > 0 ? (int)work_rows : 1;
    return n;
}

/* Runs fn(arg_i) for i in [0, n) on n threads (thread 0 is the caller). */
static int run_threads(int n, void *(*fn)(void *), void *args, size_t arg_size) {
    pthread_t tid[256];
    int started = 0;
    for (int i = 1; i < n; i++) {
        if (pthread_create(&tid[i], NULL, fn, (char *)args + (size_t)i * arg_size) != 0) break;
        started = i;
    }
    fn(args);
    for (int i = 1; i <= started; i++) pthread_join(tid[i], NULL);
    /* Any range a thread failed to start for is run here, serially. */
    for (int i = started + 1; i < n; i++) fn((char *)args + (size_t)i * arg_size);
    return n;
}

/* ------------------------------------------------------------------------- */
/* GEMM, every output                                                         */
/* ------------------------------------------------------------------------- */

typedef struct {
    int64_t M, N, K, row0, row1;
    const double *Ad, *Bd; /* decoded: Ad[i*K + k], Bd[k*N + j] */
    double *C, *S;
} gemm_job;

static void *gemm_rows(void *p) {
    gemm_job *jb = (gemm_job *)p;
    const int64_t N = jb->N, K = jb->K;
    for (int64_t i = jb->row0; i < jb->row1; i++) {
        double *c = jb->C + i * N;
        double *s = jb->S + i * N;
        for (int64_t j = 0; j < N; j++) { c[j] = 0.0; s[j] = 0.0; }
        for (int64_t k = 0; k < K; k++) { /* i-k-j: each c[j] still sums k in order */
            const double a = jb->Ad[i * K + k];
            const double *b = jb->Bd + k * N;
            for (int64_t j = 0; j < N; j++) {
                const double prod = a * b[j];
                c[j] += prod;
                s[j] += fabs(prod);
            }
        }
    }
    return NULL;
}

int oracle_gemm(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda, int a_col_major,
                const uint16_t *B, int64_t ldb, int b_col_major, int dtype, double *C, double *S,
                int nthreads) {
    if (M < 0 || N < 0 || K < 0 || (M * N > 0 && (!C || !S))) return OR_EINVAL;
    if (K > 0 && M > 0 && (!A || lda < (a_col_major ? M : K))) return OR_EINVAL;
    if (K > 0 && N > 0 && (!B || ldb < (b_col_major ? K : N))) return OR_EINVAL;
    double *Ad = (double *)malloc((size_t)(M * K + 1) * sizeof(double));
    double *Bd = (double *)malloc((size_t)(K * N + 1) * sizeof(double));
    if (!Ad || !Bd) { free(Ad); free(Bd); return OR_ENOMEM; }
    for (int64_t i = 0; i < M; i++)
        for (int64_t k = 0; k < K; k++)
            Ad[i * K + k] = dec(a_col_major ? A[k * lda + i] : A[i * lda + k], dtype);
    for (int64_t k = 0; k < K; k++)
        for (int64_t j = 0; j < N; j++)
            Bd[k * N + j] = dec(b_col_major ? B[j * ldb + k] : B[k * ldb + j], dtype);
    int n = pick_threads(nthreads, M);
    gemm_job jobs[256];
    for (int t = 0; t < n; t++) {
        jobs[t].M = M; jobs[t].N = N; jobs[t].K = K;
        jobs[t].row0 = M * t / n; jobs[t].row1 = M * (t + 1) / n;
        jobs[t].Ad = Ad; jobs[t].Bd = Bd; jobs[t].C = C; jobs[t].S = S;
    }
    run_threads(n, gemm_rows, jobs, sizeof(gemm_job));
    free(Ad); free(Bd);
    return n;
}

/* ------------------------------------------------------------------------- */
/* GEMM, selected outputs (for shapes too large to evaluate whole)            */
/* ------------------------------------------------------------------------- */

typedef struct {
    int64_t K, lda, ldb, i0, i1;
    int a_col_major, b_col_major, dtype;
    const uint16_t *A, *B;
    const int64_t *rows, *cols;
    double *c, *s;
} gemm_sample_job;

static void *gemm_samples(void *p) {
    gemm_sample_job *jb = (gemm_sample_job *)p;
    for (int64_t t = jb->i0; t < jb->i1; t++) {
        const int64_t i = jb->rows[t], j = jb->cols[t];
        double acc = 0.0, sacc = 0.0;
        for (int64_t k = 0; k < jb->K; k++) {
            const double a = dec(jb->a_col_major ? jb->A[k * jb->lda + i] : jb->A[i * jb->lda + k], jb->dtype);
            const double b = dec(jb->b_col_major ? jb->B[j * jb->ldb + k] : jb->B[k * jb->ldb + j], jb->dtype);
            acc += a * b;
            sacc += fabs(a * b);
        }
        jb->c[t] = acc;
        jb->s[t] = sacc;
    }
    return NULL;
}

int oracle_gemm_sample(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda, int a_col_major,
                       const uint16_t *B, int64_t ldb, int b_col_major, int dtype, int64_t nsamp,
                       const int64_t *rows, const int64_t *cols, double *c, double *s, int nthreads) {
    if (M < 0 || N < 0 || K < 0 || nsamp < 0 || (nsamp > 0 && (!rows || !cols || !c || !s))) return OR_EINVAL;
    for (int64_t t = 0; t < nsamp; t++)
        if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N) return OR_EINVAL;
    if (K > 0 && nsamp > 0 && (!A || !B || lda < (a_col_major ? M : K) || ldb < (b_col_major ? K : N)))
        return OR_EINVAL;
    int n = pick_threads(nthreads, nsamp);
    gemm_sample_job jobs[256];
    for (int t = 0; t < n; t++) {
        jobs[t].K = K; jobs[t].lda = lda; jobs[t].ldb = ldb;
        jobs[t].i0 = nsamp * t / n; jobs[t].i1 = nsamp * (t + 1) / n;
        jobs[t].a_col_major = a_col_major; jobs[t].b_col_major = b_col_major; jobs[t].dtype = dtype;
        jobs[t].A = A; jobs[t].B = B; jobs[t].rows = rows; jobs[t].cols = cols; jobs[t].c = c; jobs[t].s = s;
    }
    run_threads(n, gemm_samples, jobs, sizeof(gemm_sample_job));
    return n;
}

/* ------------------------------------------------------------------------- */
/* Direct convolution, NHWC input, KRSC filter, NPQK output                   */
/* ------------------------------------------------------------------------- */

typedef struct {
    int64_t N, H, W, C, K, R, S, sh, sw, ph, pw, dh, dw, P, Q;
    int dtype;
    const uint16_t *x, *w, *dy; /* forward input, filter, output gradient (NPQK) */
    /* either a contiguous range of output pixels (flat n*P*Q index) ... */
    int64_t pix0, pix1;
    double *y, *ys;
    /* ... or a list of flat NPQK output indices */
    const int64_t *idx;
    int64_t i0, i1;
} conv_job;

/* One output element: direct sum over (r, s, c) of in-bounds taps. */
static void conv_point(const conv_job *jb, int64_t n, int64_t p, int64_t q, int64_t k, double *out,
                       double *outs) {
    double acc = 0.0, sacc = 0.0;
    for (int64_t r = 0; r < jb->R; r++) {
        const int64_t h = p * jb->sh - jb->ph + r * jb->dh;
        if (h < 0 || h >= jb->H) continue;
        for (int64_t s = 0; s < jb->S; s++) {
            const int64_t w = q * jb->sw - jb->pw + s * jb->dw;
            if (w < 0 || w >= jb->W) continue;
            const uint16_t *xp = jb->x + ((n * jb->H + h) * jb->W + w) * jb->C;
            const uint16_t *wp = jb->w + ((k * jb->R + r) * jb->S + s) * jb->C;
            for (int64_t c = 0; c < jb->C; c++) {
                const double prod = dec(xp[c], jb->dtype) * dec(wp[c], jb->dtype);
                acc += prod;
                sacc += fabs(prod);
            }
        }
    }
    *out = acc;
    *outs = sacc;
}

static void *conv_pixels(void *p) {
    conv_job *jb = (conv_job *)p;
    for (int64_t pix = jb->pix0; pix < jb->pix1; pix++) {
        const int64_t n = pix / (jb->P * jb->Q), pq = pix % (jb->P * jb->Q);
        const int64_t pp = pq / jb->Q, qq = pq % jb->Q;
        for (int64_t k = 0; k < jb->K; k++) conv_point(jb, n, pp, qq, k, &jb->y[pix * jb->K + k], &jb->ys[pix * jb->K + k]);
    }
    return NULL;
}

static void *conv_points(void *p) {
    conv_job *jb = (conv_job *)p;
    for (int64_t t = jb->i0; t < jb->i1; t++) {
        int64_t f = jb->idx[t];
        const int64_t k = f % jb->K; f /= jb->K;
        const int64_t qq = f % jb->Q; f /= jb->Q;
        const int64_t pp = f % jb->P; f /= jb->P;
        conv_point(jb, f, pp, qq, k, &jb->y[t], &jb->ys[t]);
    }
    return NULL;
}

static int conv_setup(conv_job *jb, int64_t N, int64_t H, int64_t W, int64_t C, int64_t K, int64_t R, int64_t S,
                      int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw, const uint16_t *x,
                      const uint16_t *w, int dtype) {
    if (N < 0 || H < 1 || W < 1 || C < 0 || K < 0 || R < 1 || S < 1 || sh < 1 || sw < 1 || ph < 0 || pw < 0 ||
        dh < 1 || dw < 1)
        return OR_EINVAL;
    const int64_t P = (H + 2 * ph - dh * (R - 1) - 1) / sh + 1;
    const int64_t Q = (W + 2 * pw - dw * (S - 1) - 1) / sw + 1;
    if (H + 2 * ph - dh * (R - 1) - 1 < 0 || W + 2 * pw - dw * (S - 1) - 1 < 0) return OR_EINVAL;
    memset(jb, 0, sizeof *jb);
    jb->N = N; jb->H = H; jb->W = W; jb->C = C; jb->K = K; jb->R = R; jb->S = S;
    jb->sh = sh; jb->sw = sw; jb->ph = ph; jb->pw = pw; jb->dh = dh; jb->dw = dw;
    jb->P = P; jb->Q = Q; jb->dtype = dtype; jb->x = x; jb->w = w;
    return 0;
}

int oracle_conv2d_nhwc(int64_t N, int64_t H, int64_t W, int64_t C, int64_t K, int64_t R, int64_t S, int64_t sh,
                       int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw, const uint16_t *x,
                       const uint16_t *w, int dtype, double *y, double *ys, int nthreads) {
    conv_job base;
    if (conv_setup(&base, N, H, W, C, K, R, S, sh, sw, ph, pw, dh, dw, x, w, dtype) != 0) return OR_EINVAL;
    const int64_t npix = N * base.P * base.Q;
    if (npix * K > 0 && (!y || !ys)) return OR_EINVAL;
    if (npix > 0 && K > 0 && C > 0 && (!x || !w)) return OR_EINVAL;
    int n = pick_threads(nthreads, npix);
    conv_job jobs[256];
    for (int t = 0; t < n; t++) {
        jobs[t] = base;
        jobs[t].pix0 = npix * t / n; jobs[t].pix1 = npix * (t + 1) / n;
        jobs[t].y = y; jobs[t].ys = ys;
    }
    run_threads(n, conv_pixels, jobs, sizeof(conv_job));
    return n;
}

int oracle_conv2d_nhwc_sample(int64_t N, int64_t H, int64_t W, int64_t C, int64_t K, int64_t R, int64_t S,
                              int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw,
                              const uint16_t *x, const uint16_t *w, int dtype, int64_t nsamp, const int64_t *idx,
                              double *y, double *ys, int nthreads) {
    conv_job base;
    if (conv_setup(&base, N, H, W, C, K, R, S, sh, sw, ph, pw, dh, dw, x, w, dtype) != 0) return OR_EINVAL;
    if (nsamp < 0 || (nsamp > 0 && (!idx || !y || !ys))) return OR_EINVAL;
    const int64_t total = N * base.P * base.Q * K;
    for (int64_t t = 0; t < nsamp; t++)
        if (idx[t] < 0 || idx[t] >= total) return OR_EINVAL;
    if (nsamp > 0 && C > 0 && (!x || !w)) return OR_EINVAL;
    int n = pick_threads(nthreads, nsamp);
    conv_job jobs[256];
    for (int t = 0; t < n; t++) {
        jobs[t] = base;
        jobs[t].idx = idx; jobs[t].i0 = nsamp * t / n; jobs[t].i1 = nsamp * (t + 1) / n;
        jobs[t].y = y; jobs[t].ys = ys;
    }
    run_threads(n, conv_points, jobs, sizeof(conv_job));
    return n;
}

/* ------------------------------------------------------------------------- */
/* Data gradient: dx (NHWC) from dy (NPQK) and the filter (KRSC)              */
/* ------------------------------------------------------------------------- */

/* One dx element: every (r, s, k) whose forward tap lands on (h, w). */
static void dgrad_point(const conv_job *jb, int64_t n, int64_t h, int64_t w, int64_t c, double *out,
                        double *outs) {
    double acc = 0.0, sacc = 0.0;
    for (int64_t r = 0; r < jb->R; r++) {
        const int64_t pnum = h + jb->ph - r * jb->dh; /* = p * sh */
        if (pnum < 0 || pnum % jb->sh != 0) continue;
        const int64_t p = pnum / jb->sh;
        if (p >= jb->P) continue;
        for (int64_t s = 0; s < jb->S; s++) {
            const int64_t qnum = w + jb->pw - s * jb->dw; /* = q * sw */
            if (qnum < 0 || qnum % jb->sw != 0) continue;
            const int64_t q = qnum / jb->sw;
            if (q >= jb->Q) continue;
            const uint16_t *dyp = jb->dy + ((n * jb->P + p) * jb->Q + q) * jb->K;
            for (int64_t k = 0; k < jb->K; k++) {
                const double prod = dec(dyp[k], jb->dtype) * dec(jb->w[((k * jb->R + r) * jb->S + s) * jb->C + c], jb->dtype);
                acc += prod;
                sacc += fabs(prod);
            }
        }
    }
    *out = acc;
    *outs = sacc;
}

static void *dgrad_pixels(void *p) {
    conv_job *jb = (conv_job *)p;
    for (int64_t pix = jb->pix0; pix < jb->pix1; pix++) {
        const int64_t n = pix / (jb->H * jb->W), hw = pix % (jb->H * jb->W);
        const int64_t h = hw / jb->W, w = hw % jb->W;
        for (int64_t c = 0; c < jb->C; c++) dgrad_point(jb, n, h, w, c, &jb->y[pix * jb->C + c], &jb->ys[pix * jb->C + c]);
    }
    return NULL;
}

static void *dgrad_points(void *p) {
    conv_job *jb = (conv_job *)p;
    for (int64_t t = jb->i0; t < jb->i1; t++) {
        int64_t f = jb->idx[t];
        const int64_t c = f % jb->C; f /= jb->C;
        const int64_t w = f % jb->W; f /= jb->W;
        const int64_t h = f % jb->H; f /= jb->H;
        dgrad_point(jb, f, h, w, c, &jb->y[t], &jb->ys[t]);
    }
    return NULL;
}

int oracle_conv2d_dgrad_nhwc(int64_t N, int64_t H, int64_t W, int64_t C, int64_t K, int64_t R, int64_t S, int64_t sh,
                             int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw, const uint16_t *dy,
                             const uint16_t *w, int dtype, double *dx, double *dxs, int nthreads) {
    conv_job base;
    if (conv_setup(&base, N, H, W, C, K, R, S, sh, sw, ph, pw, dh, dw, NULL, w, dtype) != 0) return OR_EINVAL;
    base.dy = dy;
    const int64_t npix = N * H * W;
    if (npix * C > 0 && (!dx || !dxs)) return OR_EINVAL;
    if (npix > 0 && C > 0 && K > 0 && (!dy || !w)) return OR_EINVAL;
    int n = pick_threads(nthreads, npix);
    conv_job jobs[256];
    for (int t = 0; t < n; t++) {
        jobs[t] = base;
        jobs[t].pix0 = npix * t / n; jobs[t].pix1 = npix * (t + 1) / n;
        jobs[t].y = dx; jobs[t].ys = dxs;
    }
    run_threads(n, dgrad_pixels, jobs, sizeof(conv_job));
    return n;
}

int oracle_conv2d_dgrad_nhwc_sample(int64_t N, int64_t H, int64_t W, int64_t C, int64_t K, int64_t R, int64_t S,
                                    int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw,
                                    const uint16_t *dy, const uint16_t *w, int dtype, int64_t nsamp,
                                    const int64_t *idx, double *dx, double *dxs, int nthreads) {
    conv_job base;
    if (conv_setup(&base, N, H, W, C, K, R, S, sh, sw, ph, pw, dh, dw, NULL, w, dtype) != 0) return OR_EINVAL;
    base.dy = dy;
    if (nsamp < 0 || (nsamp > 0 && (!idx || !dx || !dxs))) return OR_EINVAL;
    const int64_t total = N * H * W * C;
    for (int64_t t = 0; t < nsamp; t++)
        if (idx[t] < 0 || idx[t] >= total) return OR_EINVAL;
    if (nsamp > 0 && K > 0 && (!dy || !w)) return OR_EINVAL;
    int n = pick_threads(nthreads, nsamp);
    conv_job jobs[256];
    for (int t = 0; t < n; t++) {
        jobs[t] = base;
        jobs[t].idx = idx; jobs[t].i0 = nsamp * t / n; jobs[t].i1 = nsamp * (t + 1) / n;
        jobs[t].y = dx; jobs[t].ys = dxs;
    }
    run_threads(n, dgrad_points, jobs, sizeof(conv_job));
    return n;
}

/* ------------------------------------------------------------------------- */
/* Filter gradient: dw (KRSC) from x (NHWC) and dy (NPQK)                     */
/* ------------------------------------------------------------------------- */

/* One dw element: every output pixel (n, p, q) whose window puts tap (r, s) inside the image. */
static void wgrad_point(const conv_job *jb, int64_t k, int64_t r, int64_t s, int64_t c, double *out, double *outs) {
    double acc = 0.0, sacc = 0.0;
    for (int64_t n = 0; n < jb->N; n++)
        for (int64_t p = 0; p < jb->P; p++) {
            const int64_t h = p * jb->sh - jb->ph + r * jb->dh;
            if (h < 0 || h >= jb->H) continue;
            for (int64_t q = 0; q < jb->Q; q++) {
                const int64_t w = q * jb->sw - jb->pw + s * jb->dw;
                if (w < 0 || w >= jb->W) continue;
                const double prod = dec(jb->dy[((n * jb->P + p) * jb->Q + q) * jb->K + k], jb->dtype) *
                                    dec(jb->x[((n * jb->H + h) * jb->W + w) * jb->C + c], jb->dtype);
                acc += prod;
                sacc += fabs(prod);
            }
        }
    *out = acc;
    *outs = sacc;
}

static void *wgrad_points(void *p) {
    conv_job *jb = (conv_job *)p;
    for (int64_t t = jb->i0; t < jb->i1; t++) {
        int64_t f = jb->idx ? jb->idx[t] : t;
        const int64_t c = f % jb->C; f /= jb->C;
        const int64_t s = f % jb->S; f /= jb->S;
        const int64_t r = f % jb->R; f /= jb->R;
        wgrad_point(jb, f, r, s, c, &jb->y[t], &jb->ys[t]);
    }
    return NULL;
}

/* idx == NULL: every element, in KRSC order (nsamp must be K*R*S*C). */
int oracle_conv2d_wgrad_nhwc_sample(int64_t N, int64_t H, int64_t W, int64_t C, int64_t K, int64_t R, int64_t S,
                                    int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw,
                                    const uint16_t *x, const uint16_t *dy, int dtype, int64_t nsamp,
                                    const int64_t *idx, double *dwt, double *dws, int nthreads) {
    conv_job base;
    if (conv_setup(&base, N, H, W, C, K, R, S, sh, sw, ph, pw, dh, dw, x, NULL, dtype) != 0) return OR_EINVAL;
    base.dy = dy;
    const int64_t total = K * R * S * C;
    if (nsamp < 0 || (nsamp > 0 && (!dwt || !dws)) || (!idx && nsamp != total)) return OR_EINVAL;
    if (idx)
        for (int64_t t = 0; t < nsamp; t++)
            if (idx[t] < 0 || idx[t] >= total) return OR_EINVAL;
    if (nsamp > 0 && N * base.P * base.Q > 0 && (!x || !dy)) return OR_EINVAL;
    int n = pick_threads(nthreads, nsamp);
    conv_job jobs[256];
    for (int t = 0; t < n; t++) {
        jobs[t] = base;
        jobs[t].idx = idx; jobs[t].i0 = nsamp * t / n; jobs[t].i1 = nsamp * (t + 1) / n;
        jobs[t].y = dwt; jobs[t].ys = dws;
    }
    run_threads(n, wgrad_points, jobs, sizeof(conv_job));
    return n;
}

int oracle_conv2d_wgrad_nhwc(int64_t N, int64_t H, int64_t W, int64_t C, int64_t K, int64_t R, int64_t S, int64_t sh,
                             int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw, const uint16_t *x,
                             const uint16_t *dy, int dtype, double *dwt, double *dws, int nthreads) {
    if (K < 0 || R < 1 || S < 1 || C < 0) return OR_EINVAL;
    return oracle_conv2d_wgrad_nhwc_sample(N, H, W, C, K, R, S, sh, sw, ph, pw, dh, dw, x, dy, dtype, K * R * S * C,
                                           NULL, dwt, dws, nthreads);
}
