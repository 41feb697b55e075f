/*
 * Driver for a sanitizer build of the float64 oracle (test infrastructure):
 * calls every exported oracle function on small deterministic inputs
 * (float32 and bfloat16 inputs, float64 and bfloat16 state, the backward)
 * so that AddressSanitizer and UndefinedBehaviorSanitizer see every loop
 * and index the tests use.  Built and run by tests/test_oracle_sanitize.py
 * together with oracle/sdm_oracle.c; prints "ok" and exits 0 when no
 * function reports an error.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int sdm_oracle_topk_rows(int64_t nrows, int sqrtN, int K, const void *x, int dtype,
                         int32_t *idx, double *wts, double *shi, double *slo, int nthreads);
void sdm_oracle_round_bf16(const double *x, double *out, int64_t n);
int sdm_oracle_recurrence(int B, int64_t T, int H, int sqrtN, int d_v, int W, int R,
                          const int32_t *Iw, const double *kw, const int32_t *Ir,
                          const double *qw, const void *v, int v_dtype, const float *alpha,
                          const float *beta, const float *M0, int state_mode, int scale_log2,
                          int c0, int c1, double *y, double *M, int nthreads);
void sdm_oracle_round_fp8(const double *x, double *out, int64_t n, int s);
int sdm_oracle_backward(int B, int64_t T, int H, int sqrtN, int d_v, int W, int R,
                        const int32_t *Iw, const double *kw, const int32_t *Ir, const double *qw,
                        const void *v, int v_dtype, const float *alpha, const float *beta,
                        const float *M0, const double *dy, const double *dMT, double *dkp,
                        double *dqp, double *dv, double *dalpha, double *dbeta, double *dM0,
                        int nthreads);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;

static double uniform(void) /* in [-1, 1): a 64-bit linear congruential step */
{
    g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(g_state >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}

static uint16_t to_bf16_bits(float f) /* truncation is enough for test inputs */
{
    union { float f; uint32_t u; } c;
    c.f = f;
    return (uint16_t)(c.u >> 16);
}

static void *xmalloc(size_t n)
{
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

#define CHECK(x)                                                   \
    do {                                                           \
        int rc_ = (x);                                             \
        if (rc_ != 0) {                                            \
            fprintf(stderr, "%s returned %d\n", #x, rc_);          \
            return 1;                                              \
        }                                                          \
    } while (0)

int main(void)
{
    const int B = 2, H = 2, S = 8, D = 12, W = 5, R = 6, threads = 3;
    const int64_t T = 37, N = (int64_t)S * S, ht = (int64_t)B * T * H;
    float *kp = xmalloc(sizeof(float) * ht * 2 * S), *qp = xmalloc(sizeof(float) * ht * 2 * S);
    float *v = xmalloc(sizeof(float) * ht * D);
    uint16_t *kb = xmalloc(2 * ht * 2 * S), *qb = xmalloc(2 * ht * 2 * S), *vb = xmalloc(2 * ht * D);
    float *alpha = xmalloc(sizeof(float) * ht), *beta = xmalloc(sizeof(float) * ht);
    float *M0 = xmalloc(sizeof(float) * H * N * D);
    for (int64_t i = 0; i < ht * 2 * S; i++) {
        kp[i] = (float)(2.0 * uniform());
        qp[i] = (float)(2.0 * uniform());
        if (i % 7 == 0) kp[i] = 0.5f; /* ties */
        kb[i] = to_bf16_bits(kp[i]);
        qb[i] = to_bf16_bits(qp[i]);
    }
    for (int64_t i = 0; i < ht * D; i++) {
        v[i] = (float)uniform();
        vb[i] = to_bf16_bits(v[i]);
    }
    for (int64_t i = 0; i < ht; i++) {
        alpha[i] = (float)(0.75 + 0.25 * uniform());
        beta[i] = (float)(0.5 + 0.5 * uniform());
    }
    for (int64_t i = 0; i < H * N * D; i++) M0[i] = (float)(0.02 * uniform());

    int32_t *Iw = xmalloc(sizeof(int32_t) * ht * W), *Ir = xmalloc(sizeof(int32_t) * ht * R);
    double *kw = xmalloc(sizeof(double) * ht * W), *qw = xmalloc(sizeof(double) * ht * R);
    double *hi = xmalloc(sizeof(double) * ht * W), *lo = xmalloc(sizeof(double) * ht * W);
    double *y = xmalloc(sizeof(double) * ht * D), *M = xmalloc(sizeof(double) * B * H * N * D);
    double *dy = xmalloc(sizeof(double) * ht * D), *dMT = xmalloc(sizeof(double) * B * H * N * D);
    double *dkp = xmalloc(sizeof(double) * ht * 2 * S), *dqp = xmalloc(sizeof(double) * ht * 2 * S);
    double *dv = xmalloc(sizeof(double) * ht * D), *da = xmalloc(sizeof(double) * ht);
    double *db = xmalloc(sizeof(double) * ht), *dM0 = xmalloc(sizeof(double) * H * N * D);
    for (int64_t i = 0; i < ht * D; i++) dy[i] = uniform();
    for (int64_t i = 0; i < B * H * N * D; i++) dMT[i] = uniform();

    for (int dt = 0; dt < 2; dt++) { /* float32, then bfloat16 inputs */
        const void *k = dt ? (const void *)kb : (const void *)kp;
        const void *q = dt ? (const void *)qb : (const void *)qp;
        const void *vv = dt ? (const void *)vb : (const void *)v;
        CHECK(sdm_oracle_topk_rows(ht, S, W, k, dt, Iw, kw, hi, lo, threads));
        CHECK(sdm_oracle_topk_rows(ht, S, R, q, dt, Ir, qw, NULL, NULL, threads));
        for (int sb = 0; sb < 3; sb++) { /* float64, bfloat16 and scaled E4M3 state */
            CHECK(sdm_oracle_recurrence(B, T, H, S, D, W, R, Iw, kw, Ir, qw, vv, dt, alpha, beta,
                                        M0, sb, sb == 2 ? -4 : 0, 0, D, y, M, threads));
            CHECK(sdm_oracle_recurrence(B, T, H, S, D, W, R, Iw, kw, Ir, qw, vv, dt, alpha, beta,
                                        M0, sb, sb == 2 ? 3 : 0, 3, 7, y, M, threads)); /* window */
        }
        CHECK(sdm_oracle_backward(B, T, H, S, D, W, R, Iw, kw, Ir, qw, vv, dt, alpha, beta, M0, dy,
                                  dt ? NULL : dMT, dkp, dqp, dv, da, db, dM0, threads));
    }
    sdm_oracle_round_bf16(y, dv, ht * D);
    sdm_oracle_round_fp8(y, dv, ht * D, -5);
    /* the full ordering of a tiny key (K = sqrtN) and the smallest shape */
    CHECK(sdm_oracle_topk_rows(4, S, S, kp, 0, Iw, kw, hi, lo, 1));
    CHECK(sdm_oracle_topk_rows(1, 1, 1, kp, 0, Iw, kw, NULL, NULL, 1));

    void *all[] = {kp, qp, v, kb, qb, vb, alpha, beta, M0, Iw, Ir, kw, qw, hi, lo, y, M,
                   dy, dMT, dkp, dqp, dv, da, db, dM0};
    for (size_t i = 0; i < sizeof all / sizeof all[0]; i++) free(all[i]);
    printf("ok\n");
    return 0;
}
