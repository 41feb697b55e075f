/*
 * SDM recurrent core: plain float64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may load this
 * library: only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do.  It shares no code, header, table or helper with the HIP library.
 *
 * What it computes, per sequence b, head h and token t (the pages' notation):
 *
 *  1. Scores.  The pre-PKM key k'_t (length 2*sqrtN) is split into the halves
 *     k'_1 = k'[0, sqrtN) and k'_2 = k'[sqrtN, 2*sqrtN); slot n = i*sqrtN + j
 *     gets the outer-sum score k'_1[i] + k'_2[j]
 *     [explainer "Sparse Delta Memory：通过稀疏性扩展线性 RNN 的状态容量",
 *      §3.1 step 1; "Technical Summary: Sparse Delta Memory (SDM)",
 *      Methodology / Core Mechanism item 2].  Same for q'_t.
 *     Scores are exact real sums: each is held as the float64 TwoSum pair
 *     (hi, lo) of the two (exactly widened) inputs, and pairs are compared
 *     lexicographically, which is the exact order of the real sums.
 *  2. Selection.  The W (resp. R) slots that come first in the order
 *     (score descending, flat index n ascending), obtained with the
 *     product-key identity the same passages state: keep the top-W of each
 *     half, then the top-W of all W*W sums of survivors.
 *  3. Weights.  k^(i) (resp. q^(i)) = softmax of the selected scores.  The
 *     pages use these weights without defining them; softmax over the
 *     selected scores is the reading adopted.
 *  4. Write [explainer §3.1 step 2; Technical Summary, Core Mechanism 3]:
 *     for every selected write slot i, m = alpha_t * M[i];
 *     M[i] = m + beta_t * k^(i) * (v_t - m).  Other rows are untouched.
 *  5. Read [explainer §3.1 step 3]: y_t = sum over the read set, in list
 *     order, of q^(i) * M[i], taken after the same token's write.
 *  Every sequence starts from the shared initial state M_0 [explainer §3.1,
 *  learned initial state paragraph; Technical Summary, Learned Initial State].
 *  7. Backward (reverse mode, float64 state) with the selected index sets
 *     held fixed -- they are piecewise constant in k' and q', so the
 *     gradient reaches k' and q' only through the softmax weights.  The
 *     explainer's training discussion (memory-efficient backward, learned
 *     initial state M_0) needs these gradients; the pages print no formulas,
 *     so they are derived here from steps 3-5 by the chain rule.  Per token,
 *     in reverse order, with G the gradient of the loss with respect to the
 *     state after the token:
 *       read:  dq_r = <dy_t, M[r]>,  G[r] += q_r dy_t
 *       write: with m = alpha M_old, new = m + beta k (v - m):
 *              dk     = <G[i], beta (v - m)>
 *              dalpha += <G[i], M_old> (1 - beta k)
 *              dbeta  += <G[i], k (v - m)>
 *              dv     += beta k G[i]
 *              G[i]    = alpha (1 - beta k) G[i],  M[i] = M_old
 *       weights: dscore_j = w_j (dw_j - sum_l w_l dw_l) (softmax), and a
 *              slot n = i sqrtN + j passes dscore to x[i] and x[sqrtN + j].
 *     After token 0, dM_0[h] = sum over sequences b of G.
 *  6. Reduced-precision state (optional).  The engineering notes of the
 *     explainer suggest storing the state in a narrower type to fit larger
 *     N; the pages fix no rule.  Reading adopted: the state is held in
 *     bfloat16 -- M_0 is rounded to bfloat16 at the start, every write
 *     computes the new row from the stored values and rounds it to
 *     bfloat16, and reads use the stored values.  Rounding is to nearest,
 *     ties to even, at bfloat16 precision (8 significant bits, the exponent
 *     range of float32, subnormal spacing 2^-133).
 *     The same notes name 8-bit states to fit N ~ 10^7 on one card; the
 *     reading adopted for that: the OCP FP8 E4M3 format (4 exponent bits,
 *     bias 7, 3 mantissa bits, largest magnitude 448, no infinities) with a
 *     power-of-two scale 2^s given per layer -- a stored code c means the
 *     value c * 2^s -- rounded to nearest, ties to even, and saturated at
 *     +-448 * 2^s; M_0, writes and reads follow the bfloat16 rule above.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -fPIC -shared.
 * (-ffp-contract=off keeps every product and sum separately rounded, so the
 * TwoSum error terms are exact.)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };

typedef struct {
    double hi, lo; /* exact score = hi + lo */
    int32_t n;     /* slot index (flat index, or index within a half) */
} cand;

/* Knuth's TwoSum: s = fl(a + b), e = (a + b) - s exactly. */
static void two_sum(double a, double b, double *s, double *e)
{
    double x = a + b;
    double bv = x - a;
    double av = x - bv;
    *s = x;
    *e = (a - av) + (b - bv);
}

/* Does a come before b?  Larger exact score first, then smaller index. */
static int precedes(const cand *a, const cand *b)
{
    if (a->hi != b->hi) return a->hi > b->hi;
    if (a->lo != b->lo) return a->lo > b->lo;
    return a->n < b->n;
}

/* keep[0..*cnt) is in canonical order; insert c if it is among the first K. */
static void topk_push(cand *keep, int *cnt, int K, const cand *c)
{
    int m = *cnt;
    if (m == K) {
        if (!precedes(c, &keep[K - 1])) return;
        m = K - 1; /* the last kept item drops out */
    }
    int p = m;
    while (p > 0 && precedes(c, &keep[p - 1])) {
        keep[p] = keep[p - 1];
        p--;
    }
    keep[p] = *c;
    if (*cnt < K) (*cnt)++;
}

static double load_value(const void *x, int dtype, int64_t i)
{
    if (dtype == ORACLE_BF16) {
        uint32_t u = (uint32_t)((const uint16_t *)x)[i] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    return (double)((const float *)x)[i];
}

/*
 * Top-K slots of one pre-PKM vector x (length 2*sqrtN) and their softmax
 * weights.  kept1/kept2 are scratch of K items each, cands of K*K items.
 */
static void topk_one(const double *x, int sqrtN, int K, cand *kept1, cand *kept2,
                     cand *out, int32_t *idx, double *wts, double *shi, double *slo)
{
    /* stage 1: top-K of each half, ties to the lower index within the half */
    int c1 = 0, c2 = 0;
    for (int i = 0; i < sqrtN; i++) {
        cand a = {x[i], 0.0, i};
        topk_push(kept1, &c1, K, &a);
        cand b = {x[sqrtN + i], 0.0, i};
        topk_push(kept2, &c2, K, &b);
    }
    /* stage 2: top-K of all K*K outer sums of the survivors */
    int co = 0;
    for (int a = 0; a < K; a++) {
        for (int b = 0; b < K; b++) {
            cand c;
            two_sum(kept1[a].hi, kept2[b].hi, &c.hi, &c.lo);
            c.n = kept1[a].n * sqrtN + kept2[b].n;
            topk_push(out, &co, K, &c);
        }
    }
    /* softmax over the K selected exact scores; out[0] holds the maximum */
    double z = 0.0;
    for (int k = 0; k < K; k++) {
        double d = (out[k].hi - out[0].hi) + (out[k].lo - out[0].lo);
        wts[k] = exp(d);
        z += wts[k];
    }
    for (int k = 0; k < K; k++) {
        wts[k] /= z;
        idx[k] = out[k].n;
        if (shi) shi[k] = out[k].hi;
        if (slo) slo[k] = out[k].lo;
    }
}

/*
 * Selection for nrows independent pre-PKM vectors x[nrows][2*sqrtN]
 * (float32, or bfloat16 bit patterns).  Writes idx[nrows][K] (canonical
 * order) and wts[nrows][K]; shi/slo (may be NULL) receive the exact scores.
 * Returns 0, or -1 on bad arguments.
 */
int sdm_oracle_topk_rows(int64_t nrows, int sqrtN, int K, const void *x, int dtype,
                         int32_t *idx, double *wts, double *shi, double *slo,
                         int nthreads)
{
    if (nrows < 0 || sqrtN < 1 || K < 1 || K > sqrtN || !x || !idx || !wts) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
    if (nthreads < 1) nthreads = 1;
    int bad = 0;
#pragma omp parallel num_threads(nthreads)
    {
        double *xv = malloc(sizeof(double) * 2 * (size_t)sqrtN);
        cand *k1 = malloc(sizeof(cand) * (size_t)K);
        cand *k2 = malloc(sizeof(cand) * (size_t)K);
        cand *o = malloc(sizeof(cand) * (size_t)K);
        if (!xv || !k1 || !k2 || !o) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t r = 0; r < nrows; r++) {
                for (int i = 0; i < 2 * sqrtN; i++)
                    xv[i] = load_value(x, dtype, r * 2 * (int64_t)sqrtN + i);
                topk_one(xv, sqrtN, K, k1, k2, o, idx + r * K, wts + r * K,
                         shi ? shi + r * K : NULL, slo ? slo + r * K : NULL);
            }
        }
        free(xv);
        free(k1);
        free(k2);
        free(o);
    }
    return bad ? -2 : 0;
}

/*
 * The recurrence for one chain (b, h) over the columns [ca, cb) of the
 * requested column window [c0, c1): init from M_0, then for every token the
 * gated delta write of the W selected rows followed by the sparse read.
 */
/* Nearest bfloat16 value of x, ties to even: x is rounded to a multiple of
   the bfloat16 spacing at its magnitude, 2^(e-8) for |x| in [2^(e-1), 2^e),
   never finer than the subnormal spacing 2^-133.  nearbyint rounds half to
   even in the default rounding mode. */
static double round_bf16(double x)
{
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    (void)frexp(x, &e);
    int q = e - 8;
    if (q < -133) q = -133;
    return ldexp(nearbyint(ldexp(x, -q)), q);
}

/* Element-wise round_bf16 (exported for the tests). */
void sdm_oracle_round_bf16(const double *x, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++) out[i] = round_bf16(x[i]);
}

/* Nearest value of the scaled E4M3 format (item 6): a = x * 2^-s is rounded
   to a multiple of the E4M3 spacing at its magnitude, 2^(e-4) for |a| in
   [2^(e-1), 2^e) (3 mantissa bits), never finer than the subnormal spacing
   2^-9; ties to even; magnitudes above 448 saturate to 448.  The result is
   scaled back by 2^s (both scalings are exact). */
static double round_fp8(double x, int s)
{
    if (x == 0.0 || !isfinite(x)) return x;
    const double a = ldexp(x, -s);
    int e;
    (void)frexp(a, &e);
    int q = e - 4;
    if (q < -9) q = -9;
    double r = ldexp(nearbyint(ldexp(a, -q)), q);
    if (r > 448.0) r = 448.0;
    if (r < -448.0) r = -448.0;
    return ldexp(r, s);
}

/* Element-wise round_fp8 with scale 2^s (exported for the tests). */
void sdm_oracle_round_fp8(const double *x, double *out, int64_t n, int s)
{
    for (int64_t i = 0; i < n; i++) out[i] = round_fp8(x[i], s);
}

/* The value the state holds for x: itself (mode 0), bfloat16 (mode 1) or
   scaled E4M3 (mode 2, scale 2^s). */
static double store_value(double x, int state_mode, int s)
{
    if (state_mode == 1) return round_bf16(x);
    if (state_mode == 2) return round_fp8(x, s);
    return x;
}

static void run_chain(int64_t T, int H, int64_t N, int d_v, int W, int R, int b, int h,
                      const int32_t *Iw, const double *kw, const int32_t *Ir,
                      const double *qw, const void *v, int v_dtype, const float *alpha,
                      const float *beta, const float *M0, int state_mode, int scale_log2,
                      int c0, int c1, int ca, int cb, double *y, double *M)
{
    const int nc = c1 - c0;
    double *Mc = M + ((int64_t)b * H + h) * N * nc; /* this chain's [N][nc] */
    for (int64_t n = 0; n < N; n++)
        for (int c = ca; c < cb; c++) {
            const double m0 = (double)M0[((int64_t)h * N + n) * d_v + c];
            Mc[n * nc + (c - c0)] = store_value(m0, state_mode, scale_log2);
        }

    for (int64_t t = 0; t < T; t++) {
        const int64_t ht = ((int64_t)b * T + t) * H + h; /* head-token index */
        const double a_t = (double)alpha[ht];
        const double b_t = (double)beta[ht];
        /* write: every selected slot, in list order (the slots are distinct) */
        for (int w = 0; w < W; w++) {
            const int64_t s = Iw[ht * W + w];
            const double k = kw[ht * W + w];
            for (int c = ca; c < cb; c++) {
                const double vt = load_value(v, v_dtype, ht * d_v + c);
                double *row = &Mc[s * nc + (c - c0)];
                const double m = a_t * (*row);     /* forget gate */
                *row = m + b_t * k * (vt - m);     /* delta + input gate */
                *row = store_value(*row, state_mode, scale_log2);
            }
        }
        /* read: on the state after this token's write */
        for (int c = ca; c < cb; c++) {
            double acc = 0.0;
            for (int r = 0; r < R; r++) {
                const int64_t s = Ir[ht * R + r];
                acc += qw[ht * R + r] * Mc[s * nc + (c - c0)];
            }
            y[ht * nc + (c - c0)] = acc;
        }
    }
}

/*
 * Token-serial recurrence from a given selection.
 *   Iw,kw [B][T][H][W], Ir,qw [B][T][H][R]   selection (from the oracle)
 *   v [B][T][H][d_v] (float32 or bf16 bits), alpha,beta [B][T][H] float32
 *   M0 [H][N][d_v] float32
 *   state_mode: 0 = float64 state, 1 = state held in bfloat16, 2 = state held
 *   in E4M3 with scale 2^scale_log2 (item 6 above)
 * Only the columns [c0, c1) of y and M are produced (columns of the state
 * never interact):  y [B][T][H][c1-c0], M [B][H][N][c1-c0], both float64.
 * Returns 0, or -1 on bad arguments.
 */
int sdm_oracle_recurrence(int B, int64_t T, int H, int sqrtN, int d_v, int W, int R,
                          const int32_t *Iw, const double *kw, const int32_t *Ir,
                          const double *qw, const void *v, int v_dtype, const float *alpha,
                          const float *beta, const float *M0, int state_mode, int scale_log2,
                          int c0, int c1, double *y, double *M, int nthreads)
{
    if (B < 1 || T < 0 || H < 1 || sqrtN < 1 || d_v < 1 || W < 1 || R < 1) return -1;
    if (W > sqrtN || R > sqrtN || c0 < 0 || c1 > d_v || c0 >= c1) return -1;
    if (!Iw || !kw || !Ir || !qw || !v || !alpha || !beta || !M0 || !y || !M) return -1;
    if (v_dtype != ORACLE_F32 && v_dtype != ORACLE_BF16) return -1;
    if (state_mode < 0 || state_mode > 2 || scale_log2 < -100 || scale_log2 > 100) return -1;
    if (nthreads < 1) nthreads = 1;
    const int64_t N = (int64_t)sqrtN * sqrtN;
    /* independent units: (chain, block of columns); CB columns per unit */
    const int CB = 8;
    const int nblk = (c1 - c0 + CB - 1) / CB;
    const int64_t units = (int64_t)B * H * nblk;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t u = 0; u < units; u++) {
        const int blk = (int)(u % nblk);
        const int64_t chain = u / nblk;
        const int b = (int)(chain / H), h = (int)(chain % H);
        const int ca = c0 + blk * CB;
        const int cb = ca + CB < c1 ? ca + CB : c1;
        run_chain(T, H, N, d_v, W, R, b, h, Iw, kw, Ir, qw, v, v_dtype, alpha, beta, M0,
                  state_mode, scale_log2, c0, c1, ca, cb, y, M);
    }
    return 0;
}

/*
 * Backward of one chain (b, h): recomputes the forward with a tape of the
 * rows each write replaced, then runs the tokens in reverse.  Gf receives
 * the gradient with respect to this chain's initial state.
 */
static int backward_chain(int64_t T, int H, int64_t N, int d_v, int W, int R, int sqrtN, int b,
                          int h, const int32_t *Iw, const double *kw, const int32_t *Ir,
                          const double *qw, const void *v, int v_dtype, const float *alpha,
                          const float *beta, const float *M0, const double *dy, const double *dMT,
                          double *dkp, double *dqp, double *dv, double *dalpha, double *dbeta,
                          double *Gf)
{
    double *M = malloc(sizeof(double) * (size_t)(N * d_v));
    double *tape = malloc(sizeof(double) * (size_t)(T * W) * (size_t)d_v);
    double *dwk = malloc(sizeof(double) * (size_t)(W > R ? W : R));
    if (!M || !tape || !dwk) {
        free(M);
        free(tape);
        free(dwk);
        return -2;
    }
    double *G = Gf;
    const int64_t S = 2 * (int64_t)sqrtN;
    for (int64_t x = 0; x < N * d_v; x++) M[x] = (double)M0[(int64_t)h * N * d_v + x];
    /* forward, recording the old row of every write */
    for (int64_t t = 0; t < T; t++) {
        const int64_t ht = ((int64_t)b * T + t) * H + h;
        const double a_t = (double)alpha[ht], b_t = (double)beta[ht];
        for (int w = 0; w < W; w++) {
            const int64_t sl = Iw[ht * W + w];
            const double k = kw[ht * W + w];
            double *row = M + sl * d_v;
            double *old = tape + (t * W + w) * d_v;
            for (int c = 0; c < d_v; c++) {
                old[c] = row[c];
                const double m = a_t * row[c];
                row[c] = m + b_t * k * (load_value(v, v_dtype, ht * d_v + c) - m);
            }
        }
    }
    /* reverse */
    const int64_t chain_off = ((int64_t)b * H + h) * N * d_v;
    for (int64_t x = 0; x < N * d_v; x++) G[x] = dMT ? dMT[chain_off + x] : 0.0;
    for (int64_t t = T - 1; t >= 0; t--) {
        const int64_t ht = ((int64_t)b * T + t) * H + h;
        const double a_t = (double)alpha[ht], b_t = (double)beta[ht];
        const double *dyt = dy + ht * d_v;
        double *dkp_t = dkp + ht * S, *dqp_t = dqp + ht * S;
        for (int64_t x = 0; x < S; x++) dkp_t[x] = dqp_t[x] = 0.0;
        /* read: on the state after this token's writes */
        double sw = 0.0;
        for (int r = 0; r < R; r++) {
            const int64_t sl = Ir[ht * R + r];
            const double q = qw[ht * R + r];
            double dq = 0.0;
            for (int c = 0; c < d_v; c++) dq += dyt[c] * M[sl * d_v + c];
            for (int c = 0; c < d_v; c++) G[sl * d_v + c] += q * dyt[c];
            dwk[r] = dq;
            sw += q * dq;
        }
        for (int r = 0; r < R; r++) {
            const double q = qw[ht * R + r];
            const double ds = q * (dwk[r] - sw);
            const int64_t n = Ir[ht * R + r];
            dqp_t[n / sqrtN] += ds;
            dqp_t[sqrtN + n % sqrtN] += ds;
        }
        /* writes (distinct slots: order is irrelevant) */
        double da = 0.0, db = 0.0;
        for (int c = 0; c < d_v; c++) dv[ht * d_v + c] = 0.0;
        sw = 0.0;
        for (int w = 0; w < W; w++) {
            const int64_t sl = Iw[ht * W + w];
            const double k = kw[ht * W + w];
            const double *old = tape + (t * W + w) * d_v;
            double *g = G + sl * d_v;
            double dk = 0.0;
            for (int c = 0; c < d_v; c++) {
                const double vt = load_value(v, v_dtype, ht * d_v + c);
                const double m = a_t * old[c];
                dk += g[c] * b_t * (vt - m);
                da += g[c] * old[c] * (1.0 - b_t * k);
                db += g[c] * k * (vt - m);
                dv[ht * d_v + c] += b_t * k * g[c];
                g[c] *= a_t * (1.0 - b_t * k);
                M[sl * d_v + c] = old[c];
            }
            dwk[w] = dk;
            sw += k * dk;
        }
        dalpha[ht] = da;
        dbeta[ht] = db;
        for (int w = 0; w < W; w++) {
            const double k = kw[ht * W + w];
            const double ds = k * (dwk[w] - sw);
            const int64_t n = Iw[ht * W + w];
            dkp_t[n / sqrtN] += ds;
            dkp_t[sqrtN + n % sqrtN] += ds;
        }
    }
    free(M);
    free(tape);
    free(dwk);
    return 0;
}

/*
 * Gradients of the token-serial core (float64 state) from a given selection.
 *   dy [B][T][H][d_v], dMT [B][H][N][d_v] (NULL: zero) upstream gradients
 *   out: dkp, dqp [B][T][H][2*sqrtN], dv [B][T][H][d_v], dalpha, dbeta
 *   [B][T][H], dM0 [H][N][d_v]  (all float64, every column)
 * Returns 0, -1 on bad arguments, -2 when out of host memory.
 */
int sdm_oracle_backward(int B, int64_t T, int H, int sqrtN, int d_v, int W, int R,
                        const int32_t *Iw, const double *kw, const int32_t *Ir, const double *qw,
                        const void *v, int v_dtype, const float *alpha, const float *beta,
                        const float *M0, const double *dy, const double *dMT, double *dkp,
                        double *dqp, double *dv, double *dalpha, double *dbeta, double *dM0,
                        int nthreads)
{
    if (B < 1 || T < 1 || H < 1 || sqrtN < 1 || d_v < 1 || W < 1 || R < 1) return -1;
    if (W > sqrtN || R > sqrtN) return -1;
    if (!Iw || !kw || !Ir || !qw || !v || !alpha || !beta || !M0 || !dy) return -1;
    if (!dkp || !dqp || !dv || !dalpha || !dbeta || !dM0) return -1;
    if (v_dtype != ORACLE_F32 && v_dtype != ORACLE_BF16) return -1;
    if (nthreads < 1) nthreads = 1;
    const int64_t N = (int64_t)sqrtN * sqrtN;
    const int64_t chains = (int64_t)B * H;
    double *Gall = malloc(sizeof(double) * (size_t)(chains * N) * (size_t)d_v);
    if (!Gall) return -2;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t ch = 0; ch < chains; ch++) {
        const int b = (int)(ch / H), h = (int)(ch % H);
        if (backward_chain(T, H, N, d_v, W, R, sqrtN, b, h, Iw, kw, Ir, qw, v, v_dtype, alpha,
                           beta, M0, dy, dMT, dkp, dqp, dv, dalpha, dbeta,
                           Gall + ch * N * d_v) != 0) {
#pragma omp atomic write
            bad = 1;
        }
    }
    if (!bad) {
        /* dM_0[h] = sum over b of the chains' initial-state gradients, b in order */
        for (int h = 0; h < H; h++)
            for (int64_t x = 0; x < N * d_v; x++) {
                double acc = 0.0;
                for (int b = 0; b < B; b++) acc += Gall[((int64_t)b * H + h) * N * d_v + x];
                dM0[(int64_t)h * N * d_v + x] = acc;
            }
    }
    free(Gall);
    return bad ? -2 : 0;
}
