/*
 * Exact-attention oracle: plain fp64 CPU reference.  TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  It shares no code, header, table or constant
 * generator with the GPU library; the dropout generator below is written
 * independently from its published definition.
 *
 * What it computes (per batch b, head h, every value in double precision):
 *
 *   S      = scale * Q K^T                      -- "Vanilla Attention", the
 *                                                  displayed equation of the
 *                                                  mrodiduger.github.io page,
 *                                                  with the caller's scale
 *   S_ij   = -inf for j > i when causal          -- masking, same page,
 *                                                  "Vanilla Attention" and
 *                                                  "Experimental Results"
 *   m_i    = max_j S_ij,  l_i = sum_j exp(S_ij - m_i),
 *   LSE_i  = m_i + ln l_i                        -- safe softmax statistics,
 *                                                  same page, "Tiling"; stored
 *                                                  as one log-sum-exp per row
 *                                                  ("Recomputation" keeps m, l)
 *   P_ij   = exp(S_ij - LSE_i)
 *   Pd_ij  = P_ij * keep_ij * c,  c = float(1/(1-p))   (inverted dropout)
 *   O      = Pd V
 *
 * Backward (the calculus of the definition above; the pages say only that
 * S and P are recomputed from the stored statistics, "Recomputation"):
 *
 *   dV  = Pd^T dO
 *   dPd = dO V^T,   dP = dPd * keep * c
 *   D_i = sum_c dO_ic O_ic
 *   dS  = P o (dP - D 1^T)
 *   dQ  = scale dS K,   dK = scale dS^T Q
 *
 * There is no tiling and no online softmax here: every row is evaluated
 * over all of its keys, with the score row materialised.
 *
 * Dropout keep bits use the Philox-4x32 counter-based generator with 10
 * rounds (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
 * 1, 2, 3", SC'11).  Counter = (col >> 3, row, h, b), key = (seed low 32,
 * seed high 32).  The four output words are eight 16-bit lanes; column col
 * uses lane col & 7 (word (col&7)>>1, low half for even col, high half for
 * odd).  An element is kept iff its lane value >= T with
 * T = round(p * 65536).  Parity with the published known-answer vectors is
 * UNPINNED (they are not available here); the GPU library implements the
 * same definition separately and must agree bit for bit.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL 1
#define ORACLE_ENOMEM 2

/* ---------------------------------------------------------------- Philox */

/* Philox-4x32 multipliers and key increments, as published in SC'11. */
static const uint32_t PHILOX_M0 = 0xD2511F53u;
static const uint32_t PHILOX_M1 = 0xCD9E8D57u;
static const uint32_t PHILOX_W0 = 0x9E3779B9u;
static const uint32_t PHILOX_W1 = 0xBB67AE85u;

/* One Philox-4x32 round: two 32x32->64 products, their high halves are
 * xored with the other two words and the round key. */
static void philox_round(uint32_t x[4], uint32_t k0, uint32_t k1)
{
    uint64_t prod0 = (uint64_t)PHILOX_M0 * (uint64_t)x[0];
    uint64_t prod1 = (uint64_t)PHILOX_M1 * (uint64_t)x[2];
    uint32_t hi0 = (uint32_t)(prod0 >> 32), lo0 = (uint32_t)prod0;
    uint32_t hi1 = (uint32_t)(prod1 >> 32), lo1 = (uint32_t)prod1;
    uint32_t y0 = hi1 ^ x[1] ^ k0;
    uint32_t y1 = lo1;
    uint32_t y2 = hi0 ^ x[3] ^ k1;
    uint32_t y3 = lo0;
    x[0] = y0; x[1] = y1; x[2] = y2; x[3] = y3;
}

/* Philox-4x32-10: ten rounds, the key is bumped by the Weyl constants
 * between rounds. */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t x[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
    uint32_t k0 = key[0], k1 = key[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) { k0 += PHILOX_W0; k1 += PHILOX_W1; }
        philox_round(x, k0, k1);
    }
    out[0] = x[0]; out[1] = x[1]; out[2] = x[2]; out[3] = x[3];
}

/* Threshold T = round(p * 65536): an element is dropped when its 16-bit
 * lane is below T. */
uint32_t oracle_drop_threshold(double p)
{
    return (uint32_t)llround(p * 65536.0);
}

/* Keep-scale c = 1/(1-p), evaluated in double and rounded once to float. */
double oracle_keep_scale(double p)
{
    return (double)(float)(1.0 / (1.0 - p));
}

static int keep_bit(uint64_t seed, int64_t b, int64_t h, int64_t row, int64_t col, uint32_t T)
{
    uint32_t ctr[4] = {(uint32_t)(col >> 3), (uint32_t)row, (uint32_t)h, (uint32_t)b};
    uint32_t key[2] = {(uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32)};
    uint32_t out[4];
    oracle_philox4x32_10(ctr, key, out);
    int lane = (int)(col & 7);
    uint32_t word = out[lane >> 1];
    uint32_t v16 = (lane & 1) ? (word >> 16) : (word & 0xFFFFu);
    return v16 >= T;
}

/* Keep mask of one (b, h) plane: mask[row * N + col] = 1 when kept. */
int oracle_dropout_mask(int64_t N, double p, uint64_t seed, int64_t b, int64_t h, uint8_t *mask)
{
    if (N < 0 || !(p >= 0.0 && p < 1.0) || (N > 0 && !mask)) return ORACLE_EINVAL;
    uint32_t T = oracle_drop_threshold(p);
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N; ++i)
        for (int64_t j = 0; j < N; ++j)
            mask[i * N + j] = (uint8_t)(p == 0.0 ? 1 : keep_bit(seed, b, h, i, j, T));
    return ORACLE_OK;
}

/* ------------------------------------------------------- one score row */

/* Fills s[0..N) with scale * q_i . k_j, -inf where masked, and returns the
 * row's log-sum-exp (two passes: max, then sum of exponentials). */
static double score_row(int64_t N, int64_t d, const double *qi, const double *k,
                        double scale, int causal, int64_t i, double *s)
{
    double m = -INFINITY;
    for (int64_t j = 0; j < N; ++j) {
        if (causal && j > i) { s[j] = -INFINITY; continue; }
        double acc = 0.0;
        const double *kj = k + j * d;
        for (int64_t c = 0; c < d; ++c) acc += qi[c] * kj[c];
        s[j] = scale * acc;
        if (s[j] > m) m = s[j];
    }
    if (m == -INFINITY) return -INFINITY;      /* no visible key */
    double l = 0.0;
    for (int64_t j = 0; j < N; ++j)
        if (s[j] != -INFINITY) l += exp(s[j] - m);
    return m + log(l);
}

/* P_ij = exp(S_ij - LSE_i) and the dropped, rescaled Pd_ij of one row. */
static void prob_row(int64_t N, const double *s, double lse, double p, uint64_t seed,
                     int64_t b, int64_t h, int64_t i, double *prob, double *pd)
{
    uint32_t T = oracle_drop_threshold(p);
    double c = p > 0.0 ? oracle_keep_scale(p) : 1.0;
    for (int64_t j = 0; j < N; ++j) {
        double pij = (s[j] == -INFINITY || lse == -INFINITY) ? 0.0 : exp(s[j] - lse);
        prob[j] = pij;
        if (p > 0.0) pd[j] = keep_bit(seed, b, h, i, j, T) ? pij * c : 0.0;
        else pd[j] = pij;
    }
}

/* ------------------------------------------------------------ forward */

/*
 * Forward of one (b, h) head for the listed rows (rows == NULL: all N rows,
 * in order).  q, k, v: [N, d] row-major.  o_out: [nrows, d], lse_out:
 * [nrows].  A row with no visible key gets O = 0, LSE = -inf.
 */
int oracle_fwd_rows(int64_t N, int64_t d, const double *q, const double *k, const double *v,
                    double scale, int causal, double p, uint64_t seed, int64_t b, int64_t h,
                    const int64_t *rows, int64_t nrows, double *o_out, double *lse_out)
{
    if (N < 0 || d <= 0 || nrows < 0 || !(p >= 0.0 && p < 1.0)) return ORACLE_EINVAL;
    if (!rows) nrows = N;
    int bad = 0;
    #pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        double *prob = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        double *pd = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        if (!s || !prob || !pd) {
            #pragma omp atomic write
            bad = 1;
        } else {
            #pragma omp for schedule(dynamic, 4)
            for (int64_t r = 0; r < nrows; ++r) {
                int64_t i = rows ? rows[r] : r;
                double *oi = o_out + r * d;
                if (i < 0 || i >= N) { bad = 1; continue; }
                double lse = score_row(N, d, q + i * d, k, scale, causal, i, s);
                lse_out[r] = lse;
                prob_row(N, s, lse, p, seed, b, h, i, prob, pd);
                for (int64_t c = 0; c < d; ++c) oi[c] = 0.0;
                for (int64_t j = 0; j < N; ++j) {
                    if (pd[j] == 0.0) continue;
                    const double *vj = v + j * d;
                    for (int64_t c = 0; c < d; ++c) oi[c] += pd[j] * vj[c];
                }
            }
        }
        free(s); free(prob); free(pd);
    }
    return bad ? ORACLE_EINVAL : ORACLE_OK;
}

/* ------------------------------------------ queries and keys of two lengths */

/*
 * Forward of one (b, h) head with Nq query rows and Nk keys: cross
 * attention, or the last Nq positions of a sequence of Nk (decoding).  When
 * causal, the last query is aligned with the last key: key j is visible to
 * query i iff j <= i + (Nk - Nq), which is the square rule when Nq == Nk; a
 * query with no visible key gets O = 0, LSE = -inf.  Dropout uses the same
 * counters as the square case with the query's own row index i.
 * q: [Nq, d]; k, v: [Nk, d]; o_out: [Nq, d]; lse_out: [Nq].
 */
int oracle_fwd_cross(int64_t Nq, int64_t Nk, int64_t d, const double *q, const double *k,
                     const double *v, double scale, int causal, double p, uint64_t seed,
                     int64_t b, int64_t h, double *o_out, double *lse_out)
{
    if (Nq < 0 || Nk < 0 || d <= 0 || !(p >= 0.0 && p < 1.0)) return ORACLE_EINVAL;
    int bad = 0;
    #pragma omp parallel
    {
        size_t n = (size_t)(Nk > 0 ? Nk : 1);
        double *s = (double *)malloc(sizeof(double) * n);
        double *prob = (double *)malloc(sizeof(double) * n);
        double *pd = (double *)malloc(sizeof(double) * n);
        if (!s || !prob || !pd) {
            #pragma omp atomic write
            bad = 1;
        } else {
            #pragma omp for schedule(dynamic, 4)
            for (int64_t i = 0; i < Nq; ++i) {
                const double *qi = q + i * d;
                const int64_t last = causal ? i + (Nk - Nq) : Nk - 1;   /* last visible key */
                /* scores and the row's log-sum-exp (max, then sum) */
                double m = -INFINITY;
                for (int64_t j = 0; j < Nk; ++j) {
                    if (j > last) { s[j] = -INFINITY; continue; }
                    double acc = 0.0;
                    for (int64_t c = 0; c < d; ++c) acc += qi[c] * k[j * d + c];
                    s[j] = acc * scale;
                    if (s[j] > m) m = s[j];
                }
                double lse = -INFINITY;
                if (m != -INFINITY) {
                    double l = 0.0;
                    for (int64_t j = 0; j < Nk; ++j)
                        if (s[j] != -INFINITY) l += exp(s[j] - m);
                    lse = m + log(l);
                }
                lse_out[i] = lse;
                prob_row(Nk, s, lse, p, seed, b, h, i, prob, pd);
                double *oi = o_out + i * d;
                for (int64_t c = 0; c < d; ++c) oi[c] = 0.0;
                for (int64_t j = 0; j < Nk; ++j) {
                    if (pd[j] == 0.0) continue;
                    for (int64_t c = 0; c < d; ++c) oi[c] += pd[j] * v[j * d + c];
                }
            }
        }
        free(s); free(prob); free(pd);
    }
    return bad ? ORACLE_ENOMEM : ORACLE_OK;
}

/* Probability rows of one head: prob, pd: [N, N]. */
int oracle_probs(int64_t N, int64_t d, const double *q, const double *k, double scale,
                 int causal, double p, uint64_t seed, int64_t b, int64_t h,
                 double *prob, double *pd)
{
    if (N < 0 || d <= 0 || !(p >= 0.0 && p < 1.0)) return ORACLE_EINVAL;
    int bad = 0;
    #pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        if (!s) {
            #pragma omp atomic write
            bad = 1;
        } else {
            #pragma omp for schedule(static)
            for (int64_t i = 0; i < N; ++i) {
                double lse = score_row(N, d, q + i * d, k, scale, causal, i, s);
                prob_row(N, s, lse, p, seed, b, h, i, prob + i * N, pd + i * N);
            }
        }
        free(s);
    }
    return bad ? ORACLE_ENOMEM : ORACLE_OK;
}

/* ----------------------------------------------------------- backward */

/*
 * Backward of one (b, h) head.  Inputs q, k, v, dout: [N, d].  Outputs
 * dq, dk, dv: [N, d]; o and lse (the forward's O [N, d] and LSE [N]) are
 * written too.  P, Pd and dS are materialised as N x N matrices.
 */
int oracle_bwd_head(int64_t N, int64_t d, const double *q, const double *k, const double *v,
                    const double *dout, double scale, int causal, double p, uint64_t seed,
                    int64_t b, int64_t h, double *dq, double *dk, double *dv,
                    double *o, double *lse)
{
    if (N < 0 || d <= 0 || !(p >= 0.0 && p < 1.0)) return ORACLE_EINVAL;
    if (N == 0) return ORACLE_OK;
    double c = p > 0.0 ? oracle_keep_scale(p) : 1.0;
    uint32_t T = oracle_drop_threshold(p);
    size_t nn = (size_t)N * (size_t)N;
    double *pd_all = (double *)malloc(sizeof(double) * nn);
    double *ds_all = (double *)malloc(sizeof(double) * nn);
    if (!pd_all || !ds_all) { free(pd_all); free(ds_all); return ORACLE_ENOMEM; }
    int bad = 0;

    /* Row pass: P, Pd, O_i, D_i, dP, dS and dQ_i of each row. */
    #pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)N);
        double *prob = (double *)malloc(sizeof(double) * (size_t)N);
        if (!s || !prob) {
            #pragma omp atomic write
            bad = 1;
        } else {
            #pragma omp for schedule(dynamic, 4)
            for (int64_t i = 0; i < N; ++i) {
                const double *qi = q + i * d, *doi = dout + i * d;
                double *pd = pd_all + (size_t)i * (size_t)N;
                double *ds = ds_all + (size_t)i * (size_t)N;
                double l = score_row(N, d, qi, k, scale, causal, i, s);
                lse[i] = l;
                prob_row(N, s, l, p, seed, b, h, i, prob, pd);
                double *oi = o + i * d;
                for (int64_t cc = 0; cc < d; ++cc) oi[cc] = 0.0;
                for (int64_t j = 0; j < N; ++j)
                    for (int64_t cc = 0; cc < d; ++cc) oi[cc] += pd[j] * v[j * d + cc];
                double Di = 0.0;
                for (int64_t cc = 0; cc < d; ++cc) Di += doi[cc] * oi[cc];
                double *dqi = dq + i * d;
                for (int64_t cc = 0; cc < d; ++cc) dqi[cc] = 0.0;
                for (int64_t j = 0; j < N; ++j) {
                    if (prob[j] == 0.0) { ds[j] = 0.0; continue; }
                    double dpd = 0.0;
                    for (int64_t cc = 0; cc < d; ++cc) dpd += doi[cc] * v[j * d + cc];
                    double keep = p > 0.0 ? (double)keep_bit(seed, b, h, i, j, T) : 1.0;
                    double dp = dpd * keep * c;
                    ds[j] = prob[j] * (dp - Di);
                    for (int64_t cc = 0; cc < d; ++cc) dqi[cc] += scale * ds[j] * k[j * d + cc];
                }
            }
        }
        free(s); free(prob);
    }
    /* Column pass: dK_j and dV_j of each key. */
    #pragma omp parallel for schedule(dynamic, 4)
    for (int64_t j = 0; j < N; ++j) {
        double *dkj = dk + j * d, *dvj = dv + j * d;
        for (int64_t cc = 0; cc < d; ++cc) { dkj[cc] = 0.0; dvj[cc] = 0.0; }
        for (int64_t i = 0; i < N; ++i) {
            double dsij = ds_all[(size_t)i * (size_t)N + (size_t)j];
            double pdij = pd_all[(size_t)i * (size_t)N + (size_t)j];
            for (int64_t cc = 0; cc < d; ++cc) {
                dkj[cc] += scale * dsij * q[i * d + cc];
                dvj[cc] += pdij * dout[i * d + cc];
            }
        }
    }
    free(pd_all); free(ds_all);
    return bad ? ORACLE_ENOMEM : ORACLE_OK;
}

/*
 * Backward of one (b, h) head with Nq query rows and Nk keys (visibility and
 * dropout counters as in oracle_fwd_cross).  Inputs q, dout: [Nq, d]; k, v:
 * [Nk, d].  Outputs dq: [Nq, d]; dk, dv: [Nk, d]; o [Nq, d] and lse [Nq].
 * The same calculus as oracle_bwd_head with P, Pd and dS materialised as
 * Nq x Nk matrices.
 */
int oracle_bwd_cross(int64_t Nq, int64_t Nk, int64_t d, const double *q, const double *k,
                     const double *v, const double *dout, double scale, int causal, double p,
                     uint64_t seed, int64_t b, int64_t h, double *dq, double *dk, double *dv,
                     double *o, double *lse)
{
    if (Nq < 0 || Nk < 0 || d <= 0 || !(p >= 0.0 && p < 1.0)) return ORACLE_EINVAL;
    double c = p > 0.0 ? oracle_keep_scale(p) : 1.0;
    uint32_t T = oracle_drop_threshold(p);
    size_t nn = (size_t)(Nq > 0 ? Nq : 1) * (size_t)(Nk > 0 ? Nk : 1);
    double *pd_all = (double *)malloc(sizeof(double) * nn);
    double *ds_all = (double *)malloc(sizeof(double) * nn);
    double *s = (double *)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
    double *prob = (double *)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
    if (!pd_all || !ds_all || !s || !prob) {
        free(pd_all); free(ds_all); free(s); free(prob);
        return ORACLE_ENOMEM;
    }
    /* Row pass (one query at a time): P, Pd, O_i, D_i, dS and dQ_i. */
    for (int64_t i = 0; i < Nq; ++i) {
        const double *qi = q + i * d, *doi = dout + i * d;
        double *pd = pd_all + (size_t)i * (size_t)Nk, *ds = ds_all + (size_t)i * (size_t)Nk;
        const int64_t last = causal ? (Nk - Nq) + i : Nk - 1;   /* last visible key */
        double m = -INFINITY;
        for (int64_t j = 0; j < Nk; ++j) {
            if (j > last) { s[j] = -INFINITY; continue; }
            double acc = 0.0;
            for (int64_t cc = 0; cc < d; ++cc) acc += qi[cc] * k[j * d + cc];
            s[j] = acc * scale;
            if (s[j] > m) m = s[j];
        }
        double li = -INFINITY;
        if (m != -INFINITY) {
            double l = 0.0;
            for (int64_t j = 0; j < Nk; ++j)
                if (s[j] != -INFINITY) l += exp(s[j] - m);
            li = m + log(l);
        }
        lse[i] = li;
        prob_row(Nk, s, li, p, seed, b, h, i, prob, pd);
        double *oi = o + i * d;
        for (int64_t cc = 0; cc < d; ++cc) oi[cc] = 0.0;
        for (int64_t j = 0; j < Nk; ++j)
            for (int64_t cc = 0; cc < d; ++cc) oi[cc] += pd[j] * v[j * d + cc];
        double Di = 0.0;
        for (int64_t cc = 0; cc < d; ++cc) Di += doi[cc] * oi[cc];
        double *dqi = dq + i * d;
        for (int64_t cc = 0; cc < d; ++cc) dqi[cc] = 0.0;
        for (int64_t j = 0; j < Nk; ++j) {
            if (prob[j] == 0.0) { ds[j] = 0.0; continue; }
            double dpd = 0.0;
            for (int64_t cc = 0; cc < d; ++cc) dpd += doi[cc] * v[j * d + cc];
            double keep = p > 0.0 ? (double)keep_bit(seed, b, h, i, j, T) : 1.0;
            ds[j] = prob[j] * (dpd * keep * c - Di);
            for (int64_t cc = 0; cc < d; ++cc) dqi[cc] += ds[j] * scale * k[j * d + cc];
        }
    }
    /* Column pass: dK_j and dV_j of each key. */
    for (int64_t j = 0; j < Nk; ++j) {
        double *dkj = dk + j * d, *dvj = dv + j * d;
        for (int64_t cc = 0; cc < d; ++cc) { dkj[cc] = 0.0; dvj[cc] = 0.0; }
        for (int64_t i = 0; i < Nq; ++i) {
            double dsij = ds_all[(size_t)i * (size_t)Nk + (size_t)j];
            double pdij = pd_all[(size_t)i * (size_t)Nk + (size_t)j];
            for (int64_t cc = 0; cc < d; ++cc) {
                dkj[cc] += dsij * scale * q[i * d + cc];
                dvj[cc] += pdij * dout[i * d + cc];
            }
        }
    }
    free(pd_all); free(ds_all); free(s); free(prob);
    return ORACLE_OK;
}

/* Number of threads OpenMP will use (for reporting). */
int oracle_num_threads(void)
{
    int n = 1;
    #pragma omp parallel
    {
        #pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
