/*
 * attn_oracle.c -- plain fp64 CPU oracle for exact scaled-dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls
 * this file; it exists so that tests, the smoke check and the bench's CPU
 * baseline can compare the HIP kernels against an obviously correct
 * definition.  It shares no code, header, table or helper with the HIP path.
 *
 * What it computes (pages cited by title and section):
 *
 *  - oracle_fwd: the definition of attention, O = softmax(S) V with
 *    S = scale * Q K^T ("FlashAttention" explainer, "What is FlashAttention?"
 *    and Step 2 "Standard Attention"), the softmax taken row by row as the
 *    numerically safe three-pass softmax (max, sum of exp(x - m), divide)
 *    written out in "13% more FLOPs, 5.7x faster", section "Softmax is the
 *    anti-tiling operation".  The per-row statistic it saves is
 *    lse = m + ln(l) (natural log), the logsumexp form of the pair (m, l)
 *    that the same page's section "The backward pass: recompute instead of
 *    read" says the forward keeps.  Causal masking keeps keys j <= i.
 *
 *  - oracle_bwd: the gradient of L = sum(O * dO) with respect to Q, K, V.
 *    The pages say only that the backward regenerates S and P from Q, K, V
 *    and the saved statistics; the formulas are the plain chain rule through
 *    the softmax Jacobian diag(p) - p p^T:
 *        P_ij  = exp(s_ij - lse_i)            (0 for masked j)
 *        dV_j  = sum_i P_ij dO_i
 *        dP_ij = dO_i . V_j
 *        D_i   = sum_j P_ij dP_ij
 *        dS_ij = P_ij (dP_ij - D_i)
 *        dQ_i  = scale * sum_j dS_ij K_j
 *        dK_j  = scale * sum_i dS_ij Q_i
 *    These are pinned by central finite differences in the tests, not by
 *    re-typing them.  The backward of the library takes the forward's stored
 *    output o as an input and forms D_i = dO_i . o_i from it; when a caller
 *    passes that stored o (o_in below), the oracle does the same, which for
 *    the exact o is the same number as sum_j P_ij dP_ij.
 *
 *  - oracle_online_softmax / oracle_fwd_online: the pages' online method in
 *    fp64 -- running max m and normaliser l updated chunk by chunk with the
 *    factor exp(m_old - m_new) ("Softmax is the anti-tiling operation"), and
 *    the output accumulator rescaled by the same factor and divided by l
 *    after the last tile ("FlashAttention's move: rescale the output, too";
 *    explainer Step 4 "Online Softmax").  The state starts at m = -inf,
 *    l = 0 with no rescale on the first chunk (explainer Step 4).  These
 *    serve the pages' worked examples (the 8-score chunked softmax, and the
 *    Step 6 exactness check of tiled against standard attention).
 *
 *  - oracle_fwd_rect: the forward definition for Nq queries against Nk keys
 *    per head, the shape of Flash-Decoding (a few new queries against a long
 *    key/value cache; explainer "Common questions").  Under the causal mask
 *    the queries are the last Nq positions: query i sees keys 0 .. i+Nk-Nq
 *    (a row that sees none gets o = 0, lse = -inf).
 *
 *  - oracle_fwd_dropout / oracle_bwd_dropout: the same two computations with
 *    dropout on the attention probabilities, which the pages fuse into the
 *    kernel and whose mask the backward regenerates from the PRNG state the
 *    forward keeps ("13% more FLOPs, 5.7x faster", section "The backward
 *    pass: recompute instead of read"; explainer Step 3 "Tiling").  The pages
 *    fix neither the generator nor the mask's layout; the reading taken:
 *        keep_ij = [R_ij >= t],  t = floor(256 p + 1/2)  (0 <= t <= 255),
 *        O_i     = sum_j keep_ij (256 / (256 - t)) P_ij v_j,
 *    lse the statistic of the undropped softmax, and R_ij one byte of
 *    Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers:
 *    as easy as 1, 2, 3", SC 2011): with key (seed mod 2^32, seed / 2^32)
 *    and counter (i, 2 floor(j/32) + floor(j/4) mod 2, bh, offset), R_ij is
 *    byte (j mod 4) of output word floor((j mod 32) / 8).  The gradient is
 *    the chain rule through the dropped weights W_ij = keep_ij r P_ij
 *    (r = 256 / (256 - t)): dV_j = sum_i W_ij dO_i, dP_ij = keep_ij r
 *    dO_i . v_j, D_i = sum_j P_ij dP_ij (= dO_i . O_i), dS = P (dP - D).
 *
 * All arithmetic is IEEE double with libm exp/log; loops run in the plain
 * index order of the formulas.  OpenMP only splits independent rows (forward)
 * or independent heads (backward) across threads.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Philox4x32-10 (Salmon et al., SC 2011): ten rounds of two 32x32->64-bit
 * products, each round mapping (c0, c1, c2, c3) with key (k0, k1) to
 * (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)), the key
 * advanced by the Weyl constants between rounds. */
static void philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        const uint64_t p0 = (uint64_t)M0 * c0, p1 = (uint64_t)M1 * c2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n1 = (uint32_t)p1;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        const uint32_t n3 = (uint32_t)p0;
        c0 = n0, c1 = n1, c2 = n2, c3 = n3;
        k0 += W0, k1 += W1;
    }
    out[0] = c0, out[1] = c1, out[2] = c2, out[3] = c3;
}

int oracle_philox4x32_10(const uint32_t* ctr, const uint32_t* key, uint32_t* out) {
    if (!ctr || !key || !out) return -1;
    philox4x32_10(ctr, key, out);
    return 0;
}

/* Dropout state: threshold t, keep factor r = 256 / (256 - t), generator key
 * and counter offset. */
struct drop {
    int t;
    double r;
    uint64_t seed;
    uint32_t offset;
};

static int drop_init(struct drop* dr, double p, uint64_t seed, uint32_t offset) {
    if (!(p >= 0.0 && p < 1.0)) return -1;
    const double tt = floor(256.0 * p + 0.5);
    if (tt > 255.0) return -1;
    dr->t = (int)tt;
    dr->r = 256.0 / (256.0 - tt);
    dr->seed = seed;
    dr->offset = offset;
    return 0;
}

/* keep_ij of head bh (1 kept, 0 dropped) */
static int drop_keep(const struct drop* dr, int64_t bh, int64_t i, int64_t j) {
    const uint32_t ctr[4] = {(uint32_t)i, (uint32_t)(2 * (j / 32) + (j / 4) % 2), (uint32_t)bh, dr->offset};
    const uint32_t key[2] = {(uint32_t)dr->seed, (uint32_t)(dr->seed >> 32)};
    uint32_t out[4];
    philox4x32_10(ctr, key, out);
    const uint32_t byte = (out[(j % 32) / 8] >> (8 * (j % 4))) & 0xFFu;
    return byte >= (uint32_t)dr->t;
}

/* The keep mask of one head, N x N bytes (1 kept, 0 dropped); the causal
 * mask is not applied here. */
int oracle_dropout_keep(double p, uint64_t seed, uint32_t offset, int64_t bh, int64_t N,
                        uint8_t* keep) {
    struct drop dr;
    if (!keep || N < 0 || bh < 0 || drop_init(&dr, p, seed, offset)) return -1;
    for (int64_t i = 0; i < N; ++i)
        for (int64_t j = 0; j < N; ++j) keep[i * N + j] = (uint8_t)drop_keep(&dr, bh, i, j);
    return 0;
}

/* Number of keys query row i may attend to: all Nk, or under the causal
 * mask keys 0 .. i + Nk - Nq (the Nq queries are the last Nq positions of
 * the Nk keys; i + 1 when Nq = Nk), none when that is negative. */
static int64_t keys_for_row(int64_t i, int64_t Nq, int64_t Nk, int causal) {
    if (!causal) return Nk;
    const int64_t n = i + Nk - Nq + 1;
    return n < 0 ? 0 : (n > Nk ? Nk : n);
}

/* One query row of the forward definition.
 * qi: d values; kh, vh: Nk x d of this (batch, head); s: scratch of Nk
 * doubles; dr: dropout state or NULL, bh the head's index (for the dropout
 * mask).  Writes oi (d values) and *lse_i; a row that sees no key gets
 * o = 0 and lse = -inf. */
static void fwd_row(const double* qi, const double* kh, const double* vh,
                    int64_t i, int64_t Nq, int64_t Nk, int64_t d, double scale, int causal,
                    const struct drop* dr, int64_t bh,
                    double* s, double* oi, double* lse_i) {
    int64_t nk = keys_for_row(i, Nq, Nk, causal);
    /* scores s_j = scale * q_i . k_j */
    for (int64_t j = 0; j < nk; ++j) {
        double acc = 0.0;
        for (int64_t c = 0; c < d; ++c) acc += qi[c] * kh[j * d + c];
        s[j] = scale * acc;
    }
    /* pass 1: row max */
    double m = -INFINITY;
    for (int64_t j = 0; j < nk; ++j)
        if (s[j] > m) m = s[j];
    /* pass 2: normaliser */
    double l = 0.0;
    for (int64_t j = 0; j < nk; ++j) l += exp(s[j] - m);
    /* pass 3: normalised weights (dropped and rescaled under dropout)
     * applied to V */
    for (int64_t c = 0; c < d; ++c) oi[c] = 0.0;
    for (int64_t j = 0; j < nk; ++j) {
        double p = exp(s[j] - m) / l;
        if (dr) p = drop_keep(dr, bh, i, j) ? dr->r * p : 0.0;
        for (int64_t c = 0; c < d; ++c) oi[c] += p * vh[j * d + c];
    }
    *lse_i = m + log(l);
}

/*
 * oracle_fwd
 *   q, k, v : [BH, N, d] fp64, row-major (d fastest)
 *   rows    : flattened row ids r = bh * N + i to compute, or NULL for all
 *             BH*N rows in order
 *   o       : [n_rows, d] fp64 output (row order of `rows`)
 *   lse     : [n_rows] fp64 output
 *   threads : OpenMP threads to use (<= 0: library default)
 * Returns 0, or -1 on a bad argument.
 */
static int fwd_rows(const double* q, const double* k, const double* v,
                    double* o, double* lse,
                    int64_t BH, int64_t Nq, int64_t Nk, int64_t d, double scale, int causal,
                    const struct drop* dr,
                    const int64_t* rows, int64_t n_rows, int threads) {
    if (!q || !k || !v || !o || !lse || BH < 0 || Nq < 0 || Nk < 0 || d <= 0) return -1;
    if (!rows) n_rows = BH * Nq;
    if (n_rows < 0) return -1;
    if (rows)
        for (int64_t t = 0; t < n_rows; ++t)
            if (rows[t] < 0 || rows[t] >= BH * Nq) return -1;
#ifdef _OPENMP
    if (threads <= 0) threads = omp_get_max_threads();
#else
    (void)threads;
#endif
    int failed = 0;
#pragma omp parallel num_threads(threads) reduction(| : failed)
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
        if (!s) {
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t t = 0; t < n_rows; ++t) {
                int64_t r = rows ? rows[t] : t;
                int64_t bh = r / Nq, i = r % Nq;
                const double* kh = k + bh * Nk * d;
                const double* vh = v + bh * Nk * d;
                fwd_row(q + r * d, kh, vh, i, Nq, Nk, d, scale, causal, dr, bh, s, o + t * d, lse + t);
            }
            free(s);
        }
    }
    return failed ? -1 : 0;
}

int oracle_fwd(const double* q, const double* k, const double* v,
               double* o, double* lse,
               int64_t BH, int64_t N, int64_t d, double scale, int causal,
               const int64_t* rows, int64_t n_rows, int threads) {
    return fwd_rows(q, k, v, o, lse, BH, N, N, d, scale, causal, NULL, rows, n_rows, threads);
}

/* oracle_fwd_rect: oracle_fwd with Nq query rows against Nk keys per head
 * (q, o: [BH, Nq, d]; k, v: [BH, Nk, d]; lse: [BH, Nq]; row ids bh * Nq + i).
 * Under the causal mask query i sees keys 0 .. i + Nk - Nq. */
int oracle_fwd_rect(const double* q, const double* k, const double* v,
                    double* o, double* lse,
                    int64_t BH, int64_t Nq, int64_t Nk, int64_t d, double scale, int causal,
                    const int64_t* rows, int64_t n_rows, int threads) {
    return fwd_rows(q, k, v, o, lse, BH, Nq, Nk, d, scale, causal, NULL, rows, n_rows, threads);
}

/* oracle_fwd_dropout: oracle_fwd with dropout probability p (quantised to
 * t / 256) and generator state (seed, offset). */
int oracle_fwd_dropout(const double* q, const double* k, const double* v,
                       double* o, double* lse,
                       int64_t BH, int64_t N, int64_t d, double scale, int causal,
                       double p, uint64_t seed, uint32_t offset,
                       const int64_t* rows, int64_t n_rows, int threads) {
    struct drop dr;
    if (drop_init(&dr, p, seed, offset)) return -1;
    return fwd_rows(q, k, v, o, lse, BH, N, N, d, scale, causal, &dr, rows, n_rows, threads);
}

/*
 * oracle_bwd
 *   q, k, v, dO : [BH, N, d] fp64
 *   o_in        : NULL, or [BH, N, d] fp64: a stored forward output to form
 *                 D_i = dO_i . o_in_i from (instead of sum_j P_ij dP_ij)
 *   o, lse      : [BH, N, d] and [BH, N] fp64 outputs (the oracle's own forward)
 *   dq, dk, dv  : [BH, N, d] fp64 outputs
 * Each head is independent; one thread owns a whole head, so dK and dV
 * accumulate without races.  Row by row: recompute s and the forward
 * statistics, form P, dP, D, dS, then add the row's terms to dQ, dK, dV.
 */
static int bwd_heads(const double* q, const double* k, const double* v, const double* dO,
                     const double* o_in,
                     double* o, double* lse, double* dq, double* dk, double* dv,
                     int64_t BH, int64_t N, int64_t d, double scale, int causal,
                     const struct drop* dr, int threads) {
    if (!q || !k || !v || !dO || !o || !lse || !dq || !dk || !dv || BH < 0 || N < 0 || d <= 0)
        return -1;
#ifdef _OPENMP
    if (threads <= 0) threads = omp_get_max_threads();
#else
    (void)threads;
#endif
    int failed = 0;
#pragma omp parallel num_threads(threads) reduction(| : failed)
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        double* p = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        double* dp = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        double* w = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        if (!s || !p || !dp || !w) {
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t bh = 0; bh < BH; ++bh) {
                const double* qh = q + bh * N * d;
                const double* kh = k + bh * N * d;
                const double* vh = v + bh * N * d;
                const double* gh = dO + bh * N * d;
                double* oh = o + bh * N * d;
                double* lh = lse + bh * N;
                double* dqh = dq + bh * N * d;
                double* dkh = dk + bh * N * d;
                double* dvh = dv + bh * N * d;
                memset(dkh, 0, sizeof(double) * (size_t)(N * d));
                memset(dvh, 0, sizeof(double) * (size_t)(N * d));
                for (int64_t i = 0; i < N; ++i) {
                    int64_t nk = keys_for_row(i, N, N, causal);
                    const double* qi = qh + i * d;
                    const double* gi = gh + i * d;
                    /* forward quantities of this row: o_i and lse_i */
                    fwd_row(qi, kh, vh, i, N, N, d, scale, causal, dr, bh, s, oh + i * d, lh + i);
                    /* s was overwritten by fwd_row with the scaled scores; P from
                     * lse, and the weights W applied to V (W = P without dropout) */
                    for (int64_t j = 0; j < nk; ++j) {
                        p[j] = exp(s[j] - lh[i]);
                        w[j] = dr ? (drop_keep(dr, bh, i, j) ? dr->r * p[j] : 0.0) : p[j];
                    }
                    /* dP_ij = d(loss)/dP_ij: dO_i . v_j, times keep_ij r under dropout */
                    for (int64_t j = 0; j < nk; ++j) {
                        double acc = 0.0;
                        for (int64_t c = 0; c < d; ++c) acc += gi[c] * vh[j * d + c];
                        dp[j] = dr ? (drop_keep(dr, bh, i, j) ? dr->r * acc : 0.0) : acc;
                    }
                    /* D_i = sum_j P_ij dP_ij, or dO_i . o_i for a given stored o */
                    double Di = 0.0;
                    if (o_in) {
                        const double* oi = o_in + (bh * N + i) * d;
                        for (int64_t c = 0; c < d; ++c) Di += gi[c] * oi[c];
                    } else {
                        for (int64_t j = 0; j < nk; ++j) Di += p[j] * dp[j];
                    }
                    /* dS, then the three gradient sums */
                    for (int64_t c = 0; c < d; ++c) dqh[i * d + c] = 0.0;
                    for (int64_t j = 0; j < nk; ++j) {
                        double ds = p[j] * (dp[j] - Di);
                        for (int64_t c = 0; c < d; ++c) {
                            dqh[i * d + c] += scale * ds * kh[j * d + c];
                            dkh[j * d + c] += scale * ds * qi[c];
                            dvh[j * d + c] += w[j] * gi[c];
                        }
                    }
                }
            }
        }
        free(s);
        free(p);
        free(dp);
        free(w);
    }
    return failed ? -1 : 0;
}

int oracle_bwd(const double* q, const double* k, const double* v, const double* dO,
               const double* o_in,
               double* o, double* lse, double* dq, double* dk, double* dv,
               int64_t BH, int64_t N, int64_t d, double scale, int causal, int threads) {
    return bwd_heads(q, k, v, dO, o_in, o, lse, dq, dk, dv, BH, N, d, scale, causal, NULL, threads);
}

/* oracle_bwd_dropout: oracle_bwd through the dropped weights (see the top of
 * the file); o and lse are the dropout forward's. */
int oracle_bwd_dropout(const double* q, const double* k, const double* v, const double* dO,
                       const double* o_in,
                       double* o, double* lse, double* dq, double* dk, double* dv,
                       int64_t BH, int64_t N, int64_t d, double scale, int causal,
                       double p, uint64_t seed, uint32_t offset, int threads) {
    struct drop dr;
    if (drop_init(&dr, p, seed, offset)) return -1;
    return bwd_heads(q, k, v, dO, o_in, o, lse, dq, dk, dv, BH, N, d, scale, causal, &dr, threads);
}

/*
 * oracle_online_softmax: softmax of x[0..n) by the pages' one-pass update,
 * reading `chunk` scores at a time.
 *   y        : n outputs, the final probabilities exp(x_j - m) / l
 *   states   : optional [n_chunks][3] = (m, l, rescale factor) after each
 *              chunk; the factor is reported as NAN for the first chunk,
 *              whose history is empty ("none yet")
 * Returns the number of chunks, or -1 on a bad argument.
 */
int64_t oracle_online_softmax(const double* x, int64_t n, int64_t chunk,
                              double* y, double* states) {
    if (!x || !y || n < 0 || chunk <= 0) return -1;
    double m = -INFINITY, l = 0.0;
    int64_t nc = 0;
    for (int64_t c0 = 0; c0 < n; c0 += chunk, ++nc) {
        int64_t c1 = c0 + chunk < n ? c0 + chunk : n;
        double mb = -INFINITY;
        for (int64_t j = c0; j < c1; ++j)
            if (x[j] > mb) mb = x[j];
        double m_new = mb > m ? mb : m;
        double lb = 0.0;
        for (int64_t j = c0; j < c1; ++j) lb += exp(x[j] - m_new);
        /* empty history: nothing to rescale */
        double alpha = (m == -INFINITY) ? NAN : exp(m - m_new);
        l = (m == -INFINITY ? 0.0 : alpha * l) + lb;
        m = m_new;
        if (states) {
            states[3 * nc + 0] = m;
            states[3 * nc + 1] = l;
            states[3 * nc + 2] = alpha;
        }
    }
    for (int64_t j = 0; j < n; ++j) y[j] = exp(x[j] - m) / l;
    return nc;
}

/*
 * oracle_fwd_online: the tiled forward of the pages in fp64 for one head.
 * For each query row, K/V tiles of `tile` keys are visited in order; each
 * tile updates (m, l) and rescales the unnormalised output accumulator by
 * exp(m_old - m_new) before adding the tile's sum of exp(s - m_new) * v;
 * the accumulator is divided by l after the last tile.
 *   q, k, v : [N, d]; o : [N, d]; lse : [N]
 */
int oracle_fwd_online(const double* q, const double* k, const double* v,
                      double* o, double* lse, int64_t N, int64_t d,
                      double scale, int causal, int64_t tile) {
    if (!q || !k || !v || !o || !lse || N < 0 || d <= 0 || tile <= 0) return -1;
    double* s = (double*)malloc(sizeof(double) * (size_t)(tile));
    if (!s) return -1;
    for (int64_t i = 0; i < N; ++i) {
        int64_t nk = keys_for_row(i, N, N, causal);
        double m = -INFINITY, l = 0.0;
        double* oi = o + i * d;
        for (int64_t c = 0; c < d; ++c) oi[c] = 0.0;
        for (int64_t j0 = 0; j0 < nk; j0 += tile) {
            int64_t j1 = j0 + tile < nk ? j0 + tile : nk;
            double mb = -INFINITY;
            for (int64_t j = j0; j < j1; ++j) {
                double acc = 0.0;
                for (int64_t c = 0; c < d; ++c) acc += q[i * d + c] * k[j * d + c];
                s[j - j0] = scale * acc;
                if (s[j - j0] > mb) mb = s[j - j0];
            }
            double m_new = mb > m ? mb : m;
            double alpha = (m == -INFINITY) ? 0.0 : exp(m - m_new);
            l *= alpha;
            for (int64_t c = 0; c < d; ++c) oi[c] *= alpha;
            for (int64_t j = j0; j < j1; ++j) {
                double pj = exp(s[j - j0] - m_new);
                l += pj;
                for (int64_t c = 0; c < d; ++c) oi[c] += pj * v[j * d + c];
            }
            m = m_new;
        }
        for (int64_t c = 0; c < d; ++c) oi[c] /= l;
        lse[i] = m + log(l);
    }
    free(s);
    return 0;
}
