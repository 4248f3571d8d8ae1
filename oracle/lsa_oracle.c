/*
 * CPU oracle for content-routed block sparse attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain reference that the
 * GPU library is checked against.  Only the test suite, the smoke check and
 * the CPU-baseline leg of the benchmark may load it; the product path never
 * calls it and shares no code, header or table with it.
 *
 * What it computes, step by step, in the order the pages give:
 *
 *   1. Block summaries.  Keys are cut into contiguous blocks of `bs` tokens
 *      and each block is summarised by its mean, the first cumulant mu_c of
 *      the SSA routing score (SSA page, jonsmirl/ssa, "Algorithm and
 *      complexity", r_c(q) = <q, mu_c> + (beta/2) q^T Sigma_c q, here with
 *      beta = 0).  The mean is summed in fp64 and rounded once to fp32
 *      ("fp32 block means").  In the non-causal image mode the queries are
 *      pooled the same way over query blocks of `bs` tokens (LLSA page,
 *      "Minimum Usage": block_size 16 for both).
 *
 *   2. Routing scores s_c = <q, mu_c>, in fp64, over the eligible blocks.
 *      Causal rows: only complete blocks that end before the local window
 *      are eligible, so that no summary mixes in a future key (SSA page,
 *      "Mathematical status" and "Known limitations": a routed set is causal
 *      only once it is cut at the query's own position; Subquadratic Sparse
 *      Attention page, "Why the layer is mathematically subquadratic":
 *      completed blocks are exposed only when their last token is before the
 *      cutoff that excludes the local window).
 *
 *   3. Top-k.  The candidates are ordered by score, descending, and exact
 *      ties go to the lower block index; the first min(k, E) are kept and
 *      emitted in ascending block order, padded with -1.  (The SSA page,
 *      "Mathematical status", notes that without a margin a deterministic
 *      index order is needed to name one top set; this build fixes it to the
 *      lowest index.)
 *
 *   4. Exact softmax attention over the selected keys only: the routed
 *      blocks plus the local causal window (SSA page, opening paragraph;
 *      Subquadratic Sparse Attention page, "Architecture": selected attention
 *      alongside a causal sliding window).  Logits (q . k_j) * scale, scale
 *      1/sqrt(D) by default as in the scaled dot-product attention that LLSA
 *      replaces.  Computed in fp64, stored as fp32.
 *
 * Readings where the pages leave a step open (all plain choices):
 *   - The window is block aligned: the query's own block (keys up to the
 *     query, inclusive) plus the window/bs - 1 blocks before it.  With
 *     beta = t / bs and E = max(0, beta - window/bs + 1), the eligible
 *     routed blocks are c in [0, E) and the window is keys [bs*E, t].  The
 *     two never overlap, and with every eligible block selected their union
 *     is exactly [0, t] (dense causal attention).
 *   - Grouped-query attention: query head h reads KV head h / (Hq / Hkv).
 *     Routing is done per query head, or, in consensus mode, once per KV
 *     group with the sum of the group's heads' scores (orc_route_consensus).
 *   - Image mode (causal == 0): query block i (tokens [i*bs, i*bs+bs)) is
 *     routed with the pooled query mean over all key blocks; every token of
 *     the block attends to the union of the selected blocks; no window.
 *
 * Indices: a causal row is r = (b*Hq + h)*N + t; an image-mode routing row
 * is r = (b*Hq + h)*(N/bs) + i.  Arrays are [B, H, N, D] row-major, D
 * fastest; bf16 arrives as raw uint16 bit patterns.
 *
 * Return codes: 0 ok, -1 bad argument, -2 an idx entry is not a valid
 * selection (out of range, not ascending, or a -1 followed by a block).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

static double bf16_to_f64(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int orc_num_threads(void) { return omp_get_max_threads(); }

/* Step 1: mean of each block of bs consecutive tokens, fp64 sum, one fp32
 * rounding.  x [B*H, N, D] bf16 -> out [B*H, N/bs, D] fp32. */
int orc_block_means(const uint16_t *x, int64_t BH, int64_t N, int64_t D,
                    int64_t bs, float *out)
{
    if (!x || !out || BH <= 0 || N <= 0 || D <= 0 || bs <= 0 || N % bs)
        return -1;
    const int64_t nb = N / bs;
#pragma omp parallel for schedule(static)
    for (int64_t hc = 0; hc < BH * nb; ++hc) {
        const int64_t bh = hc / nb, c = hc % nb;
        for (int64_t d = 0; d < D; ++d) {
            double s = 0.0;
            for (int64_t j = 0; j < bs; ++j)
                s += bf16_to_f64(x[(bh * N + c * bs + j) * D + d]);
            out[(bh * nb + c) * D + d] = (float)(s / (double)bs);
        }
    }
    return 0;
}

/* Number of routed candidates of causal query position t. */
static int64_t eligible_blocks(int64_t t, int64_t bs, int64_t window)
{
    int64_t e = t / bs - window / bs + 1;
    return e > 0 ? e : 0;
}

typedef struct {
    double s;
    int64_t c;
} cand_t;

/* Score descending, then block index ascending. */
static int cand_order(const void *pa, const void *pb)
{
    const cand_t *a = (const cand_t *)pa, *b = (const cand_t *)pb;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return (a->c > b->c) - (a->c < b->c);
}

static int idx_ascending(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

/* Step 3 for one row: buf holds the ncand candidates' scores (buf[c].s) and
 * ids; orders them, keeps the first min(k, ncand), emits them ascending and
 * -1 padded, and the k-th / (k+1)-th gap. */
static void pick_top(cand_t *buf, int64_t ncand, int64_t k, int32_t *idx_out,
                     double *gap_out)
{
    qsort(buf, (size_t)ncand, sizeof(cand_t), cand_order);
    const int64_t keep = ncand < k ? ncand : k;
    for (int64_t i = 0; i < k; ++i)
        idx_out[i] = i < keep ? (int32_t)buf[i].c : -1;
    qsort(idx_out, (size_t)keep, sizeof(int32_t), idx_ascending);
    if (gap_out)
        *gap_out = ncand > k ? buf[k - 1].s - buf[k].s : INFINITY;
}

/* Steps 2-3 for one row, given its query as doubles and the candidate count.
 * summ: [ncand, D] fp32 summaries of the row's KV head. */
static void select_top(const double *qd, const float *summ, int64_t ncand,
                       int64_t D, int64_t k, cand_t *buf, int32_t *idx_out,
                       double *gap_out)
{
    for (int64_t c = 0; c < ncand; ++c) {
        double s = 0.0;
        for (int64_t d = 0; d < D; ++d)
            s += qd[d] * (double)summ[c * D + d];
        buf[c].s = s;
        buf[c].c = c;
    }
    pick_top(buf, ncand, k, idx_out, gap_out);
}

/* Steps 2-3, causal rows.  rows: n_rows row ids (NULL = all B*Hq*N rows in
 * order).  idx: [n_rows, k].  gap (nullable): [n_rows], score of the k-th
 * selected minus score of the best unselected (+inf when nothing is left
 * out). */
int orc_route_causal(const uint16_t *q, const float *kbar, int64_t B,
                     int64_t Hq, int64_t Hkv, int64_t N, int64_t D, int64_t bs,
                     int64_t k, int64_t window, const int64_t *rows,
                     int64_t n_rows, int32_t *idx, double *gap)
{
    if (!q || !kbar || !idx || bs <= 0 || N % bs || Hkv <= 0 || Hq % Hkv ||
        k <= 0 || window < bs || window % bs)
        return -1;
    const int64_t nb = N / bs, rep = Hq / Hkv;
    const int64_t total = rows ? n_rows : B * Hq * N;
    int bad = 0;
#pragma omp parallel
    {
        cand_t *buf = (cand_t *)malloc(sizeof(cand_t) * (size_t)(nb + 1));
        double *qd = (double *)malloc(sizeof(double) * (size_t)D);
        if (!buf || !qd) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 64)
        for (int64_t i = 0; i < total; ++i) {
            if (!buf || !qd) continue;
            const int64_t r = rows ? rows[i] : i;
            if (r < 0 || r >= B * Hq * N) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            const int64_t t = r % N, bh = r / N, h = bh % Hq, b = bh / Hq;
            const int64_t g = h / rep;
            for (int64_t d = 0; d < D; ++d)
                qd[d] = bf16_to_f64(q[r * D + d]);
            const float *summ = kbar + (b * Hkv + g) * nb * D;
            select_top(qd, summ, eligible_blocks(t, bs, window), D, k, buf,
                       idx + i * k, gap ? gap + i : NULL);
        }
        free(buf);
        free(qd);
    }
    return bad ? -1 : 0;
}

/* Steps 2-3, image mode.  qbar [B, Hq, nb, D] fp32 pooled queries,
 * kbar [B, Hkv, nb, D].  rows index query blocks: (b*Hq + h)*nb + i. */
int orc_route_image(const float *qbar, const float *kbar, int64_t B,
                    int64_t Hq, int64_t Hkv, int64_t nb, int64_t D, int64_t k,
                    const int64_t *rows, int64_t n_rows, int32_t *idx,
                    double *gap)
{
    if (!qbar || !kbar || !idx || nb <= 0 || Hkv <= 0 || Hq % Hkv || k <= 0)
        return -1;
    const int64_t rep = Hq / Hkv;
    const int64_t total = rows ? n_rows : B * Hq * nb;
    int bad = 0;
#pragma omp parallel
    {
        cand_t *buf = (cand_t *)malloc(sizeof(cand_t) * (size_t)(nb + 1));
        double *qd = (double *)malloc(sizeof(double) * (size_t)D);
        if (!buf || !qd) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t i = 0; i < total; ++i) {
            if (!buf || !qd) continue;
            const int64_t r = rows ? rows[i] : i;
            if (r < 0 || r >= B * Hq * nb) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            const int64_t bh = r / nb, h = bh % Hq, b = bh / Hq;
            for (int64_t d = 0; d < D; ++d)
                qd[d] = (double)qbar[r * D + d];
            const float *summ = kbar + (b * Hkv + h / rep) * nb * D;
            select_top(qd, summ, nb, D, k, buf, idx + i * k,
                       gap ? gap + i : NULL);
        }
        free(buf);
        free(qd);
    }
    return bad ? -1 : 0;
}

/* Step 2 alone, for checking near ties: every block's score for the given
 * rows, -inf where the block is not a candidate.  scores [n_rows, nb].
 * causal != 0: q is bf16 [B,Hq,N,D], rows are causal rows.
 * causal == 0: qbar is fp32 [B,Hq,nb,D], rows are query-block rows. */
int orc_route_scores(const uint16_t *q, const float *qbar, const float *kbar,
                     int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D,
                     int64_t bs, int64_t window, int64_t causal,
                     const int64_t *rows, int64_t n_rows, double *scores)
{
    if (!kbar || !rows || !scores || bs <= 0 || N % bs || Hkv <= 0 ||
        Hq % Hkv)
        return -1;
    if (causal ? (!q || window < bs || window % bs) : !qbar)
        return -1;
    const int64_t nb = N / bs, rep = Hq / Hkv;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < n_rows; ++i) {
        const int64_t r = rows[i];
        const int64_t per = causal ? N : nb;
        if (r < 0 || r >= B * Hq * per) {
#pragma omp atomic write
            bad = 1;
            continue;
        }
        const int64_t bh = r / per, h = bh % Hq, b = bh / Hq;
        const int64_t ncand = causal ? eligible_blocks(r % per, bs, window) : nb;
        const float *summ = kbar + (b * Hkv + h / rep) * nb * D;
        for (int64_t c = 0; c < nb; ++c) {
            double s = -INFINITY;
            if (c < ncand) {
                s = 0.0;
                for (int64_t d = 0; d < D; ++d) {
                    double qv = causal ? bf16_to_f64(q[r * D + d])
                                       : (double)qbar[r * D + d];
                    s += qv * (double)summ[c * D + d];
                }
            }
            scores[i * nb + c] = s;
        }
    }
    return bad ? -1 : 0;
}

/* Consensus routing, one route per KV group: a group's score for block c is
 * the sum of the routing scores of the group's query heads,
 * sum_h <q_h, mu_c> (SSA page, "Complete 10M transformer result": a
 * cross-head consensus route; here the heads that share one KV head, so
 * that the route can be shared with them).  Candidates, top-k and tie-break
 * as in steps 2-3.
 *   causal != 0: q bf16 [B,Hq,N,D]; rows index (b*Hkv + g)*N + t.
 *   causal == 0: qbar fp32 [B,Hq,nb,D] pooled queries; rows index
 *                (b*Hkv + g)*nb + i.
 * rows NULL = every group row in order.  idx [n_rows, k]; gap (nullable) as
 * in orc_route_causal; scores (nullable) [n_rows, nb] every block's
 * consensus score, -inf where the block is not a candidate. */
int orc_route_consensus(const uint16_t *q, const float *qbar,
                        const float *kbar, int64_t B, int64_t Hq, int64_t Hkv,
                        int64_t N, int64_t D, int64_t bs, int64_t k,
                        int64_t window, int64_t causal, const int64_t *rows,
                        int64_t n_rows, int32_t *idx, double *gap,
                        double *scores)
{
    if (!kbar || !idx || bs <= 0 || N % bs || Hkv <= 0 || Hq % Hkv || k <= 0)
        return -1;
    if (causal ? (!q || window < bs || window % bs) : !qbar)
        return -1;
    const int64_t nb = N / bs, rep = Hq / Hkv;
    const int64_t per = causal ? N : nb;
    const int64_t total = rows ? n_rows : B * Hkv * per;
    int bad = 0;
#pragma omp parallel
    {
        cand_t *buf = (cand_t *)malloc(sizeof(cand_t) * (size_t)(nb + 1));
        if (!buf) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 32)
        for (int64_t i = 0; i < total; ++i) {
            if (!buf) continue;
            const int64_t r = rows ? rows[i] : i;
            if (r < 0 || r >= B * Hkv * per) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            const int64_t p = r % per, bg = r / per;
            const int64_t b = bg / Hkv, g = bg % Hkv;
            const int64_t ncand = causal ? eligible_blocks(p, bs, window) : nb;
            const float *summ = kbar + bg * nb * D;
            for (int64_t c = 0; c < ncand; ++c) {
                double s = 0.0;
                for (int64_t hh = 0; hh < rep; ++hh) {
                    const int64_t qr = ((b * Hq + g * rep + hh) * per + p) * D;
                    double sh = 0.0;
                    for (int64_t d = 0; d < D; ++d) {
                        const double qv = causal ? bf16_to_f64(q[qr + d])
                                                 : (double)qbar[qr + d];
                        sh += qv * (double)summ[c * D + d];
                    }
                    s += sh;
                }
                buf[c].s = s;
                buf[c].c = c;
            }
            if (scores)
                for (int64_t c = 0; c < nb; ++c)
                    scores[i * nb + c] = c < ncand ? buf[c].s : -INFINITY;
            pick_top(buf, ncand, k, idx + i * k, gap ? gap + i : NULL);
        }
        free(buf);
    }
    return bad ? -1 : 0;
}

/* Second-cumulant routing score (SSA page, "Algorithm and complexity"):
 *   r_c(q) = <q, mu_c> + (beta/2) q^T Sigma_c q,
 * mu_c the fp32 block mean of step 1 and Sigma_c the covariance of the
 * block's bs keys about their mean, normalised by bs (the second cumulant
 * of the block's key distribution; fp64 throughout).  beta = 0 gives the
 * step-2 score.  Causal rows only: q bf16 [B,Hq,N,D], k bf16 [B,Hkv,N,D],
 * kbar [B,Hkv,nb,D]; rows (b*Hq + h)*N + t (NULL = all).  idx [n_rows, k]
 * with the step-3 ordering; gap (nullable) as in orc_route_causal; scores
 * (nullable) [n_rows, nb], -inf where the block is not a candidate. */
int orc_route_cumulant(const uint16_t *q, const uint16_t *kk, const float *kbar,
                       int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                       int64_t D, int64_t bs, int64_t k, int64_t window,
                       double beta, const int64_t *rows, int64_t n_rows,
                       int32_t *idx, double *gap, double *scores)
{
    if (!q || !kk || !kbar || !idx || bs <= 0 || N % bs || Hkv <= 0 ||
        Hq % Hkv || k <= 0 || window < bs || window % bs)
        return -1;
    const int64_t nb = N / bs, rep = Hq / Hkv;
    const int64_t total = rows ? n_rows : B * Hq * N;
    /* Sigma_c of every block: [B*Hkv][nb][D][D] */
    double *sig = (double *)malloc(sizeof(double) * (size_t)(B * Hkv * nb * D * D));
    if (!sig)
        return -1;
#pragma omp parallel
    {
        double *m = (double *)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(static)
        for (int64_t gc = 0; gc < B * Hkv * nb; ++gc) {
            const int64_t bg = gc / nb, c = gc % nb;
            const uint16_t *blk = kk + (bg * N + c * bs) * D;
            double *S = sig + gc * D * D;
            for (int64_t d = 0; d < D; ++d) {
                double a = 0.0;
                for (int64_t j = 0; j < bs; ++j)
                    a += bf16_to_f64(blk[j * D + d]);
                m[d] = a / (double)bs;
            }
            for (int64_t d = 0; d < D; ++d)
                for (int64_t e = 0; e < D; ++e) {
                    double a = 0.0;
                    for (int64_t j = 0; j < bs; ++j)
                        a += (bf16_to_f64(blk[j * D + d]) - m[d]) *
                             (bf16_to_f64(blk[j * D + e]) - m[e]);
                    S[d * D + e] = a / (double)bs;
                }
        }
        free(m);
    }
    int bad = 0;
#pragma omp parallel
    {
        cand_t *buf = (cand_t *)malloc(sizeof(cand_t) * (size_t)(nb + 1));
        double *qd = (double *)malloc(sizeof(double) * (size_t)D);
        if (!buf || !qd) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t i = 0; i < total; ++i) {
            if (!buf || !qd) continue;
            const int64_t r = rows ? rows[i] : i;
            if (r < 0 || r >= B * Hq * N) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            const int64_t t = r % N, bh = r / N, h = bh % Hq, b = bh / Hq;
            const int64_t bg = b * Hkv + h / rep;
            const int64_t ncand = eligible_blocks(t, bs, window);
            for (int64_t d = 0; d < D; ++d)
                qd[d] = bf16_to_f64(q[r * D + d]);
            for (int64_t c = 0; c < ncand; ++c) {
                const float *mu = kbar + (bg * nb + c) * D;
                const double *S = sig + (bg * nb + c) * D * D;
                double first = 0.0, quad = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    first += qd[d] * (double)mu[d];
                for (int64_t d = 0; d < D; ++d)
                    for (int64_t e = 0; e < D; ++e)
                        quad += qd[d] * S[d * D + e] * qd[e];
                buf[c].s = first + 0.5 * beta * quad;
                buf[c].c = c;
            }
            if (scores)
                for (int64_t c = 0; c < nb; ++c)
                    scores[i * nb + c] = c < ncand ? buf[c].s : -INFINITY;
            pick_top(buf, ncand, k, idx + i * k, gap ? gap + i : NULL);
        }
        free(buf);
        free(qd);
    }
    free(sig);
    return bad ? -1 : 0;
}

/* Two-level (tree) routing (SSA page, "Algorithm and complexity": a
 * hierarchical router with fixed block size and budget, the measured tree
 * at fanout 16; "Complete 10M transformer result": a bounded hierarchical
 * router).  Nodes group F consecutive key blocks; a node's summary is the
 * mean of its F block means (fp64 sum, one fp32 rounding).  For a row with
 * E candidate blocks (causal: E(t); image mode: all nb):
 *   1. the S = floor(E / F) complete candidate nodes are scored <q, nu_s>
 *      and the best min(beam, S) are kept (score desc, index asc);
 *   2. the candidate blocks are those of the kept nodes plus the tail
 *      blocks [F*S, E) of the incomplete node;
 *   3. those blocks are scored <q, mu_c> and the top-k taken as in step 3.
 * With beam >= S every block is a candidate and the result is the flat
 * selection.  Causal: q bf16 [B,Hq,N,D], rows (b*Hq + h)*N + t.  Image
 * mode: qbar fp32 [B,Hq,nb,D], rows (b*Hq + h)*nb + i.  idx [n_rows, k].
 * Optional outputs per row: gap1 (beam-th minus (beam+1)-th node score,
 * +inf when no node is left out), gap2 (k-th minus (k+1)-th score among the
 * candidates), node_scores [n_rows, nb/F] (-inf beyond S), beam_out
 * [n_rows, beam] (kept nodes ascending, -1 padded). */
int orc_route_tree(const uint16_t *q, const float *qbar, const float *kbar,
                   int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D,
                   int64_t bs, int64_t k, int64_t window, int64_t causal,
                   int64_t F, int64_t beam, const int64_t *rows,
                   int64_t n_rows, int32_t *idx, double *gap1, double *gap2,
                   double *node_scores, int32_t *beam_out)
{
    if (!kbar || !idx || bs <= 0 || N % bs || Hkv <= 0 || Hq % Hkv || k <= 0 ||
        F <= 0 || beam <= 0)
        return -1;
    if (causal ? (!q || window < bs || window % bs) : !qbar)
        return -1;
    const int64_t nb = N / bs, rep = Hq / Hkv, nn = nb / F;
    const int64_t per = causal ? N : nb;
    const int64_t total = rows ? n_rows : B * Hq * per;
    float *nu = (float *)malloc(sizeof(float) * (size_t)((B * Hkv * nn > 0 ? B * Hkv * nn : 1) * D));
    if (!nu)
        return -1;
    for (int64_t gs = 0; gs < B * Hkv * nn; ++gs) {
        const int64_t bg = gs / nn, sn = gs % nn;
        for (int64_t d = 0; d < D; ++d) {
            double a = 0.0;
            for (int64_t i = 0; i < F; ++i)
                a += (double)kbar[(bg * nb + sn * F + i) * D + d];
            nu[gs * D + d] = (float)(a / (double)F);
        }
    }
    int bad = 0;
#pragma omp parallel
    {
        cand_t *nbuf = (cand_t *)malloc(sizeof(cand_t) * (size_t)(nn + 1));
        cand_t *cbuf = (cand_t *)malloc(sizeof(cand_t) * (size_t)(nb + 1));
        int32_t *kept = (int32_t *)malloc(sizeof(int32_t) * (size_t)beam);
        double *qd = (double *)malloc(sizeof(double) * (size_t)D);
        if (!nbuf || !cbuf || !kept || !qd) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 32)
        for (int64_t i = 0; i < total; ++i) {
            if (!nbuf || !cbuf || !kept || !qd) continue;
            const int64_t r = rows ? rows[i] : i;
            if (r < 0 || r >= B * Hq * per) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            const int64_t p = r % per, bh = r / per, h = bh % Hq, b = bh / Hq;
            const int64_t bg = b * Hkv + h / rep;
            const int64_t E = causal ? eligible_blocks(p, bs, window) : nb;
            const int64_t S = E / F;
            for (int64_t d = 0; d < D; ++d)
                qd[d] = causal ? bf16_to_f64(q[r * D + d]) : (double)qbar[r * D + d];
            /* level 1: the nodes */
            for (int64_t sn = 0; sn < S; ++sn) {
                double sc = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    sc += qd[d] * (double)nu[(bg * nn + sn) * D + d];
                nbuf[sn].s = sc;
                nbuf[sn].c = sn;
            }
            if (node_scores)
                for (int64_t sn = 0; sn < nn; ++sn)
                    node_scores[i * nn + sn] = sn < S ? nbuf[sn].s : -INFINITY;
            pick_top(nbuf, S, beam, kept, gap1 ? gap1 + i : NULL);
            if (beam_out)
                memcpy(beam_out + i * beam, kept, sizeof(int32_t) * (size_t)beam);
            /* level 2: blocks of the kept nodes, then the tail */
            int64_t nc = 0;
            for (int64_t j = 0; j < beam && kept[j] >= 0; ++j)
                for (int64_t x = 0; x < F; ++x) {
                    cbuf[nc].c = kept[j] * F + x;
                    ++nc;
                }
            for (int64_t c = S * F; c < E; ++c) {
                cbuf[nc].c = c;
                ++nc;
            }
            const float *summ = kbar + bg * nb * D;
            for (int64_t j = 0; j < nc; ++j) {
                double sc = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    sc += qd[d] * (double)summ[cbuf[j].c * D + d];
                cbuf[j].s = sc;
            }
            pick_top(cbuf, nc, k, idx + i * k, gap2 ? gap2 + i : NULL);
        }
        free(nbuf);
        free(cbuf);
        free(kept);
        free(qd);
    }
    free(nu);
    return bad ? -1 : 0;
}

/* Checks one row's selection: entries in [0, ncand), strictly ascending,
 * -1 only as trailing padding.  Returns the number of selected blocks, or
 * -1 when the row is not a valid selection. */
static int64_t check_selection(const int32_t *sel, int64_t k, int64_t ncand)
{
    int64_t n = 0;
    for (int64_t i = 0; i < k; ++i) {
        if (sel[i] < 0) {
            if (sel[i] != -1) return -1;
            continue;
        }
        if (i > 0 && sel[i - 1] < 0) return -1;     /* block after padding */
        if (sel[i] >= ncand) return -1;
        if (i > 0 && sel[i] <= sel[i - 1]) return -1;
        ++n;
    }
    return n;
}

/* Step 4 for one query: softmax over the listed key ranges, fp64. */
static void attend_ranges(const double *qd, const uint16_t *kh,
                          const uint16_t *vh, int64_t D, double scale,
                          const int64_t *lo, const int64_t *hi, int64_t nr,
                          double *acc, float *out)
{
    double m = -INFINITY;
    for (int64_t r = 0; r < nr; ++r)
        for (int64_t j = lo[r]; j < hi[r]; ++j) {
            double l = 0.0;
            for (int64_t d = 0; d < D; ++d)
                l += qd[d] * bf16_to_f64(kh[j * D + d]);
            l *= scale;
            if (l > m) m = l;
        }
    double z = 0.0;
    for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
    for (int64_t r = 0; r < nr; ++r)
        for (int64_t j = lo[r]; j < hi[r]; ++j) {
            double l = 0.0;
            for (int64_t d = 0; d < D; ++d)
                l += qd[d] * bf16_to_f64(kh[j * D + d]);
            const double p = exp(l * scale - m);
            z += p;
            for (int64_t d = 0; d < D; ++d)
                acc[d] += p * bf16_to_f64(vh[j * D + d]);
        }
    for (int64_t d = 0; d < D; ++d)
        out[d] = (float)(acc[d] / z);
}

/* Step 4.  rows: token rows (b*Hq + h)*N + t (NULL = all).  sel: [n_rows, k]
 * selections aligned with rows (image mode: the selection of the row's
 * query block).  out: [n_rows, D].  scale <= 0 means 1/sqrt(D). */
int orc_attend(const uint16_t *q, const uint16_t *kk, const uint16_t *vv,
               int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D,
               int64_t bs, int64_t k, int64_t window, int64_t causal,
               double scale, const int64_t *rows, int64_t n_rows,
               const int32_t *sel, float *out)
{
    if (!q || !kk || !vv || !sel || !out || bs <= 0 || N % bs || Hkv <= 0 ||
        Hq % Hkv || k <= 0)
        return -1;
    if (causal ? (window < bs || window % bs) : window != 0)
        return -1;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
    const int64_t nb = N / bs, rep = Hq / Hkv;
    const int64_t total = rows ? n_rows : B * Hq * N;
    int bad = 0;
#pragma omp parallel
    {
        int64_t *lo = (int64_t *)malloc(sizeof(int64_t) * (size_t)(k + 1));
        int64_t *hi = (int64_t *)malloc(sizeof(int64_t) * (size_t)(k + 1));
        double *qd = (double *)malloc(sizeof(double) * (size_t)D);
        double *acc = (double *)malloc(sizeof(double) * (size_t)D);
        if (!lo || !hi || !qd || !acc) {
#pragma omp atomic write
            bad = -1;
        }
#pragma omp for schedule(dynamic, 32)
        for (int64_t i = 0; i < total; ++i) {
            if (!lo || !hi || !qd || !acc) continue;
            const int64_t r = rows ? rows[i] : i;
            if (r < 0 || r >= B * Hq * N) {
#pragma omp atomic write
                bad = -1;
                continue;
            }
            const int64_t t = r % N, bh = r / N, h = bh % Hq, b = bh / Hq;
            const int64_t kvh = b * Hkv + h / rep;
            const int64_t ncand = causal ? eligible_blocks(t, bs, window) : nb;
            const int32_t *s = sel + i * k;
            const int64_t n = check_selection(s, k, ncand);
            if (n < 0) {
#pragma omp atomic write
                bad = -2;
                continue;
            }
            int64_t nr = 0;
            for (int64_t j = 0; j < n; ++j) {
                lo[nr] = (int64_t)s[j] * bs;
                hi[nr] = lo[nr] + bs;
                ++nr;
            }
            if (causal) {           /* window: keys [bs*E, t] */
                lo[nr] = ncand * bs;
                hi[nr] = t + 1;
                ++nr;
            }
            for (int64_t d = 0; d < D; ++d)
                qd[d] = bf16_to_f64(q[r * D + d]);
            attend_ranges(qd, kk + kvh * N * D, vv + kvh * N * D, D, scale, lo,
                          hi, nr, acc, out + i * D);
        }
        free(lo);
        free(hi);
        free(qd);
        free(acc);
    }
    return bad;
}

/* Steps 1-4 end to end for the given token rows (NULL = all): summaries of
 * every key block (and, in image mode, of every query block), routing of the
 * rows (image mode: of each row's query block), attention.  sel_out
 * (nullable): [n_rows, k] the selection used by each row.  Used to time the
 * oracle as a CPU baseline. */
int orc_forward(const uint16_t *q, const uint16_t *kk, const uint16_t *vv,
                int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D,
                int64_t bs, int64_t k, int64_t window, int64_t causal,
                double scale, const int64_t *rows, int64_t n_rows,
                int32_t *sel_out, float *out)
{
    if (!q || !kk || !vv || !out || bs <= 0 || N % bs || Hkv <= 0 ||
        Hq % Hkv || k <= 0)
        return -1;
    const int64_t nb = N / bs;
    const int64_t total = rows ? n_rows : B * Hq * N;
    int rc = -1;
    float *kbar = (float *)malloc(sizeof(float) * (size_t)(B * Hkv * nb * D));
    float *qbar = causal ? NULL
                         : (float *)malloc(sizeof(float) * (size_t)(B * Hq * nb * D));
    int32_t *sel = sel_out ? sel_out
                           : (int32_t *)malloc(sizeof(int32_t) * (size_t)(total * k));
    /* image mode: each distinct query block is routed once */
    int64_t *slot = causal ? NULL : (int64_t *)malloc(sizeof(int64_t) * (size_t)(B * Hq * nb));
    int64_t *qrows = causal ? NULL : (int64_t *)malloc(sizeof(int64_t) * (size_t)total);
    int32_t *qsel = causal ? NULL : (int32_t *)malloc(sizeof(int32_t) * (size_t)(total * k));
    if (!kbar || !sel || (!causal && (!qbar || !qrows || !slot || !qsel)))
        goto done;
    if ((rc = orc_block_means(kk, B * Hkv, N, D, bs, kbar)) != 0)
        goto done;
    if (causal) {
        rc = orc_route_causal(q, kbar, B, Hq, Hkv, N, D, bs, k, window, rows,
                              total, sel, NULL);
    } else {
        if ((rc = orc_block_means(q, B * Hq, N, D, bs, qbar)) != 0)
            goto done;
        for (int64_t i = 0; i < B * Hq * nb; ++i) slot[i] = -1;
        int64_t nq = 0;
        for (int64_t i = 0; i < total; ++i) {
            const int64_t r = rows ? rows[i] : i;
            if (r < 0 || r >= B * Hq * N) { rc = -1; goto done; }
            const int64_t qb = (r / N) * nb + (r % N) / bs;
            if (slot[qb] < 0) { slot[qb] = nq; qrows[nq++] = qb; }
        }
        rc = orc_route_image(qbar, kbar, B, Hq, Hkv, nb, D, k, qrows, nq,
                             qsel, NULL);
        if (rc != 0)
            goto done;
        for (int64_t i = 0; i < total; ++i) {
            const int64_t r = rows ? rows[i] : i;
            const int64_t s = slot[(r / N) * nb + (r % N) / bs];
            memcpy(sel + i * k, qsel + s * k, sizeof(int32_t) * (size_t)k);
        }
    }
    if (rc != 0)
        goto done;
    rc = orc_attend(q, kk, vv, B, Hq, Hkv, N, D, bs, k, window, causal, scale,
                    rows, total, sel, out);
done:
    free(kbar);
    free(qbar);
    free(slot);
    free(qrows);
    free(qsel);
    if (!sel_out) free(sel);
    return rc;
}
