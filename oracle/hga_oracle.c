/*
 * hga_oracle.c -- plain CPU oracle for the hot path of Hierarchical Global
 * Attention (HGA): chunk summaries -> per-block top-k chunk routing -> exact
 * softmax attention over the routed chunks plus the causal local block, and
 * the gradient of that attention for the active segment.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, obviously correct
 * definition that the GPU library is checked against. Only the tests, the
 * smoke check and the benchmark's CPU-baseline leg load it; the product path
 * never does, and this file shares no code with it.
 *
 * Source: arXiv 2607.15105, "Long-Context Fine-Tuning with Limited VRAM"
 * (gist.science technical summary, section 2.1 "Hierarchical Global
 * Attention", section 2.2 "segment-wise backward"; author abstract).
 *
 * Precision: inputs are float32 arrays (bf16 workloads pass the widened bf16
 * values); every sum, dot product and exponential is taken in double, in
 * plain ascending index order. Outputs are double.
 *
 * The same functions serve the second routing level, 8-token groups inside
 * the chosen chunks: oracle_summarize with C = 8 gives group summaries,
 * oracle_route_groups keeps the best groups of the routed chunks, and the
 * attention functions take group ids with C = 8 (the query block stays Bq).
 *
 * Readings of points the pages leave open (each is listed with its reason in
 * the design notes of this repository):
 *   - summary of a chunk = arithmetic mean of its C key vectors (keys only);
 *   - the query block scores with the mean of its queries over all query
 *     heads that share one key/value head (routing per block and kv head);
 *   - score = plain dot product, ranking by (score desc, chunk id asc);
 *   - candidates = every closed chunk that ends at or before the block's
 *     first query position; fewer than k candidates -> take all, pad with -1;
 *   - local window = the query block itself under the causal mask;
 *   - no sink tokens and no 8-token group level (whole chunks are attended);
 *   - softmax scale = 1/sqrt(D) unless given; lse is the natural log;
 *   - gradients flow only into the active segment's keys/values (history is
 *     detached) and never through the routing decision.
 *
 * Parallelism: OpenMP over independent output rows only; the arithmetic of
 * each output element is the same sequential loop whatever the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ threads */

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_get_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------- summarize
 * Chunk summary (technical summary 2.1, chunk selection: one compact summary
 * vector per closed fixed-size chunk, kept resident):
 *     S[g][c][d] = (1/C) * sum_{t = cC}^{cC + C - 1} K[g][t][d]
 * K is [Hkv][T][D]; S is [Hkv][n_cap][D]; rows c_begin .. c_end-1 are written.
 */
void oracle_summarize(const float *K, int64_t Hkv, int64_t T, int64_t D,
                      int64_t C, int64_t c_begin, int64_t c_end,
                      double *S, int64_t n_cap)
{
    (void)T;
    int64_t n_rows = Hkv * (c_end - c_begin);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t g = r / (c_end - c_begin);
        int64_t c = c_begin + r % (c_end - c_begin);
        for (int64_t d = 0; d < D; ++d) {
            double sum = 0.0;
            for (int64_t t = c * C; t < c * C + C; ++t)
                sum += (double)K[(g * T + t) * D + d];
            S[(g * n_cap + c) * D + d] = sum / (double)C;
        }
    }
}

/* -------------------------------------------------------------------- route
 * Chunk routing (technical summary 2.1: the current query block scores the
 * resident summaries and keeps the most relevant historical chunks; the
 * selection carries no gradient).
 *
 * For kv head g and query block b (first query at absolute position
 * P = p0 + b*Bq):
 *     qbar[d]  = mean over the G query heads h of group g and the Bq queries i
 *                of block b of Q[h][i][d]
 *     E        = { c : sink <= c * C, (c + 1) * C <= P }   closed, causally
 *                earlier, not in the sink window (the first `sink` tokens,
 *                which every block attends anyway; a multiple of C)
 *     sigma_c  = sum_d qbar[d] * S[g][c][d]
 *     keep the first min(k, |E|) chunks of E ordered by (sigma desc, c asc),
 *     write them in ascending id order, pad with -1.
 * ids is [Hkv][n_blocks][k]. If sigma_out is not NULL it receives
 * sigma_c for every c < n_cap as [Hkv][n_blocks][n_cap] (NaN for c not in E).
 *
 * Two routing variants (the pages fix neither the head granularity of the
 * query block's score nor a causal form of it; both are readings of this
 * repository, next to the default above):
 *   per_q_head != 0  one routing unit per query head h instead of per kv
 *                    head: qbar is the mean over the Bq queries of head h
 *                    alone, scored against the summaries of its kv head
 *                    h / G; ids (and sigma_out) are then [Hq][n_blocks][...].
 *   prev_block != 0  strictly causal routing: block b scores with the queries
 *                    of the block before it (positions P - Bq .. P - 1): rows
 *                    (b-1)*Bq .. b*Bq - 1 of Q for b >= 1, and the Bq rows of
 *                    Q_prev ([Hq][Bq][D], the queries just before p0) for
 *                    b = 0; Q_prev may be NULL when p0 = 0 (block 0 then has
 *                    no candidates). The candidates are unchanged.
 */
typedef struct { double sigma; int64_t c; } scored_chunk;

static int by_score_desc_then_id(const void *pa, const void *pb)
{
    const scored_chunk *a = (const scored_chunk *)pa;
    const scored_chunk *b = (const scored_chunk *)pb;
    if (a->sigma > b->sigma) return -1;
    if (a->sigma < b->sigma) return 1;
    return (a->c < b->c) ? -1 : (a->c > b->c);
}

static int by_id_asc(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

void oracle_route(const float *Q, int64_t Hq, int64_t Hkv, int64_t n_q,
                  int64_t D, int64_t p0, int64_t C, int64_t Bq,
                  const double *S, int64_t n_cap, int64_t k,
                  int32_t *ids, double *sigma_out, int64_t sink,
                  int64_t per_q_head, const float *Q_prev, int64_t prev_block)
{
    int64_t G = Hq / Hkv;
    int64_t n_blocks = n_q / Bq;
    int64_t n_units = per_q_head ? Hq : Hkv;        /* routing units per block */
    int64_t heads = per_q_head ? 1 : G;             /* query heads per unit */
#pragma omp parallel for schedule(dynamic)
    for (int64_t u = 0; u < n_units * n_blocks; ++u) {
        int64_t g = u / n_blocks, b = u % n_blocks;
        int64_t kv = per_q_head ? g / G : g;        /* summaries of this kv head */
        int64_t P = p0 + b * Bq;
        int64_t c_hi = P / C;               /* chunks c with (c+1)*C <= P */
        if (c_hi > n_cap) c_hi = n_cap;
        int64_t c_lo = (sink + C - 1) / C;  /* first chunk past the sink */
        int64_t nE = c_hi > c_lo ? c_hi - c_lo : 0;

        /* the Bq query rows this block scores with: its own, or the block's
           before it (from Q_prev for the first block) */
        const float *Qr = Q;
        int64_t r_n = n_q, r_first = b * Bq;
        if (prev_block) {
            if (b > 0) {
                r_first = (b - 1) * Bq;
            } else {
                Qr = Q_prev;
                r_n = Bq;
                r_first = 0;
            }
        }
        double *qbar = (double *)malloc((size_t)D * sizeof(double));
        for (int64_t d = 0; d < D; ++d) {
            double sum = 0.0;
            if (Qr)
                for (int64_t h = g * heads; h < g * heads + heads; ++h)
                    for (int64_t i = r_first; i < r_first + Bq; ++i)
                        sum += (double)Qr[(h * r_n + i) * D + d];
            qbar[d] = sum / (double)(heads * Bq);
        }

        scored_chunk *cand = (scored_chunk *)malloc((size_t)(nE > 0 ? nE : 1) * sizeof(scored_chunk));
        for (int64_t e = 0; e < nE; ++e) {
            int64_t c = c_lo + e;
            double sigma = 0.0;
            for (int64_t d = 0; d < D; ++d)
                sigma += qbar[d] * S[(kv * n_cap + c) * D + d];
            cand[e].sigma = sigma;
            cand[e].c = c;
        }
        if (sigma_out) {
            double *row = sigma_out + (g * n_blocks + b) * n_cap;
            for (int64_t c = 0; c < n_cap; ++c) row[c] = NAN;
            for (int64_t e = 0; e < nE; ++e) row[cand[e].c] = cand[e].sigma;
        }

        qsort(cand, (size_t)nE, sizeof(scored_chunk), by_score_desc_then_id);
        int64_t take = nE < k ? nE : k;
        int32_t *out = ids + (g * n_blocks + b) * k;
        for (int64_t r = 0; r < take; ++r) out[r] = (int32_t)cand[r].c;
        qsort(out, (size_t)take, sizeof(int32_t), by_id_asc);
        for (int64_t r = take; r < k; ++r) out[r] = -1;

        free(cand);
        free(qbar);
    }
}

/* -------------------------------------------------------------- route groups
 * Group routing, the second routing level (technical summary 2.1, group
 * selection: the chosen chunks are split into smaller groups, e.g. 8 tokens,
 * whose summaries the router scores to keep the best groups inside the chosen
 * chunks; exact attention then covers the tokens of the kept groups).
 *
 * With U tokens per group (C % U == 0) and group summaries SG[g][u] = mean of
 * the U keys of group u (oracle_summarize with C = U), for kv head g and query
 * block b (qbar as in oracle_route):
 *     Ch       = the chunk ids of chunk_ids[g][b] with sink <= c*C and
 *                c < P/C, as a set (chunks of the sink window are attended
 *                whole anyway)
 *     cand     = { u : u / (C/U) in Ch }              the groups of those chunks
 *     sigma_u  = sum_d qbar[d] * SG[g][u][d]
 *     keep the first min(m, |cand|) groups ordered by (sigma desc, u asc),
 *     write them in ascending id order, pad with -1.
 * chunk_ids is [Hkv][n_blocks][k]; gids is [Hkv][n_blocks][m]. If sigma_out is
 * not NULL it receives sigma_u for every u < n_gcap as
 * [Hkv][n_blocks][n_gcap] (NaN for groups that are not candidates).
 */
void oracle_route_groups(const float *Q, int64_t Hq, int64_t Hkv, int64_t n_q,
                         int64_t D, int64_t p0, int64_t C, int64_t Bq, int64_t U,
                         const double *SG, int64_t n_gcap,
                         const int32_t *chunk_ids, int64_t k, int64_t m,
                         int32_t *gids, double *sigma_out, int64_t sink)
{
    int64_t G = Hq / Hkv;
    int64_t n_blocks = n_q / Bq;
    int64_t per = C / U;                    /* groups per chunk */
#pragma omp parallel for schedule(dynamic)
    for (int64_t w = 0; w < Hkv * n_blocks; ++w) {
        int64_t g = w / n_blocks, b = w % n_blocks;
        int64_t P = p0 + b * Bq;

        double *qbar = (double *)malloc((size_t)D * sizeof(double));
        for (int64_t d = 0; d < D; ++d) {
            double sum = 0.0;
            for (int64_t h = g * G; h < g * G + G; ++h)
                for (int64_t i = b * Bq; i < b * Bq + Bq; ++i)
                    sum += (double)Q[(h * n_q + i) * D + d];
            qbar[d] = sum / (double)(G * Bq);
        }

        /* the distinct valid chunks of the row, in any order */
        const int32_t *row = chunk_ids + (g * n_blocks + b) * k;
        int64_t *chs = (int64_t *)malloc((size_t)(k > 0 ? k : 1) * sizeof(int64_t));
        int64_t n_ch = 0;
        for (int64_t r = 0; r < k; ++r) {
            int64_t c = row[r];
            if (c < 0 || c >= P / C || c * C < sink) continue;
            int dup = 0;
            for (int64_t q = 0; q < n_ch; ++q) dup |= chs[q] == c;
            if (!dup) chs[n_ch++] = c;
        }

        int64_t n_cand = n_ch * per;
        scored_chunk *cand = (scored_chunk *)malloc((size_t)(n_cand > 0 ? n_cand : 1) * sizeof(scored_chunk));
        for (int64_t q = 0; q < n_ch; ++q)
            for (int64_t j = 0; j < per; ++j) {
                int64_t u = chs[q] * per + j;
                double sigma = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    sigma += qbar[d] * SG[(g * n_gcap + u) * D + d];
                cand[q * per + j].sigma = sigma;
                cand[q * per + j].c = u;
            }
        if (sigma_out) {
            double *srow = sigma_out + (g * n_blocks + b) * n_gcap;
            for (int64_t u = 0; u < n_gcap; ++u) srow[u] = NAN;
            for (int64_t q = 0; q < n_cand; ++q)
                if (cand[q].c < n_gcap) srow[cand[q].c] = cand[q].sigma;
        }

        qsort(cand, (size_t)n_cand, sizeof(scored_chunk), by_score_desc_then_id);
        int64_t take = n_cand < m ? n_cand : m;
        int32_t *out = gids + (g * n_blocks + b) * m;
        for (int64_t r = 0; r < take; ++r) out[r] = (int32_t)cand[r].c;
        qsort(out, (size_t)take, sizeof(int32_t), by_id_asc);
        for (int64_t r = take; r < m; ++r) out[r] = -1;

        free(cand);
        free(chs);
        free(qbar);
    }
}

/* ---------------------------------------------------------- attended set A(i)
 * Exact-token attention (technical summary 2.1: only the exact K/V of the
 * selected units enter attention; summaries are never attention values).
 * For active query i (absolute position p = p0 + i) in block b = i / Bq with
 * first position P = p0 + b*Bq and kv head g:
 *     A(i) = [0, min(sink, P))                        the sink window
 *            united with the listed units c with 0 <= c < P/C of [cC, cC + C)
 *            united with the causal local block [P, p].
 * The listed units are taken as a set (a repeated id adds nothing), and a unit
 * inside the sink window adds nothing either (sink is a multiple of C).
 * Returns the number of positions written to pos (ascending within each part).
 */
static int64_t attended_positions(const int32_t *ids_gb, int64_t k, int64_t C,
                                  int64_t P, int64_t p, int64_t *pos,
                                  unsigned char *seen, int64_t n_seen, int64_t sink)
{
    int64_t n = 0;
    for (int64_t t = 0; t < sink && t < P; ++t) pos[n++] = t;
    memset(seen, 0, (size_t)n_seen);
    for (int64_t r = 0; r < k; ++r) {
        int64_t c = ids_gb[r];
        if (c < 0 || c >= P / C || c >= n_seen || c * C < sink || seen[c]) continue;
        seen[c] = 1;
    }
    for (int64_t c = 0; c < n_seen; ++c)
        if (seen[c])
            for (int64_t t = c * C; t < c * C + C; ++t) pos[n++] = t;
    for (int64_t t = P; t <= p; ++t) pos[n++] = t;
    return n;
}

static int is_attended(const int32_t *ids_gb, int64_t k, int64_t C,
                       int64_t P, int64_t p, int64_t j, int64_t sink)
{
    if (j >= P) return j <= p;
    if (j < sink) return 1;
    int64_t c = j / C;
    if (c >= P / C) return 0;
    for (int64_t r = 0; r < k; ++r)
        if (ids_gb[r] == c) return 1;
    return 0;
}

static double dot_fd(const float *a, const float *b, int64_t D)
{
    double s = 0.0;
    for (int64_t d = 0; d < D; ++d) s += (double)a[d] * (double)b[d];
    return s;
}

/* --------------------------------------------------------------- attend fwd
 * For every active query i of query head h (kv head g = h / G):
 *     z_j   = scale * Q[h][i] . K[g][j]           j in A(i)
 *     m     = max_j z_j
 *     l     = sum_j exp(z_j - m)
 *     O[h][i] = (sum_j exp(z_j - m) V[g][j]) / l
 *     lse[h][i] = m + ln l
 * unit_mask ([Hq][n_blocks], may be NULL) limits the work to chosen
 * (head, block) units; other rows of O/lse are left untouched.
 * per_q_head != 0: ids is [Hq][n_blocks][k] and query head h attends the
 * chunks of its own row ids[h][b] (per-query-head routing); otherwise row
 * ids[h / G][b] serves all G heads of a kv head.
 */
void oracle_attend_fwd(const float *Q, const float *K, const float *V,
                       int64_t Hq, int64_t Hkv, int64_t D, int64_t T,
                       int64_t p0, int64_t n_q, int64_t C, int64_t Bq,
                       const int32_t *ids, int64_t k, double scale,
                       const uint8_t *unit_mask, double *O, double *lse, int64_t sink,
                       int64_t per_q_head)
{
    int64_t G = Hq / Hkv;
    int64_t n_blocks = n_q / Bq;
    int64_t n_chunks = T / C;
#pragma omp parallel
    {
        int64_t *pos = (int64_t *)malloc((size_t)(T + 1) * sizeof(int64_t));
        double *z = (double *)malloc((size_t)(T + 1) * sizeof(double));
        double *acc = (double *)malloc((size_t)D * sizeof(double));
        unsigned char *seen = (unsigned char *)malloc((size_t)n_chunks + 1);
#pragma omp for schedule(dynamic)
        for (int64_t row = 0; row < Hq * n_q; ++row) {
            int64_t h = row / n_q, i = row % n_q;
            int64_t b = i / Bq, g = h / G;
            if (unit_mask && !unit_mask[h * n_blocks + b]) continue;
            int64_t P = p0 + b * Bq, p = p0 + i;
            const int32_t *ids_gb = ids + ((per_q_head ? h : g) * n_blocks + b) * k;
            int64_t n = attended_positions(ids_gb, k, C, P, p, pos, seen, n_chunks, sink);
            const float *q = Q + (h * n_q + i) * D;

            double m = -INFINITY;
            for (int64_t a = 0; a < n; ++a) {
                z[a] = scale * dot_fd(q, K + (g * T + pos[a]) * D, D);
                if (z[a] > m) m = z[a];
            }
            double l = 0.0;
            for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
            for (int64_t a = 0; a < n; ++a) {
                double e = exp(z[a] - m);
                l += e;
                const float *v = V + (g * T + pos[a]) * D;
                for (int64_t d = 0; d < D; ++d) acc[d] += e * (double)v[d];
            }
            for (int64_t d = 0; d < D; ++d) O[(h * n_q + i) * D + d] = acc[d] / l;
            lse[h * n_q + i] = m + log(l);
        }
        free(seen); free(acc); free(z); free(pos);
    }
}

/* --------------------------------------------------------------- attend bwd
 * Gradient of the attention above for an upstream gradient dO, with the
 * routed ids held constant (no gradient through routing) and every key/value
 * before p0 detached (segment-wise backward, technical summary 2.2):
 *     P_ij   = exp(z_j - lse_i)
 *     Delta_i = sum_j P_ij dO_i . V_j  ( = dO_i . O_i )
 *     dS_ij  = P_ij (dO_i . V_j - Delta_i)
 *     dQ_i   = scale * sum_{j in A(i)} dS_ij K_j
 *     dK_j   = scale * sum_{(h,i) : j in A(i)} dS_ij Q_i      p0 <= j < p0+n_q
 *     dV_j   =         sum_{(h,i) : j in A(i)} P_ij dO_i      p0 <= j < p0+n_q
 * dQ is [Hq][n_q][D]; dK, dV are [Hkv][n_q][D] indexed by j - p0.
 * dq_mask ([Hq][n_blocks]) and dkv_mask ([Hkv][n_q/C]) may be NULL; masked-out
 * rows are left untouched. lse and O are recomputed here from Q, K, V.
 * per_q_head: the id rows as in oracle_attend_fwd.
 */
void oracle_attend_bwd(const float *Q, const float *K, const float *V,
                       const float *dO,
                       int64_t Hq, int64_t Hkv, int64_t D, int64_t T,
                       int64_t p0, int64_t n_q, int64_t C, int64_t Bq,
                       const int32_t *ids, int64_t k, double scale,
                       const uint8_t *dq_mask, const uint8_t *dkv_mask,
                       double *dQ, double *dK, double *dV, int64_t sink, int64_t per_q_head)
{
    int64_t G = Hq / Hkv;
    int64_t n_blocks = n_q / Bq;
    int64_t n_chunks = T / C;
    double *lse = (double *)malloc((size_t)(Hq * n_q) * sizeof(double));
    double *Obuf = (double *)malloc((size_t)(Hq * n_q * D) * sizeof(double));
    double *Delta = (double *)malloc((size_t)(Hq * n_q) * sizeof(double));

    /* pass 1: lse, O and Delta for every active query */
    oracle_attend_fwd(Q, K, V, Hq, Hkv, D, T, p0, n_q, C, Bq, ids, k, scale,
                      NULL, Obuf, lse, sink, per_q_head);
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < Hq * n_q; ++row) {
        double s = 0.0;
        for (int64_t d = 0; d < D; ++d)
            s += (double)dO[row * D + d] * Obuf[row * D + d];
        Delta[row] = s;
    }

    /* pass 2: dQ, query by query over its attended set */
#pragma omp parallel
    {
        int64_t *pos = (int64_t *)malloc((size_t)(T + 1) * sizeof(int64_t));
        double *acc = (double *)malloc((size_t)D * sizeof(double));
        unsigned char *seen = (unsigned char *)malloc((size_t)n_chunks + 1);
#pragma omp for schedule(dynamic)
        for (int64_t row = 0; row < Hq * n_q; ++row) {
            int64_t h = row / n_q, i = row % n_q;
            int64_t b = i / Bq, g = h / G;
            if (dq_mask && !dq_mask[h * n_blocks + b]) continue;
            int64_t P = p0 + b * Bq, p = p0 + i;
            const int32_t *ids_gb = ids + ((per_q_head ? h : g) * n_blocks + b) * k;
            int64_t n = attended_positions(ids_gb, k, C, P, p, pos, seen, n_chunks, sink);
            const float *q = Q + row * D;
            const float *go = dO + row * D;
            for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
            for (int64_t a = 0; a < n; ++a) {
                const float *kj = K + (g * T + pos[a]) * D;
                const float *vj = V + (g * T + pos[a]) * D;
                double Pij = exp(scale * dot_fd(q, kj, D) - lse[row]);
                double dS = Pij * (dot_fd(go, vj, D) - Delta[row]);
                for (int64_t d = 0; d < D; ++d) acc[d] += dS * (double)kj[d];
            }
            for (int64_t d = 0; d < D; ++d) dQ[row * D + d] = scale * acc[d];
        }
        free(seen); free(acc); free(pos);
    }

    /* pass 3: dK, dV, key by key over every (head, query) that attends it */
#pragma omp parallel
    {
        double *ak = (double *)malloc((size_t)D * sizeof(double));
        double *av = (double *)malloc((size_t)D * sizeof(double));
#pragma omp for schedule(dynamic)
        for (int64_t kr = 0; kr < Hkv * n_q; ++kr) {
            int64_t g = kr / n_q, jj = kr % n_q, j = p0 + jj;
            if (dkv_mask && !dkv_mask[g * (n_q / C) + jj / C]) continue;
            const float *kj = K + (g * T + j) * D;
            const float *vj = V + (g * T + j) * D;
            for (int64_t d = 0; d < D; ++d) { ak[d] = 0.0; av[d] = 0.0; }
            for (int64_t h = g * G; h < g * G + G; ++h) {
                for (int64_t i = 0; i < n_q; ++i) {
                    int64_t b = i / Bq, P = p0 + b * Bq, p = p0 + i;
                    const int64_t row_u = per_q_head ? h : g;
                    if (!is_attended(ids + (row_u * n_blocks + b) * k, k, C, P, p, j, sink))
                        continue;
                    int64_t row = h * n_q + i;
                    const float *q = Q + row * D;
                    const float *go = dO + row * D;
                    double Pij = exp(scale * dot_fd(q, kj, D) - lse[row]);
                    double dS = Pij * (dot_fd(go, vj, D) - Delta[row]);
                    for (int64_t d = 0; d < D; ++d) {
                        ak[d] += dS * (double)q[d];
                        av[d] += Pij * (double)go[d];
                    }
                }
            }
            for (int64_t d = 0; d < D; ++d) {
                dK[kr * D + d] = scale * ak[d];
                dV[kr * D + d] = av[d];
            }
        }
        free(av); free(ak);
    }
    free(Delta); free(Obuf); free(lse);
}

/* ------------------------------------------------------------- attend decode
 * Routed generation (technical summary 2.1 applied to one token at a time; the
 * pages note the method also serves generation). Token i of a decode step
 * sits at position p = p0 + i (p0 need not be a multiple of C); its local
 * window is the part of its own, still open chunk up to p, and it routes on
 * its own (ids [Hkv][n_q][k], e.g. oracle_route with Bq = 1):
 *     Pc   = C * floor(p / C)                      start of the open chunk
 *     A(p) = [0, min(sink, Pc))  U  union_{c in ids[g][i], sink <= cC, c < Pc/C}
 *            [cC, cC + C)  U  [Pc, p]
 * and O, lse as in oracle_attend_fwd. For a block of 64 queries starting a
 * chunk this is the prefill definition itself.
 */
void oracle_attend_decode(const float *Q, const float *K, const float *V,
                          int64_t Hq, int64_t Hkv, int64_t D, int64_t T,
                          int64_t p0, int64_t n_q, int64_t C,
                          const int32_t *ids, int64_t k, double scale, int64_t sink,
                          double *O, double *lse)
{
    int64_t G = Hq / Hkv;
    int64_t n_chunks = T / C;
#pragma omp parallel
    {
        int64_t *pos = (int64_t *)malloc((size_t)(T + 1) * sizeof(int64_t));
        double *z = (double *)malloc((size_t)(T + 1) * sizeof(double));
        double *acc = (double *)malloc((size_t)D * sizeof(double));
        unsigned char *seen = (unsigned char *)malloc((size_t)n_chunks + 1);
#pragma omp for schedule(dynamic)
        for (int64_t row = 0; row < Hq * n_q; ++row) {
            int64_t h = row / n_q, i = row % n_q, g = h / G;
            int64_t p = p0 + i, Pc = C * (p / C);
            int64_t n = 0;
            for (int64_t t = 0; t < sink && t < Pc; ++t) pos[n++] = t;
            memset(seen, 0, (size_t)n_chunks + 1);
            const int32_t *row_ids = ids + (g * n_q + i) * k;
            for (int64_t r = 0; r < k; ++r) {
                int64_t c = row_ids[r];
                if (c < 0 || c >= Pc / C || c * C < sink || seen[c]) continue;
                seen[c] = 1;
            }
            for (int64_t c = 0; c < n_chunks; ++c)
                if (seen[c])
                    for (int64_t t = c * C; t < c * C + C; ++t) pos[n++] = t;
            for (int64_t t = Pc; t <= p; ++t) pos[n++] = t;

            const float *q = Q + row * D;
            double m = -INFINITY;
            for (int64_t a = 0; a < n; ++a) {
                z[a] = scale * dot_fd(q, K + (g * T + pos[a]) * D, D);
                if (z[a] > m) m = z[a];
            }
            double l = 0.0;
            for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
            for (int64_t a = 0; a < n; ++a) {
                double e = exp(z[a] - m);
                l += e;
                const float *vj = V + (g * T + pos[a]) * D;
                for (int64_t d = 0; d < D; ++d) acc[d] += e * (double)vj[d];
            }
            for (int64_t d = 0; d < D; ++d) O[row * D + d] = acc[d] / l;
            lse[row] = m + log(l);
        }
        free(seen); free(acc); free(z); free(pos);
    }
}
