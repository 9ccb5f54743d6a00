/*
 * oasis_oracle.c -- plain, slow CPU oracle of the OasisKV decode hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library may include,
 * link or call this file; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no code, header, table or
 * helper with the HIP path and works on the un-paged logical layout
 * (keys and values of one (sequence, KV head) row as [ctx][D] arrays), so it
 * never sees the page table that the GPU path has to get right.
 *
 * All arithmetic is IEEE double.  Inputs arrive as doubles (the caller widens
 * bf16 or fp32 values exactly).
 *
 * Sources (the pages of "OasisKV: Scaling In-Decode KV Cache Beyond HBM with
 * Lookahead Sparse Prefetching", arXiv 2608.08097):
 *   - abstract: only the KV of the most relevant tokens stays in HBM; a
 *     lookahead (draft) token predicts the blocks the next step needs; they
 *     are prefetched before the next decode step; 2,048-token KV budget.
 *   - metalmedia.ai summary, five-step flow, step 3: the prediction is
 *     compared with the blocks already on the GPU, only the missing ones are
 *     pulled, with a per-step upper bound on the transfer.
 *   - same page, Figure 7 caption: block-wise sparsification into a working
 *     set; the draft query scans keys to predict the next step's top-K blocks;
 *     attention runs over the sparse working set.
 *   - same page, Figure 9 caption: per-KV-head table from GPU working-set
 *     block to CPU logical block.
 *   - same page, Table 2 caption: the cap bounds the blocks fetched per step
 *     by a fetch ratio; LRU eviction.
 *   - same page, glossary entry on capped eviction: only as many blocks may be
 *     newly pulled per step as the compute window allows.
 * The pages do not give the block score.  This library fixes it as the exact
 * maximum, over the block's valid tokens and over every lookahead query row of
 * the KV head's query group, of q.k / sqrt(D).  Readings of the points the
 * pages leave open are stated at each function.
 *
 * Parity pins: every function here is checked in tests/test_oracle_*.py
 * against hand-worked examples, closed forms, library routines on special
 * cases and brute-force enumeration on tiny rows.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <limits.h>

#define ORC_OK 0
#define ORC_EINVAL 1
#define ORC_ENOMEM 3

/* ------------------------------------------------------------------------ */
/* Block score (Figure 7 caption: the draft query scans the keys to predict
 * the next step's top-K blocks; score rule fixed by this library).
 *
 *   scores[n] = max over lookahead rows j < n_q and tokens t of block n with
 *               t < ctx  of  (sum_d q[j][d] * k[t][d]) / sqrt(D)
 *   scores[n] = -inf for nb <= n < W, where nb = ceil(ctx / bs).
 *
 * q: [n_q][D] -- all lookahead query vectors of the row's group (every draft,
 *    every query head of the KV head's GQA group).
 * k: [ctx][D] -- the row's keys in token order.                              */
int oracle_score_row(int ctx, int D, int bs, int n_q, const double *q,
                     const double *k, int W, double *scores)
{
    if (ctx < 0 || D <= 0 || bs <= 0 || n_q <= 0 || W < 0) return ORC_EINVAL;
    int nb = (ctx + bs - 1) / bs;
    if (nb > W) return ORC_EINVAL;
    double inv_sqrt_d = 1.0 / sqrt((double)D);
    for (int n = 0; n < W; ++n) {
        if (n >= nb) { scores[n] = -INFINITY; continue; }
        double best = -INFINITY;
        int t_end = (n + 1) * bs < ctx ? (n + 1) * bs : ctx;
        for (int t = n * bs; t < t_end; ++t) {
            for (int j = 0; j < n_q; ++j) {
                double dot = 0.0;
                for (int d = 0; d < D; ++d) dot += q[(size_t)j * D + d] * k[(size_t)t * D + d];
                double logit = dot * inv_sqrt_d;
                if (logit > best) best = logit;
            }
        }
        scores[n] = best;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Top-K selection (Figure 7 caption: "top-K blocks"; abstract: a 2,048-token
 * budget, i.e. K = budget / block size blocks per KV head).
 * Readings: only blocks n < nb compete; order by score descending and, for
 * equal scores, by block index ascending; the first min(K, nb) win; the set is
 * written in ascending block order and padded with -1 up to K.              */
typedef struct { double s; int n; } scored_block;

static int cmp_score_desc_index_asc(const void *a, const void *b)
{
    const scored_block *x = (const scored_block *)a, *y = (const scored_block *)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->n > y->n) - (x->n < y->n);
}

static int cmp_int_asc(const void *a, const void *b)
{
    int x = *(const int *)a, y = *(const int *)b;
    return (x > y) - (x < y);
}

int oracle_select_row(int nb, int K, const double *scores, int *sel)
{
    if (nb < 0 || K < 0) return ORC_EINVAL;
    scored_block *all = (scored_block *)malloc(sizeof(scored_block) * (size_t)(nb > 0 ? nb : 1));
    if (!all) return ORC_ENOMEM;
    for (int n = 0; n < nb; ++n) { all[n].s = scores[n]; all[n].n = n; }
    qsort(all, (size_t)nb, sizeof(scored_block), cmp_score_desc_index_asc);
    int m = nb < K ? nb : K;
    for (int i = 0; i < m; ++i) sel[i] = all[i].n;
    qsort(sel, (size_t)m, sizeof(int), cmp_int_asc);
    for (int i = m; i < K; ++i) sel[i] = -1;
    free(all);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Resident diff, fetch cap and capped LRU eviction for one row
 * (five-step flow step 3; Figure 9 caption; Table 2 caption; glossary entry
 * on capped eviction).
 *
 * State: slot_block[K] (block held by each working-set slot, -1 = empty) and
 * last_use[K] (step at which the slot's block was last used).
 * Readings of what the pages leave open:
 *   - a block is "used" at a step when it is selected and already resident
 *     (a hit) or when it is fetched;
 *   - misses M = selected blocks not resident; when more than `cap` miss, the
 *     highest-scoring ones are fetched (ties to the lower block index);
 *   - the fetched set F goes out in ascending block order;
 *   - destinations: empty slots in ascending order first; if F needs more,
 *     evict exactly that many resident blocks that are NOT selected, least
 *     recently used first (ties to the lower block index, then to the lower
 *     slot), in that order;
 *   - a selected block is never evicted.
 * Outputs fetch_block[i] = F[i], fetch_slot[i] = its slot, -1 padded to cap.
 * Returns |F| through *count.                                               */
typedef struct { int key; int n; int slot; } lru_cand;

static int cmp_lru(const void *a, const void *b)
{
    const lru_cand *x = (const lru_cand *)a, *y = (const lru_cand *)b;
    if (x->key != y->key) return (x->key > y->key) - (x->key < y->key);
    if (x->n != y->n) return (x->n > y->n) - (x->n < y->n);
    /* one block resident in two slots (a table no plan produces, but one a
       caller may pass): the lower slot goes first */
    return (x->slot > y->slot) - (x->slot < y->slot);
}

static int in_list(int v, const int *list, int len)
{
    for (int i = 0; i < len; ++i) if (list[i] == v) return 1;
    return 0;
}

int oracle_plan_row(int K, int cap, int step, const int *sel, const double *scores,
                    int *slot_block, int *last_use, int *fetch_block, int *fetch_slot,
                    int *count)
{
    if (K < 0 || cap < 0) return ORC_EINVAL;
    int kk = K > 0 ? K : 1;
    int *T = (int *)malloc(sizeof(int) * (size_t)kk);
    scored_block *M = (scored_block *)malloc(sizeof(scored_block) * (size_t)kk);
    int *F = (int *)malloc(sizeof(int) * (size_t)kk);
    int *dest = (int *)malloc(sizeof(int) * (size_t)kk);
    lru_cand *cand = (lru_cand *)malloc(sizeof(lru_cand) * (size_t)kk);
    if (!T || !M || !F || !dest || !cand) {
        free(T); free(M); free(F); free(dest); free(cand);
        return ORC_ENOMEM;
    }

    /* T: the selected set. */
    int nT = 0;
    for (int i = 0; i < K; ++i) if (sel[i] >= 0) T[nT++] = sel[i];

    /* Hits refresh their slot's last use. */
    for (int j = 0; j < K; ++j)
        if (slot_block[j] >= 0 && in_list(slot_block[j], T, nT)) last_use[j] = step;

    /* Misses, ranked by (score desc, index asc); F = the first cap, ascending. */
    int nM = 0;
    for (int i = 0; i < nT; ++i)
        if (!in_list(T[i], slot_block, K)) { M[nM].s = scores[T[i]]; M[nM].n = T[i]; ++nM; }
    qsort(M, (size_t)nM, sizeof(scored_block), cmp_score_desc_index_asc);
    int nF = nM < cap ? nM : cap;
    for (int i = 0; i < nF; ++i) F[i] = M[i].n;
    qsort(F, (size_t)nF, sizeof(int), cmp_int_asc);

    /* Destinations: empty slots ascending, then LRU victims among the
     * resident blocks that were not selected. */
    int nd = 0;
    for (int j = 0; j < K && nd < nF; ++j) if (slot_block[j] < 0) dest[nd++] = j;
    if (nd < nF) {
        int nc = 0;
        for (int j = 0; j < K; ++j)
            if (slot_block[j] >= 0 && !in_list(slot_block[j], T, nT)) {
                cand[nc].key = last_use[j]; cand[nc].n = slot_block[j]; cand[nc].slot = j; ++nc;
            }
        qsort(cand, (size_t)nc, sizeof(lru_cand), cmp_lru);
        for (int i = 0; i < nc && nd < nF; ++i) dest[nd++] = cand[i].slot;
    }
    if (nd < nF) { /* cannot happen for a valid state; report it */
        free(T); free(M); free(F); free(dest); free(cand);
        return ORC_EINVAL;
    }

    for (int i = 0; i < nF; ++i) {
        slot_block[dest[i]] = F[i];
        last_use[dest[i]] = step;
        fetch_block[i] = F[i];
        fetch_slot[i] = dest[i];
    }
    for (int i = nF; i < cap; ++i) { fetch_block[i] = -1; fetch_slot[i] = -1; }
    *count = nF;
    free(T); free(M); free(F); free(dest); free(cand);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Sparse decode attention over the working set (Figure 7 caption: attention
 * runs over the sparse KV working set).
 *
 * For each query head h of the group: softmax over every valid token t
 * (t < ctx) of the listed blocks of q_h.k_t / sqrt(D), then the weighted sum
 * of v_t.  blocks[i] < 0 marks an empty slot.  With no token at all the
 * output is zero (reading: the pages never reach that case).
 * q: [G][D]; k, v: [ctx][D]; out: [G][D].                                   */
int oracle_attn_row(int G, int D, int bs, int ctx, const double *q, const double *k,
                    const double *v, int n_blk, const int *blocks, double *out)
{
    if (G <= 0 || D <= 0 || bs <= 0 || ctx < 0 || n_blk < 0) return ORC_EINVAL;
    size_t cap_tokens = (size_t)(n_blk > 0 ? n_blk : 1) * (size_t)bs;
    double *logit = (double *)malloc(sizeof(double) * cap_tokens);
    int *tok = (int *)malloc(sizeof(int) * cap_tokens);
    if (!logit || !tok) { free(logit); free(tok); return ORC_ENOMEM; }
    double inv_sqrt_d = 1.0 / sqrt((double)D);

    int nt = 0;
    for (int i = 0; i < n_blk; ++i) {
        int n = blocks[i];
        if (n < 0) continue;
        for (int t = n * bs; t < (n + 1) * bs && t < ctx; ++t) tok[nt++] = t;
    }
    for (int h = 0; h < G; ++h) {
        double *o = out + (size_t)h * D;
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        if (nt == 0) continue;
        double mx = -INFINITY;
        for (int i = 0; i < nt; ++i) {
            double dot = 0.0;
            for (int d = 0; d < D; ++d) dot += q[(size_t)h * D + d] * k[(size_t)tok[i] * D + d];
            logit[i] = dot * inv_sqrt_d;
            if (logit[i] > mx) mx = logit[i];
        }
        double denom = 0.0;
        for (int i = 0; i < nt; ++i) { logit[i] = exp(logit[i] - mx); denom += logit[i]; }
        for (int i = 0; i < nt; ++i) {
            double p = logit[i] / denom;
            for (int d = 0; d < D; ++d) o[d] += p * v[(size_t)tok[i] * D + d];
        }
    }
    free(logit); free(tok);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* ------------------------------------------------------------------------ */
/* Compressed keys (Figure 7 caption: beside the sparse working set, the GPU
 * holds the keys compressed by per-block min/max pooling, and the draft query
 * scans those to predict the next step's top-K blocks).
 *
 * Reading of "min/max pooling": per block and per dimension d, the smallest
 * and the largest k[t][d] over the block's valid tokens t < ctx.
 *
 * ck: [W][2][D]; ck[n][0][d] = min, ck[n][1][d] = max for n < nb.  Blocks
 * n >= nb are not written.                                                  */
int oracle_pool_keys_row(int ctx, int D, int bs, const double *k, int W, double *ck)
{
    if (ctx < 0 || D <= 0 || bs <= 0 || W < 0) return ORC_EINVAL;
    int nb = (ctx + bs - 1) / bs;
    if (nb > W) return ORC_EINVAL;
    for (int n = 0; n < nb; ++n) {
        int t_end = (n + 1) * bs < ctx ? (n + 1) * bs : ctx;
        double *mn = ck + (size_t)n * 2 * D;
        double *mx = mn + D;
        for (int d = 0; d < D; ++d) {
            double lo = k[(size_t)(n * bs) * D + d], hi = lo;
            for (int t = n * bs + 1; t < t_end; ++t) {
                double x = k[(size_t)t * D + d];
                if (x < lo) lo = x;
                if (x > hi) hi = x;
            }
            mn[d] = lo;
            mx[d] = hi;
        }
    }
    return ORC_OK;
}

/* Block score from the compressed keys (Figure 7 caption).  The pages name
 * the pooling but not the score; the reading taken here is the largest value
 * q.x / sqrt(D) can reach for a key x inside the block's box
 * min <= x <= max: per dimension the larger of q_d * min_d and q_d * max_d,
 * summed over d.  Every valid token of the block lies in the box, so this is
 * an upper bound of the exact block score, equal to it when the block has
 * one token.  Maximised over the lookahead rows j < n_q, as the exact score.
 *
 * q: [n_q][D]; ck: [W][2][D] as written by oracle_pool_keys_row.
 * scores[n] = -inf for nb <= n < W.                                         */
int oracle_score_minmax_row(int ctx, int D, int bs, int n_q, const double *q,
                            const double *ck, int W, double *scores)
{
    if (ctx < 0 || D <= 0 || bs <= 0 || n_q <= 0 || W < 0) return ORC_EINVAL;
    int nb = (ctx + bs - 1) / bs;
    if (nb > W) return ORC_EINVAL;
    double inv_sqrt_d = 1.0 / sqrt((double)D);
    for (int n = 0; n < W; ++n) {
        if (n >= nb) { scores[n] = -INFINITY; continue; }
        const double *mn = ck + (size_t)n * 2 * D;
        const double *mx = mn + D;
        double best = -INFINITY;
        for (int j = 0; j < n_q; ++j) {
            double sum = 0.0;
            for (int d = 0; d < D; ++d) {
                double a = q[(size_t)j * D + d] * mn[d];
                double b = q[(size_t)j * D + d] * mx[d];
                sum += a > b ? a : b;
            }
            double bound = sum * inv_sqrt_d;
            if (bound > best) best = bound;
        }
        scores[n] = best;
    }
    return ORC_OK;
}

/* Whole-batch drivers: the same per-row functions over every (sequence, KV
 * head) row, rows in parallel with OpenMP (rows are independent).
 *
 * Logical layouts (ctx_max = max context, per-sequence ctx_len[b]):
 *   q_look [B][n_look][Hq][D], q [B][Hq][D], K and V [B][Hkv][ctx_max][D],
 *   scores [B][Hkv][W], sel [B][Hkv][K], slot_block / last_use [B][Hkv][K],
 *   fetch_block / fetch_slot [B][Hkv][cap], fetch_count [B][Hkv],
 *   out [B][Hq][D].
 * Query heads h of KV head g are h = g*G .. g*G+G-1, G = Hq / Hkv.           */
static void gather_group_queries(const double *q_look, int n_look, int Hq, int D,
                                 int b, int g, int G, double *dst)
{
    /* rows ordered (draft j, head-in-group r) */
    for (int j = 0; j < n_look; ++j)
        for (int r = 0; r < G; ++r)
            memcpy(dst + ((size_t)j * G + r) * D,
                   q_look + (((size_t)b * n_look + j) * Hq + (size_t)g * G + r) * D,
                   sizeof(double) * (size_t)D);
}

int oracle_score(int B, int Hq, int Hkv, int D, int bs, int ctx_max, int W,
                 const int *ctx_len, int n_look, const double *q_look, const double *K,
                 double *scores)
{
    if (B < 0 || Hkv <= 0 || Hq % Hkv) return ORC_EINVAL;
    int G = Hq / Hkv;
    int rows = B * Hkv, err = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < rows; ++r) {
        int b = r / Hkv, g = r % Hkv;
        double *qg = (double *)malloc(sizeof(double) * (size_t)n_look * G * D);
        int e = ORC_ENOMEM;
        if (qg) {
            gather_group_queries(q_look, n_look, Hq, D, b, g, G, qg);
            e = oracle_score_row(ctx_len[b], D, bs, n_look * G, qg,
                                 K + ((size_t)b * Hkv + g) * ctx_max * D, W,
                                 scores + ((size_t)b * Hkv + g) * W);
            free(qg);
        }
        if (e) {
#pragma omp atomic write
            err = e;
        }
    }
    return err;
}

/* Compressed keys of every row: K [B][Hkv][ctx_max][D] -> ck [B][Hkv][W][2][D]. */
int oracle_pool_keys(int B, int Hkv, int D, int bs, int ctx_max, int W, const int *ctx_len,
                     const double *K, double *ck)
{
    if (B < 0 || Hkv <= 0) return ORC_EINVAL;
    int rows = B * Hkv, err = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < rows; ++r) {
        int b = r / Hkv;
        int e = ctx_len[b] > ctx_max ? ORC_EINVAL
              : oracle_pool_keys_row(ctx_len[b], D, bs, K + (size_t)r * ctx_max * D, W,
                                     ck + (size_t)r * W * 2 * D);
        if (e) {
#pragma omp atomic write
            err = e;
        }
    }
    return err;
}

/* Compressed-key scores of every row: q_look [B][n_look][Hq][D],
 * ck [B][Hkv][W][2][D] -> scores [B][Hkv][W]. */
int oracle_score_minmax(int B, int Hq, int Hkv, int D, int bs, int W, const int *ctx_len,
                        int n_look, const double *q_look, const double *ck, double *scores)
{
    if (B < 0 || Hkv <= 0 || Hq % Hkv) return ORC_EINVAL;
    int G = Hq / Hkv;
    int rows = B * Hkv, err = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < rows; ++r) {
        int b = r / Hkv, g = r % Hkv;
        double *qg = (double *)malloc(sizeof(double) * (size_t)n_look * G * D);
        int e = ORC_ENOMEM;
        if (qg) {
            gather_group_queries(q_look, n_look, Hq, D, b, g, G, qg);
            e = oracle_score_minmax_row(ctx_len[b], D, bs, n_look * G, qg,
                                        ck + (size_t)r * W * 2 * D, W, scores + (size_t)r * W);
            free(qg);
        }
        if (e) {
#pragma omp atomic write
            err = e;
        }
    }
    return err;
}

int oracle_select(int B, int Hkv, int bs, int W, int K, const int *ctx_len,
                  const double *scores, int *sel)
{
    int rows = B * Hkv, err = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < rows; ++r) {
        int b = r / Hkv;
        int nb = (ctx_len[b] + bs - 1) / bs;
        int e = nb > W ? ORC_EINVAL
                       : oracle_select_row(nb, K, scores + (size_t)r * W, sel + (size_t)r * K);
        if (e) {
#pragma omp atomic write
            err = e;
        }
    }
    return err;
}

int oracle_plan(int B, int Hkv, int W, int K, int cap, int step, const int *sel,
                const double *scores, int *slot_block, int *last_use,
                int *fetch_block, int *fetch_slot, int *fetch_count)
{
    int rows = B * Hkv, err = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < rows; ++r) {
        int e = oracle_plan_row(K, cap, step, sel + (size_t)r * K, scores + (size_t)r * W,
                                slot_block + (size_t)r * K, last_use + (size_t)r * K,
                                fetch_block + (size_t)r * cap, fetch_slot + (size_t)r * cap,
                                fetch_count + r);
        if (e) {
#pragma omp atomic write
            err = e;
        }
    }
    return err;
}

int oracle_attn(int B, int Hq, int Hkv, int D, int bs, int ctx_max, const int *ctx_len,
                const double *q, const double *K, const double *V, int n_blk,
                const int *blocks, double *out)
{
    if (B < 0 || Hkv <= 0 || Hq % Hkv) return ORC_EINVAL;
    int G = Hq / Hkv;
    int rows = B * Hkv, err = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < rows; ++r) {
        int b = r / Hkv, g = r % Hkv;
        size_t kv_off = ((size_t)b * Hkv + g) * ctx_max * D;
        int e = oracle_attn_row(G, D, bs, ctx_len[b], q + ((size_t)b * Hq + (size_t)g * G) * D,
                                K + kv_off, V + kv_off, n_blk, blocks + (size_t)r * n_blk,
                                out + ((size_t)b * Hq + (size_t)g * G) * D);
        if (e) {
#pragma omp atomic write
            err = e;
        }
    }
    return err;
}

/* One whole decode step of one layer, row by row: score with the lookahead
 * queries, select the top K, plan against the resident state (which it
 * updates), then attend with the true query over the working set the plan
 * leaves (the slot table).  Rows run in parallel. */
int oracle_decode_step(int B, int Hq, int Hkv, int D, int bs, int ctx_max, int W,
                       const int *ctx_len, int n_look, const double *q_look,
                       const double *q, const double *K, const double *V, int K_blocks,
                       int cap, int step, double *scores, int *sel, int *slot_block,
                       int *last_use, int *fetch_block, int *fetch_slot, int *fetch_count,
                       double *out)
{
    if (B < 0 || Hkv <= 0 || Hq % Hkv) return ORC_EINVAL;
    int G = Hq / Hkv;
    int rows = B * Hkv, err = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < rows; ++r) {
        int b = r / Hkv, g = r % Hkv;
        size_t kv_off = ((size_t)b * Hkv + g) * ctx_max * D;
        int nb = (ctx_len[b] + bs - 1) / bs;
        double *qg = (double *)malloc(sizeof(double) * (size_t)n_look * G * D);
        int e = ORC_ENOMEM;
        if (qg) {
            gather_group_queries(q_look, n_look, Hq, D, b, g, G, qg);
            e = oracle_score_row(ctx_len[b], D, bs, n_look * G, qg, K + kv_off, W,
                                 scores + (size_t)r * W);
            free(qg);
        }
        if (!e) e = oracle_select_row(nb, K_blocks, scores + (size_t)r * W, sel + (size_t)r * K_blocks);
        if (!e) e = oracle_plan_row(K_blocks, cap, step, sel + (size_t)r * K_blocks,
                                    scores + (size_t)r * W, slot_block + (size_t)r * K_blocks,
                                    last_use + (size_t)r * K_blocks, fetch_block + (size_t)r * cap,
                                    fetch_slot + (size_t)r * cap, fetch_count + r);
        if (!e) e = oracle_attn_row(G, D, bs, ctx_len[b], q + ((size_t)b * Hq + (size_t)g * G) * D,
                                    K + kv_off, V + kv_off, K_blocks,
                                    slot_block + (size_t)r * K_blocks,
                                    out + ((size_t)b * Hq + (size_t)g * G) * D);
        if (e) {
#pragma omp atomic write
            err = e;
        }
    }
    return err;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of the following parallel regions (for timing the oracle on one core
 * or on all of them); returns the count now in effect. */
int oracle_set_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    extern int omp_get_max_threads(void);
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}
