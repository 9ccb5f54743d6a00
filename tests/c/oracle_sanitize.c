/* oracle_sanitize.c -- drives every entry point of the CPU oracle
 * (oracle/oasis_oracle.c) on small inputs and edge cases: ragged and empty
 * contexts, widths past the context, selections shorter than K, empty and
 * padded block lists, cap 0 and cap K, evictions, invalid sizes.  Built with
 * AddressSanitizer and UndefinedBehaviorSanitizer by the CPU tests, so that
 * an out-of-bounds access, a leak or undefined arithmetic in the oracle fails
 * the run; the values themselves are checked by the Python pins. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_score_row(int ctx, int D, int bs, int n_q, const double *q, const double *k, int W,
                     double *scores);
int oracle_select_row(int nb, int K, const double *scores, int *sel);
int oracle_plan_row(int K, int cap, int step, const int *sel, const double *scores,
                    int *slot_block, int *last_use, int *fetch_block, int *fetch_slot, int *count);
int oracle_attn_row(int G, int D, int bs, int ctx, const double *q, const double *k,
                    const double *v, int n_blk, const int *blocks, double *out);
int oracle_pool_keys_row(int ctx, int D, int bs, const double *k, int W, double *ck);
int oracle_score_minmax_row(int ctx, int D, int bs, int n_q, const double *q, const double *ck,
                            int W, double *scores);
int oracle_score(int B, int Hq, int Hkv, int D, int bs, int ctx_max, int W, const int *ctx_len,
                 int n_look, const double *q_look, const double *K, double *scores);
int oracle_pool_keys(int B, int Hkv, int D, int bs, int ctx_max, int W, const int *ctx_len,
                     const double *K, double *ck);
int oracle_score_minmax(int B, int Hq, int Hkv, int D, int bs, int W, const int *ctx_len,
                        int n_look, const double *q_look, const double *ck, double *scores);
int oracle_select(int B, int Hkv, int bs, int W, int K, const int *ctx_len, const double *scores,
                  int *sel);
int oracle_plan(int B, int Hkv, int W, int K, int cap, int step, const int *sel,
                const double *scores, int *slot_block, int *last_use, int *fetch_block,
                int *fetch_slot, int *fetch_count);
int oracle_attn(int B, int Hq, int Hkv, int D, int bs, int ctx_max, const int *ctx_len,
                const double *q, const double *K, const double *V, int n_blk, const int *blocks,
                double *out);
int oracle_decode_step(int B, int Hq, int Hkv, int D, int bs, int ctx_max, int W,
                       const int *ctx_len, int n_look, const double *q_look, const double *q,
                       const double *K, const double *V, int K_blocks, int cap, int step,
                       double *scores, int *sel, int *slot_block, int *last_use, int *fetch_block,
                       int *fetch_slot, int *fetch_count, double *out);
int oracle_set_threads(int n);

static unsigned rng = 12345u;
static double urand(void) { rng = rng * 1664525u + 1013904223u; return (rng >> 8) / 16777216.0 - 0.5; }

/* heap buffers of exactly the size a call may touch, so ASan sees overruns */
static double *dbuf(size_t n) {
    double *p = (double *)malloc(sizeof(double) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) p[i] = urand();
    return p;
}
static int *ibuf(size_t n, int v) {
    int *p = (int *)malloc(sizeof(int) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) p[i] = v;
    return p;
}

#define CHECK(x)                                                          \
    do {                                                                  \
        if (!(x)) { fprintf(stderr, "check failed: %s (line %d)\n", #x, __LINE__); return 1; } \
    } while (0)

static int rows(void) {
    const int D = 8, bs = 16;
    const int ctxs[] = {0, 1, 15, 16, 37, 64};
    for (size_t c = 0; c < sizeof(ctxs) / sizeof(ctxs[0]); ++c) {
        const int ctx = ctxs[c], nb = (ctx + bs - 1) / bs, W = nb + 2, n_q = 3;
        double *q = dbuf((size_t)n_q * D), *k = dbuf((size_t)(ctx ? ctx : 1) * D);
        double *v = dbuf((size_t)(ctx ? ctx : 1) * D);
        double *s = dbuf((size_t)W), *ck = dbuf((size_t)W * 2 * D), *sm = dbuf((size_t)W);
        CHECK(oracle_score_row(ctx, D, bs, n_q, q, k, W, s) == 0);
        for (int n = nb; n < W; ++n) CHECK(isinf(s[n]) && s[n] < 0);
        CHECK(oracle_pool_keys_row(ctx, D, bs, k, W, ck) == 0);
        CHECK(oracle_score_minmax_row(ctx, D, bs, n_q, q, ck, W, sm) == 0);
        for (int K = 1; K <= nb + 2; ++K) {
            int *sel = ibuf((size_t)K, 7);
            CHECK(oracle_select_row(nb, K, s, sel) == 0);
            for (int cap = 0; cap <= K; ++cap) {
                int *sb = ibuf((size_t)K, -1), *lu = ibuf((size_t)K, -7);
                /* a resident set with a block past the selection, to force evictions */
                if (K > 1) { sb[0] = nb + 1; lu[0] = 3; }
                int *fb = ibuf((size_t)(cap ? cap : 1), 0), *fs = ibuf((size_t)(cap ? cap : 1), 0);
                int cnt = -1;
                CHECK(oracle_plan_row(K, cap, 5, sel, s, sb, lu, fb, fs, &cnt) == 0);
                CHECK(cnt >= 0 && cnt <= cap);
                free(sb); free(lu); free(fb); free(fs);
            }
            double *o = dbuf((size_t)2 * D);
            CHECK(oracle_attn_row(2, D, bs, ctx, q, k, v, K, sel, o) == 0);
            free(sel); free(o);
        }
        /* an empty list and an all-padding list give zeros */
        int pad[3] = {-1, -1, -1};
        double *o = dbuf((size_t)2 * D);
        CHECK(oracle_attn_row(2, D, bs, ctx, q, k, v, 3, pad, o) == 0);
        for (int i = 0; i < 2 * D; ++i) CHECK(o[i] == 0.0);
        CHECK(oracle_attn_row(2, D, bs, ctx, q, k, v, 0, pad, o) == 0);
        free(q); free(k); free(v); free(s); free(ck); free(sm); free(o);
    }
    /* invalid sizes are refused without touching the buffers */
    double x[4] = {0};
    int ix[4] = {0};
    CHECK(oracle_score_row(-1, 8, 16, 1, x, x, 1, x) != 0);
    CHECK(oracle_select_row(-1, 2, x, ix) != 0);
    CHECK(oracle_plan_row(-1, 0, 0, ix, x, ix, ix, ix, ix, ix) != 0);
    CHECK(oracle_attn_row(0, 8, 16, 4, x, x, x, 1, ix, x) != 0);
    CHECK(oracle_pool_keys_row(-3, 8, 16, x, 1, x) != 0);
    CHECK(oracle_score_minmax_row(4, 8, 16, 0, x, x, 1, x) != 0);
    return 0;
}

static int batch(void) {
    const int B = 3, Hq = 4, Hkv = 2, D = 8, bs = 16, ctx_max = 48, W = 4, n_look = 2;
    const int ctx_len[3] = {37, 16, 0};
    const int Kb = 2, cap = 1;
    double *ql = dbuf((size_t)B * n_look * Hq * D), *q = dbuf((size_t)B * Hq * D);
    double *K = dbuf((size_t)B * Hkv * ctx_max * D), *V = dbuf((size_t)B * Hkv * ctx_max * D);
    double *s = dbuf((size_t)B * Hkv * W), *ck = dbuf((size_t)B * Hkv * W * 2 * D);
    double *sm = dbuf((size_t)B * Hkv * W), *o = dbuf((size_t)B * Hq * D);
    int *sel = ibuf((size_t)B * Hkv * Kb, 0), *sb = ibuf((size_t)B * Hkv * Kb, -1);
    int *lu = ibuf((size_t)B * Hkv * Kb, -100), *fb = ibuf((size_t)B * Hkv * cap, 0);
    int *fs = ibuf((size_t)B * Hkv * cap, 0), *fc = ibuf((size_t)B * Hkv, 0);
    oracle_set_threads(2);
    CHECK(oracle_score(B, Hq, Hkv, D, bs, ctx_max, W, ctx_len, n_look, ql, K, s) == 0);
    CHECK(oracle_pool_keys(B, Hkv, D, bs, ctx_max, W, ctx_len, K, ck) == 0);
    CHECK(oracle_score_minmax(B, Hq, Hkv, D, bs, W, ctx_len, n_look, ql, ck, sm) == 0);
    CHECK(oracle_select(B, Hkv, bs, W, Kb, ctx_len, s, sel) == 0);
    CHECK(oracle_plan(B, Hkv, W, Kb, cap, 0, sel, s, sb, lu, fb, fs, fc) == 0);
    CHECK(oracle_attn(B, Hq, Hkv, D, bs, ctx_max, ctx_len, q, K, V, Kb, sb, o) == 0);
    for (int step = 1; step < 4; ++step)
        CHECK(oracle_decode_step(B, Hq, Hkv, D, bs, ctx_max, W, ctx_len, n_look, ql, q, K, V, Kb,
                                 cap, step, s, sel, sb, lu, fb, fs, fc, o) == 0);
    for (int i = 0; i < B * Hkv; ++i) CHECK(fc[i] <= cap);
    free(ql); free(q); free(K); free(V); free(s); free(ck); free(sm); free(o);
    free(sel); free(sb); free(lu); free(fb); free(fs); free(fc);
    return 0;
}

int main(void) {
    if (rows() || batch()) return 1;
    printf("oracle sanitize ok\n");
    return 0;
}
