/* One decode step of the hot path through the C ABI alone (include/oasis.h),
 * from plain C: no Python, no torch.  Tiny shape: 2 sequences, 8 query / 2 KV
 * heads, D 64, contexts 1000 and 777 tokens (63 and 49 blocks), K = 16 blocks,
 * cap 4, one lookahead query.  Inputs come from a fixed linear congruential
 * generator; the program checks what must hold whatever the inputs:
 *   - scores finite for valid blocks, -inf past the context;
 *   - the selection ascending, without repeats, of valid blocks, and each
 *     selected score >= every unselected one;
 *   - from an empty working set with cap 4: 4 blocks fetched per row, into
 *     slots 0..3, each selected and among the 4 best-scoring of the selection;
 *   - attention over the working set finite and a convex combination of V
 *     (each output within the min/max of V over the attended tokens).
 * Exit status 0 when every check passes; the tests run it on an MI355X. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "oasis.h"

#define B 2
#define HQ 8
#define HKV 2
#define D 64
#define BS 16
#define W 64
#define K 16
#define CAP 4
#define PAGES (B * W)

static uint32_t lcg = 12345u;
static float urand(void) { lcg = lcg * 1664525u + 1013904223u; return ((lcg >> 8) & 0xffffff) / 16777216.0f; }
static float nrand(void) { float s = 0.f; for (int i = 0; i < 12; ++i) s += urand(); return s - 6.f; }
static uint16_t to_bf16(float f) { uint32_t u; memcpy(&u, &f, 4); u += 0x7fffu + ((u >> 16) & 1u); return (uint16_t)(u >> 16); }
static float from_bf16(uint16_t h) { uint32_t u = (uint32_t)h << 16; float f; memcpy(&f, &u, 4); return f; }

#define CHECK_HIP(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_)); return 2; } } while (0)
#define CHECK_OASIS(x) do { int e_ = (x); if (e_) { fprintf(stderr, "%s: %s (%s)\n", #x, oasis_status_string(e_), oasis_last_error()); return 3; } } while (0)
#define EXPECT(c, ...) do { if (!(c)) { fprintf(stderr, __VA_ARGS__); fputc('\n', stderr); return 1; } } while (0)

static void *dev_copy(const void *h, size_t n) {
    void *d = NULL;
    if (hipMalloc(&d, n) != hipSuccess) return NULL;
    if (h && hipMemcpy(d, h, n, hipMemcpyHostToDevice) != hipSuccess) return NULL;
    return d;
}

int main(void) {
    const int ctx[B] = {1000, 777};
    /* key pool [page][Hkv][BS*D] in 8-dimension slices, value pool [page][Hkv][D][BS] */
    static uint16_t kp[PAGES][HKV][BS * D], vp[PAGES][HKV][D][BS];
    static float vlog[B][HKV][W * BS][D];              /* V by logical token, for the check */
    static uint16_t ql[B][HQ][D], q[B][HQ][D];
    int32_t bt[B][W];
    for (int b = 0; b < B; ++b)
        for (int n = 0; n < W; ++n) bt[b][n] = (b * W + n * 37) % PAGES;   /* a permutation */
    for (int b = 0; b < B; ++b)
        for (int n = 0; n < W; ++n)
            for (int g = 0; g < HKV; ++g)
                for (int t = 0; t < BS; ++t)
                    for (int d = 0; d < D; ++d) {
                        const int p = bt[b][n];
                        kp[p][g][((d / 8) * BS + t) * 8 + d % 8] = to_bf16(nrand());
                        const uint16_t v = to_bf16(nrand());
                        vp[p][g][d][t] = v;
                        vlog[b][g][n * BS + t][d] = from_bf16(v);
                    }
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < HQ; ++h)
            for (int d = 0; d < D; ++d) { q[b][h][d] = to_bf16(nrand()); ql[b][h][d] = to_bf16(nrand()); }

    oasis_shape s = {B, HQ, HKV, D, BS, W, PAGES};
    const float scale = 1.0f / sqrtf((float)D);
    const size_t ws_bytes = oasis_attn_workspace_bytes(&s, 1, K);
    EXPECT(ws_bytes > 0, "workspace size 0");
    int32_t sb0[B][HKV][K], lu0[B][HKV][K];
    for (int i = 0; i < B * HKV * K; ++i) { ((int32_t *)sb0)[i] = -1; ((int32_t *)lu0)[i] = INT32_MIN; }

    void *d_kp = dev_copy(kp, sizeof kp), *d_vp = dev_copy(vp, sizeof vp), *d_bt = dev_copy(bt, sizeof bt);
    void *d_ctx = dev_copy(ctx, sizeof ctx), *d_ql = dev_copy(ql, sizeof ql), *d_q = dev_copy(q, sizeof q);
    void *d_sb = dev_copy(sb0, sizeof sb0), *d_lu = dev_copy(lu0, sizeof lu0);
    void *d_scores = dev_copy(NULL, sizeof(float) * B * HKV * W), *d_sel = dev_copy(NULL, sizeof(int32_t) * B * HKV * K);
    void *d_fb = dev_copy(NULL, sizeof(int32_t) * B * HKV * CAP), *d_fs = dev_copy(NULL, sizeof(int32_t) * B * HKV * CAP);
    void *d_fc = dev_copy(NULL, sizeof(int32_t) * B * HKV), *d_out = dev_copy(NULL, sizeof(uint16_t) * B * HQ * D);
    void *d_ws = dev_copy(NULL, ws_bytes);
    EXPECT(d_kp && d_vp && d_bt && d_ctx && d_ql && d_q && d_sb && d_lu && d_scores && d_sel && d_fb &&
           d_fs && d_fc && d_out && d_ws, "hipMalloc failed");

    CHECK_OASIS(oasis_score_blocks(&s, d_ql, 1, d_kp, d_bt, d_ctx, scale, d_scores, NULL));
    CHECK_OASIS(oasis_select_topk(&s, d_scores, d_ctx, K, d_sel, NULL));
    CHECK_OASIS(oasis_plan_fetch(&s, d_sel, d_scores, K, CAP, 0, d_sb, d_lu, d_fb, d_fs, d_fc, NULL));
    CHECK_OASIS(oasis_sparse_decode_attn(&s, d_q, 1, d_kp, d_vp, d_bt, d_sb, K, d_sb, d_ctx, scale,
                                         d_out, d_ws, ws_bytes, NULL));
    CHECK_HIP(hipDeviceSynchronize());

    static float scores[B][HKV][W];
    int32_t sel[B][HKV][K], sb[B][HKV][K], fb[B][HKV][CAP], fs[B][HKV][CAP], fc[B][HKV];
    static uint16_t out[B][HQ][D];
    CHECK_HIP(hipMemcpy(scores, d_scores, sizeof scores, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(sel, d_sel, sizeof sel, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(sb, d_sb, sizeof sb, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(fb, d_fb, sizeof fb, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(fs, d_fs, sizeof fs, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(fc, d_fc, sizeof fc, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(out, d_out, sizeof out, hipMemcpyDeviceToHost));

    for (int b = 0; b < B; ++b)
        for (int g = 0; g < HKV; ++g) {
            const int nb = (ctx[b] + BS - 1) / BS;
            for (int n = 0; n < W; ++n)
                EXPECT(n < nb ? isfinite(scores[b][g][n]) : isinf(scores[b][g][n]) && scores[b][g][n] < 0,
                       "score b%d g%d n%d = %g", b, g, n, scores[b][g][n]);
            float min_sel = INFINITY, max_unsel = -INFINITY;
            int is_sel[W] = {0};
            for (int i = 0; i < K; ++i) {
                const int n = sel[b][g][i];
                EXPECT(n >= 0 && n < nb && (i == 0 || n > sel[b][g][i - 1]), "selection b%d g%d", b, g);
                is_sel[n] = 1;
                if (scores[b][g][n] < min_sel) min_sel = scores[b][g][n];
            }
            for (int n = 0; n < nb; ++n)
                if (!is_sel[n] && scores[b][g][n] > max_unsel) max_unsel = scores[b][g][n];
            EXPECT(min_sel >= max_unsel, "top-K order b%d g%d", b, g);
            EXPECT(fc[b][g] == CAP, "fetch count b%d g%d = %d", b, g, fc[b][g]);
            for (int i = 0; i < CAP; ++i) {
                const int n = fb[b][g][i];
                EXPECT(n >= 0 && is_sel[n] && fs[b][g][i] == i && sb[b][g][i] == n &&
                       (i == 0 || n > fb[b][g][i - 1]), "fetch list b%d g%d", b, g);
                int above = 0;              /* selected blocks scoring strictly higher */
                for (int j = 0; j < K; ++j) above += scores[b][g][sel[b][g][j]] > scores[b][g][n];
                EXPECT(above < CAP, "fetched block %d is not among the %d best b%d g%d", n, CAP, b, g);
            }
            for (int i = CAP; i < K; ++i) EXPECT(sb[b][g][i] == -1, "slot %d not empty", i);
            for (int h = g * (HQ / HKV); h < (g + 1) * (HQ / HKV); ++h)
                for (int d = 0; d < D; ++d) {
                    float lo = INFINITY, hi = -INFINITY;
                    for (int i = 0; i < CAP; ++i)
                        for (int t = 0; t < BS; ++t) {
                            const int tok = fb[b][g][i] * BS + t;
                            if (tok >= ctx[b]) continue;
                            const float v = vlog[b][g][tok][d];
                            lo = v < lo ? v : lo;
                            hi = v > hi ? v : hi;
                        }
                    const float o = from_bf16(out[b][h][d]);
                    /* slack: bf16 rounding of the output, half an ulp of the bound */
                    const float slack = 1e-3f + fmaxf(fabsf(lo), fabsf(hi)) * 0.00390625f;
                    EXPECT(isfinite(o) && o >= lo - slack && o <= hi + slack,
                           "attention b%d h%d d%d = %g outside [%g, %g]", b, h, d, o, lo, hi);
                }
        }
    printf("abi_step ok: %d rows, K %d, cap %d\n", B * HKV, K, CAP);
    return 0;
}
