/* abi_validate.c -- the host-side argument validation of every entry point of
 * include/oasis.h, from plain C: NULL and misaligned pointers, zero, negative,
 * unsupported and extreme sizes (up to INT32_MAX, where size arithmetic could
 * overflow), unknown flags, undersized workspaces.  Every call here is refused
 * (or is a documented no-op) before anything is enqueued, so no GPU is
 * needed.  The CPU tests build the library's ABI unit with AddressSanitizer
 * and UndefinedBehaviorSanitizer and run this program against it: a read
 * past a buffer, a signed overflow or a misaligned access in the validation
 * fails the run.  Exit status 0 when every status is the expected one. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "oasis.h"

static int failures = 0;

#define EXPECT(call, want)                                                                  \
    do {                                                                                    \
        int got_ = (call);                                                                  \
        if (got_ != (want)) {                                                               \
            fprintf(stderr, "line %d: %s returned %s, expected %s (%s)\n", __LINE__, #call,  \
                    oasis_status_string(got_), oasis_status_string(want), oasis_last_error()); \
            ++failures;                                                                     \
        }                                                                                   \
    } while (0)

static oasis_shape shape(int32_t batch, int32_t hq, int32_t hkv, int32_t d, int32_t bs, int32_t w,
                         int32_t pages) {
    oasis_shape s = {batch, hq, hkv, d, bs, w, pages};
    return s;
}

int main(void) {
    /* never dereferenced: every call below fails validation, or has nothing to do */
    uint16_t *const P16 = (uint16_t *)(uintptr_t)4096;
    int32_t *const PI = (int32_t *)(uintptr_t)4096;
    float *const PF = (float *)(uintptr_t)4096;
    void *const PV = (void *)(uintptr_t)4096;
    uint16_t *const MIS = (uint16_t *)(uintptr_t)4104;      /* 8-byte aligned only */
    const oasis_shape ok = shape(2, 8, 2, 128, 16, 64, 128);
    const oasis_shape big = shape(65535, 32, 1, 128, 16, INT32_MAX, INT32_MAX);
    oasis_shape s;

    /* shapes every call shares */
    EXPECT(oasis_score_blocks(NULL, P16, 1, P16, PI, PI, 0.1f, PF, NULL), OASIS_ERR_INVALID);
    s = shape(-1, 8, 2, 128, 16, 64, 128);
    EXPECT(oasis_score_blocks(&s, P16, 1, P16, PI, PI, 0.1f, PF, NULL), OASIS_ERR_INVALID);
    s = shape(2, 7, 2, 128, 16, 64, 128);
    EXPECT(oasis_score_blocks(&s, P16, 1, P16, PI, PI, 0.1f, PF, NULL), OASIS_ERR_INVALID);
    s = shape(2, 8, 0, 128, 16, 64, 128);
    EXPECT(oasis_score_blocks(&s, P16, 1, P16, PI, PI, 0.1f, PF, NULL), OASIS_ERR_INVALID);
    s = shape(2, 8, 2, 96, 16, 64, 128);
    EXPECT(oasis_score_blocks(&s, P16, 1, P16, PI, PI, 0.1f, PF, NULL), OASIS_ERR_UNSUPPORTED);
    s = shape(2, 8, 2, 128, 32, 64, 128);
    EXPECT(oasis_score_blocks(&s, P16, 1, P16, PI, PI, 0.1f, PF, NULL), OASIS_ERR_UNSUPPORTED);
    s = shape(70000, 8, 2, 128, 16, 64, 128);
    EXPECT(oasis_score_blocks(&s, P16, 1, P16, PI, PI, 0.1f, PF, NULL), OASIS_ERR_UNSUPPORTED);
    s = shape(INT32_MAX, INT32_MAX, INT32_MAX, 128, 16, INT32_MAX, INT32_MAX);
    EXPECT(oasis_score_blocks(&s, P16, 1, P16, PI, PI, 0.1f, PF, NULL), OASIS_ERR_UNSUPPORTED);

    /* scoring */
    EXPECT(oasis_score_blocks(&ok, P16, 0, P16, PI, PI, 0.1f, PF, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_score_blocks(&ok, P16, 5, P16, PI, PI, 0.1f, PF, NULL), OASIS_ERR_UNSUPPORTED);
    EXPECT(oasis_score_blocks(&ok, P16, INT32_MAX, P16, PI, PI, 0.1f, PF, NULL), OASIS_ERR_UNSUPPORTED);
    EXPECT(oasis_score_blocks(&ok, P16, 1, P16, PI, PI, 0.0f, PF, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_score_blocks(&ok, P16, 1, P16, PI, PI, -1.0f, PF, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_score_blocks(&ok, NULL, 1, P16, PI, PI, 0.1f, PF, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_score_blocks(&ok, MIS, 1, P16, PI, PI, 0.1f, PF, NULL), OASIS_ERR_INVALID);
    s = shape(0, 8, 2, 128, 16, 64, 128);
    EXPECT(oasis_score_blocks(&s, NULL, 1, NULL, NULL, NULL, 0.1f, NULL, NULL), OASIS_OK);
    EXPECT(oasis_pool_keys(&ok, P16, PI, PI, 2, P16, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_pool_keys(&ok, P16, PI, PI, -1, P16, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_pool_keys(&ok, P16, PI, PI, 0, NULL, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_pool_keys(&ok, P16, PI, PI, 0, MIS, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_score_blocks_minmax(&ok, P16, 1, P16, P16, NULL, PI, 0.1f, PF, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_score_blocks_minmax(&ok, P16, 1, MIS, NULL, NULL, PI, 0.1f, PF, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_score_blocks_minmax(&ok, P16, 17, P16, NULL, NULL, PI, 0.1f, PF, NULL), OASIS_ERR_UNSUPPORTED);

    /* select and plan */
    EXPECT(oasis_select_topk(&ok, PF, PI, 0, PI, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_select_topk(&ok, PF, PI, INT32_MAX, PI, NULL), OASIS_ERR_UNSUPPORTED);
    EXPECT(oasis_select_topk(&big, PF, PI, 8, PI, NULL), OASIS_ERR_UNSUPPORTED);
    EXPECT(oasis_select_topk(&ok, NULL, PI, 8, PI, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_plan_fetch(&ok, PI, PF, 8, 9, 0, PI, PI, PI, PI, PI, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_plan_fetch(&ok, PI, PF, 8, -1, 0, PI, PI, PI, PI, PI, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_plan_fetch(&ok, PI, PF, 8, 2, 0, PI, PI, NULL, PI, PI, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_plan_fetch(&ok, PI, PF, 8, 2, 0, PI, PI, PI, PI, NULL, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_plan_fetch(&ok, PI, PF, INT32_MAX, 2, 0, PI, PI, PI, PI, PI, NULL), OASIS_ERR_UNSUPPORTED);
    EXPECT(oasis_select_plan(&ok, PF, PI, 8, 9, 0, PI, PI, PI, PI, PI, PI, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_select_plan(&big, PF, PI, 8, 2, 0, PI, PI, PI, PI, PI, PI, NULL), OASIS_ERR_UNSUPPORTED);
    EXPECT(oasis_select_plan_ex(&ok, PF, PI, 8, 2, INT32_MIN, PI, NULL, PI, PI, PI, PI, PI, NULL),
           OASIS_ERR_INVALID);

    /* the two-pass selection of wide rows */
    s = shape(2, 8, 2, 128, 16, 8193, 128);
    const size_t sws = oasis_select_workspace_bytes(&s, 128);
    if (sws != (size_t)2 * 2 * 5 * 128 * 8) { fprintf(stderr, "select workspace %zu\n", sws); ++failures; }
    s.table_width = 8192;
    if (oasis_select_workspace_bytes(&s, 128) != 0) { fprintf(stderr, "8192 needs none\n"); ++failures; }
    s.table_width = 8193;
    if (oasis_select_workspace_bytes(&ok, 128) != 0) { fprintf(stderr, "narrow rows need none\n"); ++failures; }
    (void)oasis_select_workspace_bytes(&big, INT32_MAX);
    (void)oasis_select_workspace_bytes(&big, 1);
    (void)oasis_select_workspace_bytes(NULL, 1);
    EXPECT(oasis_select_plan_ws(&s, PF, PI, 128, 2, 0, NULL, PI, PI, PI, PI, PI, PI, NULL, 0, NULL),
           OASIS_ERR_NOMEM);
    EXPECT(oasis_select_plan_ws(&s, PF, PI, 128, 2, 0, NULL, PI, PI, PI, PI, PI, PI, PV, sws - 1, NULL),
           OASIS_ERR_NOMEM);
    EXPECT(oasis_select_plan_ws(&s, PF, PI, 128, 2, 0, NULL, PI, PI, PI, PI, PI, PI,
                                (void *)(uintptr_t)4100, sws, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_select_plan_ws(&s, PF, PI, 0, 2, 0, NULL, PI, PI, PI, PI, PI, PI, PV, sws, NULL),
           OASIS_ERR_INVALID);
    EXPECT(oasis_select_plan_ws(&s, PF, PI, 2000, 2, 0, NULL, PI, PI, PI, PI, PI, PI, PV, sws, NULL),
           OASIS_ERR_UNSUPPORTED);
    EXPECT(oasis_select_plan_ws(&s, PF, PI, 128, 129, 0, NULL, PI, PI, PI, PI, PI, PI, PV, sws, NULL),
           OASIS_ERR_INVALID);
    EXPECT(oasis_select_plan_ws(&s, PF, PI, 128, 2, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL, PV,
                                sws, NULL), OASIS_ERR_INVALID);            /* select only, no sel */
    EXPECT(oasis_select_plan_ws(&s, PF, PI, 128, 2, 0, NULL, PI, PI, NULL, PI, PI, PI, PV, sws, NULL),
           OASIS_ERR_INVALID);                                             /* plan without last_use */
    s = shape(2, 8, 2, 128, 16, 1048577, 128);
    EXPECT(oasis_select_plan_ws(&s, PF, PI, 128, 2, 0, NULL, PI, PI, PI, PI, PI, PI, PV, (size_t)-1,
                                NULL), OASIS_ERR_UNSUPPORTED);             /* wider than 8192 * 64 */
    s = shape(0, 8, 2, 128, 16, 65536, 128);
    EXPECT(oasis_select_plan_ws(&s, NULL, NULL, 128, 2, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                                NULL, 0, NULL), OASIS_OK);

    /* planning from one table copy into another: the tables are required, and
       an output array is its input array or shares no entry with the inputs
       (ok: 4 rows x 8 entries = 32 per array) */
    EXPECT(oasis_select_plan_next(&ok, PF, PI, 8, 2, 0, NULL, PI, NULL, PI + 100, PI + 200, PI + 300,
                                  PI, PI, PI, NULL, 0, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_select_plan_next(&ok, PF, PI, 8, 2, 0, NULL, PI, PI + 100, PI + 200, NULL, PI + 300,
                                  PI, PI, PI, NULL, 0, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_select_plan_next(&ok, PF, PI, 8, 2, 0, NULL, PI, PI + 100, PI + 200, PI + 101,
                                  PI + 300, PI, PI, PI, NULL, 0, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_select_plan_next(&ok, PF, PI, 8, 2, 0, NULL, PI, PI + 100, PI + 200, PI + 231,
                                  PI + 300, PI, PI, PI, NULL, 0, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_select_plan_next(&ok, PF, PI, 8, 2, 0, NULL, PI, PI + 100, PI + 200, PI + 100,
                                  PI + 116, PI, PI, PI, NULL, 0, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_select_plan_next(&ok, PF, PI, 8, 2, 0, NULL, PI, PI + 100, PI + 200, PI + 300,
                                  PI + 300, PI, PI, PI, NULL, 0, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_select_plan_next(&ok, PF, PI, 8, 9, 0, NULL, PI, PI + 100, PI + 200, PI + 300,
                                  PI + 400, PI, PI, PI, NULL, 0, NULL), OASIS_ERR_INVALID);
    s = shape(0, 8, 2, 128, 16, 64, 128);
    EXPECT(oasis_select_plan_next(&s, NULL, NULL, 8, 2, 0, NULL, NULL, PI, PI + 100, PI, PI + 100,
                                  NULL, NULL, NULL, NULL, 0, NULL), OASIS_OK);   /* in place, no rows */

    /* attention: workspace sizes at the extremes must not overflow */
    (void)oasis_attn_workspace_bytes(&big, 1, INT32_MAX);
    (void)oasis_attn_workspace_bytes(&big, INT32_MAX, 1);
    (void)oasis_attn_workspace_bytes(&ok, 1, INT32_MAX);
    (void)oasis_attn_workspace_bytes(&ok, 8, INT32_MAX);
    (void)oasis_attn_workspace_bytes(NULL, 1, 1);
    s = shape(65535, 4, 1, 128, 16, 64, 128);
    (void)oasis_attn_workspace_bytes(&s, 8, INT32_MAX);
    const size_t ws = oasis_attn_workspace_bytes(&ok, 1, 128);
    if (ws == 0) { fprintf(stderr, "workspace size 0 for a valid shape\n"); ++failures; }
    EXPECT(oasis_sparse_decode_attn(&ok, P16, 0, P16, P16, PI, PI, 128, PI, PI, 0.1f, P16, PV, ws, NULL),
           OASIS_ERR_INVALID);
    EXPECT(oasis_sparse_decode_attn(&ok, P16, 1, P16, P16, PI, PI, 0, PI, PI, 0.1f, P16, PV, ws, NULL),
           OASIS_ERR_INVALID);
    EXPECT(oasis_sparse_decode_attn(&ok, P16, 9, P16, P16, PI, PI, 128, PI, PI, 0.1f, P16, PV, ws, NULL),
           OASIS_ERR_UNSUPPORTED);
    EXPECT(oasis_sparse_decode_attn(&ok, P16, INT32_MAX, P16, P16, PI, PI, INT32_MAX, PI, PI, 0.1f, P16,
                                    PV, ws, NULL), OASIS_ERR_UNSUPPORTED);
    EXPECT(oasis_sparse_decode_attn(&ok, P16, 1, P16, P16, PI, PI, 128, PI, PI, 0.1f, P16, PV, ws - 1,
                                    NULL), OASIS_ERR_NOMEM);
    EXPECT(oasis_sparse_decode_attn(&ok, P16, 1, P16, P16, PI, NULL, 128, NULL, PI, 0.1f, P16, PV, ws,
                                    NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_sparse_decode_attn(&ok, P16, 1, P16, MIS, PI, PI, 128, PI, PI, 0.1f, P16, PV, ws, NULL),
           OASIS_ERR_INVALID);
    EXPECT(oasis_sparse_decode_attn(&ok, P16, 1, P16, P16, PI, PI, 128, PI, PI, 0.1f, P16,
                                    (void *)(uintptr_t)4100, ws, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_sparse_decode_attn_ex(&ok, P16, 1, P16, P16, PI, PI, 128, PI, PI, 0.1f, P16, PV, ws,
                                       8, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_sparse_decode_attn_noalloc(&ok, P16, 1, P16, P16, PI, PI, 128, PI, PI, 0.1f, P16, 8,
                                            NULL), OASIS_ERR_INVALID);
    s = shape(4096, 32, 8, 128, 16, 64, 128);                /* 32,768 rows: above the array */
    EXPECT(oasis_sparse_decode_attn_noalloc(&s, P16, 1, P16, P16, PI, PI, 1024, PI, PI, 0.1f, P16, 0,
                                            NULL), OASIS_ERR_NOMEM);
    EXPECT(oasis_sparse_decode_attn_noalloc(&big, P16, 1, P16, P16, PI, PI, INT32_MAX, PI, PI, 0.1f,
                                            P16, 0, NULL), OASIS_ERR_UNSUPPORTED);
    EXPECT(oasis_sparse_decode_attn(&ok, P16, 1, P16, P16, PI, PI, 65537, PI, PI, 0.1f, P16, PV,
                                    (size_t)-1, NULL), OASIS_ERR_UNSUPPORTED);
    if (oasis_attn_workspace_bytes(&ok, 1, 65537) != 0 || oasis_attn_workspace_bytes(&ok, 1, 65536) == 0) {
        fprintf(stderr, "workspace size at the list limit\n");
        ++failures;
    }

    /* host tier */
    void *host = PV;
    EXPECT(oasis_hostpool_create(0, &host), OASIS_ERR_INVALID);
    if (host != NULL) { fprintf(stderr, "host pointer not cleared on failure\n"); ++failures; }
    EXPECT(oasis_hostpool_create(64, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_hostpool_device_pointer(NULL, &host), OASIS_ERR_INVALID);
    EXPECT(oasis_hostpool_device_pointer(PV, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_hostpool_destroy(NULL), OASIS_OK);
    EXPECT(oasis_fetch_blocks(&ok, P16, P16, 0, PI, PI, PI, 2, PI, P16, P16, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_fetch_blocks(&ok, P16, P16, 64, PI, PI, PI, 65, PI, P16, P16, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_fetch_blocks(&ok, P16, P16, 64, PI, PI, PI, -1, PI, P16, P16, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_fetch_blocks(&ok, P16, P16, 64, NULL, PI, PI, 2, PI, P16, P16, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_fetch_blocks(&ok, MIS, P16, 64, PI, PI, PI, 2, PI, P16, P16, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_fetch_blocks(&ok, NULL, NULL, 64, NULL, NULL, NULL, 0, NULL, NULL, NULL, NULL), OASIS_OK);

    /* the layer step */
    oasis_layer layer;
    oasis_step_sync sync;
    memset(&layer, 0, sizeof(layer));
    memset(&sync, 0, sizeof(sync));
    EXPECT(oasis_layer_step(NULL, P16, P16, PF, 0, &sync), OASIS_ERR_INVALID);
    EXPECT(oasis_layer_step(&layer, P16, P16, PF, 0, NULL), OASIS_ERR_INVALID);
    EXPECT(oasis_layer_step(&layer, P16, P16, PF, 0, &sync), OASIS_ERR_INVALID);   /* no events */
    sync.scored = PV;
    sync.attended = PV;
    layer.slot_block_next = PI;                                        /* without last_use_next */
    EXPECT(oasis_layer_step(&layer, P16, P16, PF, 0, &sync), OASIS_ERR_INVALID);

    /* status text */
    if (strcmp(oasis_status_string(OASIS_ERR_NOMEM), "OASIS_ERR_NOMEM") != 0 ||
        strcmp(oasis_status_string(-5), "OASIS_ERR_UNKNOWN") != 0 || !oasis_version()[0]) {
        fprintf(stderr, "status strings\n");
        ++failures;
    }
    if (failures) return 1;
    printf("abi validation ok\n");
    return 0;
}
