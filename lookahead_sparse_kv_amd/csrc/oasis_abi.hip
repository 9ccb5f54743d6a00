// oasis_abi.hip -- the extern "C" entry points declared in include/oasis.h:
// host-side argument validation, then one launch per call on the caller's
// stream.  No allocation, no synchronisation, no printing.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <mutex>

#include "oasis.h"
#include "oasis_launch.h"

#ifndef OASIS_HOSTPOOL_FLAGS
#define OASIS_HOSTPOOL_FLAGS (hipHostMallocMapped | hipHostMallocPortable)
#endif

namespace {

thread_local char g_err[512] = "";

// The completion event of the stage oasis_layer_step is enqueueing: the
// stage's last kernel launch records it (oasis::LaunchStop).  Null outside
// oasis_layer_step, so the public calls launch as they always do.
thread_local oasis::LaunchStop *t_stage_stop = nullptr;

int fail(int status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_err[0] = '\0';
    return OASIS_OK;
}

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

int check_hip(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(OASIS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// Shape checks shared by every call.
int check_shape(const oasis_shape *s, const char *fn) {
    if (!s) return fail(OASIS_ERR_INVALID, "%s: shape is NULL", fn);
    if (s->batch < 0 || s->num_q_heads <= 0 || s->num_kv_heads <= 0 || s->head_dim <= 0 ||
        s->block_size <= 0 || s->table_width < 0 || s->num_pages < 0)
        return fail(OASIS_ERR_INVALID, "%s: negative or zero dimension in shape", fn);
    if (s->num_q_heads % s->num_kv_heads)
        return fail(OASIS_ERR_INVALID, "%s: num_q_heads %d is not a multiple of num_kv_heads %d", fn,
                    s->num_q_heads, s->num_kv_heads);
    if (s->block_size != oasis::kBlockTokens)
        return fail(OASIS_ERR_UNSUPPORTED, "%s: block_size %d (only 16 is implemented)", fn,
                    s->block_size);
    if (s->head_dim != 64 && s->head_dim != 128)
        return fail(OASIS_ERR_UNSUPPORTED, "%s: head_dim %d (64 or 128 are implemented)", fn,
                    s->head_dim);
    if ((long long)s->batch * s->num_kv_heads > 65535)
        return fail(OASIS_ERR_UNSUPPORTED, "%s: batch * num_kv_heads above 65535", fn);
    return OASIS_OK;
}

// The kernels read these buffers 16 bytes per lane.
bool misaligned16(const void *p) { return reinterpret_cast<uintptr_t>(p) % 16 != 0; }

}  // namespace

extern "C" {

const char *oasis_status_string(int status) {
    switch (status) {
        case OASIS_OK: return "OASIS_OK";
        case OASIS_ERR_INVALID: return "OASIS_ERR_INVALID";
        case OASIS_ERR_UNSUPPORTED: return "OASIS_ERR_UNSUPPORTED";
        case OASIS_ERR_NOMEM: return "OASIS_ERR_NOMEM";
        case OASIS_ERR_HIP: return "OASIS_ERR_HIP";
        default: return "OASIS_ERR_UNKNOWN";
    }
}

const char *oasis_last_error(void) { return g_err; }

const char *oasis_version(void) { return "oasis-mi355x 0.1 (gfx950)"; }

int oasis_score_blocks(const oasis_shape *s, const uint16_t *q_look, int32_t n_look,
                       const uint16_t *k_pool, const int32_t *block_table, const int32_t *ctx_len,
                       float scale, float *scores, void *stream) {
    const char *fn = "oasis_score_blocks";
    if (int e = check_shape(s, fn)) return e;
    if (n_look < 1) return fail(OASIS_ERR_INVALID, "%s: n_look %d < 1", fn, n_look);
    const int G = s->num_q_heads / s->num_kv_heads;
    if ((long long)n_look * G > oasis::kMaxRowsQ)
        return fail(OASIS_ERR_UNSUPPORTED, "%s: n_look * group = %lld above %d", fn,
                    (long long)n_look * G, oasis::kMaxRowsQ);
    if (!(scale > 0.f) || !isfinite(scale))
        return fail(OASIS_ERR_INVALID, "%s: scale must be finite and > 0", fn);
    if (s->batch == 0 || s->table_width == 0) return ok();
    if (!q_look || !k_pool || !block_table || !ctx_len || !scores)
        return fail(OASIS_ERR_INVALID, "%s: NULL pointer argument", fn);
    if (misaligned16(q_look) || misaligned16(k_pool))
        return fail(OASIS_ERR_INVALID, "%s: q_look and k_pool must be 16-byte aligned", fn);
    oasis::ScoreArgs a{q_look, k_pool, block_table, ctx_len, scores, scale,
                       s->batch, s->num_q_heads, s->num_kv_heads, G, s->table_width,
                       s->num_pages, n_look, n_look * G};
    return check_hip(oasis::launch_score_blocks(a, s->head_dim, as_stream(stream), t_stage_stop), fn);
}

int oasis_pool_keys(const oasis_shape *s, const uint16_t *k_pool, const int32_t *block_table,
                    const int32_t *ctx_len, int32_t last_only, uint16_t *ck, void *stream) {
    const char *fn = "oasis_pool_keys";
    if (int e = check_shape(s, fn)) return e;
    if (last_only != 0 && last_only != 1)
        return fail(OASIS_ERR_INVALID, "%s: last_only must be 0 or 1, got %d", fn, last_only);
    if (s->batch == 0 || s->table_width == 0) return ok();
    if (!k_pool || !block_table || !ctx_len || !ck)
        return fail(OASIS_ERR_INVALID, "%s: NULL pointer argument", fn);
    if (misaligned16(ck) || misaligned16(k_pool))
        return fail(OASIS_ERR_INVALID, "%s: k_pool and ck must be 16-byte aligned", fn);
    oasis::PoolArgs a{k_pool, block_table, ctx_len, ck, s->batch, s->num_kv_heads, s->table_width,
                      s->num_pages, last_only};
    return check_hip(oasis::launch_pool_keys(a, s->head_dim, as_stream(stream)), fn);
}

int oasis_score_blocks_minmax(const oasis_shape *s, const uint16_t *q_look, int32_t n_look,
                              uint16_t *ck, const uint16_t *k_pool, const int32_t *block_table,
                              const int32_t *ctx_len, float scale, float *scores, void *stream) {
    const char *fn = "oasis_score_blocks_minmax";
    if (int e = check_shape(s, fn)) return e;
    if (n_look < 1) return fail(OASIS_ERR_INVALID, "%s: n_look %d < 1", fn, n_look);
    const int G = s->num_q_heads / s->num_kv_heads;
    if ((long long)n_look * G > oasis::kMaxRowsQ)
        return fail(OASIS_ERR_UNSUPPORTED, "%s: n_look * group = %lld above %d", fn,
                    (long long)n_look * G, oasis::kMaxRowsQ);
    if (!(scale > 0.f) || !isfinite(scale))
        return fail(OASIS_ERR_INVALID, "%s: scale must be finite and > 0", fn);
    if (s->batch == 0 || s->table_width == 0) return ok();
    if (!q_look || !ck || !ctx_len || !scores)
        return fail(OASIS_ERR_INVALID, "%s: NULL pointer argument", fn);
    if (!k_pool != !block_table)
        return fail(OASIS_ERR_INVALID, "%s: k_pool and block_table must both be set or both NULL",
                    fn);
    if (misaligned16(ck) || misaligned16(k_pool) || misaligned16(q_look))
        return fail(OASIS_ERR_INVALID, "%s: q_look, ck and k_pool must be 16-byte aligned", fn);
    oasis::MinmaxArgs a{q_look, ck, k_pool, block_table, ctx_len, scores, scale, s->batch,
                        s->num_q_heads, s->num_kv_heads, G, s->table_width, s->num_pages, n_look,
                        n_look * G};
    return check_hip(oasis::launch_score_minmax(a, s->head_dim, as_stream(stream), t_stage_stop), fn);
}

int oasis_select_topk(const oasis_shape *s, const float *scores, const int32_t *ctx_len,
                      int32_t k_blocks, int32_t *sel, void *stream) {
    const char *fn = "oasis_select_topk";
    if (int e = check_shape(s, fn)) return e;
    if (k_blocks < 1) return fail(OASIS_ERR_INVALID, "%s: k_blocks %d < 1", fn, k_blocks);
    if (k_blocks > oasis::kMaxKBlocks)
        return fail(OASIS_ERR_UNSUPPORTED, "%s: k_blocks %d above %d", fn, k_blocks,
                    oasis::kMaxKBlocks);
    if (s->table_width > oasis::kMaxSelectWidth)
        return fail(OASIS_ERR_UNSUPPORTED, "%s: table_width %d above %d", fn, s->table_width,
                    oasis::kMaxSelectWidth);
    if (s->batch == 0) return ok();
    if (!scores || !ctx_len || !sel) return fail(OASIS_ERR_INVALID, "%s: NULL pointer argument", fn);
    const int rows = s->batch * s->num_kv_heads;
    if (oasis::row_select_plan_fits(s->table_width, k_blocks, 1)) {
        oasis::SelectPlanArgs a{scores, ctx_len, sel, nullptr, nullptr, nullptr, nullptr, nullptr,
                                rows, s->num_kv_heads, s->table_width, k_blocks, 0, 0};
        return check_hip(oasis::launch_row_select_plan(a, 1, as_stream(stream), t_stage_stop), fn);
    }
    oasis::SelectArgs a{scores, ctx_len, sel, rows, s->num_kv_heads, s->table_width, k_blocks};
    return check_hip(oasis::launch_select_topk(a, as_stream(stream)), fn);
}

int oasis_plan_fetch(const oasis_shape *s, const int32_t *sel, const float *scores,
                     int32_t k_blocks, int32_t cap, int32_t step, int32_t *slot_block,
                     int32_t *last_use, int32_t *fetch_block, int32_t *fetch_slot,
                     int32_t *fetch_count, void *stream) {
    const char *fn = "oasis_plan_fetch";
    if (int e = check_shape(s, fn)) return e;
    if (k_blocks < 1) return fail(OASIS_ERR_INVALID, "%s: k_blocks %d < 1", fn, k_blocks);
    if (k_blocks > oasis::kMaxKBlocks)
        return fail(OASIS_ERR_UNSUPPORTED, "%s: k_blocks %d above %d", fn, k_blocks,
                    oasis::kMaxKBlocks);
    if (cap < 0 || cap > k_blocks)
        return fail(OASIS_ERR_INVALID, "%s: cap %d outside [0, k_blocks = %d]", fn, cap, k_blocks);
    if (s->batch == 0) return ok();
    if (!sel || !scores || !slot_block || !last_use || !fetch_count)
        return fail(OASIS_ERR_INVALID, "%s: NULL pointer argument", fn);
    if (cap > 0 && (!fetch_block || !fetch_slot))
        return fail(OASIS_ERR_INVALID, "%s: NULL fetch list with cap %d", fn, cap);
    const int rows = s->batch * s->num_kv_heads;
    oasis::SelectPlanArgs a{scores, nullptr, const_cast<int32_t *>(sel), slot_block, last_use,
                            fetch_block, fetch_slot, fetch_count, rows, s->num_kv_heads,
                            s->table_width, k_blocks, cap, step, nullptr, slot_block, last_use};
    return check_hip(oasis::launch_row_select_plan(a, 2, as_stream(stream), t_stage_stop), fn);
}

int oasis_select_plan(const oasis_shape *s, const float *scores, const int32_t *ctx_len,
                      int32_t k_blocks, int32_t cap, int32_t step, int32_t *sel,
                      int32_t *slot_block, int32_t *last_use, int32_t *fetch_block,
                      int32_t *fetch_slot, int32_t *fetch_count, void *stream) {
    return oasis_select_plan_ex(s, scores, ctx_len, k_blocks, cap, step, nullptr, sel, slot_block,
                                last_use, fetch_block, fetch_slot, fetch_count, stream);
}

// Select + plan where the plan starts from the table (sb_in, lu_in) and
// writes (slot_block, last_use): the same arrays when planning in place.
static int select_plan_one_pass(const char *fn, const oasis_shape *s, const float *scores,
                                const int32_t *ctx_len, int32_t k_blocks, int32_t cap, int32_t step,
                                const int32_t *step_dev, int32_t *sel, const int32_t *sb_in,
                                const int32_t *lu_in, int32_t *slot_block, int32_t *last_use,
                                int32_t *fetch_block, int32_t *fetch_slot, int32_t *fetch_count,
                                void *stream) {
    if (int e = check_shape(s, fn)) return e;
    if (k_blocks < 1) return fail(OASIS_ERR_INVALID, "%s: k_blocks %d < 1", fn, k_blocks);
    if (k_blocks > oasis::kMaxKBlocks)
        return fail(OASIS_ERR_UNSUPPORTED, "%s: k_blocks %d above %d", fn, k_blocks,
                    oasis::kMaxKBlocks);
    if (s->table_width > oasis::kMaxSelectWidth)
        return fail(OASIS_ERR_UNSUPPORTED, "%s: table_width %d above %d", fn, s->table_width,
                    oasis::kMaxSelectWidth);
    if (cap < 0 || cap > k_blocks)
        return fail(OASIS_ERR_INVALID, "%s: cap %d outside [0, k_blocks = %d]", fn, cap, k_blocks);
    if (s->batch == 0) return ok();
    if (!scores || !ctx_len || !sel || !slot_block || !last_use || !fetch_count || !sb_in || !lu_in)
        return fail(OASIS_ERR_INVALID, "%s: NULL pointer argument", fn);
    if (cap > 0 && (!fetch_block || !fetch_slot))
        return fail(OASIS_ERR_INVALID, "%s: NULL fetch list with cap %d", fn, cap);
    const int rows = s->batch * s->num_kv_heads;
    oasis::SelectPlanArgs a{scores, ctx_len, sel, slot_block, last_use, fetch_block, fetch_slot,
                            fetch_count, rows, s->num_kv_heads, s->table_width, k_blocks, cap,
                            step, step_dev, sb_in, lu_in};
    if (oasis::row_select_plan_fits(s->table_width, k_blocks, 3))
        return check_hip(oasis::launch_row_select_plan(a, 3, as_stream(stream), t_stage_stop), fn);
    if (oasis::row_select_plan_fits(s->table_width, k_blocks, 1)) {
        if (int e = check_hip(oasis::launch_row_select_plan(a, 1, as_stream(stream)), fn)) return e;
    } else {
        oasis::SelectArgs sa{scores, ctx_len, sel, rows, s->num_kv_heads, s->table_width, k_blocks};
        if (int e = check_hip(oasis::launch_select_topk(sa, as_stream(stream)), fn)) return e;
    }
    return check_hip(oasis::launch_row_select_plan(a, 2, as_stream(stream), t_stage_stop), fn);
}

int oasis_select_plan_ex(const oasis_shape *s, const float *scores, const int32_t *ctx_len,
                         int32_t k_blocks, int32_t cap, int32_t step, const int32_t *step_dev,
                         int32_t *sel, int32_t *slot_block, int32_t *last_use,
                         int32_t *fetch_block, int32_t *fetch_slot, int32_t *fetch_count,
                         void *stream) {
    return select_plan_one_pass("oasis_select_plan", s, scores, ctx_len, k_blocks, cap, step,
                                step_dev, sel, slot_block, last_use, slot_block, last_use,
                                fetch_block, fetch_slot, fetch_count, stream);
}

size_t oasis_select_workspace_bytes(const oasis_shape *s, int32_t k_blocks) {
    if (!s || s->batch < 0 || s->num_kv_heads <= 0 || s->table_width < 0 || k_blocks < 1 ||
        k_blocks > oasis::kMaxKBlocks || (long long)s->batch * s->num_kv_heads > 65535 ||
        s->table_width <= oasis::kTwoPassMinWidth ||
        s->table_width > oasis::two_pass_max_width(k_blocks))
        return 0;
    int cw = 0, chunks = 0;
    oasis::two_pass_plan(s->table_width, k_blocks, &cw, &chunks);
    return (size_t)s->batch * s->num_kv_heads * chunks * k_blocks * 8;
}

// oasis_select_plan_ws with the plan starting from (sb_in, lu_in).
static int select_plan_any_width(const char *fn, const oasis_shape *s, const float *scores,
                                 const int32_t *ctx_len, int32_t k_blocks, int32_t cap,
                                 int32_t step, const int32_t *step_dev, int32_t *sel,
                                 const int32_t *sb_in, const int32_t *lu_in, int32_t *slot_block,
                                 int32_t *last_use, int32_t *fetch_block, int32_t *fetch_slot,
                                 int32_t *fetch_count, void *workspace, size_t workspace_bytes,
                                 void *stream) {
    if (int e = check_shape(s, fn)) return e;
    if (k_blocks < 1) return fail(OASIS_ERR_INVALID, "%s: k_blocks %d < 1", fn, k_blocks);
    if (k_blocks > oasis::kMaxKBlocks)
        return fail(OASIS_ERR_UNSUPPORTED, "%s: k_blocks %d above %d", fn, k_blocks,
                    oasis::kMaxKBlocks);
    const bool plan = slot_block != nullptr;
    if (plan && (cap < 0 || cap > k_blocks))
        return fail(OASIS_ERR_INVALID, "%s: cap %d outside [0, k_blocks = %d]", fn, cap, k_blocks);
    if (s->table_width > oasis::two_pass_max_width(k_blocks))
        return fail(OASIS_ERR_UNSUPPORTED, "%s: table_width %d above %lld for k_blocks %d", fn,
                    s->table_width, oasis::two_pass_max_width(k_blocks), k_blocks);
    if (s->batch == 0) return ok();
    if (!scores || !ctx_len || !sel) return fail(OASIS_ERR_INVALID, "%s: NULL pointer argument", fn);
    if (plan && (!last_use || !fetch_count || !sb_in || !lu_in ||
                 (cap > 0 && (!fetch_block || !fetch_slot))))
        return fail(OASIS_ERR_INVALID, "%s: NULL plan buffer", fn);
    if (s->table_width <= oasis::kTwoPassMinWidth) {      // one pass; no workspace needed
        if (plan)
            return select_plan_one_pass(fn, s, scores, ctx_len, k_blocks, cap, step, step_dev,
                                        sel, sb_in, lu_in, slot_block, last_use, fetch_block,
                                        fetch_slot, fetch_count, stream);
        return oasis_select_topk(s, scores, ctx_len, k_blocks, sel, stream);
    }
    const size_t need = oasis_select_workspace_bytes(s, k_blocks);
    if (!workspace || workspace_bytes < need)
        return fail(OASIS_ERR_NOMEM, "%s: workspace %zu bytes, %zu needed", fn, workspace_bytes, need);
    if (reinterpret_cast<uintptr_t>(workspace) % 8)
        return fail(OASIS_ERR_INVALID, "%s: workspace must be 8-byte aligned", fn);
    const int rows = s->batch * s->num_kv_heads;
    int cw = 0, chunks = 0;
    oasis::two_pass_plan(s->table_width, k_blocks, &cw, &chunks);
    uint32_t *cand_key = static_cast<uint32_t *>(workspace);
    int32_t *cand_idx = reinterpret_cast<int32_t *>(cand_key + (size_t)rows * chunks * k_blocks);
    oasis::SelectPlanArgs a{scores, ctx_len, sel, slot_block, last_use, fetch_block, fetch_slot,
                            fetch_count, rows, s->num_kv_heads, s->table_width, k_blocks,
                            plan ? cap : 0, step, step_dev, sb_in, lu_in};
    return check_hip(oasis::launch_two_pass_select_plan(a, plan ? 3 : 1, cand_key, cand_idx,
                                                        as_stream(stream), t_stage_stop), fn);
}

int oasis_select_plan_ws(const oasis_shape *s, const float *scores, const int32_t *ctx_len,
                         int32_t k_blocks, int32_t cap, int32_t step, const int32_t *step_dev,
                         int32_t *sel, int32_t *slot_block, int32_t *last_use,
                         int32_t *fetch_block, int32_t *fetch_slot, int32_t *fetch_count,
                         void *workspace, size_t workspace_bytes, void *stream) {
    return select_plan_any_width("oasis_select_plan_ws", s, scores, ctx_len, k_blocks, cap, step,
                                 step_dev, sel, slot_block, last_use, slot_block, last_use,
                                 fetch_block, fetch_slot, fetch_count, workspace,
                                 workspace_bytes, stream);
}

// [a, a + n) and [b, b + n) (int32 entries) share an entry
static bool overlap(const int32_t *a, const int32_t *b, size_t n) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + n * sizeof(int32_t) && y < x + n * sizeof(int32_t);
}

int oasis_select_plan_next(const oasis_shape *s, const float *scores, const int32_t *ctx_len,
                           int32_t k_blocks, int32_t cap, int32_t step, const int32_t *step_dev,
                           int32_t *sel, const int32_t *slot_block_in, const int32_t *last_use_in,
                           int32_t *slot_block, int32_t *last_use, int32_t *fetch_block,
                           int32_t *fetch_slot, int32_t *fetch_count, void *workspace,
                           size_t workspace_bytes, void *stream) {
    const char *fn = "oasis_select_plan_next";
    if (int e = check_shape(s, fn)) return e;
    if (!slot_block || !last_use || !slot_block_in || !last_use_in)
        return fail(OASIS_ERR_INVALID, "%s: NULL working-set table", fn);
    if (k_blocks >= 1) {
        // each output array is either the matching input array itself (in
        // place) or shares no entry with any input array
        const size_t n = (size_t)(s->batch < 0 ? 0 : s->batch) * s->num_kv_heads * k_blocks;
        const int32_t *outs[2] = {slot_block, last_use}, *ins[2] = {slot_block_in, last_use_in};
        for (int o = 0; o < 2; ++o)
            for (int i = 0; i < 2; ++i)
                if (!(o == i && outs[o] == ins[i]) && overlap(outs[o], ins[i], n))
                    return fail(OASIS_ERR_INVALID,
                                "%s: an output table overlaps an input table without being it", fn);
        if (overlap(slot_block, last_use, n))
            return fail(OASIS_ERR_INVALID, "%s: slot_block and last_use overlap", fn);
    }
    return select_plan_any_width(fn, s, scores, ctx_len, k_blocks, cap, step, step_dev, sel,
                                 slot_block_in, last_use_in, slot_block, last_use, fetch_block,
                                 fetch_slot, fetch_count, workspace, workspace_bytes, stream);
}

size_t oasis_attn_workspace_bytes(const oasis_shape *s, int32_t n_q, int32_t n_blk) {
    if (!s || s->batch < 0 || s->num_kv_heads <= 0 || s->num_q_heads <= 0 || s->head_dim <= 0 ||
        n_q < 1 || n_blk < 1 || n_blk > oasis::kMaxAttnBlocks || s->num_q_heads % s->num_kv_heads ||
        (long long)s->batch * s->num_kv_heads > 65535 ||
        (long long)n_q * (s->num_q_heads / s->num_kv_heads) > oasis::kMaxAttnRowsQ)
        return 0;
    const int rows = s->batch * s->num_kv_heads;
    const int nrq = n_q * (s->num_q_heads / s->num_kv_heads);
    int splits = 1, per = 1;
    oasis::attn_split_plan(rows, n_blk, &splits, &per);
    // partials, then a hand-over flag and an epoch per row (16-byte padded)
    return (size_t)rows * splits * nrq * (s->head_dim + 2) * sizeof(float) +
           (((size_t)rows * 2 * sizeof(uint32_t) + 15) & ~(size_t)15);
}

// A token per attention call: the two workgroups of a row exchange it in the
// row's flag to find which of them merges (the flag need not start at any
// particular value, and returns to 0 after the call).  The call count is
// spread over the 32 bits by an odd multiplier, and the top and bottom bits
// are set, so a token is never 0 and never a small integer such as a block
// index left in a reused allocation.
static uint32_t next_attn_token() {
    static std::atomic<uint32_t> calls{0};
    const uint32_t t = calls.fetch_add(1, std::memory_order_relaxed) + 1;
    return (t * 0x9E3779B1u) | 0x80000001u;
}

int oasis_sparse_decode_attn(const oasis_shape *s, const uint16_t *q, int32_t n_q,
                             const uint16_t *k_pool, const uint16_t *v_pool,
                             const int32_t *page_table, const int32_t *blk, int32_t n_blk,
                             const int32_t *blk_logical, const int32_t *ctx_len, float scale,
                             uint16_t *out, void *workspace, size_t workspace_bytes,
                             void *stream) {
    return oasis_sparse_decode_attn_ex(s, q, n_q, k_pool, v_pool, page_table, blk, n_blk,
                                       blk_logical, ctx_len, scale, out, workspace,
                                       workspace_bytes, 0, stream);
}

int oasis_sparse_decode_attn_ex(const oasis_shape *s, const uint16_t *q, int32_t n_q,
                                const uint16_t *k_pool, const uint16_t *v_pool,
                                const int32_t *page_table, const int32_t *blk, int32_t n_blk,
                                const int32_t *blk_logical, const int32_t *ctx_len, float scale,
                                uint16_t *out, void *workspace, size_t workspace_bytes,
                                int32_t flags, void *stream) {
    const char *fn = "oasis_sparse_decode_attn";
    if (int e = check_shape(s, fn)) return e;
    if (flags & ~OASIS_ATTN_SHARE_GPU) return fail(OASIS_ERR_INVALID, "%s: unknown flags 0x%x", fn, flags);
    if (n_q < 1) return fail(OASIS_ERR_INVALID, "%s: n_q %d < 1", fn, n_q);
    if (n_blk < 1) return fail(OASIS_ERR_INVALID, "%s: n_blk %d < 1", fn, n_blk);
    if (n_blk > oasis::kMaxAttnBlocks)
        return fail(OASIS_ERR_UNSUPPORTED, "%s: n_blk %d above %d", fn, n_blk, oasis::kMaxAttnBlocks);
    const int G = s->num_q_heads / s->num_kv_heads;
    if ((long long)n_q * G > oasis::kMaxAttnRowsQ)
        return fail(OASIS_ERR_UNSUPPORTED, "%s: n_q * group = %lld above %d", fn,
                    (long long)n_q * G, oasis::kMaxAttnRowsQ);
    if (!(scale > 0.f) || !isfinite(scale))
        return fail(OASIS_ERR_INVALID, "%s: scale must be finite and > 0", fn);
    if (s->batch == 0) return ok();
    if (!q || !k_pool || !v_pool || !page_table || !ctx_len || !out)
        return fail(OASIS_ERR_INVALID, "%s: NULL pointer argument", fn);
    if (!blk && !blk_logical)
        return fail(OASIS_ERR_INVALID, "%s: blk and blk_logical are both NULL", fn);
    if (misaligned16(q) || misaligned16(k_pool) || misaligned16(v_pool))
        return fail(OASIS_ERR_INVALID, "%s: q, k_pool and v_pool must be 16-byte aligned", fn);
    const size_t need = oasis_attn_workspace_bytes(s, n_q, n_blk);
    if (!workspace || workspace_bytes < need)
        return fail(OASIS_ERR_NOMEM, "%s: workspace %zu bytes, %zu needed", fn, workspace_bytes, need);
    if (misaligned16(workspace))
        return fail(OASIS_ERR_INVALID, "%s: workspace must be 16-byte aligned", fn);
    const int rows = s->batch * s->num_kv_heads;
    int splits = 1, per = 1;
    oasis::attn_split_plan(rows, n_blk, &splits, &per);
    const int nrq = n_q * G;
    float *part_o = static_cast<float *>(workspace);
    float *part_ml = part_o + (size_t)rows * splits * nrq * s->head_dim;
    uint32_t *row_flag = reinterpret_cast<uint32_t *>(part_ml + (size_t)rows * splits * nrq * 2);
    uint32_t *row_epoch = row_flag + rows;
    oasis::AttnArgs a{q, k_pool, v_pool, page_table, blk, blk_logical, ctx_len, out,
                      part_o, part_ml, row_flag, row_epoch, next_attn_token(),
                      scale * 1.4426950408889634f,
                      s->batch, s->num_q_heads, s->num_kv_heads, G, s->table_width,
                      s->num_pages, n_q, nrq, n_blk, splits, per};
    return check_hip(oasis::launch_sparse_decode_attn(a, s->head_dim, (flags & OASIS_ATTN_SHARE_GPU) != 0,
                                                      as_stream(stream), t_stage_stop), fn);
}

}  // extern "C"

// Device-resident workspace of oasis_sparse_decode_attn_noalloc, for callers
// that cannot allocate.  In host code the name `scratch` is only a host-side
// stand-in for the array: its device address on each GPU comes from
// hipGetSymbolAddress (with that GPU current), kept in g_scratch_ptr, and
// only that address is ever handed to a kernel.
static __device__ __align__(256) unsigned char scratch[OASIS_ATTN_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::once_flag g_scratch_once[kMaxScratchDevices];
void *g_scratch_ptr[kMaxScratchDevices];
hipError_t g_scratch_err[kMaxScratchDevices];

// The current device's scratch address (looked up once per device).
int scratch_for_current_device(void **ptr, const char *fn) {
    int device = -1;
    if (int e = check_hip(hipGetDevice(&device), fn)) return e;
    if (device < 0 || device >= kMaxScratchDevices)
        return fail(OASIS_ERR_UNSUPPORTED, "%s: device %d above the %d this library keeps scratch for",
                    fn, device, kMaxScratchDevices);
    std::call_once(g_scratch_once[device], [device] {
        void *p = nullptr;
        g_scratch_err[device] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[device] = g_scratch_err[device] == hipSuccess ? p : nullptr;
    });
    if (g_scratch_err[device] != hipSuccess || !g_scratch_ptr[device])
        return fail(OASIS_ERR_HIP, "%s: hipGetSymbolAddress of the scratch array on device %d: %s",
                    fn, device, hipGetErrorString(g_scratch_err[device]));
    *ptr = g_scratch_ptr[device];
    return OASIS_OK;
}

}  // namespace

extern "C" {

int oasis_sparse_decode_attn_noalloc(const oasis_shape *s, const uint16_t *q, int32_t n_q,
                                     const uint16_t *k_pool, const uint16_t *v_pool,
                                     const int32_t *page_table, const int32_t *blk, int32_t n_blk,
                                     const int32_t *blk_logical, const int32_t *ctx_len,
                                     float scale, uint16_t *out, int32_t flags, void *stream) {
    const char *fn = "oasis_sparse_decode_attn_noalloc";
    if (int e = check_shape(s, fn)) return e;
    if (flags & ~OASIS_ATTN_SHARE_GPU) return fail(OASIS_ERR_INVALID, "%s: unknown flags 0x%x", fn, flags);
    if (n_q < 1) return fail(OASIS_ERR_INVALID, "%s: n_q %d < 1", fn, n_q);
    if (n_blk < 1) return fail(OASIS_ERR_INVALID, "%s: n_blk %d < 1", fn, n_blk);
    const size_t need = oasis_attn_workspace_bytes(s, n_q, n_blk);
    if (need == 0)       // nothing to do, or a shape the attention call refuses: it says which
        return oasis_sparse_decode_attn_ex(s, q, n_q, k_pool, v_pool, page_table, blk, n_blk,
                                           blk_logical, ctx_len, scale, out, nullptr, 0, flags,
                                           stream);
    if (need > OASIS_ATTN_SCRATCH_BYTES)
        return fail(OASIS_ERR_NOMEM, "%s: this shape needs %zu bytes of workspace, above the %u "
                    "bytes of the static scratch array; call oasis_sparse_decode_attn with a "
                    "workspace of your own", fn, need, (unsigned)OASIS_ATTN_SCRATCH_BYTES);
    void *ws = nullptr;
    if (int e = scratch_for_current_device(&ws, fn)) return e;
    return oasis_sparse_decode_attn_ex(s, q, n_q, k_pool, v_pool, page_table, blk, n_blk,
                                       blk_logical, ctx_len, scale, out, ws,
                                       OASIS_ATTN_SCRATCH_BYTES, flags, stream);
}

int oasis_layer_step(const oasis_layer *L, const uint16_t *q_look_next, const uint16_t *q,
                     float *scores, int32_t step, const oasis_step_sync *sync) {
    const char *fn = "oasis_layer_step";
    if (!L || !sync) return fail(OASIS_ERR_INVALID, "%s: NULL layer or sync", fn);
    if (!sync->scored || (sync->plan_stream != sync->attn_stream && !sync->attended))
        return fail(OASIS_ERR_INVALID, "%s: the scored / attended events are required", fn);
    hipStream_t ss = as_stream(sync->score_stream), as = as_stream(sync->attn_stream),
                ps = as_stream(sync->plan_stream);
    const auto ev = [](void *e) { return reinterpret_cast<hipEvent_t>(e); };
    // Each stage's completion event is recorded by its last kernel launch;
    // a stage that launched nothing records it as a command of its own.
    const auto run_stage = [&](void *event, hipStream_t stream, auto &&enqueue) -> int {
        oasis::LaunchStop st;
        st.event = ev(event);
        t_stage_stop = event ? &st : nullptr;
        const int e = enqueue();
        t_stage_stop = nullptr;
        if (e) return e;
        if (event && !st.used) return check_hip(hipEventRecord(ev(event), stream), fn);
        return OASIS_OK;
    };
    if (sync->inputs) {
        if (int e = check_hip(hipEventRecord(ev(sync->inputs), as), fn)) return e;
        if (int e = check_hip(hipStreamWaitEvent(ss, ev(sync->inputs), 0), fn)) return e;
    }
    if (sync->score_after)
        if (int e = check_hip(hipStreamWaitEvent(ss, ev(sync->score_after), 0), fn)) return e;
    const uint16_t *skp = L->score_k_pool ? L->score_k_pool : L->k_pool;
    // Two copies of the working-set table (slot_block_next set): the plan of
    // step s writes copy s & 1 (copy 1 = the *_next arrays) from copy
    // (s - 1) & 1, which this call's attention (of step s - 1) reads.
    const bool two = L->slot_block_next != nullptr;
    if (two != (L->last_use_next != nullptr))
        return fail(OASIS_ERR_INVALID, "%s: slot_block_next and last_use_next go together", fn);
    const bool odd = (step & 1) != 0;
    int32_t *sb_out = two && odd ? L->slot_block_next : L->slot_block;
    int32_t *lu_out = two && odd ? L->last_use_next : L->last_use;
    int32_t *sb_cur = two && !odd ? L->slot_block_next : L->slot_block;
    int32_t *lu_cur = two && !odd ? L->last_use_next : L->last_use;
    int e = run_stage(sync->scored, ss, [&] {
        return L->ck ? oasis_score_blocks_minmax(&L->shape, q_look_next, L->n_look, L->ck,
                                                 L->refresh ? skp : nullptr,
                                                 L->refresh ? L->block_table : nullptr, L->ctx_len,
                                                 L->scale, scores, ss)
                     : oasis_score_blocks(&L->shape, q_look_next, L->n_look, skp, L->block_table,
                                          L->ctx_len, L->scale, scores, ss);
    });
    if (e) return e;
    if (sync->attn_after)
        if ((e = check_hip(hipStreamWaitEvent(as, ev(sync->attn_after), 0), fn))) return e;
    e = run_stage(ps != as ? sync->attended : nullptr, as, [&] {
        return oasis_sparse_decode_attn_ex(&L->shape, q, L->n_q, L->k_pool, L->v_pool,
                                           L->block_table, sb_cur, L->k_blocks, sb_cur, L->ctx_len,
                                           L->scale, L->out, L->workspace, L->workspace_bytes,
                                           L->attn_flags, as);
    });
    if (e) return e;
    // the plan rewrites the table copy that the attention waited for here
    // last read: this call's attention, or with two copies (plan_after set)
    // the attention of the call before
    if (ps != as) {
        void *after = two && sync->plan_after ? sync->plan_after : sync->attended;
        if ((e = check_hip(hipStreamWaitEvent(ps, ev(after), 0), fn))) return e;
    }
    if (ps != ss)
        if ((e = check_hip(hipStreamWaitEvent(ps, ev(sync->scored), 0), fn))) return e;
    return run_stage(sync->planned, ps, [&] {
        return oasis_select_plan_next(&L->shape, scores, L->ctx_len, L->k_blocks, L->cap, step,
                                      nullptr, L->sel, sb_cur, lu_cur, sb_out, lu_out,
                                      L->fetch_block, L->fetch_slot, L->fetch_count,
                                      L->select_workspace, L->select_workspace_bytes, ps);
    });
}

int oasis_hostpool_create(size_t bytes, void **host_ptr) {
    const char *fn = "oasis_hostpool_create";
    if (!host_ptr) return fail(OASIS_ERR_INVALID, "%s: host_ptr is NULL", fn);
    *host_ptr = nullptr;
    if (bytes == 0) return fail(OASIS_ERR_INVALID, "%s: zero bytes", fn);
    void *p = nullptr;
    const hipError_t e = hipHostMalloc(&p, bytes, OASIS_HOSTPOOL_FLAGS);
    if (e != hipSuccess || !p) {
        (void)hipGetLastError();
        return fail(OASIS_ERR_NOMEM, "%s: hipHostMalloc of %zu bytes failed: %s", fn, bytes,
                    hipGetErrorString(e));
    }
    *host_ptr = p;
    return ok();
}

int oasis_hostpool_device_pointer(void *host_ptr, void **device_ptr) {
    const char *fn = "oasis_hostpool_device_pointer";
    if (!host_ptr || !device_ptr) return fail(OASIS_ERR_INVALID, "%s: NULL pointer argument", fn);
    *device_ptr = nullptr;
    return check_hip(hipHostGetDevicePointer(device_ptr, host_ptr, 0), fn);
}

int oasis_hostpool_destroy(void *host_ptr) {
    const char *fn = "oasis_hostpool_destroy";
    if (!host_ptr) return ok();
    return check_hip(hipHostFree(host_ptr), fn);
}

int oasis_fetch_blocks(const oasis_shape *s, const uint16_t *host_k, const uint16_t *host_v,
                       int32_t host_blocks, const int32_t *fetch_block, const int32_t *fetch_slot,
                       const int32_t *fetch_count, int32_t cap, const int32_t *ws_page_table,
                       uint16_t *ws_k_pool, uint16_t *ws_v_pool, void *stream) {
    const char *fn = "oasis_fetch_blocks";
    if (int e = check_shape(s, fn)) return e;
    if (host_blocks < 1) return fail(OASIS_ERR_INVALID, "%s: host_blocks %d < 1", fn, host_blocks);
    if (cap < 0 || cap > s->table_width)
        return fail(OASIS_ERR_INVALID, "%s: cap %d outside [0, table_width = %d]", fn, cap,
                    s->table_width);
    if (s->batch == 0 || cap == 0) return ok();
    if (!host_k || !host_v || !fetch_block || !fetch_slot || !fetch_count || !ws_page_table ||
        !ws_k_pool || !ws_v_pool)
        return fail(OASIS_ERR_INVALID, "%s: NULL pointer argument", fn);
    if (misaligned16(host_k) || misaligned16(host_v) || misaligned16(ws_k_pool) ||
        misaligned16(ws_v_pool))
        return fail(OASIS_ERR_INVALID, "%s: host and working-set pools must be 16-byte aligned", fn);
    oasis::FetchArgs a{host_k, host_v, fetch_block, fetch_slot, fetch_count, ws_page_table,
                       ws_k_pool, ws_v_pool, s->batch, s->num_kv_heads, host_blocks,
                       s->table_width, cap, s->num_pages};
    return check_hip(oasis::launch_fetch_blocks(a, s->head_dim, as_stream(stream)), fn);
}

}  // extern "C"
