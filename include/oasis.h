/*
 * oasis.h -- C ABI of the OasisKV decode hot path for MI355X (gfx950).
 *
 * The method ("OasisKV: Scaling In-Decode KV Cache Beyond HBM with Lookahead
 * Sparse Prefetching", arXiv 2608.08097): a lookahead (draft) query predicts,
 * one decode step ahead, which KV blocks the next step will attend to; only
 * those blocks are kept in a bounded HBM working set under a token budget,
 * and the missing ones are fetched under a per-step cap.  One decode step of
 * one layer is four calls, each a hand-written HIP kernel:
 *
 *   oasis_score_blocks       lookahead-query block scores over the paged keys
 *   oasis_select_topk        top-K blocks per KV head under the budget
 *   oasis_plan_fetch         resident diff + fetch cap + LRU eviction, which
 *                            updates the per-head working-set table
 *   oasis_sparse_decode_attn sparse paged decode attention over the working set
 *                            (oasis_sparse_decode_attn_ex: the same with launch hints)
 *
 * and, for the pages' own compressed-key scorer, oasis_pool_keys (min/max
 * pooling of the keys) and oasis_score_blocks_minmax (scores from them).
 * oasis_select_plan runs select and plan as one launch (oasis_select_plan_ex:
 * with the step number partly in device memory); oasis_layer_step enqueues a
 * whole overlapped layer-step (score, attention, select + plan and the event
 * edges between their streams) in one call; oasis_hostpool_* and
 * oasis_fetch_blocks are the pinned host tier and its capped fetch.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Pointers are DEVICE pointers unless a comment says otherwise.  Every
 *    buffer is caller-owned; no call allocates device memory.
 *  - bf16 tensors are passed as uint16_t bit patterns.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Calls
 *    only enqueue work and never synchronise.
 *  - Arguments are validated on the host before anything is enqueued; a
 *    failing call enqueues nothing and returns a non-zero status, with detail
 *    text from oasis_last_error() (thread-local).  Device-side faults surface
 *    at the caller's next synchronisation.
 *  - Device-resident indices (block tables, context lengths, block lists) are
 *    bounds-checked inside the kernels: a page id outside [0, num_pages) or a
 *    negative list entry makes that block count as absent (score -inf, not
 *    attended) instead of being dereferenced; a context longer than
 *    table_width * block_size is clamped to it.
 *  - Calls are reentrant; the library keeps no state besides the error text
 *    and a count of attention calls (the source of their tokens).
 *
 * Layouts (row-major, innermost last):
 *  - lookahead queries  q_look  [B][n_look][Hq][D]    bf16
 *  - true queries       q       [B][n_q][Hq][D]       bf16
 *  - key pool           k_pool  [num_pages][Hkv][bs*D]   bf16; each (page, head)
 *                       tile in 8-dimension slices [D/8][bs][8]: element
 *                       (token t, dim d) at ((d / 8) * bs + t) * 8 + d % 8, so a
 *                       16-byte-per-lane load of an MFMA operand reads 1 KiB of
 *                       contiguous memory
 *  - value pool         v_pool  [num_pages][Hkv][D][bs]  bf16 (dim-major tile)
 *  - block table        [B][table_width]  int32, logical block -> page
 *  - context lengths    ctx_len [B]       int32, tokens
 *  - scores             [B][Hkv][table_width]  fp32
 *  - compressed keys    ck      [B][Hkv][ceil(W/16)][2D/8][16][8] bf16: per row,
 *                       tiles of 16 blocks; in a tile, slice s holds elements
 *                       8s .. 8s+7 of every block's [min(D) | max(D)] vector, so
 *                       (block n, element e) is at tile n/16, slice e/8,
 *                       position (n % 16) * 8 + e % 8
 *  - selection          sel     [B][Hkv][K]     int32, ascending, -1 padded
 *  - working-set table  slot_block, last_use [B][Hkv][K] int32
 *  - fetch list         fetch_block, fetch_slot [B][Hkv][cap] int32, -1 padded;
 *                       fetch_count [B][Hkv] int32
 *  - output             out     [B][n_q][Hq][D]       bf16
 * Query head h belongs to KV head h / G, G = Hq / Hkv (grouped-query attention).
 */
#ifndef OASIS_H
#define OASIS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum oasis_status {
    OASIS_OK = 0,
    OASIS_ERR_INVALID = 1,      /* null pointer, negative size, inconsistent shape   */
    OASIS_ERR_UNSUPPORTED = 2,  /* valid but outside what the kernels implement     */
    OASIS_ERR_NOMEM = 3,        /* workspace too small / host pool allocation failed */
    OASIS_ERR_HIP = 4           /* the HIP runtime reported an error                 */
};

typedef struct oasis_shape {
    int32_t batch;          /* B, sequences (0 allowed: the call does nothing)          */
    int32_t num_q_heads;    /* Hq                                                        */
    int32_t num_kv_heads;   /* Hkv; Hq must be a multiple of Hkv                         */
    int32_t head_dim;       /* D: 64 or 128                                              */
    int32_t block_size;     /* tokens per KV block: 16                                   */
    int32_t table_width;    /* W, entries per block-table row (blocks per sequence max)  */
    int32_t num_pages;      /* pages in k_pool / v_pool                                  */
} oasis_shape;

/*
 * Lookahead block scoring.  Figure 7 caption of the pages (metalmedia.ai
 * summary of OasisKV): the draft query scans the keys to predict the next
 * step's top-K blocks.  The pages leave the score open; this library fixes it:
 *
 *   scores[b][g][n] = max over drafts j < n_look, query heads h of KV head g,
 *                     and tokens t of block n with 16n + t < ctx_len[b] of
 *                     scale * (q_look[b][j][h] . k_t)
 *   scores[b][g][n] = -inf for n >= ceil(ctx_len[b] / bs) (up to table_width).
 *
 * bf16 inputs, fp32 accumulation.  Requires D in {64, 128}, bs = 16,
 * 1 <= n_look and n_look * G <= 16, q_look and k_pool 16-byte aligned.  scale
 * is normally 1/sqrt(D) and must be > 0.
 */
int oasis_score_blocks(const oasis_shape *s, const uint16_t *q_look, int32_t n_look,
                       const uint16_t *k_pool, const int32_t *block_table,
                       const int32_t *ctx_len, float scale, float *scores, void *stream);

/*
 * Compressed keys by per-block min/max pooling.  Figure 7 caption: beside the
 * sparse KV working set the GPU keeps the keys compressed by per-block min/max
 * pooling, for the draft query to scan.
 *
 *   min[b][g][n][d], max[b][g][n][d] = min and max of k_t[d] over the tokens
 *   t of block n with 16n + t < ctx_len[b]      (ck layout: see "Layouts" above)
 *
 * last_only = 0 writes every block n < ceil(ctx_len[b] / bs); last_only = 1
 * only block ceil(ctx_len[b] / bs) - 1 of each sequence (the one a decode step
 * appends its token to; it is recomputed from the pool, so the call may be
 * repeated).  Blocks at or past the context are not written.  A page id
 * outside [0, num_pages) is not read: that block is written as an empty box
 * (min = +inf, max = -inf), which oasis_score_blocks_minmax scores -inf.  The
 * values are bf16 keys themselves, so the pooling is exact.
 * Requires D in {64, 128}, bs = 16, k_pool and ck 16-byte aligned;
 * last_only must be 0 or 1.
 */
int oasis_pool_keys(const oasis_shape *s, const uint16_t *k_pool, const int32_t *block_table,
                    const int32_t *ctx_len, int32_t last_only, uint16_t *ck, void *stream);

/*
 * Lookahead block scoring from the compressed keys (Figure 7 caption: the
 * draft query scans the compressed keys to predict the next step's top-K
 * blocks).  The pages name the pooling, not the score; this library takes the
 * largest value q . x can reach inside the block's box min <= x <= max:
 *
 *   scores[b][g][n] = max over drafts j < n_look and query heads h of KV head g
 *                     of scale * sum_d max(q_d * min_d, q_d * max_d),
 *                     q = q_look[b][j][h], (min, max) = block n of row (b, g) in ck
 *   scores[b][g][n] = -inf for n >= ceil(ctx_len[b] / bs) and for empty boxes.
 *
 * An upper bound of oasis_score_blocks' exact score, equal to it for a block
 * of one token; it reads 2D values per block instead of 16D.  bf16 inputs,
 * fp32 accumulation.  The output feeds oasis_select_topk / oasis_select_plan
 * unchanged.
 *
 * k_pool and block_table (both set, or both NULL): in the same launch, the
 * last block of each sequence (ceil(ctx_len[b] / bs) - 1, the one a decode
 * step appends its token to) is first re-pooled from the key pool exactly as
 * oasis_pool_keys(last_only = 1) would, its row of ck is written, and it is
 * scored from the fresh values.  This keeps ck current for decode without a
 * separate launch.  ck is only read when both are NULL.
 *
 * Requires D in {64, 128}, bs = 16, 1 <= n_look, n_look * G <= 16, scale > 0;
 * q_look, ck and k_pool 16-byte aligned.
 */
int oasis_score_blocks_minmax(const oasis_shape *s, const uint16_t *q_look, int32_t n_look,
                              uint16_t *ck, const uint16_t *k_pool, const int32_t *block_table,
                              const int32_t *ctx_len, float scale, float *scores, void *stream);

/*
 * Per-KV-head top-K.  Figure 7 caption ("top-K blocks"); abstract (a
 * 2,048-token KV budget, i.e. K = budget / bs blocks per KV head).
 * Among blocks n < ceil(ctx_len[b] / bs), the k_blocks largest scores win;
 * equal scores go to the lower block index (-0.0 equals +0.0).  sel is written
 * in ascending block order, padded with -1 when fewer blocks exist.
 * Requires 1 <= k_blocks <= 1024 and table_width <= 15360.  Scores must not be NaN.
 */
int oasis_select_topk(const oasis_shape *s, const float *scores, const int32_t *ctx_len,
                      int32_t k_blocks, int32_t *sel, void *stream);

/*
 * Resident diff + fetch cap + capped LRU eviction, one row per (sequence,
 * KV head).  Pages: five-step flow step 3 (compare the prediction with the
 * blocks already on the GPU and pull only the missing ones, with a per-step
 * bound); Figure 9 caption (per-KV-head table from working-set block to CPU
 * logical block); Table 2 caption (the cap is a fetch ratio; LRU eviction).
 *
 * slot_block[b][g][j] is the logical block held by working-set slot j (-1 =
 * empty) and last_use[b][g][j] the step it was last used; both are read and
 * updated in place.  For each row:
 *   1. resident selected blocks (hits) get last_use = step;
 *   2. the selected blocks that are not resident (misses) are ranked by score
 *      (descending, ties to the lower index); the first min(#misses, cap) are
 *      fetched and listed in ascending block order;
 *   3. their destinations are the empty slots in ascending order, then -- if
 *      more are needed -- exactly that many resident blocks that are not
 *      selected, least recently used first (ties to the lower block index);
 *      a selected block is never evicted;
 *   4. slot_block / last_use of each destination become (block, step).
 * fetch_block[i] / fetch_slot[i] (i < fetch_count) list the fetched blocks and
 * their slots, -1 padded up to cap.  `scores` is the scoring output [B][Hkv][W].
 * Requires 1 <= k_blocks <= 1024, 0 <= cap <= k_blocks; when cap == 0 the
 * fetch_block / fetch_slot pointers may be NULL.  Precondition: no row of
 * slot_block holds a block twice (no plan produces such a row).  Where one
 * does and enough blocks can still be evicted, the plan is still the one
 * above, the copies of a block ranked for eviction by slot (lower first).
 */
int oasis_plan_fetch(const oasis_shape *s, const int32_t *sel, const float *scores,
                     int32_t k_blocks, int32_t cap, int32_t step, int32_t *slot_block,
                     int32_t *last_use, int32_t *fetch_block, int32_t *fetch_slot,
                     int32_t *fetch_count, void *stream);

/*
 * oasis_select_topk followed by oasis_plan_fetch on the same row, as one
 * launch when k_blocks <= 512 and table_width <= 8192 (one workgroup per row;
 * the selection never leaves the chip between the two), else as the two calls.
 * Results are identical to the two calls; `sel` receives the selection.
 * Same arguments, requirements and errors as the two calls together.
 */
int oasis_select_plan(const oasis_shape *s, const float *scores, const int32_t *ctx_len,
                      int32_t k_blocks, int32_t cap, int32_t step, int32_t *sel,
                      int32_t *slot_block, int32_t *last_use, int32_t *fetch_block,
                      int32_t *fetch_slot, int32_t *fetch_count, void *stream);

/*
 * oasis_select_plan with the step number partly in device memory: the plan
 * uses step + *step_dev (step_dev may be NULL: step alone).  For callers that
 * capture the decode step in a HIP graph and replay it: kernel arguments are
 * fixed at capture, so the step number that the LRU order needs comes from a
 * counter the graph advances on the device.  Same results as
 * oasis_select_plan called with that sum.
 */
int oasis_select_plan_ex(const oasis_shape *s, const float *scores, const int32_t *ctx_len,
                         int32_t k_blocks, int32_t cap, int32_t step, const int32_t *step_dev,
                         int32_t *sel, int32_t *slot_block, int32_t *last_use,
                         int32_t *fetch_block, int32_t *fetch_slot, int32_t *fetch_count,
                         void *stream);

/*
 * Top-K (and the plan) of rows of up to 65,536 blocks and more, with a
 * workspace.  Rows of at most 8,192 blocks take the one-pass kernels of
 * oasis_select_plan (the workspace is then not needed; pass NULL).  Wider
 * rows take two passes: each row is split into chunks of at least 2,048
 * blocks, one workgroup per chunk writes the chunk's top-K to the workspace
 * as candidates, then one workgroup per row selects the top-K of its
 * candidates (every block of the row's top-K is among its chunk's top-K, and
 * candidates are kept in block order, so ties still go to the lower block)
 * and plans it.  Results are those of oasis_select_topk / oasis_plan_fetch.
 * slot_block == NULL selects only (last_use, fetch_block, fetch_slot,
 * fetch_count and cap are then unused).  Requires 1 <= k_blocks <= 1024,
 * table_width <= 8192 * (8192 / k_blocks) (65,536 at k_blocks = 1024), and a
 * workspace of oasis_select_workspace_bytes() bytes, 8-byte aligned, any
 * contents (OASIS_ERR_NOMEM if smaller).  step_dev as in oasis_select_plan_ex.
 */
size_t oasis_select_workspace_bytes(const oasis_shape *s, int32_t k_blocks);
int oasis_select_plan_ws(const oasis_shape *s, const float *scores, const int32_t *ctx_len,
                         int32_t k_blocks, int32_t cap, int32_t step, const int32_t *step_dev,
                         int32_t *sel, int32_t *slot_block, int32_t *last_use,
                         int32_t *fetch_block, int32_t *fetch_slot, int32_t *fetch_count,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * oasis_select_plan_ws with the plan starting from the working-set table
 * (slot_block_in, last_use_in) and writing the planned table to (slot_block,
 * last_use).  An output array is either its input array itself (in place,
 * as oasis_select_plan_ws) or shares no entry with either input array; the
 * inputs are only read.  Keeping two copies of the table and planning from
 * one into the other lets the plan of step t + 1 run while the attention of
 * step t still reads the table of step t (flow step 4 and Figure 8 caption:
 * the next step's prediction overlaps the current step's attention), instead
 * of waiting for it.  Results are those of oasis_select_plan_ws on a copy of
 * the input table.  Same requirements and errors, plus OASIS_ERR_INVALID for
 * NULL table arrays or for tables that overlap otherwise than in place.
 */
int oasis_select_plan_next(const oasis_shape *s, const float *scores, const int32_t *ctx_len,
                           int32_t k_blocks, int32_t cap, int32_t step, const int32_t *step_dev,
                           int32_t *sel, const int32_t *slot_block_in, const int32_t *last_use_in,
                           int32_t *slot_block, int32_t *last_use, int32_t *fetch_block,
                           int32_t *fetch_slot, int32_t *fetch_count, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * Bytes of device workspace oasis_sparse_decode_attn needs for this shape:
 * room for the partial results of a row's shares (per row and share: max,
 * sum and the D-wide output of each query row), then a 32-bit hand-over flag
 * and a 32-bit hand-over epoch per row (B * Hkv rows each), padded to 16
 * bytes.  The workspace needs no initialisation.  Where a row is split
 * between two workgroups, each publishes its partial as 64-bit words that
 * carry a tag (the call's token mixed with the row's epoch) beside each
 * value, then reads its partner's: the one that finds its partner's words
 * all tagged merges; when neither does, an exchange of the tag in the row's
 * flag picks the one that waits for its partner's words.  A merging
 * workgroup advances the row's epoch, so the tag changes from call to call
 * even where the token does not (a call replayed from a captured graph), and
 * words left by other calls or shapes do not carry it.  One workspace serves
 * one call at a time.  Returns 0 for an invalid shape.
 */
size_t oasis_attn_workspace_bytes(const oasis_shape *s, int32_t n_q, int32_t n_blk);

/*
 * Sparse paged decode attention over the working set.  Figure 7 caption:
 * attention runs over the sparse KV working set.  For each sequence b, query
 * row i < n_q and head h of KV head g:
 *
 *   out[b][i][h] = sum_t softmax_t(scale * q[b][i][h] . k_t) v_t
 *
 * over every valid token t of the row's listed blocks.  Entry e of row
 * (b, g) names the block
 *   blk[b][g][e]  -- an index into page_table row b (-1 = empty entry);
 *                    blk == NULL means entry e is index e itself;
 *   blk_logical[b][g][e] -- its logical block number (token 16*l + t is valid
 *                    while < ctx_len[b]; -1 = empty entry);
 * full-pool mode passes the block table as page_table and the selected (or
 * resident) logical blocks as both blk and blk_logical; working-set mode
 * passes the slot -> page table and blk = NULL, blk_logical = slot_block.
 * The n_q query rows of a sequence are independent: with the normal query
 * and the draft queries of a speculative step as rows i = 0 .. n_q - 1, one
 * call attends them all in a single pass over the sparse KV (Figure 7
 * caption: the attention kernel takes the normal and the draft queries
 * together).
 * A row with no valid token outputs zeros.  bf16 in and out, fp32 softmax and
 * accumulation.  Requires D in {64, 128}, bs = 16, 1 <= n_q, n_q * G <= 32,
 * 1 <= n_blk <= 65536, scale > 0, q, k_pool, v_pool and workspace 16-byte aligned, and
 * workspace_bytes >= oasis_attn_workspace_bytes().
 *
 * Launch shape (results agree to fp32 rounding whichever is taken), by rows
 * (B * Hkv) and query rows per KV head (n_q * G):
 *   - 256 rows or more, at most 16 query rows: one workgroup per row merges
 *     its waves in LDS;
 *   - 128 to 255 rows, and at least 31 listed entries per row: two
 *     workgroups per row (8 waves each up to 16 query rows; 4 waves with two
 *     column tiles for 17..32 query rows while their partials fit in 64 KiB
 *     of LDS), the second to finish merging both through the workspace;
 *   - otherwise split-K waves and a second merge launch.
 */
int oasis_sparse_decode_attn(const oasis_shape *s, const uint16_t *q, int32_t n_q,
                             const uint16_t *k_pool, const uint16_t *v_pool,
                             const int32_t *page_table, const int32_t *blk, int32_t n_blk,
                             const int32_t *blk_logical, const int32_t *ctx_len, float scale,
                             uint16_t *out, void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * oasis_sparse_decode_attn with launch hints.  flags = 0 is that call.
 * OASIS_ATTN_SHARE_GPU: another launch (the next step's scoring) runs beside
 * this one; from 128 rows attention then keeps to one workgroup (one CU) per
 * row, which leaves CUs to the concurrent launch.  Other bits:
 * OASIS_ERR_INVALID.
 */
#define OASIS_ATTN_SHARE_GPU 1
int oasis_sparse_decode_attn_ex(const oasis_shape *s, const uint16_t *q, int32_t n_q,
                                const uint16_t *k_pool, const uint16_t *v_pool,
                                const int32_t *page_table, const int32_t *blk, int32_t n_blk,
                                const int32_t *blk_logical, const int32_t *ctx_len, float scale,
                                uint16_t *out, void *workspace, size_t workspace_bytes,
                                int32_t flags, void *stream);

/*
 * oasis_sparse_decode_attn_ex without a workspace argument and without any
 * allocation, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * split partials and hand-over flags live in a static device array of
 * OASIS_ATTN_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends; its address on the current device is looked up on
 * the first call there.  Same inputs, outputs, results and launch shapes as
 * oasis_sparse_decode_attn_ex.
 * Errors: as oasis_sparse_decode_attn_ex, plus OASIS_ERR_NOMEM when the shape
 * needs more than OASIS_ATTN_SCRATCH_BYTES (oasis_attn_workspace_bytes tells);
 * OASIS_ERR_HIP if the array's address cannot be had.  The array keeps the
 * last call's contents and nothing in it needs clearing (the hand-over flags
 * need no initial value; the array starts at zero and each call returns its
 * flags to zero).  Calls that overlap on one GPU (on different streams, or
 * from different threads) share the array and race: serialise them.
 */
#define OASIS_ATTN_SCRATCH_BYTES (16u << 20)
int oasis_sparse_decode_attn_noalloc(const oasis_shape *s, const uint16_t *q, int32_t n_q,
                                     const uint16_t *k_pool, const uint16_t *v_pool,
                                     const int32_t *page_table, const int32_t *blk, int32_t n_blk,
                                     const int32_t *blk_logical, const int32_t *ctx_len,
                                     float scale, uint16_t *out, int32_t flags, void *stream);

/*
 * Pinned host KV pool, the tier the working set is fetched from.  The pages
 * keep the full KV cache in CPU memory and hold only a bounded working set in
 * HBM (abstract; Figure 7 caption).  oasis_hostpool_create allocates `bytes`
 * of page-locked host memory mapped into the device address space (host
 * pointer in *host_ptr; OASIS_ERR_NOMEM if the allocation fails);
 * oasis_hostpool_device_pointer gives the address kernels use for it;
 * oasis_hostpool_destroy frees it (after all work that reads it is done).
 * The caller fills the pool from the host.
 */
int oasis_hostpool_create(size_t bytes, void **host_ptr);
int oasis_hostpool_device_pointer(void *host_ptr, void **device_ptr);
int oasis_hostpool_destroy(void *host_ptr);

/*
 * Capped fetch host -> HBM.  Five-step flow step 3 (pull only the missing
 * blocks, bounded per step), Figure 8 caption (the transfer runs in the
 * background before that layer's attention at the next step), Figure 9
 * caption (working-set slots of each KV head).  For every row (b, g) and
 * i < fetch_count[b][g] (clamped to [0, cap]), copies logical block
 * fetch_block[b][g][i] of the host pool into working-set slot
 * fetch_slot[b][g][i], i.e. into page ws_page_table[b][slot] of the working-set
 * pools, for KV head g.  Layouts: host_k [B][Hkv][host_blocks][bs*D] (tiles in
 * the key pool's slice order) and
 * host_v [B][Hkv][host_blocks][D][bs] (device-mapped pointers from
 * oasis_hostpool_device_pointer); ws_page_table [B][table_width];
 * ws_k_pool [num_pages][Hkv][bs*D], ws_v_pool [num_pages][Hkv][D][bs].  Here
 * s->table_width is the number of slots K and s->num_pages the working-set
 * pages.  Entries with a block outside [0, host_blocks), a slot outside
 * [0, K) or a page outside [0, num_pages) are skipped.  The fetch lists are
 * those oasis_plan_fetch writes; the call reads them on the device, so no host
 * synchronisation is needed.  Requires 0 <= cap <= K and the four pools
 * 16-byte aligned.
 *
 * This is the path's fetch-issue call: enqueued on a side stream, it issues
 * the step's capped host -> HBM transfer.  It is a gather kernel rather than
 * a series of copy-engine copies (hipMemcpyAsync of each listed tile): the
 * copy engines pay a fixed cost per copy that 4 KiB tiles cannot amortise
 * (about 1.8 GB/s against 55 GB/s for the gather on MI355X), and a list of
 * copies would have to come back to the host first.
 */
int oasis_fetch_blocks(const oasis_shape *s, const uint16_t *host_k, const uint16_t *host_v,
                       int32_t host_blocks, const int32_t *fetch_block, const int32_t *fetch_slot,
                       const int32_t *fetch_count, int32_t cap, const int32_t *ws_page_table,
                       uint16_t *ws_k_pool, uint16_t *ws_v_pool, void *stream);

/*
 * One layer of the overlapped decode step, enqueued by one call: the three
 * calls of a step and the event waits and records that order them across
 * streams (flow step 4 and Figure 8 caption: the next step's prediction runs
 * ahead of, and overlaps, the current step's attention).  For host loops
 * whose kernels are short enough that a dozen runtime calls per layer and
 * step would bound the step.
 *
 * oasis_layer holds what does not change from step to step (caller-owned
 * device buffers, as in the calls named below); ck == NULL selects exact
 * scoring (oasis_score_blocks), else the compressed keys
 * (oasis_score_blocks_minmax, re-pooling each sequence's last block first
 * when refresh != 0).  oasis_step_sync holds hipStream_t / hipEvent_t
 * handles passed as void*; an event that is NULL is skipped.  The call
 * enqueues, in this order:
 *
 *   attn_stream:  record inputs (if set)
 *   score_stream: wait inputs (if set); wait score_after; scoring of
 *                 q_look_next into scores; record scored
 *   attn_stream:  wait attn_after; oasis_sparse_decode_attn_ex(attn_flags) of
 *                 q over the working set slot_block (full-pool mode: the block
 *                 table as page table); record attended if plan_stream differs
 *   plan_stream:  if it differs from attn_stream, wait attended (plan_after
 *                 with two table copies); if it differs from score_stream,
 *                 wait scored; oasis_select_plan_next(step) from scores, the
 *                 table read and written in place (slot_block / last_use) or,
 *                 with two copies, from one copy into the other; record planned
 *
 * and nothing else: the results are those of the three calls in that order.
 * Errors: the first failing call's status; the calls before it stay enqueued.
 */
typedef struct {
    oasis_shape shape;                 /* full-pool shape: num_pages = key pool pages */
    const uint16_t *k_pool, *v_pool;
    const int32_t *block_table, *ctx_len;
    uint16_t *ck;                      /* compressed keys, or NULL for exact scoring */
    int32_t refresh, n_look, n_q, k_blocks, cap, attn_flags;
    float scale;
    int32_t *sel, *slot_block, *last_use, *fetch_block, *fetch_slot, *fetch_count;
    uint16_t *out;
    void *workspace;
    size_t workspace_bytes;
    const uint16_t *score_k_pool;      /* scoring (and the re-pooling of the last block)
                                          reads this key pool when set, attention reads
                                          k_pool: keys kept in two pools by step parity,
                                          so that one step's keys can be rewritten while
                                          the step before is attended; NULL: k_pool */
    void *select_workspace;            /* oasis_select_plan_ws workspace (NULL where the
                                          table width needs none) */
    size_t select_workspace_bytes;
    int32_t *slot_block_next, *last_use_next;
                                       /* a second copy of the working-set table, or both
                                          NULL: the plan of step s writes copy s & 1 (copy 1
                                          = these arrays, copy 0 = slot_block / last_use)
                                          from copy (s - 1) & 1, which the attention of the
                                          call reads; so the next step's plan need not wait
                                          for this step's attention.  Both copies must hold
                                          the table before the first call; steps of
                                          consecutive calls must be consecutive */
} oasis_layer;

typedef struct {
    void *score_stream, *attn_stream, *plan_stream;
    void *score_after, *attn_after;    /* events waited on first (NULL: none) */
    void *scored, *attended, *planned; /* events recorded */
    void *inputs;                      /* recorded on attn_stream and waited on by score_stream
                                          before scoring, so that scoring sees q_look_next,
                                          ctx_len and appended keys written on attn_stream
                                          (the caller's stream) before the call; NULL: the
                                          caller orders those writes itself */
    void *plan_after;                  /* with two table copies: the event the previous
                                          call's attention recorded (`attended` then), which
                                          the plan waits for instead of this call's
                                          `attended`: that attention last read the copy the
                                          plan writes.  NULL: this call's `attended` */
} oasis_step_sync;

int oasis_layer_step(const oasis_layer *L, const uint16_t *q_look_next, const uint16_t *q,
                     float *scores, int32_t step, const oasis_step_sync *sync);

/* Human-readable name of a status code (static storage). */
const char *oasis_status_string(int status);

/* Detail text of the calling thread's last failed call ("" if none). */
const char *oasis_last_error(void);

/* Library version string (static storage). */
const char *oasis_version(void);

#ifdef __cplusplus
}
#endif

#endif /* OASIS_H */
