// oasis_launch.h -- argument blocks and launchers of the gfx950 kernels.
// Host-side validation lives in oasis_abi.hip; the launchers assume valid
// arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stddef.h>
#include <stdint.h>

namespace oasis {

struct ScoreArgs {
    const uint16_t *q_look;
    const uint16_t *k_pool;
    const int32_t *block_table;
    const int32_t *ctx_len;
    float *scores;
    float scale;
    int batch, hq, hkv, group, width, num_pages, n_look, n_rows_q;
};

struct SelectArgs {
    const float *scores;
    const int32_t *ctx_len;
    int32_t *sel;
    int rows, hkv, width, k;
};

struct SelectPlanArgs {
    const float *scores;
    const int32_t *ctx_len;
    int32_t *sel;          // select: output (may be null when planning too); plan only: input
    int32_t *slot_block;
    int32_t *last_use;
    int32_t *fetch_block;
    int32_t *fetch_slot;
    int32_t *fetch_count;
    int rows, hkv, width, k, cap, step;
    const int32_t *step_dev;   // if set, *step_dev is added to step (read on the device)
    // the working-set table the plan starts from (the plan writes slot_block /
    // last_use): the same arrays when planning in place
    const int32_t *slot_block_in;
    const int32_t *last_use_in;
};

// Candidates of the two-pass selection of wide rows: each row split into
// `chunks` chunks of chunk_w blocks; per (row, chunk) the chunk's top-K as
// order-preserving keys and block indices, in ascending block order, padded
// with key 0 and index -1.
struct ChunkArgs {
    const float *scores;
    const int32_t *ctx_len;
    uint32_t *cand_key;    // [rows][chunks][k]
    int32_t *cand_idx;     // [rows][chunks][k]
    int rows, hkv, width, k, chunk_w, chunks;
};

struct FetchArgs {
    const uint16_t *host_k;       // device-mapped pinned host pool, [B][Hkv][host_blocks][bs*D], key tiles in slices
    const uint16_t *host_v;       // [B][Hkv][host_blocks][D][bs]
    const int32_t *fetch_block;
    const int32_t *fetch_slot;
    const int32_t *fetch_count;
    const int32_t *ws_page_table; // [B][k_slots] slot -> working-set page
    uint16_t *ws_k;               // [ws_pages][Hkv][bs*D], key tiles in slices
    uint16_t *ws_v;               // [ws_pages][Hkv][D][bs]
    int batch, hkv, host_blocks, k_slots, cap, ws_pages;
};

struct AttnArgs {
    const uint16_t *q;
    const uint16_t *k_pool;
    const uint16_t *v_pool;
    const int32_t *page_table;
    const int32_t *blk;
    const int32_t *blk_logical;
    const int32_t *ctx_len;
    uint16_t *out;
    float *part_o;    // [rows][splits][n_rows_q][D]
    float *part_ml;   // [rows][splits][n_rows_q][2]
    uint32_t *row_flag;    // [rows] hand-over flags of a row's two workgroups (any initial value)
    uint32_t *row_epoch;   // [rows] hand-over epochs, advanced by each call (any initial value)
    uint32_t token;        // nonzero, different from call to call
    float scale_log2;
    int batch, hq, hkv, group, width, num_pages, n_q, n_rows_q, n_blk, splits, per_split;
};

// Min/max pooling of the paged keys into ck [B][Hkv][W][2][D] (all blocks, or
// only the last block of each sequence).
struct PoolArgs {
    const uint16_t *k_pool;
    const int32_t *block_table;
    const int32_t *ctx_len;
    uint16_t *ck;
    int batch, hkv, width, num_pages, last_only;
};

// Block scores from the compressed keys; with k_pool set, the last block of
// each sequence is first re-pooled from the key pool (ck written) and scored
// from the fresh values.
struct MinmaxArgs {
    const uint16_t *q_look;
    uint16_t *ck;
    const uint16_t *k_pool;        // NULL: no refresh
    const int32_t *block_table;
    const int32_t *ctx_len;
    float *scores;
    float scale;
    int batch, hq, hkv, group, width, num_pages, n_look, n_rows_q;
};

// Compressed keys: each row's blocks in tiles of 16, a tile stored as
// [2D/8 slices][16 blocks][8]: slice s holds elements 8s .. 8s+7 of every
// block's [min | max] vector.  Element offset of slice s of block n of `row`:
__host__ __device__ inline size_t ck_slice_offset(int row, int width, int n, int s, int D) {
    const size_t tiles = (size_t)(width + 15) / 16;
    return (((size_t)row * tiles + n / 16) * (size_t)(2 * D / 8) + s) * 128 + (size_t)(n % 16) * 8;
}

// An event recorded by the completion of a stage's last kernel, as part of that
// launch (hipExtLaunchKernelGGL's stop event) rather than as a separate record
// command behind it: in a schedule of three streams tied by events, separate
// record commands doubled the period of a layer-step in a probe.  `used` tells
// whether a launch took it (a stage that launches nothing leaves it to the
// caller).
struct LaunchStop {
    hipEvent_t event = nullptr;
    bool used = false;
};

// Launch `kernel`; with `stop` (not yet used), the launch also records its
// event when the kernel completes.
template <typename F, typename... Args>
inline void launch_k(F kernel, dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                     LaunchStop *stop, Args... args) {
    if (stop && stop->event && !stop->used) {
        hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, stream, nullptr, stop->event, 0u,
                              args...);
        stop->used = true;
    } else {
        hipLaunchKernelGGL(kernel, grid, block, lds, stream, args...);
    }
}

hipError_t launch_score_blocks(const ScoreArgs &a, int head_dim, hipStream_t stream,
                               LaunchStop *stop = nullptr);
hipError_t launch_pool_keys(const PoolArgs &a, int head_dim, hipStream_t stream);
hipError_t launch_score_minmax(const MinmaxArgs &a, int head_dim, hipStream_t stream,
                               LaunchStop *stop = nullptr);
hipError_t launch_select_topk(const SelectArgs &a, hipStream_t stream);
// One workgroup per row (256 threads; 1024 for rows wider than kWideRowMinWidth);
// mode 1 = select, 2 = plan, 3 = select then plan.
bool row_select_plan_fits(int width, int k, int mode);
hipError_t launch_row_select_plan(const SelectPlanArgs &a, int mode, hipStream_t stream,
                                  LaunchStop *stop = nullptr);
// Rows wider than this (in blocks) are selected by a 1024-thread build of the
// same kernels (select_plan_wide.hip).
#ifndef OASIS_WIDE_ROW_MIN_WIDTH
#define OASIS_WIDE_ROW_MIN_WIDTH 2048
#endif
constexpr int kWideRowMinWidth = OASIS_WIDE_ROW_MIN_WIDTH;
namespace wide {
hipError_t launch_row_select_plan(const SelectPlanArgs &a, int mode, hipStream_t stream,
                                  LaunchStop *stop = nullptr);
size_t row_shared_bytes();       // static LDS of the 1024-thread build's row state
}
size_t row_shared_bytes();       // the same for the 256-thread build
// Two-pass selection (and plan) of rows wider than kTwoPassMinWidth blocks:
// the chunk kernel, then one workgroup per row over the candidates.
void two_pass_plan(int width, int k, int *chunk_w, int *chunks);
hipError_t launch_two_pass_select_plan(const SelectPlanArgs &a, int mode, uint32_t *cand_key,
                                       int32_t *cand_idx, hipStream_t stream,
                                       LaunchStop *stop = nullptr);
namespace wide {
hipError_t launch_chunk_select(const ChunkArgs &a, hipStream_t stream);
hipError_t launch_merge_select_plan(const SelectPlanArgs &a, int mode, const uint32_t *cand_key,
                                    const int32_t *cand_idx, int ncand, hipStream_t stream,
                                    LaunchStop *stop = nullptr);
}
hipError_t launch_chunk_select(const ChunkArgs &a, hipStream_t stream);
hipError_t launch_merge_select_plan(const SelectPlanArgs &a, int mode, const uint32_t *cand_key,
                                    const int32_t *cand_idx, int ncand, hipStream_t stream,
                                    LaunchStop *stop = nullptr);
hipError_t launch_fetch_blocks(const FetchArgs &a, int head_dim, hipStream_t stream);
hipError_t launch_sparse_decode_attn(const AttnArgs &a, int head_dim, bool share_gpu, hipStream_t stream,
                                     LaunchStop *stop = nullptr);

// Split-K plan of the attention kernel: how many splits per row and entries per split.
void attn_split_plan(int rows, int n_blk, int *splits, int *per_split);

constexpr int kBlockTokens = 16;   // tokens per KV block
constexpr int kMaxRowsQ = 16;     // lookahead rows per KV head in one MFMA tile (scoring)
constexpr int kMaxAttnRowsQ = 32; // query rows per KV head in attention (two MFMA tiles)
constexpr int kMaxAttnBlocks = 65536;  // list entries per row in attention (keeps the split plan's int sums in range)
constexpr int kMaxKBlocks = 1024; // K limit of select / plan
constexpr int kRowSelectMaxWidth = 8192;  // widest table the row select keeps in LDS
constexpr int kFusedMaxWidth = 8192;      // fused select + plan: table width limit (and the LDS bound of row_select_plan_fits)
constexpr int kFusedMaxK = 512;           // fused select + plan: K limit
constexpr int kMaxSelectWidth = 15360;   // keys of a row staged in LDS (60 KiB)
constexpr int kMaxCandidates = 8192;     // candidates of a row in the two-pass selection (LDS)
constexpr int kMinChunkWidth = 2048;     // blocks per chunk of the two-pass selection, at least
// widest row of the two-pass selection: chunks of at most kRowSelectMaxWidth
// blocks, at most kMaxCandidates / K of them
__host__ __device__ constexpr long long two_pass_max_width(int k) {
    return (long long)kRowSelectMaxWidth * (kMaxCandidates / (k > 0 ? k : 1));
}
#ifndef OASIS_TWO_PASS_MIN_WIDTH
#define OASIS_TWO_PASS_MIN_WIDTH 8192    // up to here one fused launch is faster (13.1 against 17.8 us at 8,192)
#endif
constexpr int kTwoPassMinWidth = OASIS_TWO_PASS_MIN_WIDTH;   // rows wider than this: two passes

}  // namespace oasis
