// score_blocks.hip -- lookahead-query block scoring over the paged key pool.
//
// OasisKV (metalmedia.ai summary), Figure 7 caption: the draft query scans
// the keys to predict the next step's top-K blocks.  Score of block n of KV
// head g: the max over its valid tokens t and over every lookahead row
// (draft j, query head h of the group) of scale * q_jh . k_t.
//
// Design (gfx950): the scan is a skinny dense contraction (16 tokens x D
// against at most 16 lookahead rows per block), so each 16-token block is one
// 16x16 MFMA output tile: A = the block's key tile (token = M, head dim = K),
// B = the group's lookahead rows (head dim = K, row = N), D / 32 MFMAs of
// 16x16x32 bf16 with fp32 accumulation.  The kernel is bound by streaming the
// keys from HBM: every key byte is read exactly once, 16 bytes per lane per
// load, the whole 4 KiB (D = 128) tile of a block by one wave.  The key tiles
// are stored in 8-dimension slices so that every load instruction reads 1 KiB
// of contiguous memory (with a 16-row x 64-byte pattern per load the same
// stream measured 10-15% slower).  A wave owns a
// chunk of consecutive blocks of one (sequence, KV head) row and streams it in
// groups: the next group's loads are issued (as buffer loads that can never
// fault) before the current group is reduced.  The max over a tile is reduced
// across lanes four blocks at a time so that each lane exchange serves
// several blocks.
#include "oasis_device.h"
#include "oasis_launch.h"

namespace oasis {

#ifndef OASIS_SCORE_CHUNK
#define OASIS_SCORE_CHUNK 8          // blocks per wave (4 and 8 alike, 16 +0.5% per step, 32 +1%)
#endif
#ifndef OASIS_SCORE_CPOL
#define OASIS_SCORE_CPOL 2           // keys are streamed once per step: non-temporal loads
#endif
#ifndef OASIS_SCORE_GROUP
#define OASIS_SCORE_GROUP 4          // blocks loaded together (a multiple of 4)
#endif
constexpr int kScoreChunk = OASIS_SCORE_CHUNK;
constexpr int kScoreGroup = OASIS_SCORE_GROUP;
constexpr int kScoreWaves = 4;       // waves per workgroup
static_assert(kScoreChunk % kScoreGroup == 0 && kScoreGroup % 4 == 0 && kScoreChunk <= kWave,
              "chunk must split into groups of four-block reductions");

template <int D>
struct KeyGroup {
    u32x4 k[kScoreGroup][D / 32];
};

template <int D>
__global__ __launch_bounds__(kScoreWaves * kWave) void score_blocks_kernel(ScoreArgs a) {
    constexpr int KK = D / 32;
    constexpr uint32_t kTileBytes = kBlockTokens * D * 2;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // uniform: keeps row indices scalar
    const int row = blockIdx.y;                       // b * hkv + g
    const int b = row / a.hkv;
    const int g = row - b * a.hkv;
    const int n0 = (blockIdx.x * kScoreWaves + wave) * kScoreChunk;
    if (n0 >= a.width) return;
    const int r16 = lane & 15;
    const int j4 = lane >> 4;

    int ctx = a.ctx_len[b];
    ctx = ctx < 0 ? 0 : (ctx > a.width * kBlockTokens ? a.width * kBlockTokens : ctx);
    const int nb = (ctx + kBlockTokens - 1) / kBlockTokens;

    // B operand: lookahead row r16 (draft r16 / G, head g*G + r16 % G), head-dim
    // slice 32*kk + 8*j4 .. +8.  Rows past n_rows_q are zero and masked below.
    bf16x8 qv[KK];
    const bool col_ok = r16 < a.n_rows_q;
    if (col_ok) {
        const int jd = r16 / a.group;
        const int hr = r16 - jd * a.group;
        const uint16_t *qp = a.q_look +
            (((size_t)b * a.n_look + jd) * a.hq + (size_t)g * a.group + hr) * D + 8 * j4;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qv[kk] = as_bf16x8(load_u32x4(qp + 32 * kk));
    } else {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qv[kk] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
    }

    // Page of block n0 + lane (lanes < chunk); -1 when past the context or out of range.
    int pg = -1;
    if (lane < kScoreChunk) {
        const int n = n0 + lane;
        if (n < nb) {
            const int p = a.block_table[(size_t)b * a.width + n];
            if (p >= 0 && p < a.num_pages) pg = p;
        }
    }

    const size_t page_stride = (size_t)a.hkv * kBlockTokens * D;
    const uint16_t *head_base = a.k_pool + (size_t)g * kBlockTokens * D;
    // A operand: token r16 of the tile, head-dim slice 32*kk + 8*j4 .. +8.  The
    // tile is stored in 8-dimension slices ([D/8][16][8]), so that slice is at
    // (4*kk + j4) * 256 + r16 * 16 bytes: lane * 16 + kk * 1 KiB, and each load
    // instruction reads 1 KiB of contiguous memory.
    const uint32_t koff = (uint32_t)lane * 16;
    float *out = a.scores + (size_t)row * a.width;
    const float NEG_INF = -__builtin_inff();

    // Absent blocks get a zero-byte resource: their loads return zeros without
    // touching memory, so every load is issued and the next group streams in
    // while the current one is reduced.
    auto load_group = [&](KeyGroup<D> &kg, int c) {
#pragma unroll
        for (int u = 0; u < kScoreGroup; ++u) {
            const int p = readlane_i(pg, c + u);
            const rsrc_t r = p >= 0 ? make_rsrc(head_base + (size_t)p * page_stride, kTileBytes)
                                    : make_rsrc(a.k_pool, 0u);
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) kg.k[u][kk] = buf_load16<OASIS_SCORE_CPOL>(r, koff, 1024 * kk);
        }
    };

    KeyGroup<D> cur, nxt;
    load_group(cur, 0);
#pragma unroll
    for (int c = 0; c < kScoreChunk; c += kScoreGroup) {
        if (c + kScoreGroup < kScoreChunk) load_group(nxt, c + kScoreGroup);
        float v[kScoreGroup];
#pragma unroll
        for (int u = 0; u < kScoreGroup; ++u) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) acc = mfma16x16x32(as_bf16x8(cur.k[u][kk]), qv[kk], acc);
            // rows 4*j4 + i of the tile are tokens; keep the valid ones
            const int valid = ctx - (n0 + c + u) * kBlockTokens - 4 * j4;
            float m = NEG_INF;
#pragma unroll
            for (int i = 0; i < 4; ++i) m = (i < valid) ? fmaxf(m, acc[i]) : m;
            v[u] = (col_ok && readlane_i(pg, c + u) >= 0) ? m : NEG_INF;
        }
        // Reduce four blocks at a time across the wave: halve the block set per
        // exchange (lane bit 5, then bit 4), then finish within 16-lane groups.
#pragma unroll
        for (int q = 0; q < kScoreGroup; q += 4) {
            float a0 = (lane & 32) ? v[q + 2] : v[q + 0];
            float a1 = (lane & 32) ? v[q + 3] : v[q + 1];
            const float s0 = (lane & 32) ? v[q + 0] : v[q + 2];
            const float s1 = (lane & 32) ? v[q + 1] : v[q + 3];
            a0 = fmaxf(a0, shfl_xor_f(s0, 32));
            a1 = fmaxf(a1, shfl_xor_f(s1, 32));
            float x = (lane & 16) ? a1 : a0;
            const float y = (lane & 16) ? a0 : a1;
            x = fmaxf(x, shfl_xor_f(y, 16));
            x = fmaxf(x, shfl_xor_f(x, 8));
            x = fmaxf(x, shfl_xor_f(x, 4));
            x = fmaxf(x, shfl_xor_f(x, 2));
            x = fmaxf(x, shfl_xor_f(x, 1));
            const int n = n0 + c + q + (((lane >> 5) << 1) | ((lane >> 4) & 1));
            if (r16 == 0 && n < a.width) out[n] = x * a.scale;
        }
        if (c + kScoreGroup < kScoreChunk) cur = nxt;
    }
}

hipError_t launch_score_blocks(const ScoreArgs &a, int head_dim, hipStream_t stream,
                               LaunchStop *stop) {
    const int rows = a.batch * a.hkv;
    if (rows == 0 || a.width == 0) return hipSuccess;
    const int per_wg = kScoreWaves * kScoreChunk;
    dim3 grid((a.width + per_wg - 1) / per_wg, rows);
    dim3 block(kScoreWaves * kWave);
    if (head_dim == 128)
        launch_k(score_blocks_kernel<128>, grid, block, 0, stream, stop, a);
    else
        launch_k(score_blocks_kernel<64>, grid, block, 0, stream, stop, a);
    return hipGetLastError();
}

}  // namespace oasis
