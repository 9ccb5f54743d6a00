// score_minmax.hip -- lookahead block scores from the min/max-pooled keys.
//
// OasisKV (metalmedia.ai summary), Figure 7 caption: the draft query scans the
// compressed keys (per-block min/max pooling) to predict the next step's top-K
// blocks.  The score of block n for one lookahead row q is the largest value
// q . x can reach for x in the block's box min <= x <= max:
//   sum_d max(q_d * min_d, q_d * max_d) = q- . min + q+ . max,
// where q+ keeps the non-negative and q- the negative components of q.  It is
// maximised over the KV head's lookahead rows and scaled, as the exact score.
//
// Design (gfx950): the right-hand form is one dot product of length 2D, so a
// 16 x 16 MFMA tile covers 16 lookahead rows (A = [q- | q+], bf16, split by
// sign bit once per wave) against 16 blocks (B = the compressed rows
// [min | max], stored by tiles of 16 blocks in 8-element slices, 8 KiB per
// tile at D = 128); D/16 v_mfma_f32_16x16x32_bf16 per tile.  A wave takes one
// tile (16 consecutive blocks) of one row, issues all its loads (raw buffer
// loads bounded to the row's valid blocks, non-temporal: each compressed key
// is read once per step), then reduces the tile's columns over the lookahead
// rows with two lane exchanges.  One tile per wave (8 KiB) keeps more waves in
// flight and leaves a shorter tail than four: 22.3 against 23.7 us per launch
// at 16 x 32K.
// A block written as an empty box (min > max, for a page outside the pool)
// scores -inf.  The bytes are 1/8 of the exact scorer's at bs = 16.
//
// With the key pool given, one more wave per row re-pools the row's last
// block (the one a decode step appends to) from the pool, writes it, and
// scores it itself; the tile waves leave that block's score to it, so no
// wave reads compressed keys another wave writes.
#include "oasis_device.h"
#include "oasis_launch.h"
#include "pool_block.h"

#ifndef OASIS_MINMAX_CPOL
#define OASIS_MINMAX_CPOL 2      // non-temporal: each compressed key is read once per step
#endif

namespace oasis {

#ifndef OASIS_MM_WAVES
#define OASIS_MM_WAVES 4
#endif
constexpr int kMmWaves = OASIS_MM_WAVES;   // waves per workgroup
#ifndef OASIS_MM_TILES
#define OASIS_MM_TILES 1
#endif
constexpr int kMmTiles = OASIS_MM_TILES;   // 16-block tiles per wave
constexpr int kMmBlocksPerWave = kMmTiles * kBlockTokens;

// Refresh wave of one row: pool the last block (ceil(ctx / 16) - 1) from the
// key pool with the same helper as oasis_pool_keys (a group of lanes per
// 8-dimension slice), write its compressed slices, and score the block from
// the fresh values.
template <int D>
__device__ __forceinline__ void refresh_last_block(const MinmaxArgs &a, int row) {
    using G = PoolGeom<D>;
    constexpr int kRowsPerLane = kMaxRowsQ / G::kLanes;   // lookahead rows per lane
    constexpr uint32_t kTileBytes = kBlockTokens * D * 2;
    const int lane = threadIdx.x & (kWave - 1);
    const int b = row / a.hkv;
    const int g = row - b * a.hkv;
    long long ctx = a.ctx_len[b];
    const long long cmax = (long long)a.width * kBlockTokens;
    ctx = ctx < 0 ? 0 : (ctx > cmax ? cmax : ctx);
    const int nb = (int)((ctx + kBlockTokens - 1) / kBlockTokens);
    if (nb == 0) return;
    const int n = nb - 1;
    const int nt = (int)(ctx - (long long)n * kBlockTokens);
    const int s = lane / G::kLanes;          // the slice this lane pools and scores
    const int t0 = lane % G::kLanes;
    float *out = a.scores + (size_t)row * a.width;
    uint16_t *ck_min = a.ck + ck_slice_offset(row, a.width, n, s, D);
    uint16_t *ck_max = a.ck + ck_slice_offset(row, a.width, n, G::kSlices + s, D);
    const int page = a.block_table[(size_t)b * a.width + n];
    if (page < 0 || page >= a.num_pages) {
        if (t0 == 0) {
            *reinterpret_cast<u32x4 *>(ck_min) =
                u32x4{kBf16PosInfPair, kBf16PosInfPair, kBf16PosInfPair, kBf16PosInfPair};
            *reinterpret_cast<u32x4 *>(ck_max) =
                u32x4{kBf16NegInfPair, kBf16NegInfPair, kBf16NegInfPair, kBf16NegInfPair};
        }
        if (lane == 0) out[n] = -__builtin_inff();
        return;
    }
    u32x4 v[G::kLoads];
    pool_load<D, 0>(make_rsrc(a.k_pool + ((size_t)page * a.hkv + g) * kBlockTokens * D, kTileBytes),
                    pool_lane_offset<D>(lane), v);
    float mn[8], mx[8];
    pool_slice<D>(v, nt, lane, mn, mx);
    if (t0 == 0) {
        *reinterpret_cast<u32x4 *>(ck_min) = pack_exact_bf16x8(mn);
        *reinterpret_cast<u32x4 *>(ck_max) = pack_exact_bf16x8(mx);
    }
    // Lane (s, t0) bounds slice s for lookahead rows t0 + kLanes * k; the
    // slices are then summed (lanes of equal t0) and the rows maximised.
    float part[kRowsPerLane];
#pragma unroll
    for (int k = 0; k < kRowsPerLane; ++k) {
        const int r = t0 + G::kLanes * k;
        part[k] = 0.f;
        if (r < a.n_rows_q) {
            const int jd = r / a.group;
            const int hr = r - jd * a.group;
            const u32x4 qw = load_u32x4(a.q_look +
                (((size_t)b * a.n_look + jd) * a.hq + (size_t)g * a.group + hr) * D + 8 * s);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float q0 = bf16_bits_to_float(qw[w] & 0xffffu);
                const float q1 = bf16_bits_to_float(qw[w] >> 16);
                part[k] += q0 < 0.f ? q0 * mn[2 * w] : q0 * mx[2 * w];
                part[k] += q1 < 0.f ? q1 * mn[2 * w + 1] : q1 * mx[2 * w + 1];
            }
        }
    }
#pragma unroll
    for (int off = G::kLanes; off < kWave; off <<= 1)
#pragma unroll
        for (int k = 0; k < kRowsPerLane; ++k) part[k] += shfl_xor_f(part[k], off);
    float best = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < kRowsPerLane; ++k)
        if (t0 + G::kLanes * k < a.n_rows_q) best = fmaxf(best, part[k]);
#pragma unroll
    for (int off = 1; off < G::kLanes; off <<= 1) best = fmaxf(best, shfl_xor_f(best, off));
    if (lane == 0) out[n] = best * a.scale;
}

template <int D>
__global__ __launch_bounds__(kMmWaves * kWave) void score_minmax_kernel(MinmaxArgs a) {
    constexpr int QK = D / 32;         // 32-wide k-steps of one half (q- or q+)
    constexpr int KK = 2 * QK;         // k-steps of a tile
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int r16 = lane & 15;
    const int j4 = lane >> 4;
    const long long gw = (long long)blockIdx.x * kMmWaves + wave;
    const int chunks = (a.width + kMmBlocksPerWave - 1) / kMmBlocksPerWave;
    const int rows = a.batch * a.hkv;
    const bool refresh = a.k_pool != nullptr;
    if (gw >= (long long)rows * chunks) {         // the refresh waves, one per row
        const long long r = gw - (long long)rows * chunks;
        if (refresh && r < rows) refresh_last_block<D>(a, (int)r);
        return;
    }
    const int row = (int)(gw / chunks);
    const int n0 = (int)(gw - (long long)row * chunks) * kMmBlocksPerWave;
    const int b = row / a.hkv;
    const int g = row - b * a.hkv;
    long long ctx = a.ctx_len[b];
    const long long cmax = (long long)a.width * kBlockTokens;
    ctx = ctx < 0 ? 0 : (ctx > cmax ? cmax : ctx);
    const int nb = (int)((ctx + kBlockTokens - 1) / kBlockTokens);

    // Compressed tiles n0/16 .. n0/16 + kMmTiles - 1 (16 blocks each, in 8-element slices):
    // the B operand of k-step kk (block r16, elements 32*kk + 8*j4 .. +8) is
    // slice 4*kk + j4, at lane * 16 + kk * 1 KiB of the tile, so each load
    // reads 1 KiB of contiguous memory.  The resource ends at the last tile
    // holding a valid block; blocks past the context inside that tile are
    // read but their scores are -inf (a column of the MFMA output depends on
    // its own block only).
    constexpr uint32_t kTileBytes = kBlockTokens * 2 * D * 2;
    const int valid_tiles = nb > n0 ? (nb - n0 + kBlockTokens - 1) / kBlockTokens : 0;
    const uint16_t *base = a.ck + ck_slice_offset(row, a.width, n0, 0, D);
    const rsrc_t r = make_rsrc(base, (uint32_t)(valid_tiles < kMmTiles ? valid_tiles : kMmTiles) *
                                         kTileBytes);
    // The tile index sits in the per-lane offset, so the range check cuts at
    // whole tiles; the k-step offset (< 8 KiB) stays inside the tile.
    u32x4 kb[kMmTiles][KK];
#pragma unroll
    for (int t = 0; t < kMmTiles; ++t) {
        const uint32_t boff = (uint32_t)t * kTileBytes + (uint32_t)lane * 16;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) kb[t][kk] = buf_load16<OASIS_MINMAX_CPOL>(r, boff, 1024 * kk);
    }

    // A operand: lookahead row r16 (draft r16 / G, head g*G + r16 % G), dims
    // 32*kk + 8*j4 .. +8, split by sign: k-steps 0 .. QK-1 carry q-, the rest q+.
    bf16x8 qa[KK];
    if (r16 < a.n_rows_q) {
        const int jd = r16 / a.group;
        const int hr = r16 - jd * a.group;
        const uint16_t *qp = a.q_look +
            (((size_t)b * a.n_look + jd) * a.hq + (size_t)g * a.group + hr) * D + 8 * j4;
#pragma unroll
        for (int kk = 0; kk < QK; ++kk) {
            const u32x4 w = load_u32x4(qp + 32 * kk);
            u32x4 neg, pos;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t m = ((w[e] & 0x80008000u) >> 15) * 0xffffu;   // sign of each half
                neg[e] = w[e] & m;
                pos[e] = w[e] & ~m;
            }
            qa[kk] = as_bf16x8(neg);
            qa[QK + kk] = as_bf16x8(pos);
        }
    } else {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qa[kk] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
    }

    const float NEG_INF = -__builtin_inff();
    float *out = a.scores + (size_t)row * a.width;
#pragma unroll
    for (int t = 0; t < kMmTiles; ++t) {
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) s = mfma16x16x32(qa[kk], as_bf16x8(kb[t][kk]), s);
        // s[i] = bound of lookahead row 4*j4 + i on block r16 of the tile
        float m = NEG_INF;
#pragma unroll
        for (int i = 0; i < 4; ++i) m = (4 * j4 + i < a.n_rows_q) ? fmaxf(m, s[i]) : m;
        m = max_xor32(max_xor16(m));
        const int n = n0 + t * kBlockTokens + r16;
        if (j4 == 0 && n < a.width && !(refresh && n == nb - 1)) {   // the refresh wave scores nb - 1
            // lanes j4 = 0 hold min[0..7] (k-step 0) and max[0..7] (k-step QK) of block r16
            const float mn0 = bf16_bits_to_float(kb[t][0][0] & 0xffffu);
            const float mx0 = bf16_bits_to_float(kb[t][QK][0] & 0xffffu);
            out[n] = (n < nb && !(mn0 > mx0)) ? m * a.scale : NEG_INF;
        }
    }
}

hipError_t launch_score_minmax(const MinmaxArgs &a, int head_dim, hipStream_t stream,
                               LaunchStop *stop) {
    const long long rows = (long long)a.batch * a.hkv;
    const long long chunks = (a.width + kMmBlocksPerWave - 1) / kMmBlocksPerWave;
    const long long waves = rows * chunks + (a.k_pool ? rows : 0);
    if (waves == 0) return hipSuccess;
    const dim3 grid((unsigned)((waves + kMmWaves - 1) / kMmWaves));
    const dim3 block(kMmWaves * kWave);
    if (head_dim == 128)
        launch_k(score_minmax_kernel<128>, grid, block, 0, stream, stop, a);
    else
        launch_k(score_minmax_kernel<64>, grid, block, 0, stream, stop, a);
    return hipGetLastError();
}

}  // namespace oasis
