// pool_keys.hip -- min/max pooling of the paged keys into the compressed-key cache.
//
// OasisKV (metalmedia.ai summary), Figure 7 caption: beside the sparse KV
// working set the GPU keeps the keys compressed by per-block min/max pooling,
// and the draft query scans those.  Per (sequence, KV head, block n) and per
// dimension d:
//   ck[b][g][n][0][d] = min, ck[b][g][n][1][d] = max over the valid tokens
//   (16n + t < ctx_len[b]) of the block.
// Both are bf16 values of the keys themselves, so the pooling is exact.
//
// Design: a wave pools four consecutive blocks of one (sequence, KV head)
// row.  The loads of all four key tiles are issued first (non-temporal: the
// whole pool is streamed once), then each tile is reduced as the shared
// pooling helper describes: a group of lanes per 8-dimension slice, min/max in
// registers over the lane's tokens, DPP folds over the group.  A page outside
// the pool is not read: the block is written as an empty box (min = +inf,
// max = -inf), which the compressed scorer turns into -inf.  The last-block
// mode re-pools only block ceil(ctx / 16) - 1 of each sequence: the one a
// decode step appends its token to.
#include "oasis_device.h"
#include "oasis_launch.h"
#include "pool_block.h"

namespace oasis {

constexpr int kPoolWaves = 4;
constexpr int kPoolChunk = 4;           // blocks per wave
#ifndef OASIS_POOL_CPOL
#define OASIS_POOL_CPOL 2               // key tiles: non-temporal (each is read once)
#endif

template <int D>
__global__ __launch_bounds__(kPoolWaves * kWave) void pool_keys_kernel(PoolArgs a) {
    using G = PoolGeom<D>;
    constexpr uint32_t kTileBytes = kBlockTokens * D * 2;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const long long gw = (long long)blockIdx.x * kPoolWaves + wave;
    const int rows = a.batch * a.hkv;
    const int chunks = (a.width + kPoolChunk - 1) / kPoolChunk;
    int row, n0 = 0;
    if (a.last_only) {
        if (gw >= rows) return;
        row = (int)gw;
    } else {
        row = (int)(gw / chunks);
        if (row >= rows) return;
        n0 = (int)(gw - (long long)row * chunks) * kPoolChunk;
    }
    const int b = row / a.hkv;
    const int g = row - b * a.hkv;
    long long ctx = a.ctx_len[b];
    const long long cmax = (long long)a.width * kBlockTokens;
    ctx = ctx < 0 ? 0 : (ctx > cmax ? cmax : ctx);
    const int nb = (int)((ctx + kBlockTokens - 1) / kBlockTokens);
    int count;
    if (a.last_only) {
        n0 = nb - 1;
        count = nb > 0 ? 1 : 0;
    } else {
        count = nb - n0 < kPoolChunk ? nb - n0 : kPoolChunk;
    }
    if (count <= 0) return;

    const uint32_t off = pool_lane_offset<D>(lane);
    u32x4 v[kPoolChunk][G::kLoads];
    bool present[kPoolChunk];
#pragma unroll
    for (int u = 0; u < kPoolChunk; ++u) {
        const int page = u < count ? a.block_table[(size_t)b * a.width + n0 + u] : -1;
        present[u] = page >= 0 && page < a.num_pages;
        const rsrc_t r = present[u]
            ? make_rsrc(a.k_pool + ((size_t)page * a.hkv + g) * kBlockTokens * D, kTileBytes)
            : make_rsrc(a.k_pool, 0u);
        pool_load<D, OASIS_POOL_CPOL>(r, off, v[u]);
    }
    const int s = lane / G::kLanes;
    const bool writer = lane % G::kLanes == 0;
#pragma unroll
    for (int u = 0; u < kPoolChunk; ++u) {
        if (u >= count) break;
        const int n = n0 + u;
        u32x4 pmn = {kBf16PosInfPair, kBf16PosInfPair, kBf16PosInfPair, kBf16PosInfPair};
        u32x4 pmx = {kBf16NegInfPair, kBf16NegInfPair, kBf16NegInfPair, kBf16NegInfPair};
        if (present[u]) {
            long long nt = ctx - (long long)n * kBlockTokens;
            nt = nt > kBlockTokens ? kBlockTokens : nt;
            float mn[8], mx[8];
            pool_slice<D>(v[u], (int)nt, lane, mn, mx);
            pmn = pack_exact_bf16x8(mn);
            pmx = pack_exact_bf16x8(mx);
        }
        if (writer) {
            *reinterpret_cast<u32x4 *>(a.ck + ck_slice_offset(row, a.width, n, s, D)) = pmn;
            *reinterpret_cast<u32x4 *>(a.ck + ck_slice_offset(row, a.width, n, G::kSlices + s, D)) = pmx;
        }
    }
}

hipError_t launch_pool_keys(const PoolArgs &a, int head_dim, hipStream_t stream) {
    const long long rows = (long long)a.batch * a.hkv;
    const long long waves = a.last_only ? rows : rows * ((a.width + kPoolChunk - 1) / kPoolChunk);
    if (waves == 0) return hipSuccess;
    const dim3 grid((unsigned)((waves + kPoolWaves - 1) / kPoolWaves));
    const dim3 block(kPoolWaves * kWave);
    if (head_dim == 128)
        hipLaunchKernelGGL(pool_keys_kernel<128>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(pool_keys_kernel<64>, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace oasis
