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
// Design: the whole-pool build gives a wave one compressed tile (16
// consecutive blocks of a row); the loads of four blocks are in flight while
// the previous four are reduced, as the shared pooling helper describes (a
// group of lanes per 8-dimension slice, min/max in registers over the lane's
// tokens, DPP folds over the group); the tile is staged in LDS and written in
// 1 KiB contiguous stores.  A page outside the pool is not read: the block is
// written as an empty box (min = +inf, max = -inf), which the compressed
// scorer turns into -inf.  The last-block mode re-pools only block
// ceil(ctx / 16) - 1 of each sequence: the one a decode step appends its
// token to.
#include "oasis_device.h"
#include "oasis_launch.h"
#include "pool_block.h"

namespace oasis {

#ifndef OASIS_POOL_WAVES
#define OASIS_POOL_WAVES 4
#endif
constexpr int kPoolWaves = OASIS_POOL_WAVES;   // waves per workgroup
#ifndef OASIS_POOL_CPOL
#define OASIS_POOL_CPOL 2               // key tiles: non-temporal (each is read once)
#endif

// Last-block mode: one wave per row re-pools block ceil(ctx / 16) - 1.
template <int D>
__global__ __launch_bounds__(kPoolWaves * kWave) void pool_keys_kernel(PoolArgs a) {
    using G = PoolGeom<D>;
    constexpr uint32_t kTileBytes = kBlockTokens * D * 2;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const long long gw = (long long)blockIdx.x * kPoolWaves + wave;
    const int rows = a.batch * a.hkv;
    if (gw >= rows) return;
    const int row = (int)gw;
    const int b = row / a.hkv;
    const int g = row - b * a.hkv;
    long long ctx = a.ctx_len[b];
    const long long cmax = (long long)a.width * kBlockTokens;
    ctx = ctx < 0 ? 0 : (ctx > cmax ? cmax : ctx);
    const int nb = (int)((ctx + kBlockTokens - 1) / kBlockTokens);
    if (nb <= 0) return;
    const int n = nb - 1;
    const int page = a.block_table[(size_t)b * a.width + n];
    const bool present = page >= 0 && page < a.num_pages;
    const int s = lane / G::kLanes;
    u32x4 pmn = {kBf16PosInfPair, kBf16PosInfPair, kBf16PosInfPair, kBf16PosInfPair};
    u32x4 pmx = {kBf16NegInfPair, kBf16NegInfPair, kBf16NegInfPair, kBf16NegInfPair};
    if (present) {
        u32x4 v[G::kLoads];
        pool_load<D, 0>(make_rsrc(a.k_pool + ((size_t)page * a.hkv + g) * kBlockTokens * D, kTileBytes),
                        pool_lane_offset<D>(lane), v);
        long long nt = ctx - (long long)n * kBlockTokens;
        nt = nt > kBlockTokens ? kBlockTokens : nt;
        float mn[8], mx[8];
        pool_slice<D>(v, (int)nt, lane, mn, mx);
        pmn = pack_exact_bf16x8(mn);
        pmx = pack_exact_bf16x8(mx);
    }
    if (lane % G::kLanes == 0) {
        *reinterpret_cast<u32x4 *>(a.ck + ck_slice_offset(row, a.width, n, s, D)) = pmn;
        *reinterpret_cast<u32x4 *>(a.ck + ck_slice_offset(row, a.width, n, G::kSlices + s, D)) = pmx;
    }
}

// The whole-pool build: a wave pools one compressed tile (16 consecutive
// blocks of a row), four blocks at a time with the next four loading, and
// stages the results in its own LDS region laid out as the tile is in memory
// ([2D/8 slices][16 blocks][8 elements], a slice padded to 17 entries so
// that the 16 writer lanes hit different banks).  The tile then leaves in
// 1 KiB contiguous non-temporal stores instead of 16-byte slices 256 bytes
// apart (which cost a third of the kernel's time).  Blocks past the context
// are not written, as in the per-block kernel.
constexpr int kPoolTileBlocks = 16;      // blocks per compressed tile
#ifndef OASIS_POOL_GROUP
#define OASIS_POOL_GROUP 4
#endif
constexpr int kPoolGroup = OASIS_POOL_GROUP;   // blocks loaded together
#ifndef OASIS_POOL_CONTIG
#define OASIS_POOL_CONTIG 1
#endif
// Tile loads of 1 KiB contiguous per instruction (lane l, load i: bytes
// 1024 i + 16 l), put through the wave's LDS into the pooling layout; the
// pooling layout loaded directly reads 16 runs of 64 bytes per instruction,
// which HBM serves more slowly.  A slice is padded from 256 to 272 bytes in
// LDS so that the lanes reading one token group hit different banks.
constexpr int kPoolSliceLds = 272;

#ifndef OASIS_POOL_WGS
#define OASIS_POOL_WGS 0            // > 0: that many workgroups, each wave walking tiles grid-stride
#endif

template <int D>
__global__ __launch_bounds__(kPoolWaves * kWave) void pool_tiles_kernel(PoolArgs a) {
    using G = PoolGeom<D>;
    constexpr uint32_t kTileBytes = kBlockTokens * D * 2;
    constexpr int kSlots = 2 * G::kSlices;                      // min slices, then max slices
    constexpr int kPad = kPoolTileBlocks + 1;
    constexpr int kEntries = kSlots * kPoolTileBlocks;          // 16-byte entries of a tile
    __shared__ u32x4 stage[kPoolWaves][kSlots * kPad];
#if OASIS_POOL_CONTIG
    __shared__ u32x4 xpose[kPoolWaves][G::kSlices * kPoolSliceLds / 16];
#endif
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int rows = a.batch * a.hkv;
    const int tiles = (a.width + kPoolTileBlocks - 1) / kPoolTileBlocks;
    const long long total = (long long)rows * tiles;
    const long long stride = OASIS_POOL_WGS > 0 ? (long long)gridDim.x * kPoolWaves : total;
    for (long long gw = (long long)blockIdx.x * kPoolWaves + wave; gw < total; gw += stride) {
    const int row = (int)(gw / tiles);
    const int n0 = (int)(gw - (long long)row * tiles) * kPoolTileBlocks;
    const int b = row / a.hkv;
    const int g = row - b * a.hkv;
    // the tile's 16 page numbers in one vector load (lane j: block n0 + j, if
    // in the table), issued beside the context length: blocks past the
    // context are dropped below
    const int page_v = n0 + lane < a.width && lane < kPoolTileBlocks
                           ? a.block_table[(size_t)b * a.width + n0 + lane] : -1;
    long long ctx = a.ctx_len[b];
    const long long cmax = (long long)a.width * kBlockTokens;
    ctx = ctx < 0 ? 0 : (ctx > cmax ? cmax : ctx);
    const int nb = (int)((ctx + kBlockTokens - 1) / kBlockTokens);
    const int count = nb - n0 < kPoolTileBlocks ? nb - n0 : kPoolTileBlocks;
    if (count <= 0) continue;

#if OASIS_POOL_CONTIG
    const uint32_t off = (uint32_t)lane * 16u;
    u32x4 *xp = xpose[wave];
    // where this lane's loads go in the transposition buffer, and where the
    // pooling layout is read back from (16-byte units)
    const int pool_off = (int)pool_lane_offset<D>(lane);
    int wr_at[G::kLoads], rd_at[G::kLoads];
#pragma unroll
    for (int i = 0; i < G::kLoads; ++i) {
        const int bw = 1024 * i + 16 * lane;
        const int br = pool_off + i * G::kLanes * 16;
        wr_at[i] = ((bw >> 8) * kPoolSliceLds + (bw & 255)) >> 4;
        rd_at[i] = ((br >> 8) * kPoolSliceLds + (br & 255)) >> 4;
    }
#else
    const uint32_t off = pool_lane_offset<D>(lane);
#endif
    const int s = lane / G::kLanes;
    const bool writer = lane % G::kLanes == 0;
    u32x4 *st = stage[wave];
    u32x4 v[2][kPoolGroup][G::kLoads];
    bool present[kPoolTileBlocks];
    auto issue = [&](int buf, int grp) {
#pragma unroll
        for (int u = 0; u < kPoolGroup; ++u) {
            const int j = grp * kPoolGroup + u;
            const int page = j < count ? readlane_i(page_v, j) : -1;
            present[j] = page >= 0 && page < a.num_pages;
            const rsrc_t r = present[j]
                ? make_rsrc(a.k_pool + ((size_t)page * a.hkv + g) * kBlockTokens * D, kTileBytes)
                : make_rsrc(a.k_pool, 0u);
#if OASIS_POOL_CONTIG
#pragma unroll
            for (int i = 0; i < G::kLoads; ++i)
                v[buf][u][i] = buf_load16<OASIS_POOL_CPOL>(r, off, 1024 * i);
#else
            pool_load<D, OASIS_POOL_CPOL>(r, off, v[buf][u]);
#endif
        }
    };
    issue(0, 0);
#pragma unroll
    for (int grp = 0; grp < kPoolTileBlocks / kPoolGroup; ++grp) {
        if (grp + 1 < kPoolTileBlocks / kPoolGroup) issue((grp + 1) & 1, grp + 1);
#pragma unroll
        for (int u = 0; u < kPoolGroup; ++u) {
            const int j = grp * kPoolGroup + u;
            if (j >= count) break;
            u32x4 pmn = {kBf16PosInfPair, kBf16PosInfPair, kBf16PosInfPair, kBf16PosInfPair};
            u32x4 pmx = {kBf16NegInfPair, kBf16NegInfPair, kBf16NegInfPair, kBf16NegInfPair};
            if (present[j]) {
                long long nt = ctx - (long long)(n0 + j) * kBlockTokens;
                nt = nt > kBlockTokens ? kBlockTokens : nt;
                float mn[8], mx[8];
#if OASIS_POOL_CONTIG
                // the tile through LDS into the pooling layout (this wave's own
                // region: its LDS accesses are performed in order)
                u32x4 w[G::kLoads];
#pragma unroll
                for (int i = 0; i < G::kLoads; ++i) xp[wr_at[i]] = v[grp & 1][u][i];
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll
                for (int i = 0; i < G::kLoads; ++i) w[i] = xp[rd_at[i]];
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");   // read before the next block's writes
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
                pool_slice<D>(w, (int)nt, lane, mn, mx);
#else
                pool_slice<D>(v[grp & 1][u], (int)nt, lane, mn, mx);
#endif
                pmn = pack_exact_bf16x8(mn);
                pmx = pack_exact_bf16x8(mx);
            }
            if (writer) {
                st[s * kPad + j] = pmn;
                st[(G::kSlices + s) * kPad + j] = pmx;
            }
        }
    }
    // the wave reads back what its own lanes staged
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    u32x4 *tile = reinterpret_cast<u32x4 *>(a.ck + ck_slice_offset(row, a.width, n0, 0, D));
#pragma unroll
    for (int i = 0; i < kEntries / kWave; ++i) {
        const int e = i * kWave + lane;                 // slot e / 16, block e % 16
        const int j = e % kPoolTileBlocks;
        if (j < count) __builtin_nontemporal_store(st[(e / kPoolTileBlocks) * kPad + j], &tile[e]);
    }
    // the next tile's staging overwrites what these stores read
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
}

hipError_t launch_pool_keys(const PoolArgs &a, int head_dim, hipStream_t stream) {
    const long long rows = (long long)a.batch * a.hkv;
    const dim3 block(kPoolWaves * kWave);
    if (!a.last_only) {
        const long long waves = rows * ((a.width + kPoolTileBlocks - 1) / kPoolTileBlocks);
        if (waves == 0) return hipSuccess;
        long long wgs = (waves + kPoolWaves - 1) / kPoolWaves;
        if (OASIS_POOL_WGS > 0 && wgs > OASIS_POOL_WGS) wgs = OASIS_POOL_WGS;
        const dim3 grid((unsigned)wgs);
        if (head_dim == 128)
            hipLaunchKernelGGL(pool_tiles_kernel<128>, grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL(pool_tiles_kernel<64>, grid, block, 0, stream, a);
        return hipGetLastError();
    }
    if (rows == 0) return hipSuccess;
    const dim3 grid((unsigned)((rows + kPoolWaves - 1) / kPoolWaves));
    if (head_dim == 128)
        hipLaunchKernelGGL(pool_keys_kernel<128>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(pool_keys_kernel<64>, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace oasis
