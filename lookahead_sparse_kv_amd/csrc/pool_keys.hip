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
// consecutive blocks of a row), reads it block by block with the next block
// in flight, folds each column of a block over its tokens with packed 16-bit
// integer min/max, stages the tile in LDS and writes it in 1 KiB contiguous
// stores (pool_tiles_kernel below).  A page outside the pool is not read: the block is
// written as an empty box (min = +inf, max = -inf), which the compressed
// scorer turns into -inf.  The last-block mode re-pools only block
// ceil(ctx / 16) - 1 of each sequence: the one a decode step appends its
// token to.
#include "oasis_device.h"
#include "oasis_launch.h"
#include "pool_block.h"

namespace oasis {

#ifndef OASIS_POOL_WAVES
#define OASIS_POOL_WAVES 8
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

// Min and max of bf16 bit patterns, two per 32-bit word, with packed 16-bit
// integer min/max and no conversion to float.  Read as signed 16-bit
// integers, the non-negative values (+0 up to +inf) are in their float order
// and every negative value lies below them; read as unsigned, the negative
// values (-0 up to -inf) are in order of magnitude, above every non-negative
// one.  So over a set of keys:
//   float min = (signed min < 0) ? unsigned max : signed min
//   float max = (signed max < 0) ? unsigned min : signed max
// (a negative signed min means the set holds a negative value, whose largest
// magnitude is the unsigned max; a negative signed max means every value is
// negative, and the smallest magnitude is the unsigned min).  A zero of
// either sign may come out for a set holding both zeros; they are equal.
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

struct BoxFold {
    // identities: no key beats them (the largest key is +inf = 0x7f80, the
    // largest unsigned pattern -inf = 0xff80)
    uint32_t smin = 0x7fff7fffu, smax = 0x80008000u, umin = 0xffffffffu, umax = 0u;

    __device__ __forceinline__ void add(uint32_t x) {
        const s16x2 xs = __builtin_bit_cast(s16x2, x);
        const u16x2 xu = __builtin_bit_cast(u16x2, x);
        smin = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(s16x2, smin), xs));
        smax = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(s16x2, smax), xs));
        umin = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, umin), xu));
        umax = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, umax), xu));
    }
    __device__ __forceinline__ void add_pair(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
        smin = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(s16x2, smin), __builtin_bit_cast(s16x2, a)));
        smax = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(s16x2, smax), __builtin_bit_cast(s16x2, b)));
        umin = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, umin), __builtin_bit_cast(u16x2, c)));
        umax = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, umax), __builtin_bit_cast(u16x2, d)));
    }
    // 0xffff in each half whose sign bit is set
    static __device__ __forceinline__ uint32_t neg_halves(uint32_t x) {
        return __builtin_bit_cast(uint32_t, __builtin_bit_cast(s16x2, x) >> (s16x2){15, 15});
    }
    __device__ __forceinline__ uint32_t min_bits() const {
        const uint32_t m = neg_halves(smin);
        return (umax & m) | (smin & ~m);
    }
    __device__ __forceinline__ uint32_t max_bits() const {
        const uint32_t m = neg_halves(smax);
        return (umin & m) | (smax & ~m);
    }
};

// The whole-pool build: a wave pools one compressed tile (16 consecutive
// blocks of a row), one block at a time with the next block's loads in
// flight.  Each block is loaded 1 KiB contiguous per
// instruction (lane l, load i: bytes 1024 i + 16 l of the tile) and written
// to the wave's own LDS region as it lies in memory, with a slice padded from
// 256 to 272 bytes.  Lane c then reads back one column of the tile (the
// 32-bit word holding dimensions 2p and 2p + 1 of slice s, c = 4 s + p) for
// every token, one 4-byte read per token (the 32 lanes of a read hit 32
// different banks), and folds it with packed 16-bit min/max (BoxFold), so no
// lane exchange is needed.  At D = 64 the tile has 32 columns: lanes 32..63
// take tokens 8..15 of the same columns, and the two halves are folded
// together by one row swap.  The tile's results are staged in LDS laid out
// as the compressed tile is in memory ([2D/8 slices][16 blocks][8 elements],
// a slice padded to 17 entries) and leave in 1 KiB contiguous device-scope
// stores.  Blocks past the context are not written, as in the per-block
// kernel.
//
// The build reads 1 GiB and writes an eighth of that: the writes, not the
// arithmetic, are what it has to fit around.  Measured over a 1 GiB pool,
// the reads alone take 163 us and the writes added 50 us with non-temporal
// stores and eight blocks in flight per wave on twelve waves per CU; with
// device-scope stores (sc1), one block in flight per wave and eight waves per
// CU (one 8-wave workgroup: its 104 KiB of LDS leave room for no second) the
// build took 193-196 us, and 204-208 us taking four pools in turn (as a
// build over the layers does: the address translations of each pool are
// cold).  More in flight, more waves (twelve per CU) or fewer (four) were
// each slower.  Giving the eight waves of a workgroup the same tile of the
// eight KV heads, so that they read the same 16 pages (32 KiB contiguous per
// page between them), took it to 191 us and 200 us over four pools.
constexpr int kPoolTileBlocks = 16;      // blocks per compressed tile
#ifndef OASIS_POOL_GROUP
#define OASIS_POOL_GROUP 1
#endif
constexpr int kPoolGroup = OASIS_POOL_GROUP;   // blocks loaded together
constexpr int kPoolSliceLds = 272;             // a 256-byte slice padded in LDS

#ifndef OASIS_POOL_STORE_CPOL
#define OASIS_POOL_STORE_CPOL 16        // compressed tiles: device-scope stores (sc1)
#endif

#ifndef OASIS_POOL_HEAD_MAJOR
#define OASIS_POOL_HEAD_MAJOR 1         // the waves of a workgroup take one tile of every KV head
#endif

#ifndef OASIS_POOL_WGS
#define OASIS_POOL_WGS 0            // > 0: that many workgroups, each wave walking tiles grid-stride
#endif

template <int D>
__global__ __launch_bounds__(kPoolWaves * kWave) void pool_tiles_kernel(PoolArgs a) {
    constexpr uint32_t kTileBytes = kBlockTokens * D * 2;
    constexpr int kSlices = D / 8;
    constexpr int kLoads = (int)kTileBytes / 1024;              // 1 KiB loads per block
    constexpr int kCols = D / 2;                                // 32-bit columns of a token
    constexpr int kTpl = kBlockTokens * kCols / kWave;          // tokens per lane: 16 (D 128), 8 (D 64)
    static_assert(kCols * (kBlockTokens / kTpl) == kWave, "a lane per (column, token range)");
    constexpr int kSlots = 2 * kSlices;                         // min slices, then max slices
    constexpr int kPad = kPoolTileBlocks + 1;
    constexpr int kEntries = kSlots * kPoolTileBlocks;          // 16-byte entries of a tile
    __shared__ u32x4 stage[kPoolWaves][kSlots * kPad];
    __shared__ u32x4 xpose[kPoolWaves][kSlices * kPoolSliceLds / 16];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int rows = a.batch * a.hkv;
    const int tiles = (a.width + kPoolTileBlocks - 1) / kPoolTileBlocks;
    const long long total = (long long)rows * tiles;
    const long long stride = OASIS_POOL_WGS > 0 ? (long long)gridDim.x * kPoolWaves : total;
    // where this lane's loads go in the wave's LDS region (16-byte units; load
    // i goes 1 KiB = four padded slices further), and the column it reads back
    // (32-bit units): slice s = c / 4, word p = c % 4, tokens from t0
    const uint32_t off = (uint32_t)lane * 16u;
    const int wr_at = ((lane >> 4) * kPoolSliceLds + ((16 * lane) & 255)) >> 4;
    constexpr int kWrStep = 4 * kPoolSliceLds / 16;
    const int col = lane % kCols;
    const int cs = col >> 2, cp = col & 3;
    const int t0 = (lane / kCols) * kTpl;
    const int rd_at = (cs * kPoolSliceLds + t0 * 16 + cp * 4) >> 2;
    u32x4 *xp = xpose[wave];
    const uint32_t *xw = reinterpret_cast<const uint32_t *>(xp);
    uint32_t *sw = reinterpret_cast<uint32_t *>(stage[wave]);
    const bool writer = lane < kCols;
    for (long long gw = (long long)blockIdx.x * kPoolWaves + wave; gw < total; gw += stride) {
#if OASIS_POOL_HEAD_MAJOR
    // consecutive waves take the KV heads of one (sequence, tile): a page's
    // tiles of every head are read together
    const long long bt = gw / a.hkv;
    const int g = (int)(gw - bt * a.hkv);
    const int b = (int)(bt / tiles);
    const int n0 = (int)(bt - (long long)b * tiles) * kPoolTileBlocks;
    const int row = b * a.hkv + g;
#else
    const int row = (int)(gw / tiles);
    const int n0 = (int)(gw - (long long)row * tiles) * kPoolTileBlocks;
    const int b = row / a.hkv;
    const int g = row - b * a.hkv;
#endif
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

    u32x4 v[2][kPoolGroup][kLoads];
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
#pragma unroll
            for (int i = 0; i < kLoads; ++i)
                v[buf][u][i] = buf_load16<OASIS_POOL_CPOL>(r, off, 1024 * i);
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
            uint32_t mn = kBf16PosInfPair, mx = kBf16NegInfPair;       // the empty box
            if (present[j]) {
                // the block through this wave's own LDS region (its LDS
                // accesses are performed in order)
#pragma unroll
                for (int i = 0; i < kLoads; ++i) xp[wr_at + kWrStep * i] = v[grp & 1][u][i];
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
                const long long left = ctx - (long long)(n0 + j) * kBlockTokens;
                const int nt = left > kBlockTokens ? kBlockTokens : (int)left;   // >= 1: j < count
                BoxFold f;
                if (nt >= kBlockTokens) {
#pragma unroll
                    for (int t = 0; t < kTpl; ++t) f.add(xw[rd_at + 4 * t]);
                } else {
#pragma unroll
                    for (int t = 0; t < kTpl; ++t) {
                        const uint32_t x = xw[rd_at + 4 * t];
                        if (t0 + t < nt) f.add(x);
                    }
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");   // read before the next block's writes
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
                if (kTpl < kBlockTokens) {
                    // the other token half of the same column, in lane ^ 32: a
                    // row swap of two copies of a word leaves the word of the
                    // lane and of its partner in the two results, in every lane
                    const auto s0 = __builtin_amdgcn_permlane32_swap(f.smin, f.smin, false, false);
                    const auto s1 = __builtin_amdgcn_permlane32_swap(f.smax, f.smax, false, false);
                    const auto s2 = __builtin_amdgcn_permlane32_swap(f.umin, f.umin, false, false);
                    const auto s3 = __builtin_amdgcn_permlane32_swap(f.umax, f.umax, false, false);
                    f.smin = (uint32_t)s0[0];
                    f.smax = (uint32_t)s1[0];
                    f.umin = (uint32_t)s2[0];
                    f.umax = (uint32_t)s3[0];
                    f.add_pair((uint32_t)s0[1], (uint32_t)s1[1], (uint32_t)s2[1], (uint32_t)s3[1]);
                }
                mn = f.min_bits();
                mx = f.max_bits();
            }
            if (writer) {
                sw[(cs * kPad + j) * 4 + cp] = mn;
                sw[((kSlices + cs) * kPad + j) * 4 + cp] = mx;
            }
        }
    }
    // the wave reads back what its own lanes staged
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    const rsrc_t out = make_rsrc(a.ck + ck_slice_offset(row, a.width, n0, 0, D), kEntries * 16);
    const u32x4 *st = stage[wave];
#pragma unroll
    for (int i = 0; i < kEntries / kWave; ++i) {
        const int e = i * kWave + lane;                 // slot e / 16, block e % 16
        const int j = e % kPoolTileBlocks;
        if (j < count)
            __builtin_amdgcn_raw_buffer_store_b128(st[(e / kPoolTileBlocks) * kPad + j], out,
                                                   (uint32_t)lane * 16u, i * kWave * 16,
                                                   OASIS_POOL_STORE_CPOL);
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
