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
// Design: one wave per block.  The 4 KiB key tile, stored in 8-dimension
// slices ([D/8][16][8]), is read 16 B per lane, so one load instruction covers
// four slices (1 KiB contiguous): lane l holds 8 dimensions of token l % 16,
// and the 16 tokens of each slice are folded by lane exchanges.  A page
// outside the pool is not read: the block is written as an empty box
// (min = +inf, max = -inf), which the compressed scorer turns into -inf.  The last-block mode refreshes only block ceil(ctx / 16) - 1 of each
// sequence: the one a decode step appends its token to.
#include "oasis_device.h"
#include "oasis_launch.h"

namespace oasis {

constexpr int kPoolWaves = 4;

template <int D>
__global__ __launch_bounds__(kPoolWaves * kWave) void pool_keys_kernel(PoolArgs a) {
    constexpr int NI = D / 32;                   // load instructions: 4 slices of 8 dims each
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const long long gw = (long long)blockIdx.x * kPoolWaves + wave;
    const int rows = a.batch * a.hkv;
    int row, n;
    if (a.last_only) {
        if (gw >= rows) return;
        row = (int)gw;
        n = -1;
    } else {
        row = (int)(gw / a.width);
        if (row >= rows) return;
        n = (int)(gw - (long long)row * a.width);
    }
    const int b = row / a.hkv;
    const int g = row - b * a.hkv;
    long long ctx = a.ctx_len[b];
    const long long cmax = (long long)a.width * kBlockTokens;
    ctx = ctx < 0 ? 0 : (ctx > cmax ? cmax : ctx);
    const int nb = (int)((ctx + kBlockTokens - 1) / kBlockTokens);
    if (a.last_only) n = nb - 1;
    if (n < 0 || n >= nb) return;
    long long nt = ctx - (long long)n * kBlockTokens;
    nt = nt > kBlockTokens ? kBlockTokens : nt;

    // The tile is stored in 8-dimension slices ([D/8][16][8]): load i, lane l
    // reads token t = l % 16 of slice 4i + l / 16 (1 KiB contiguous per load).
    const int t = lane & 15;
    const int g4 = lane >> 4;
    const int page = a.block_table[(size_t)b * a.width + n];
    if (page < 0 || page >= a.num_pages) {
        if (t == 0) {
            const u32x4 pinf = {0x7f807f80u, 0x7f807f80u, 0x7f807f80u, 0x7f807f80u};
            const u32x4 ninf = {0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                *reinterpret_cast<u32x4 *>(a.ck + ck_slice_offset(row, a.width, n, 4 * i + g4, D)) = pinf;
                *reinterpret_cast<u32x4 *>(a.ck + ck_slice_offset(row, a.width, n, D / 8 + 4 * i + g4, D)) = ninf;
            }
        }
        return;
    }
    const uint16_t *tile = a.k_pool + ((size_t)page * a.hkv + g) * kBlockTokens * D;
    u32x4 v[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i)
        v[i] = *reinterpret_cast<const u32x4 *>(tile + (size_t)i * 512 + lane * 8);
    float mn[NI][8], mx[NI][8];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const bool ok = t < nt;
            const float lo = bf16_bits_to_float(v[i][w] & 0xffffu);
            const float hi = bf16_bits_to_float(v[i][w] >> 16);
            mn[i][2 * w] = ok ? lo : __builtin_inff();
            mx[i][2 * w] = ok ? lo : -__builtin_inff();
            mn[i][2 * w + 1] = ok ? hi : __builtin_inff();
            mx[i][2 * w + 1] = ok ? hi : -__builtin_inff();
        }
    }
    // fold the 16 tokens of each slice (lanes of one 16-lane group)
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                mn[i][e] = fminf(mn[i][e], shfl_xor_f(mn[i][e], off));
                mx[i][e] = fmaxf(mx[i][e], shfl_xor_f(mx[i][e], off));
            }
        }
    }
    if (t == 0) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            u32x4 pmn, pmx;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                // exact: every value is a bf16 key element
                pmn[w] = (__builtin_bit_cast(uint32_t, mn[i][2 * w]) >> 16) |
                         (__builtin_bit_cast(uint32_t, mn[i][2 * w + 1]) & 0xffff0000u);
                pmx[w] = (__builtin_bit_cast(uint32_t, mx[i][2 * w]) >> 16) |
                         (__builtin_bit_cast(uint32_t, mx[i][2 * w + 1]) & 0xffff0000u);
            }
            *reinterpret_cast<u32x4 *>(a.ck + ck_slice_offset(row, a.width, n, 4 * i + g4, D)) = pmn;
            *reinterpret_cast<u32x4 *>(a.ck + ck_slice_offset(row, a.width, n, D / 8 + 4 * i + g4, D)) = pmx;
        }
    }
}

hipError_t launch_pool_keys(const PoolArgs &a, int head_dim, hipStream_t stream) {
    const long long rows = (long long)a.batch * a.hkv;
    const long long waves = a.last_only ? rows : rows * a.width;
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
