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
// Design: one wave per block.  The 4 KiB key tile (token-major) is read 16 B
// per lane, so one load instruction covers 64 lanes x 16 B = 4 tokens at
// D = 128 (8 at D = 64), contiguous in memory; each lane keeps the running
// min and max of its 8 dimensions and the token groups are folded by lane
// exchanges.  A page outside the pool is not read: the block is written as an
// empty box (min = +inf, max = -inf), which the compressed scorer turns into
// -inf.  The last-block mode refreshes only block ceil(ctx / 16) - 1 of each
// sequence: the one a decode step appends its token to.
#include "oasis_device.h"
#include "oasis_launch.h"

namespace oasis {

constexpr int kPoolWaves = 4;

template <int D>
__global__ __launch_bounds__(kPoolWaves * kWave) void pool_keys_kernel(PoolArgs a) {
    constexpr int CH = D / 8;                    // 16-byte chunks per token
    constexpr int TPL = kWave / CH;              // tokens per load instruction
    constexpr int NL = kBlockTokens / TPL;       // loads per lane
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

    const int c = lane % CH;         // dims 8c .. 8c + 7
    const int tg = lane / CH;        // tokens tg, tg + TPL, ...
    uint16_t *out = a.ck + ((size_t)row * a.width + n) * 2 * D;
    const int page = a.block_table[(size_t)b * a.width + n];
    if (page < 0 || page >= a.num_pages) {
        if (tg == 0) {
            const u32x4 pinf = {0x7f807f80u, 0x7f807f80u, 0x7f807f80u, 0x7f807f80u};
            const u32x4 ninf = {0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};
            *reinterpret_cast<u32x4 *>(out + 8 * c) = pinf;
            *reinterpret_cast<u32x4 *>(out + D + 8 * c) = ninf;
        }
        return;
    }
    const uint16_t *tile = a.k_pool + ((size_t)page * a.hkv + g) * kBlockTokens * D;
    float mn[8], mx[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) { mn[e] = __builtin_inff(); mx[e] = -__builtin_inff(); }
    u32x4 v[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int t = tg + TPL * i;
        v[i] = t < nt ? *reinterpret_cast<const u32x4 *>(tile + (size_t)t * D + 8 * c)
                      : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        if (tg + TPL * i < nt) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float lo = bf16_bits_to_float(v[i][w] & 0xffffu);
                const float hi = bf16_bits_to_float(v[i][w] >> 16);
                mn[2 * w] = fminf(mn[2 * w], lo);
                mx[2 * w] = fmaxf(mx[2 * w], lo);
                mn[2 * w + 1] = fminf(mn[2 * w + 1], hi);
                mx[2 * w + 1] = fmaxf(mx[2 * w + 1], hi);
            }
        }
    }
    // fold the token groups (lanes c, c + CH, c + 2 CH, ...)
#pragma unroll
    for (int off = CH; off < kWave; off <<= 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            mn[e] = fminf(mn[e], shfl_xor_f(mn[e], off));
            mx[e] = fmaxf(mx[e], shfl_xor_f(mx[e], off));
        }
    }
    if (tg == 0) {
        u32x4 pmn, pmx;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            // exact: every value is a bf16 key element
            pmn[w] = (__builtin_bit_cast(uint32_t, mn[2 * w]) >> 16) |
                     (__builtin_bit_cast(uint32_t, mn[2 * w + 1]) & 0xffff0000u);
            pmx[w] = (__builtin_bit_cast(uint32_t, mx[2 * w]) >> 16) |
                     (__builtin_bit_cast(uint32_t, mx[2 * w + 1]) & 0xffff0000u);
        }
        *reinterpret_cast<u32x4 *>(out + 8 * c) = pmn;
        *reinterpret_cast<u32x4 *>(out + D + 8 * c) = pmx;
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
