// fetch_blocks.hip -- the capped fetch of working-set blocks from the pinned
// host KV pool into HBM.
//
// OasisKV (metalmedia.ai summary): five-step flow step 3 (only the missing
// blocks are pulled, under a per-step bound that keeps the transfer within the
// PCIe budget), Figure 8 caption (the transfer runs in the background before
// that layer's attention at the next step), Figure 9 caption (working-set
// slots map to CPU logical blocks per KV head).
//
// Design: the planner leaves the fetch list in device memory.  Instead of
// bringing it back to the host and issuing one copy per block, a kernel on a
// side stream reads each listed block straight from the device-mapped pinned
// host pool over PCIe and writes it into its working-set slot: one wave per
// (row, list entry), 4 KiB of keys and 4 KiB of values per block (D = 128),
// 16 bytes per lane per load, all loads of a block issued before any store.
// The kernel needs no host synchronisation and uses few CUs; it overlaps the
// scoring and attention of the following layers.
#include "oasis_device.h"
#include "oasis_launch.h"

namespace oasis {

constexpr int kFetchWaves = 4;

template <int D>
__global__ __launch_bounds__(kFetchWaves * kWave) void fetch_blocks_kernel(FetchArgs a) {
    constexpr int kTileVec = kBlockTokens * D * 2 / 16;   // 16-byte vectors per tile
    constexpr int kPer = kTileVec / kWave;                 // per lane
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const long long gw = (long long)blockIdx.x * kFetchWaves + wave;
    const int rows = a.batch * a.hkv;
    const int row = (int)(gw / a.cap);
    if (row >= rows) return;
    const int i = (int)(gw - (long long)row * a.cap);
    int cnt = a.fetch_count[row];
    cnt = cnt < 0 ? 0 : (cnt > a.cap ? a.cap : cnt);
    if (i >= cnt) return;
    const int blk = a.fetch_block[(size_t)row * a.cap + i];
    const int slot = a.fetch_slot[(size_t)row * a.cap + i];
    if (blk < 0 || blk >= a.host_blocks || slot < 0 || slot >= a.k_slots) return;
    const int b = row / a.hkv;
    const int g = row - b * a.hkv;
    const int page = a.ws_page_table[(size_t)b * a.k_slots + slot];
    if (page < 0 || page >= a.ws_pages) return;

    const size_t tile = (size_t)kBlockTokens * D;
    const u32x4 *src_k = reinterpret_cast<const u32x4 *>(a.host_k + ((size_t)row * a.host_blocks + blk) * tile);
    const u32x4 *src_v = reinterpret_cast<const u32x4 *>(a.host_v + ((size_t)row * a.host_blocks + blk) * tile);
    u32x4 *dst_k = reinterpret_cast<u32x4 *>(a.ws_k + ((size_t)page * a.hkv + g) * tile);
    u32x4 *dst_v = reinterpret_cast<u32x4 *>(a.ws_v + ((size_t)page * a.hkv + g) * tile);
    u32x4 kr[kPer], vr[kPer];
#pragma unroll
    for (int c = 0; c < kPer; ++c) {
        kr[c] = src_k[c * kWave + lane];
        vr[c] = src_v[c * kWave + lane];
    }
#pragma unroll
    for (int c = 0; c < kPer; ++c) {
        dst_k[c * kWave + lane] = kr[c];
        dst_v[c * kWave + lane] = vr[c];
    }
}

hipError_t launch_fetch_blocks(const FetchArgs &a, int head_dim, hipStream_t stream) {
    const long long waves = (long long)a.batch * a.hkv * a.cap;
    if (waves == 0) return hipSuccess;
    const dim3 grid((unsigned)((waves + kFetchWaves - 1) / kFetchWaves));
    const dim3 block(kFetchWaves * kWave);
    if (head_dim == 128)
        hipLaunchKernelGGL(fetch_blocks_kernel<128>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(fetch_blocks_kernel<64>, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace oasis
