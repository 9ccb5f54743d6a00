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
// host pool over PCIe and writes it into its working-set slot: 4 KiB of keys
// and 4 KiB of values per block (D = 128), 16 bytes per lane per load.  The
// grid is a small fixed number of waves that walk the list two entries at a
// time, all loads of both entries issued before any store: the bus is kept
// full with few waves, so the kernel holds few of the wave slots the
// concurrent scoring and attention of the following layers need, and it needs
// no host synchronisation.
#include "oasis_device.h"
#include "oasis_launch.h"

#ifndef OASIS_FETCH_WAVES
#define OASIS_FETCH_WAVES 64
#endif

namespace oasis {

constexpr int kFetchWaves = 4;                       // waves per workgroup
constexpr int kFetchGridWaves = OASIS_FETCH_WAVES;   // waves in the grid, at most

// Source and destination tiles of list entry e (row = e / cap), or ok = false
// for padding, out-of-range entries and invalid ids.
template <int D>
struct FetchEntry {
    const u32x4 *src_k, *src_v;
    u32x4 *dst_k, *dst_v;
    bool ok;
};

template <int D>
__device__ __forceinline__ FetchEntry<D> fetch_entry(const FetchArgs &a, long long e, long long total) {
    FetchEntry<D> f{nullptr, nullptr, nullptr, nullptr, false};
    if (e >= total) return f;
    const int row = (int)(e / a.cap);
    const int i = (int)(e - (long long)row * a.cap);
    int cnt = a.fetch_count[row];
    cnt = cnt < 0 ? 0 : (cnt > a.cap ? a.cap : cnt);
    if (i >= cnt) return f;
    const int blk = a.fetch_block[(size_t)row * a.cap + i];
    const int slot = a.fetch_slot[(size_t)row * a.cap + i];
    if (blk < 0 || blk >= a.host_blocks || slot < 0 || slot >= a.k_slots) return f;
    const int b = row / a.hkv;
    const int g = row - b * a.hkv;
    const int page = a.ws_page_table[(size_t)b * a.k_slots + slot];
    if (page < 0 || page >= a.ws_pages) return f;
    const size_t tile = (size_t)kBlockTokens * D;
    f.src_k = reinterpret_cast<const u32x4 *>(a.host_k + ((size_t)row * a.host_blocks + blk) * tile);
    f.src_v = reinterpret_cast<const u32x4 *>(a.host_v + ((size_t)row * a.host_blocks + blk) * tile);
    f.dst_k = reinterpret_cast<u32x4 *>(a.ws_k + ((size_t)page * a.hkv + g) * tile);
    f.dst_v = reinterpret_cast<u32x4 *>(a.ws_v + ((size_t)page * a.hkv + g) * tile);
    f.ok = true;
    return f;
}

template <int D>
__global__ __launch_bounds__(kFetchWaves * kWave) void fetch_blocks_kernel(FetchArgs a) {
    constexpr int kTileVec = kBlockTokens * D * 2 / 16;   // 16-byte vectors per tile
    constexpr int kPer = kTileVec / kWave;                 // per lane
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const long long nw = (long long)gridDim.x * kFetchWaves;
    const long long total = (long long)a.batch * a.hkv * a.cap;
    for (long long e = (long long)blockIdx.x * kFetchWaves + wave; e < total; e += 2 * nw) {
        const FetchEntry<D> f0 = fetch_entry<D>(a, e, total);
        const FetchEntry<D> f1 = fetch_entry<D>(a, e + nw, total);
        u32x4 k0[kPer], v0[kPer], k1[kPer], v1[kPer];
        if (f0.ok) {
#pragma unroll
            for (int c = 0; c < kPer; ++c) {
                k0[c] = f0.src_k[c * kWave + lane];
                v0[c] = f0.src_v[c * kWave + lane];
            }
        }
        if (f1.ok) {
#pragma unroll
            for (int c = 0; c < kPer; ++c) {
                k1[c] = f1.src_k[c * kWave + lane];
                v1[c] = f1.src_v[c * kWave + lane];
            }
        }
        if (f0.ok) {
#pragma unroll
            for (int c = 0; c < kPer; ++c) {
                f0.dst_k[c * kWave + lane] = k0[c];
                f0.dst_v[c * kWave + lane] = v0[c];
            }
        }
        if (f1.ok) {
#pragma unroll
            for (int c = 0; c < kPer; ++c) {
                f1.dst_k[c * kWave + lane] = k1[c];
                f1.dst_v[c * kWave + lane] = v1[c];
            }
        }
    }
}

hipError_t launch_fetch_blocks(const FetchArgs &a, int head_dim, hipStream_t stream) {
    const long long entries = (long long)a.batch * a.hkv * a.cap;
    if (entries == 0) return hipSuccess;
    const long long waves = entries < kFetchGridWaves ? entries : kFetchGridWaves;
    const dim3 grid((unsigned)((waves + kFetchWaves - 1) / kFetchWaves));
    const dim3 block(kFetchWaves * kWave);
    if (head_dim == 128)
        hipLaunchKernelGGL(fetch_blocks_kernel<128>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(fetch_blocks_kernel<64>, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace oasis
