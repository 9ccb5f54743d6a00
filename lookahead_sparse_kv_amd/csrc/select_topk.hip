// select_topk.hip -- per-KV-head top-K block selection.
//
// OasisKV (metalmedia.ai summary), Figure 7 caption: the next step's top-K
// blocks; abstract: a 2,048-token KV budget, K = budget / 16 blocks per KV
// head.  Ties go to the lower block index; the set is written ascending.
//
// Design: one workgroup per (sequence, KV head) row.  Scores become
// order-preserving 32-bit keys in LDS; four 8-bit radix passes (LDS histogram
// + workgroup scan) find the K-th largest key tau exactly.  Every key above
// tau is taken, and of the keys equal to tau the lowest-index ones fill the
// rest; an ordered workgroup scan over index-contiguous chunks writes the
// winners in ascending order.  The result is exact and deterministic (no
// floating-point arithmetic, no atomics whose order matters).
#include "oasis_device.h"
#include "oasis_launch.h"

namespace oasis {

constexpr int kSelThreads = 256;

// Larger float -> larger key; -0.0 maps to +0.0 so that the two compare equal.
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive scan of one int per thread over a 256-thread workgroup.
__device__ __forceinline__ int block_inclusive_scan(int v, int *wave_sums) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int t = __shfl_up(v, d, kWave);
        if (lane >= d) v += t;
    }
    if (lane == kWave - 1) wave_sums[wave] = v;
    __syncthreads();
    int off = 0;
    for (int w = 0; w < wave; ++w) off += wave_sums[w];
    __syncthreads();
    return v + off;
}

__global__ __launch_bounds__(kSelThreads) void select_topk_kernel(SelectArgs a) {
    extern __shared__ uint32_t keys[];           // [width]
    __shared__ int hist[256];
    __shared__ int wave_sums[kSelThreads / kWave];
    __shared__ int s_digit, s_above;

    const int tid = threadIdx.x;
    const int row = blockIdx.x;
    const int b = row / a.hkv;
    int ctx = a.ctx_len[b];
    ctx = ctx < 0 ? 0 : ctx;
    int nb = (ctx + kBlockTokens - 1) / kBlockTokens;
    nb = nb > a.width ? a.width : nb;
    const float *srow = a.scores + (size_t)row * a.width;
    int32_t *out = a.sel + (size_t)row * a.k;

    if (nb <= a.k) {                              // every valid block is selected
        for (int i = tid; i < a.k; i += kSelThreads) out[i] = i < nb ? i : -1;
        return;
    }
    for (int n = tid; n < nb; n += kSelThreads) keys[n] = order_key(srow[n]);
    __syncthreads();

    uint32_t prefix = 0, mask = 0;
    int krem = a.k;                               // how many still to take at/below the prefix
    for (int shift = 24; shift >= 0; shift -= 8) {
        hist[tid] = 0;
        __syncthreads();
        for (int n = tid; n < nb; n += kSelThreads) {
            const uint32_t u = keys[n];
            if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1);
        }
        __syncthreads();
        // thread t looks at digit 255 - t: inclusive scan = keys with digit >= 255 - t
        const int c = hist[255 - tid];
        const int incl = block_inclusive_scan(c, wave_sums);
        const int excl = incl - c;
        if (excl < krem && krem <= incl) { s_digit = 255 - tid; s_above = excl; }
        __syncthreads();
        prefix |= (uint32_t)s_digit << shift;
        mask |= 255u << shift;
        krem -= s_above;
        __syncthreads();
    }
    const uint32_t tau = prefix;                  // the K-th largest key; krem of its copies are taken

    const int E = (nb + kSelThreads - 1) / kSelThreads;
    const int lo = tid * E;
    const int hi = lo + E < nb ? lo + E : nb;
    int c_gt = 0, c_eq = 0;
    for (int n = lo; n < hi; ++n) {
        const uint32_t u = keys[n];
        c_gt += u > tau;
        c_eq += u == tau;
    }
    const int eq_before = block_inclusive_scan(c_eq, wave_sums) - c_eq;
    int take_eq = krem - eq_before;
    take_eq = take_eq < 0 ? 0 : (take_eq > c_eq ? c_eq : take_eq);
    const int c_sel = c_gt + take_eq;
    int pos = block_inclusive_scan(c_sel, wave_sums) - c_sel;
    int er = eq_before;
    for (int n = lo; n < hi; ++n) {
        const uint32_t u = keys[n];
        bool take = u > tau;
        if (u == tau) { take = er < krem; ++er; }
        if (take) out[pos++] = n;
    }
}

hipError_t launch_select_topk(const SelectArgs &a, hipStream_t stream) {
    if (a.rows == 0) return hipSuccess;
    const size_t shmem = (size_t)(a.width > 0 ? a.width : 1) * sizeof(uint32_t);
    hipLaunchKernelGGL(select_topk_kernel, dim3(a.rows), dim3(kSelThreads), shmem, stream, a);
    return hipGetLastError();
}

}  // namespace oasis
