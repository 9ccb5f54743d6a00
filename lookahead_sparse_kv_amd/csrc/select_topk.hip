// select_topk.hip -- per-KV-head top-K block selection.
//
// OasisKV (metalmedia.ai summary), Figure 7 caption: the next step's top-K
// blocks; abstract: a 2,048-token KV budget, K = budget / 16 blocks per KV
// head.  Ties go to the lower block index; the set is written ascending.
//
// Design: one 1024-thread workgroup per (sequence, KV head) row.  Thread t
// holds the order-preserving 32-bit keys of blocks t, t + 1024, ... in
// registers (at most 15 per thread).  The K-th largest key tau is found bit
// by bit from the top: a candidate prefix survives when at least K keys are
// >= it; each count is a wavefront ballot + popcount per register slot (on
// the scalar unit) summed over the 16 waves through LDS, one barrier a step.
// Every key above tau is taken, and of the keys equal to tau the lowest-index
// ones fill the rest; register slot i of thread t is block 1024 i + t, so a
// ballot prefix per slot followed by a scan over the waves walks the blocks
// in ascending order and writes the winners in place.  Exact and
// deterministic: integer compares only, no atomics.
#include "oasis_device.h"
#include "oasis_launch.h"

namespace oasis {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kSelPerThread = (kMaxSelectWidth + kSelThreads - 1) / kSelThreads;

// Larger float -> larger key; -0.0 maps to +0.0 so that the two compare equal.
// Every non-NaN float maps to a key >= 0x007fffff, so 0 marks "no block".
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int popc_lt(uint64_t mask, int lane) {
    return __popcll(mask & ((1ull << lane) - 1ull));
}

__global__ __launch_bounds__(kSelThreads) void select_topk_kernel(SelectArgs a) {
    __shared__ int counts[2][kSelWaves];
    __shared__ int wsum_a[kSelWaves], wsum_b[kSelWaves];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int row = blockIdx.x;
    const int b = row / a.hkv;
    int ctx = a.ctx_len[b];
    ctx = ctx < 0 ? 0 : ctx;
    int nb = ctx / kBlockTokens + (ctx % kBlockTokens != 0);   // ceil, no overflow
    nb = nb > a.width ? a.width : nb;
    const float *srow = a.scores + (size_t)row * a.width;
    int32_t *out = a.sel + (size_t)row * a.k;

    if (nb <= a.k) {                              // every valid block is selected
        for (int i = tid; i < a.k; i += kSelThreads) out[i] = i < nb ? i : -1;
        return;
    }
    const int E = (nb + kSelThreads - 1) / kSelThreads;   // register slots in use (uniform)
    uint32_t key[kSelPerThread];
#pragma unroll
    for (int i = 0; i < kSelPerThread; ++i) {
        const int n = i * kSelThreads + tid;
        key[i] = (i < E && n < nb) ? order_key(srow[n]) : 0u;
    }

    // tau = the largest key value with at least K keys >= tau (the K-th largest key)
    uint32_t tau = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = tau | (1u << bit);
        int c = 0;
#pragma unroll
        for (int i = 0; i < kSelPerThread; ++i)
            if (i < E) c += __popcll(__ballot(key[i] >= cand));
        if (lane == 0) counts[bit & 1][wave] = c;
        __syncthreads();
        int total = 0;
#pragma unroll
        for (int w = 0; w < kSelWaves; ++w) total += counts[bit & 1][w];
        if (total >= a.k) tau = cand;
    }

    // How many keys lie strictly above tau; the rest of K are copies of tau.
    int c_gt = 0;
#pragma unroll
    for (int i = 0; i < kSelPerThread; ++i)
        if (i < E) c_gt += __popcll(__ballot(key[i] > tau));
    if (lane == 0) counts[1][wave] = c_gt;       // counts[1] is free again after the last step's barrier
    __syncthreads();
    int gt_total = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) gt_total += counts[1][w];
    const int krem = a.k - gt_total;

    // Walk the blocks in ascending order, one register slot (1024 blocks) at a time.
    int eq_base = 0, out_base = 0;
#pragma unroll
    for (int i = 0; i < kSelPerThread; ++i) {
        if (i >= E) break;                        // uniform across the workgroup
        const uint32_t u = key[i];
        const uint64_t eqm = __ballot(u == tau);
        if (lane == 0) wsum_a[wave] = __popcll(eqm);
        __syncthreads();
        int eq_before = eq_base, eq_slab = 0;
#pragma unroll
        for (int w = 0; w < kSelWaves; ++w) {
            const int c = wsum_a[w];
            eq_before += (w < wave) ? c : 0;
            eq_slab += c;
        }
        eq_before += popc_lt(eqm, lane);
        const bool take = (u > tau) || (u == tau && eq_before < krem);
        const uint64_t tm = __ballot(take);
        if (lane == 0) wsum_b[wave] = __popcll(tm);
        __syncthreads();
        int pos = out_base, take_slab = 0;
#pragma unroll
        for (int w = 0; w < kSelWaves; ++w) {
            const int c = wsum_b[w];
            pos += (w < wave) ? c : 0;
            take_slab += c;
        }
        pos += popc_lt(tm, lane);
        if (take) out[pos] = i * kSelThreads + tid;
        eq_base += eq_slab;
        out_base += take_slab;
        __syncthreads();                          // wsum_a / wsum_b are reused next slab
    }
}

hipError_t launch_select_topk(const SelectArgs &a, hipStream_t stream) {
    if (a.rows == 0) return hipSuccess;
    hipLaunchKernelGGL(select_topk_kernel, dim3(a.rows), dim3(kSelThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace oasis
