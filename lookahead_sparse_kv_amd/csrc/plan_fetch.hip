// plan_fetch.hip -- resident diff, fetch cap and capped LRU eviction.
//
// OasisKV (metalmedia.ai summary): five-step flow step 3 (compare the
// prediction with the blocks already on the GPU, pull only the missing ones,
// bound the transfer per step); Figure 9 caption (a per-KV-head table maps
// each GPU working-set block to a CPU logical block); Table 2 caption (the
// cap is a fetch ratio of the budget; LRU eviction); glossary entry on capped
// eviction.
//
// One workgroup per (sequence, KV head) row; the row's selection and its
// slot table sit in LDS.  Every ranking is a count of the elements that beat
// an element (integer compares, plus fp32 score compares for the misses), so
// each thread decides its own elements independently and the result is exact
// and deterministic.  Per row the work is O(K^2) compares with K <= 1024.
#include "oasis_device.h"
#include "oasis_launch.h"

namespace oasis {

constexpr int kPlanThreads = 256;

__global__ __launch_bounds__(kPlanThreads) void plan_fetch_kernel(PlanArgs a) {
    extern __shared__ int sm[];
    const int K = a.k;
    int *sel = sm;              // [K] selected blocks (-1 = none)
    int *sb = sel + K;          // [K] slot -> block, as read
    int *lu = sb + K;           // [K] slot -> last use, as read
    int *sb_new = lu + K;       // [K]
    int *lu_new = sb_new + K;   // [K]
    int *flag = lu_new + K;     // [K] per selected entry: 1 = miss
    int *fetched = flag + K;    // [K] per selected entry: 1 = miss that is fetched
    int *hitslot = fetched + K; // [K] per slot: 1 = holds a selected block
    int *dest = hitslot + K;    // [K] destination slot of the p-th fetched block
    __shared__ int s_nfree, s_nfetch;

    const int tid = threadIdx.x;
    const int row = blockIdx.x;
    const float *srow = a.scores + (size_t)row * a.width;
    if (tid == 0) { s_nfree = 0; s_nfetch = 0; }
    for (int i = tid; i < K; i += kPlanThreads) {
        const int s = a.sel[(size_t)row * K + i];
        sel[i] = (s >= 0 && s < a.width) ? s : -1;
        sb[i] = a.slot_block[(size_t)row * K + i];
        lu[i] = a.last_use[(size_t)row * K + i];
        dest[i] = -1;
    }
    __syncthreads();

    // Hits and misses.
    for (int j = tid; j < K; j += kPlanThreads) {
        const int blk = sb[j];
        int hit = 0;
        if (blk >= 0)
            for (int i = 0; i < K; ++i) hit |= (sel[i] == blk);
        hitslot[j] = hit;
        sb_new[j] = blk;
        lu_new[j] = hit ? a.step : lu[j];
        if (blk < 0) atomicAdd(&s_nfree, 1);
    }
    for (int i = tid; i < K; i += kPlanThreads) {
        const int blk = sel[i];
        int resident = 0;
        if (blk >= 0)
            for (int j = 0; j < K; ++j) resident |= (sb[j] == blk);
        flag[i] = (blk >= 0 && !resident) ? 1 : 0;
        fetched[i] = 0;
    }
    __syncthreads();

    // Rank the misses by (score desc, block asc); the first `cap` are fetched.
    for (int i = tid; i < K; i += kPlanThreads) {
        if (flag[i] != 1) continue;
        const int blk = sel[i];
        const float s = srow[blk];
        int rank = 0;
        for (int i2 = 0; i2 < K; ++i2) {
            if (flag[i2] == 0 || i2 == i) continue;
            const int b2 = sel[i2];
            const float s2 = srow[b2];
            rank += (s2 > s) || (s2 == s && b2 < blk);
        }
        if (rank < a.cap) { fetched[i] = 1; atomicAdd(&s_nfetch, 1); }
    }
    __syncthreads();
    const int nF = s_nfetch;
    const int nfree = s_nfree;

    // Destinations: free slots ascending, then LRU victims among the
    // unselected resident blocks ordered by (last use, block).
    for (int j = tid; j < K; j += kPlanThreads) {
        if (sb[j] < 0) {
            int pos = 0;
            for (int j2 = 0; j2 < j; ++j2) pos += (sb[j2] < 0);
            if (pos < nF) dest[pos] = j;
        } else if (!hitslot[j] && nF > nfree) {
            const int l0 = lu[j], b0 = sb[j];
            int rank = 0;
            for (int j2 = 0; j2 < K; ++j2) {
                if (sb[j2] < 0 || hitslot[j2] || j2 == j) continue;
                rank += (lu[j2] < l0) || (lu[j2] == l0 && sb[j2] < b0);
            }
            if (rank < nF - nfree) dest[nfree + rank] = j;
        }
    }
    __syncthreads();

    // The p-th fetched block in ascending block order goes to dest[p].
    for (int i = tid; i < K; i += kPlanThreads) {
        if (!fetched[i]) continue;
        const int blk = sel[i];
        int p = 0;
        for (int i2 = 0; i2 < K; ++i2) p += (fetched[i2] && sel[i2] < blk);
        const int d = dest[p];
        a.fetch_block[(size_t)row * a.cap + p] = blk;
        a.fetch_slot[(size_t)row * a.cap + p] = d;
        if (d >= 0) { sb_new[d] = blk; lu_new[d] = a.step; }
    }
    for (int p = nF + tid; p < a.cap; p += kPlanThreads) {
        a.fetch_block[(size_t)row * a.cap + p] = -1;
        a.fetch_slot[(size_t)row * a.cap + p] = -1;
    }
    if (tid == 0) a.fetch_count[row] = nF;
    __syncthreads();
    for (int j = tid; j < K; j += kPlanThreads) {
        a.slot_block[(size_t)row * K + j] = sb_new[j];
        a.last_use[(size_t)row * K + j] = lu_new[j];
    }
}

hipError_t launch_plan_fetch(const PlanArgs &a, hipStream_t stream) {
    if (a.rows == 0) return hipSuccess;
    const size_t shmem = (size_t)9 * a.k * sizeof(int);
    hipLaunchKernelGGL(plan_fetch_kernel, dim3(a.rows), dim3(kPlanThreads), shmem, stream, a);
    return hipGetLastError();
}

}  // namespace oasis
