// plan_fetch.hip -- resident diff, fetch cap and capped LRU eviction.
//
// OasisKV (metalmedia.ai summary): five-step flow step 3 (compare the
// prediction with the blocks already on the GPU, pull only the missing ones,
// bound the transfer per step); Figure 9 caption (a per-KV-head table maps
// each GPU working-set block to a CPU logical block); Table 2 caption (the
// cap is a fetch ratio of the budget; LRU eviction); glossary entry on capped
// eviction.
//
// One workgroup per (sequence, KV head) row; the row's selection, the scores
// of the selected blocks and the slot table sit in LDS, padded to a multiple
// of 16 entries.  Every ranking is a count of the elements that beat an
// element (integer compares, plus fp32 score compares for the misses), so each
// thread decides its own element independently and the result is exact and
// deterministic.  The counting loops read LDS 16 bytes at a time and are
// unrolled so that many reads are in flight; per row the work is O(K^2)
// compares with K <= 1024.
#include "oasis_device.h"
#include "oasis_launch.h"

namespace oasis {

constexpr int kPlanThreads = 256;
constexpr int kPad = 16;

__device__ __forceinline__ int4 ld4(const int *p) { return *reinterpret_cast<const int4 *>(p); }
__device__ __forceinline__ float4 ld4f(const float *p) { return *reinterpret_cast<const float4 *>(p); }

__global__ __launch_bounds__(kPlanThreads) void plan_fetch_kernel(PlanArgs a) {
    extern __shared__ int sm[];
    const int K = a.k;
    const int Kp = (K + kPad - 1) / kPad * kPad;
    int *sel = sm;                     // selected blocks (-1 = none; pad -1)
    float *sel_score = reinterpret_cast<float *>(sel + Kp);
    int *miss = sel + 2 * Kp;          // 1 = selected and not resident (pad 0)
    int *fetched = sel + 3 * Kp;       // 1 = miss that is fetched (pad 0)
    int *sb = sel + 4 * Kp;            // slot -> block as read (-1 = empty; pad -2)
    int *lu = sel + 5 * Kp;            // slot -> last use as read
    int *cand = sel + 6 * Kp;          // 1 = resident and not selected: may be evicted (pad 0)
    int *sb_new = sel + 7 * Kp;
    int *lu_new = sel + 8 * Kp;
    int *dest = sel + 9 * Kp;          // destination slot of the p-th fetched block
    __shared__ int s_nfree, s_nfetch;

    const int tid = threadIdx.x;
    const int row = blockIdx.x;
    const float *srow = a.scores + (size_t)row * a.width;
    if (tid == 0) { s_nfree = 0; s_nfetch = 0; }
    for (int i = tid; i < Kp; i += kPlanThreads) {
        if (i < K) {
            const int s = a.sel[(size_t)row * K + i];
            const bool ok = s >= 0 && s < a.width;
            sel[i] = ok ? s : -1;
            sel_score[i] = ok ? srow[s] : 0.f;
            const int blk = a.slot_block[(size_t)row * K + i];
            sb[i] = blk < 0 ? -1 : blk;
            lu[i] = a.last_use[(size_t)row * K + i];
        } else {
            sel[i] = -1;
            sel_score[i] = 0.f;
            sb[i] = -2;
            lu[i] = 0;
        }
        miss[i] = 0;
        fetched[i] = 0;
        cand[i] = 0;
        dest[i] = -1;
    }
    __syncthreads();

    // Hits refresh their slot; unselected residents become eviction candidates.
    for (int j = tid; j < K; j += kPlanThreads) {
        const int blk = sb[j];
        bool hit = false;
        if (blk >= 0) {
#pragma unroll 4
            for (int i = 0; i < Kp; i += 4) {
                const int4 v = ld4(sel + i);
                hit |= (v.x == blk) | (v.y == blk) | (v.z == blk) | (v.w == blk);
            }
        }
        cand[j] = (blk >= 0 && !hit) ? 1 : 0;
        sb_new[j] = blk;
        lu_new[j] = hit ? a.step : lu[j];
        if (blk == -1) atomicAdd(&s_nfree, 1);
    }
    // Misses: selected blocks held by no slot.
    for (int i = tid; i < K; i += kPlanThreads) {
        const int blk = sel[i];
        bool resident = false;
        if (blk >= 0) {
#pragma unroll 4
            for (int j = 0; j < Kp; j += 4) {
                const int4 v = ld4(sb + j);
                resident |= (v.x == blk) | (v.y == blk) | (v.z == blk) | (v.w == blk);
            }
        }
        miss[i] = (blk >= 0 && !resident) ? 1 : 0;
    }
    __syncthreads();

    // Rank the misses by (score desc, block asc); the first `cap` are fetched.
    for (int i = tid; i < K; i += kPlanThreads) {
        if (!miss[i]) continue;
        const int blk = sel[i];
        const float s = sel_score[i];
        int rank = 0;
#pragma unroll 4
        for (int i2 = 0; i2 < Kp; i2 += 4) {
            const int4 m = ld4(miss + i2);
            const int4 b2 = ld4(sel + i2);
            const float4 s2 = ld4f(sel_score + i2);
            rank += m.x & ((s2.x > s) | ((s2.x == s) & (b2.x < blk)));
            rank += m.y & ((s2.y > s) | ((s2.y == s) & (b2.y < blk)));
            rank += m.z & ((s2.z > s) | ((s2.z == s) & (b2.z < blk)));
            rank += m.w & ((s2.w > s) | ((s2.w == s) & (b2.w < blk)));
        }
        if (rank < a.cap) { fetched[i] = 1; atomicAdd(&s_nfetch, 1); }
    }
    __syncthreads();
    const int nF = s_nfetch;
    const int nfree = s_nfree;

    // Destinations: free slots ascending, then LRU victims among the
    // unselected resident blocks ordered by (last use, block).
    for (int j = tid; j < K; j += kPlanThreads) {
        if (sb[j] == -1) {
            int pos = 0;
#pragma unroll 4
            for (int j2 = 0; j2 < Kp; j2 += 4) {
                const int4 v = ld4(sb + j2);
                pos += (v.x == -1) & (j2 < j);
                pos += (v.y == -1) & (j2 + 1 < j);
                pos += (v.z == -1) & (j2 + 2 < j);
                pos += (v.w == -1) & (j2 + 3 < j);
            }
            if (pos < nF) dest[pos] = j;
        } else if (cand[j] && nF > nfree) {
            const int l0 = lu[j], b0 = sb[j];
            int rank = 0;
#pragma unroll 4
            for (int j2 = 0; j2 < Kp; j2 += 4) {
                const int4 c = ld4(cand + j2);
                const int4 l2 = ld4(lu + j2);
                const int4 b2 = ld4(sb + j2);
                rank += c.x & ((l2.x < l0) | ((l2.x == l0) & (b2.x < b0)));
                rank += c.y & ((l2.y < l0) | ((l2.y == l0) & (b2.y < b0)));
                rank += c.z & ((l2.z < l0) | ((l2.z == l0) & (b2.z < b0)));
                rank += c.w & ((l2.w < l0) | ((l2.w == l0) & (b2.w < b0)));
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
#pragma unroll 4
        for (int i2 = 0; i2 < Kp; i2 += 4) {
            const int4 f = ld4(fetched + i2);
            const int4 b2 = ld4(sel + i2);
            p += (f.x & (b2.x < blk)) + (f.y & (b2.y < blk)) + (f.z & (b2.z < blk)) + (f.w & (b2.w < blk));
        }
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
    const int Kp = (a.k + kPad - 1) / kPad * kPad;
    const size_t shmem = (size_t)10 * Kp * sizeof(int);
    hipLaunchKernelGGL(plan_fetch_kernel, dim3(a.rows), dim3(kPlanThreads), shmem, stream, a);
    return hipGetLastError();
}

}  // namespace oasis
