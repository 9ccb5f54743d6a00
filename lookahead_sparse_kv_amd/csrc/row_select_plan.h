// row_select_plan.h -- workgroup-level top-K selection and fetch planning of
// one (sequence, KV head) row, shared by the select, plan and fused kernels.
//
// OasisKV (metalmedia.ai summary): Figure 7 caption (the next step's top-K
// blocks), abstract (2,048-token KV budget), five-step flow step 3 (diff
// against the GPU-resident blocks and pull only the missing ones under a
// per-step bound), Figure 9 caption (per-KV-head working-set table), Table 2
// caption (fetch-ratio cap, LRU eviction).
//
// Selection (kRowThreads threads, keys in LDS): scores become order-preserving
// 32-bit keys (-0.0 equals +0.0).  The K-th largest key tau is found exactly by
// a radix select over three digits (11, 11 and 10 bits): an LDS histogram of
// the keys that still match the prefix, a workgroup scan over the bins from the
// top, and the bin where the count crosses the remaining K.  Keys above tau are
// taken, and copies of tau fill the rest in ascending block order (ordered
// scans over index-contiguous chunks), so ties go to the lower index and the
// set comes out ascending.
//
// Plan: every ranking is a count of the elements that beat an element
// (integer compares, plus fp32 score compares between misses), each thread
// deciding its own element; LDS is read 16 bytes at a time.  Exact and
// deterministic; O(K^2) compares per row.
#pragma once

#include "oasis_device.h"
#include "oasis_launch.h"

namespace oasis {

constexpr int kRowThreads = 256;
constexpr int kRowWaves = kRowThreads / kWave;
constexpr int kHistBins = 2048;          // widest radix digit: 11 bits
constexpr int kPlanPadding = 16;

__device__ __forceinline__ uint32_t score_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;            // -0.0 == +0.0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Scores of one row into LDS as keys.  A thread's loads (8 per round) are all
// issued before the first is used, so the row costs one memory latency per
// 2,048 blocks instead of one per 256.
__device__ __forceinline__ void load_row_keys(const float *srow, int nb, uint32_t *keys) {
    constexpr int U = 8;
    for (int n0 = 0; n0 < nb; n0 += kRowThreads * U) {
        float v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int n = n0 + u * kRowThreads + (int)threadIdx.x;
            v[u] = n < nb ? srow[n] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int n = n0 + u * kRowThreads + (int)threadIdx.x;
            if (n < nb) keys[n] = score_key(v[u]);
        }
    }
}

// Inclusive scan of one int per thread over the workgroup (two barriers).
__device__ __forceinline__ int row_inclusive_scan(int v, int *wave_sums) {
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
#pragma unroll
    for (int w = 0; w < kRowWaves; ++w) off += (w < wave) ? wave_sums[w] : 0;
    __syncthreads();
    return v + off;
}

struct RowShared {
    int hist[kHistBins];
    int wave_sums[kRowWaves];
    int digit, above, total;
};

// Top-K of `nb` keys (keys[0..nb), already in LDS) into sel[0..K): ascending,
// -1 padded.  Ends with a barrier; sel may then be read by every thread.
__device__ __forceinline__ void row_select(const uint32_t *keys, int nb, int K, int *sel,
                                           RowShared &sh) {
    const int tid = threadIdx.x;
    if (nb <= K) {
        for (int i = tid; i < K; i += kRowThreads) sel[i] = i < nb ? i : -1;
        __syncthreads();
        return;
    }
    uint32_t prefix = 0, pmask = 0;
    int krem = K;                                 // still to take among keys matching the prefix
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const int nbins = pass == 2 ? 1024 : 2048;
        for (int i = tid; i < nbins; i += kRowThreads) sh.hist[i] = 0;
        __syncthreads();
        for (int n = tid; n < nb; n += kRowThreads) {
            const uint32_t u = keys[n];
            if ((u & pmask) == prefix) atomicAdd(&sh.hist[(u >> shift) & (uint32_t)(nbins - 1)], 1);
        }
        __syncthreads();
        // thread t owns `per` bins counted from the top: bins hi, hi-1, .., lo
        const int per = nbins / kRowThreads;
        const int hi = nbins - 1 - tid * per;
        int local = 0;
        for (int j = 0; j < per; ++j) local += sh.hist[hi - j];
        const int incl = row_inclusive_scan(local, sh.wave_sums);
        int acc = incl - local;                   // keys in bins above hi
        if (acc < krem && krem <= incl) {
            for (int j = 0; j < per; ++j) {
                const int c = sh.hist[hi - j];
                if (acc + c >= krem) { sh.digit = hi - j; sh.above = acc; break; }
                acc += c;
            }
        }
        __syncthreads();
        prefix |= (uint32_t)sh.digit << shift;
        pmask |= (uint32_t)(nbins - 1) << shift;
        krem -= sh.above;
        __syncthreads();                          // digit / above are rewritten next pass
    }
    const uint32_t tau = prefix;                  // the K-th largest key; krem copies of it are taken

    const int E = (nb + kRowThreads - 1) / kRowThreads;
    const int lo = tid * E;
    const int hi = lo + E < nb ? lo + E : nb;
    int c_gt = 0, c_eq = 0;
    for (int n = lo; n < hi; ++n) {
        const uint32_t u = keys[n];
        c_gt += u > tau;
        c_eq += u == tau;
    }
    const int eq_before = row_inclusive_scan(c_eq, sh.wave_sums) - c_eq;
    int take_eq = krem - eq_before;
    take_eq = take_eq < 0 ? 0 : (take_eq > c_eq ? c_eq : take_eq);
    const int c_sel = c_gt + take_eq;
    int pos = row_inclusive_scan(c_sel, sh.wave_sums) - c_sel;
    int er = eq_before;
    for (int n = lo; n < hi; ++n) {
        const uint32_t u = keys[n];
        bool take = u > tau;
        if (u == tau) { take = er < krem; ++er; }
        if (take) sel[pos++] = n;
    }
    __syncthreads();
}

__device__ __forceinline__ int4 ld_i4(const int *p) { return *reinterpret_cast<const int4 *>(p); }
__device__ __forceinline__ float4 ld_f4(const float *p) { return *reinterpret_cast<const float4 *>(p); }

// LDS of the plan: 9 arrays of Kp = roundup(K, 16) ints after `sel` (Kp ints).
__host__ __device__ __forceinline__ int plan_pad(int K) {
    return (K + kPlanPadding - 1) / kPlanPadding * kPlanPadding;
}

// The plan of one row.  sel[0..K) (LDS) holds the selection; sel_score(i) gives
// the fp32 score of sel[i]; slot_block / last_use / fetch_* point at this
// row's part of the global arrays.  `pl` is 9 * Kp ints of LDS.
template <class ScoreOf>
__device__ __forceinline__ void row_plan(int *sel, ScoreOf sel_score_of, int K, int cap, int step,
                                         int32_t *slot_block, int32_t *last_use,
                                         int32_t *fetch_block, int32_t *fetch_slot,
                                         int32_t *fetch_count, int *pl, RowShared &sh) {
    const int tid = threadIdx.x;
    const int Kp = plan_pad(K);
    float *sel_score = reinterpret_cast<float *>(pl);
    int *miss = pl + Kp;
    int *fetched = pl + 2 * Kp;
    int *sb = pl + 3 * Kp;         // slot -> block as read (-1 = empty; pad -2)
    int *lu = pl + 4 * Kp;
    int *cand = pl + 5 * Kp;       // resident and not selected: may be evicted
    int *sb_new = pl + 6 * Kp;
    int *lu_new = pl + 7 * Kp;
    int *dest = pl + 8 * Kp;       // destination slot of the p-th fetched block

    if (tid == 0) { sh.digit = 0; sh.above = 0; }    // reused as counters: free slots, fetches
    for (int i = tid; i < Kp; i += kRowThreads) {
        if (i < K) {
            const int s = sel[i];
            sel_score[i] = s >= 0 ? sel_score_of(s) : 0.f;
            const int blk = slot_block[i];
            sb[i] = blk < 0 ? -1 : blk;
            lu[i] = last_use[i];
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

    for (int j = tid; j < K; j += kRowThreads) {      // hits and eviction candidates
        const int blk = sb[j];
        bool hit = false;
        if (blk >= 0) {
#pragma unroll 4
            for (int i = 0; i < Kp; i += 4) {
                const int4 v = ld_i4(sel + i);
                hit |= (v.x == blk) | (v.y == blk) | (v.z == blk) | (v.w == blk);
            }
        }
        cand[j] = (blk >= 0 && !hit) ? 1 : 0;
        sb_new[j] = blk;
        lu_new[j] = hit ? step : lu[j];
        if (blk == -1) atomicAdd(&sh.digit, 1);
    }
    for (int i = tid; i < K; i += kRowThreads) {      // misses
        const int blk = sel[i];
        bool resident = false;
        if (blk >= 0) {
#pragma unroll 4
            for (int j = 0; j < Kp; j += 4) {
                const int4 v = ld_i4(sb + j);
                resident |= (v.x == blk) | (v.y == blk) | (v.z == blk) | (v.w == blk);
            }
        }
        miss[i] = (blk >= 0 && !resident) ? 1 : 0;
    }
    __syncthreads();

    for (int i = tid; i < K; i += kRowThreads) {      // rank misses: (score desc, block asc)
        if (!miss[i]) continue;
        const int blk = sel[i];
        const float s = sel_score[i];
        int rank = 0;
#pragma unroll 4
        for (int i2 = 0; i2 < Kp; i2 += 4) {
            const int4 m = ld_i4(miss + i2);
            const int4 b2 = ld_i4(sel + i2);
            const float4 s2 = ld_f4(sel_score + i2);
            rank += m.x & ((s2.x > s) | ((s2.x == s) & (b2.x < blk)));
            rank += m.y & ((s2.y > s) | ((s2.y == s) & (b2.y < blk)));
            rank += m.z & ((s2.z > s) | ((s2.z == s) & (b2.z < blk)));
            rank += m.w & ((s2.w > s) | ((s2.w == s) & (b2.w < blk)));
        }
        if (rank < cap) { fetched[i] = 1; atomicAdd(&sh.above, 1); }
    }
    __syncthreads();
    const int nfree = sh.digit;
    const int nF = sh.above;

    for (int j = tid; j < K; j += kRowThreads) {      // free slots, then LRU victims
        if (sb[j] == -1) {
            int pos = 0;
#pragma unroll 4
            for (int j2 = 0; j2 < Kp; j2 += 4) {
                const int4 v = ld_i4(sb + j2);
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
                const int4 c = ld_i4(cand + j2);
                const int4 l2 = ld_i4(lu + j2);
                const int4 b2 = ld_i4(sb + j2);
                rank += c.x & ((l2.x < l0) | ((l2.x == l0) & (b2.x < b0)));
                rank += c.y & ((l2.y < l0) | ((l2.y == l0) & (b2.y < b0)));
                rank += c.z & ((l2.z < l0) | ((l2.z == l0) & (b2.z < b0)));
                rank += c.w & ((l2.w < l0) | ((l2.w == l0) & (b2.w < b0)));
            }
            if (rank < nF - nfree) dest[nfree + rank] = j;
        }
    }
    __syncthreads();

    for (int i = tid; i < K; i += kRowThreads) {      // p-th fetched block (ascending) -> dest[p]
        if (!fetched[i]) continue;
        const int blk = sel[i];
        int p = 0;
#pragma unroll 4
        for (int i2 = 0; i2 < Kp; i2 += 4) {
            const int4 f = ld_i4(fetched + i2);
            const int4 b2 = ld_i4(sel + i2);
            p += (f.x & (b2.x < blk)) + (f.y & (b2.y < blk)) + (f.z & (b2.z < blk)) + (f.w & (b2.w < blk));
        }
        const int d = dest[p];
        fetch_block[p] = blk;
        fetch_slot[p] = d;
        if (d >= 0) { sb_new[d] = blk; lu_new[d] = step; }
    }
    for (int p = nF + tid; p < cap; p += kRowThreads) {
        fetch_block[p] = -1;
        fetch_slot[p] = -1;
    }
    if (tid == 0) *fetch_count = nF;
    __syncthreads();
    for (int j = tid; j < K; j += kRowThreads) {
        slot_block[j] = sb_new[j];
        last_use[j] = lu_new[j];
    }
}

}  // namespace oasis
