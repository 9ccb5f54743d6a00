// select_plan_wave.hip -- one wave per (sequence, KV head) row: top-K
// selection and the resident-diff / fetch-cap / LRU plan without a single
// workgroup barrier, fused into one launch.
//
// OasisKV (metalmedia.ai summary): Figure 7 caption (the next step's top-K
// blocks), abstract (2,048-token budget), five-step flow step 3 (diff against
// the GPU-resident blocks, pull only the missing ones under a per-step bound),
// Figure 9 caption (per-KV-head working-set table), Table 2 caption (fetch
// ratio cap, LRU eviction).
//
// Select: lane l holds the order-preserving keys of blocks l, l + 64, ... in
// registers (KPL per lane).  tau, the K-th largest key, is found bit by bit
// from the top; each candidate is counted with one ballot + popcount per
// register (scalar unit), so a step costs ~2 KPL instructions and no
// synchronisation.  Keys above tau win, and copies of tau fill the rest in
// ascending block order; register i of lane l is block 64 i + l, so ballot
// prefixes walk the blocks in ascending order.
//
// Plan: the selection, its scores and the slot table live in this wave's
// LDS region; every ranking is a count of beating elements (integer compares,
// fp32 score compares for the misses) read 16 bytes at a time.  Same rules as
// plan_fetch.hip.  Exact and deterministic.
#include "oasis_device.h"
#include "oasis_launch.h"

namespace oasis {

constexpr int kWaveRowsPerGroup = 4;          // rows (waves) per workgroup
constexpr int kPlanPad = 16;

__device__ __forceinline__ uint32_t order_key_w(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;             // -0.0 == +0.0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int popc_below(uint64_t mask, int lane) {
    return __popcll(mask & ((1ull << lane) - 1ull));
}

// Order LDS traffic between the phases of one wave.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int4 lds4(const int *p) { return *reinterpret_cast<const int4 *>(p); }
__device__ __forceinline__ float4 lds4f(const float *p) { return *reinterpret_cast<const float4 *>(p); }

// Top-K of one row into sel_lds[0..K) (ascending, -1 padded) and, if
// sel_out != nullptr, to global memory.
template <int KPL>
__device__ __forceinline__ void wave_select(const float *srow, int nb, int K, int *sel_lds, int32_t *sel_out) {
    const int lane = threadIdx.x & (kWave - 1);
    if (nb <= K) {
        for (int i = lane; i < K; i += kWave) {
            const int v = i < nb ? i : -1;
            sel_lds[i] = v;
            if (sel_out) sel_out[i] = v;
        }
        return;
    }
    const int E = (nb + kWave - 1) / kWave;   // registers in use (uniform)
    uint32_t key[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const int n = i * kWave + lane;
        key[i] = (i < E && n < nb) ? order_key_w(srow[n]) : 0u;   // 0: below every real key
    }
    uint32_t tau = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = tau | (1u << bit);
        int c = 0;
#pragma unroll
        for (int i = 0; i < KPL; ++i)
            if (i < E) c += __popcll(__ballot(key[i] >= cand));
        if (c >= K) tau = cand;
    }
    int gt = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i)
        if (i < E) gt += __popcll(__ballot(key[i] > tau));
    const int krem = K - gt;                  // copies of tau to take, lowest index first
    int eq_base = 0, out_base = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        if (i < E) {
            const uint32_t u = key[i];
            const uint64_t eqm = __ballot(u == tau);
            const bool take = (u > tau) || (u == tau && eq_base + popc_below(eqm, lane) < krem);
            const uint64_t tm = __ballot(take);
            const int pos = out_base + popc_below(tm, lane);
            if (take) {
                sel_lds[pos] = i * kWave + lane;
                if (sel_out) sel_out[pos] = i * kWave + lane;
            }
            eq_base += __popcll(eqm);
            out_base += __popcll(tm);
        }
    }
}

// The plan of one row.  `sel` (K entries) is already in LDS; `lds` is this
// wave's scratch of 9 * Kp ints.
__device__ __forceinline__ void wave_plan(const int *sel, const float *srow, int width, int K, int cap, int step,
                          int32_t *slot_block, int32_t *last_use, int32_t *fetch_block,
                          int32_t *fetch_slot, int32_t *fetch_count, int *lds) {
    const int lane = threadIdx.x & (kWave - 1);
    const int Kp = (K + kPlanPad - 1) / kPlanPad * kPlanPad;
    float *sel_score = reinterpret_cast<float *>(lds);
    int *miss = lds + Kp;
    int *fetched = lds + 2 * Kp;
    int *sb = lds + 3 * Kp;        // slot -> block as read (-1 = empty; pad -2)
    int *lu = lds + 4 * Kp;
    int *cand = lds + 5 * Kp;      // resident and not selected
    int *sb_new = lds + 6 * Kp;
    int *lu_new = lds + 7 * Kp;
    int *dest = lds + 8 * Kp;
    int *sel_p = const_cast<int *>(sel);

    for (int i = lane; i < Kp; i += kWave) {
        if (i < K) {
            int s = sel_p[i];
            s = (s >= 0 && s < width) ? s : -1;
            sel_p[i] = s;
            sel_score[i] = s >= 0 ? srow[s] : 0.f;
            const int blk = slot_block[i];
            sb[i] = blk < 0 ? -1 : blk;
            lu[i] = last_use[i];
        } else {
            sel_p[i] = -1;
            sel_score[i] = 0.f;
            sb[i] = -2;
            lu[i] = 0;
        }
        miss[i] = 0;
        fetched[i] = 0;
        cand[i] = 0;
        dest[i] = -1;
    }
    wave_sync();

    int nfree = 0;
    for (int j0 = 0; j0 < K; j0 += kWave) {            // hits and eviction candidates
        const int j = j0 + lane;
        const int blk = j < K ? sb[j] : -2;
        bool hit = false;
        if (blk >= 0) {
#pragma unroll 4
            for (int i = 0; i < Kp; i += 4) {
                const int4 v = lds4(sel_p + i);
                hit |= (v.x == blk) | (v.y == blk) | (v.z == blk) | (v.w == blk);
            }
        }
        if (j < K) {
            cand[j] = (blk >= 0 && !hit) ? 1 : 0;
            sb_new[j] = blk;
            lu_new[j] = hit ? step : lu[j];
        }
        nfree += __popcll(__ballot(blk == -1));
    }
    for (int i0 = 0; i0 < K; i0 += kWave) {            // misses
        const int i = i0 + lane;
        const int blk = i < K ? sel_p[i] : -1;
        bool resident = false;
        if (blk >= 0) {
#pragma unroll 4
            for (int j = 0; j < Kp; j += 4) {
                const int4 v = lds4(sb + j);
                resident |= (v.x == blk) | (v.y == blk) | (v.z == blk) | (v.w == blk);
            }
        }
        if (i < K) miss[i] = (blk >= 0 && !resident) ? 1 : 0;
    }
    wave_sync();

    int nF = 0;
    for (int i0 = 0; i0 < K; i0 += kWave) {            // rank misses: (score desc, block asc)
        const int i = i0 + lane;
        bool take = false;
        if (i < K && miss[i]) {
            const int blk = sel_p[i];
            const float s = sel_score[i];
            int rank = 0;
#pragma unroll 4
            for (int i2 = 0; i2 < Kp; i2 += 4) {
                const int4 m = lds4(miss + i2);
                const int4 b2 = lds4(sel_p + i2);
                const float4 s2 = lds4f(sel_score + i2);
                rank += m.x & ((s2.x > s) | ((s2.x == s) & (b2.x < blk)));
                rank += m.y & ((s2.y > s) | ((s2.y == s) & (b2.y < blk)));
                rank += m.z & ((s2.z > s) | ((s2.z == s) & (b2.z < blk)));
                rank += m.w & ((s2.w > s) | ((s2.w == s) & (b2.w < blk)));
            }
            take = rank < cap;
        }
        if (i < K) fetched[i] = take ? 1 : 0;
        nF += __popcll(__ballot(take));
    }
    wave_sync();

    // destinations: free slots ascending, then LRU victims by (last use, block)
    int free_base = 0;
    for (int j0 = 0; j0 < K; j0 += kWave) {
        const int j = j0 + lane;
        const int blk = j < K ? sb[j] : -2;
        const uint64_t fm = __ballot(blk == -1);
        if (blk == -1) {
            const int pos = free_base + popc_below(fm, lane);
            if (pos < nF) dest[pos] = j;
        } else if (j < K && cand[j] && nF > nfree) {
            const int l0 = lu[j];
            int rank = 0;
#pragma unroll 4
            for (int j2 = 0; j2 < Kp; j2 += 4) {
                const int4 c = lds4(cand + j2);
                const int4 l2 = lds4(lu + j2);
                const int4 b2 = lds4(sb + j2);
                rank += c.x & ((l2.x < l0) | ((l2.x == l0) & (b2.x < blk)));
                rank += c.y & ((l2.y < l0) | ((l2.y == l0) & (b2.y < blk)));
                rank += c.z & ((l2.z < l0) | ((l2.z == l0) & (b2.z < blk)));
                rank += c.w & ((l2.w < l0) | ((l2.w == l0) & (b2.w < blk)));
            }
            if (rank < nF - nfree) dest[nfree + rank] = j;
        }
        free_base += __popcll(fm);
    }
    wave_sync();

    for (int i0 = 0; i0 < K; i0 += kWave) {            // p-th fetched block (ascending) -> dest[p]
        const int i = i0 + lane;
        if (i < K && fetched[i]) {
            const int blk = sel_p[i];
            int p = 0;
#pragma unroll 4
            for (int i2 = 0; i2 < Kp; i2 += 4) {
                const int4 f = lds4(fetched + i2);
                const int4 b2 = lds4(sel_p + i2);
                p += (f.x & (b2.x < blk)) + (f.y & (b2.y < blk)) + (f.z & (b2.z < blk)) + (f.w & (b2.w < blk));
            }
            const int d = dest[p];
            fetch_block[p] = blk;
            fetch_slot[p] = d;
            if (d >= 0) { sb_new[d] = blk; lu_new[d] = step; }
        }
    }
    for (int p = nF + lane; p < cap; p += kWave) {
        fetch_block[p] = -1;
        fetch_slot[p] = -1;
    }
    if (lane == 0) *fetch_count = nF;
    wave_sync();
    for (int j = lane; j < K; j += kWave) {
        slot_block[j] = sb_new[j];
        last_use[j] = lu_new[j];
    }
}

__device__ __forceinline__ int row_blocks(const int32_t *ctx_len, int b, int width) {
    int ctx = ctx_len[b];
    ctx = ctx < 0 ? 0 : ctx;
    const int nb = (ctx + kBlockTokens - 1) / kBlockTokens;
    return nb > width ? width : nb;
}

// mode 1 = select only, 2 = plan only, 3 = select then plan.
template <int KPL, int MODE>
__global__ __launch_bounds__(kWaveRowsPerGroup * kWave) void wave_select_plan_kernel(SelectPlanArgs a) {
    extern __shared__ int lds_all[];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int row = blockIdx.x * kWaveRowsPerGroup + wave;
    if (row >= a.rows) return;
    const int K = a.k;
    const int Kp = (K + kPlanPad - 1) / kPlanPad * kPlanPad;
    int *lds = lds_all + (size_t)wave * 10 * Kp;
    int *sel_lds = lds;
    const float *srow = a.scores + (size_t)row * a.width;
    if (MODE & 1) {
        const int nb = row_blocks(a.ctx_len, row / a.hkv, a.width);
        wave_select<KPL>(srow, nb, K, sel_lds, a.sel ? a.sel + (size_t)row * K : nullptr);
    } else {
        const int lane = threadIdx.x & (kWave - 1);
        for (int i = lane; i < K; i += kWave) sel_lds[i] = a.sel[(size_t)row * K + i];
    }
    if (MODE & 2) {
        wave_sync();
        const size_t r = (size_t)row * K;
        wave_plan(sel_lds, srow, a.width, K, a.cap, a.step, a.slot_block + r, a.last_use + r,
                  a.fetch_block + (size_t)row * a.cap, a.fetch_slot + (size_t)row * a.cap,
                  a.fetch_count + row, lds + Kp);
    }
}

template <int MODE>
static hipError_t launch_mode(const SelectPlanArgs &a, hipStream_t stream) {
    const int Kp = (a.k + kPlanPad - 1) / kPlanPad * kPlanPad;
    const size_t shmem = (size_t)kWaveRowsPerGroup * 10 * Kp * sizeof(int);
    const dim3 grid((a.rows + kWaveRowsPerGroup - 1) / kWaveRowsPerGroup);
    const dim3 block(kWaveRowsPerGroup * kWave);
    hipLaunchKernelGGL((wave_select_plan_kernel<kWaveMaxWidth / kWave, MODE>), grid, block, shmem,
                       stream, a);
    return hipGetLastError();
}

bool wave_select_plan_fits(int width, int k, bool needs_select) {
    return k <= kWaveMaxK && (!needs_select || width <= kWaveMaxWidth);
}

hipError_t launch_wave_select_plan(const SelectPlanArgs &a, int mode, hipStream_t stream) {
    if (a.rows == 0) return hipSuccess;
    switch (mode) {
        case 1: return launch_mode<1>(a, stream);
        case 2: return launch_mode<2>(a, stream);
        default: return launch_mode<3>(a, stream);
    }
}

}  // namespace oasis
