// select_plan_impl.h -- the select, plan and fused select + plan kernels and
// their launcher: one workgroup per (sequence, KV head) row
// (row_select_plan.h).  Included by select_plan.hip (256 threads per row) and
// by select_plan_wide.hip (OASIS_ROW_WIDE: 1024 threads per row, namespace
// oasis::wide, for rows of more than kWideRowMinWidth blocks).
//
// The fused kernel keeps the row's keys, its selection and its slot table on
// chip (LDS and registers) from start to end: the selection never goes back
// to HBM before it is planned, the slot table is read while the selection
// runs, and the launch between the two steps disappears.  When the selection
// is a threshold (no tie to split) it is planned without being compacted
// first (row_threshold_plan).
#pragma once
#include "row_select_plan.h"

namespace oasis {
#ifdef OASIS_ROW_WIDE
namespace wide {
#endif


// MODE 1 = select, 2 = plan (selection read from a.sel), 3 = select then plan.
template <int MODE>
__global__ __launch_bounds__(kRowThreads) void row_select_plan_kernel(SelectPlanArgs a) {
    extern __shared__ __attribute__((aligned(16))) int dyn[];   // 16-byte vector reads
    __shared__ RowShared sh;
    const int tid = threadIdx.x;
    const int row = blockIdx.x;
    const int K = a.k;
    const int Kp = plan_pad(K);
    int *sel = dyn;                                               // Kp
    int *pl = sel + Kp;                                           // 11 Kp (plan)
    uint32_t *keys = reinterpret_cast<uint32_t *>(MODE & 2 ? pl + 11 * Kp : pl);   // width
    const float *srow = a.scores + (size_t)row * a.width;
    const size_t rk = (size_t)row * K;

    PlanPrefetch pf;
    if (MODE & 2) plan_prefetch(a.slot_block_in + rk, a.last_use_in + rk, K, pf);   // in flight during the select
    const int step = (MODE & 2) ? a.step + (a.step_dev ? *a.step_dev : 0) : 0;
    int32_t *fb = a.fetch_block + (size_t)row * a.cap;
    int32_t *fs = a.fetch_slot + (size_t)row * a.cap;
    if (MODE & 1) {
        uint32_t kr[kKeyRegs];
        const int nb = load_row_keys(srow, a.width, a.ctx_len + row / a.hkv, keys, kr);
        __syncthreads();
        if (MODE == 3 && nb > K && nb <= kKeyRegs * kRowThreads) {
            // the resident marks follow the keys
            uint32_t *res_bits = keys + (a.width > 0 ? a.width : 1);
            const RowCut cut = row_find_cut<true>(keys, nb, K, sh, kr,
                                                  ResidentMarks{res_bits, a.width, K, &pf});
            if (cut.all_ties) {
                row_threshold_plan(kr, nb, cut.tau, keys, res_bits, K, a.cap, step, pf,
                                   a.sel ? a.sel + rk : nullptr, sel, a.slot_block + rk, a.last_use + rk,
                                   fb, fs, a.fetch_count + row, pl, sh);
                return;
            }
            row_compact<true>(keys, nb, sel, sh, kr, cut);
        } else if (nb <= kKeyRegs * kRowThreads) {
            row_select<true>(keys, nb, K, sel, sh, kr);
        } else {
            row_select(keys, nb, K, sel, sh);
        }
        if (a.sel)
            for (int i = tid; i < K; i += kRowThreads) a.sel[rk + i] = sel[i];
    } else {
        for (int i = tid; i < K; i += kRowThreads) {
            const int s = a.sel[rk + i];
            sel[i] = (s >= 0 && s < a.width) ? s : -1;
        }
        __syncthreads();
    }
    if (MODE & 2) {
        if (MODE & 1)
            row_plan(sel, [&](int s) { return key_to_score(keys[s]); }, K, a.cap, step, pf,
                     a.slot_block + rk, a.last_use + rk, fb, fs, a.fetch_count + row, pl, sh,
                     true, reinterpret_cast<int *>(keys), a.width);
        else
            row_plan(sel, [&](int s) { return srow[s]; }, K, a.cap, step, pf, a.slot_block + rk,
                     a.last_use + rk, fb, fs, a.fetch_count + row, pl, sh);
    }
}

// Pass 1 of the two-pass selection: workgroup (row, c) selects the exact
// top-K of blocks [c * chunk_w, (c + 1) * chunk_w) of the row's valid blocks
// and writes them as candidates (keys and block indices, ascending, padded).
__global__ __launch_bounds__(kRowThreads) void row_chunk_select_kernel(ChunkArgs a) {
    extern __shared__ __attribute__((aligned(16))) int dyn[];   // 16-byte vector reads
    __shared__ RowShared sh;
    constexpr int U = kKeyRegs;
    const int tid = threadIdx.x;
    const int row = blockIdx.x / a.chunks;
    const int c = blockIdx.x - row * a.chunks;
    const int K = a.k;
    int *sel = dyn;                                               // plan_pad(K)
    uint32_t *keys = reinterpret_cast<uint32_t *>(dyn + plan_pad(K));   // chunk_w
    const int n0 = c * a.chunk_w;
    const float *srow = a.scores + (size_t)row * a.width + n0;
    const int span = a.width - n0 < a.chunk_w ? a.width - n0 : a.chunk_w;
    const int ctx_raw = a.ctx_len[row / a.hkv];
    const int ctx = ctx_raw < 0 ? 0 : ctx_raw;
    const int cb = ctx / kBlockTokens + (ctx % kBlockTokens != 0);   // ceil, no overflow
    const int nb = cb > a.width ? a.width : cb;
    const int len = nb - n0 < 0 ? 0 : (nb - n0 < span ? nb - n0 : span);
    // the chunk's keys: U loads per thread in flight, from indices clamped
    // into the chunk; the first round also stays in registers
    static_assert(U == kKeyRegs, "the first round of keys is the register set");
    uint32_t kr[kKeyRegs];
    for (int i0 = 0; i0 < len; i0 += U * kRowThreads) {
        float v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = i0 + u * kRowThreads + tid;
            v[u] = srow[i < len ? i : len - 1];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = i0 + u * kRowThreads + tid;
            const uint32_t k = score_key(v[u]);
            if (i0 == 0) kr[u] = k;
            if (i < len) keys[i] = k;
        }
    }
    __syncthreads();
    if (len <= kKeyRegs * kRowThreads)
        row_select<true>(keys, len, K, sel, sh, kr);
    else
        row_select(keys, len, K, sel, sh);
    uint32_t *ck = a.cand_key + ((size_t)row * a.chunks + c) * K;
    int32_t *ci = a.cand_idx + ((size_t)row * a.chunks + c) * K;
    for (int i = tid; i < K; i += kRowThreads) {
        const int s = sel[i];
        ck[i] = s >= 0 ? keys[s] : 0u;
        ci[i] = s >= 0 ? n0 + s : -1;
    }
}

// Pass 2: one workgroup per row selects the top-K of the row's `ncand`
// candidates (the chunks' top-K sets in chunk order, so positions ascend with
// block index and the lower position wins a tie exactly when the lower block
// does) and, with MODE 3, plans it as the fused kernel does.  Every block of
// the row's top-K is among its chunk's top-K, so the result is the row's.
template <int MODE>
__global__ __launch_bounds__(kRowThreads) void row_merge_select_plan_kernel(
        SelectPlanArgs a, const uint32_t *cand_key, const int32_t *cand_idx, int ncand) {
    extern __shared__ __attribute__((aligned(16))) int dyn[];   // 16-byte vector reads
    __shared__ RowShared sh;
    const int tid = threadIdx.x;
    const int row = blockIdx.x;
    const int K = a.k;
    const int Kp = plan_pad(K);
    int *sel = dyn;                                               // Kp
    int *pl = sel + Kp;                                           // 11 Kp (plan)
    uint32_t *keys = reinterpret_cast<uint32_t *>(MODE & 2 ? pl + 11 * Kp : pl);   // ncand
    const size_t rk = (size_t)row * K;
    PlanPrefetch pf;
    if (MODE & 2) plan_prefetch(a.slot_block_in + rk, a.last_use_in + rk, K, pf);
    const int ctx_raw = a.ctx_len[row / a.hkv];
    const int ctx = ctx_raw < 0 ? 0 : ctx_raw;
    const int cb = ctx / kBlockTokens + (ctx % kBlockTokens != 0);
    const int nb = cb > a.width ? a.width : cb;
    const uint32_t *rk_key = cand_key + (size_t)row * ncand;
    const int32_t *rk_idx = cand_idx + (size_t)row * ncand;
    if (nb <= K) {
        for (int i = tid; i < K; i += kRowThreads) sel[i] = i < nb ? i : -1;
        __syncthreads();
    } else {
        if (ncand <= kKeyRegs * kRowThreads) {
            // the candidates in registers only, key n = u * kRowThreads + tid
            // (the register select reads no key from LDS)
            uint32_t kr[kKeyRegs];
#pragma unroll
            for (int u = 0; u < kKeyRegs; ++u) {
                const int n = u * kRowThreads + tid;
                kr[u] = rk_key[n < ncand ? n : ncand - 1];
            }
            row_select<true>(keys, ncand, K, sel, sh, kr);
        } else {
            for (int i = tid; i < ncand; i += kRowThreads) keys[i] = rk_key[i];
            __syncthreads();
            row_select(keys, ncand, K, sel, sh);
        }
        // positions -> blocks (positions ascend with block index; a position
        // padded with key 0 is never taken: there are at least K valid ones)
        for (int i = tid; i < K; i += kRowThreads) {
            const int p = sel[i];
            sel[i] = p >= 0 ? rk_idx[p] : -1;
        }
        __syncthreads();
    }
    if (a.sel)
        for (int i = tid; i < K; i += kRowThreads) a.sel[rk + i] = sel[i];
    if (MODE & 2) {
        const int step = a.step + (a.step_dev ? *a.step_dev : 0);
        const float *srow = a.scores + (size_t)row * a.width;
        row_plan(sel, [&](int s) { return srow[s]; }, K, a.cap, step, pf, a.slot_block + rk,
                 a.last_use + rk, a.fetch_block + (size_t)row * a.cap,
                 a.fetch_slot + (size_t)row * a.cap, a.fetch_count + row, pl, sh, true);
    }
}

hipError_t launch_chunk_select(const ChunkArgs &a, hipStream_t stream) {
    const size_t lds = (size_t)(plan_pad(a.k) + a.chunk_w) * 4;
    hipLaunchKernelGGL(row_chunk_select_kernel, dim3(a.rows * a.chunks), dim3(kRowThreads), lds,
                       stream, a);
    return hipGetLastError();
}

hipError_t launch_merge_select_plan(const SelectPlanArgs &a, int mode, const uint32_t *cand_key,
                                    const int32_t *cand_idx, int ncand, hipStream_t stream,
                                    LaunchStop *stop) {
    const int Kp = plan_pad(a.k);
    if (mode == 3)
        launch_k(row_merge_select_plan_kernel<3>, dim3(a.rows), dim3(kRowThreads),
                 (size_t)(12 * Kp + ncand) * 4, stream, stop, a, cand_key, cand_idx, ncand);
    else
        launch_k(row_merge_select_plan_kernel<1>, dim3(a.rows), dim3(kRowThreads),
                 (size_t)(Kp + ncand) * 4, stream, stop, a, cand_key, cand_idx, ncand);
    return hipGetLastError();
}

size_t row_shared_bytes() { return sizeof(RowShared); }

#ifndef OASIS_ROW_WIDE
bool row_select_plan_fits(int width, int k, int mode) {
    if (k > kMaxKBlocks) return false;
    if (mode == 1) return width <= kRowSelectMaxWidth;
    if (mode == 2) return true;
    // the fused launch's LDS: the selection, the plan's arrays, the keys and
    // their resident marks, beside the static row state of the build that
    // takes the row, within 64 KiB
    const size_t shared = width > kWideRowMinWidth ? wide::row_shared_bytes() : sizeof(RowShared);
    return width <= kFusedMaxWidth && k <= kFusedMaxK &&
           (size_t)(12 * plan_pad(k) + width + (width + 31) / 32) * 4 + shared <= 65536;
}
#endif

#ifndef OASIS_ROW_WIDE
// Chunks of at least kMinChunkWidth blocks, few enough that their K
// candidates each fit kMaxCandidates; chunk widths a multiple of 64.
void two_pass_plan(int width, int k, int *chunk_w, int *chunks) {
    const int cmax = kMaxCandidates / k;
    int cw = (width + cmax - 1) / cmax;
    cw = cw < kMinChunkWidth ? kMinChunkWidth : (cw + 63) / 64 * 64;
    *chunk_w = cw;
    *chunks = (width + cw - 1) / cw;
}

// mode 1 = select, 3 = select then plan (the plan in the same launch when
// its LDS fits beside the candidates, else a plan launch after it).
hipError_t launch_two_pass_select_plan(const SelectPlanArgs &a, int mode, uint32_t *cand_key,
                                       int32_t *cand_idx, hipStream_t stream, LaunchStop *stop) {
    if (a.rows == 0) return hipSuccess;
    int cw = 0, chunks = 0;
    two_pass_plan(a.width, a.k, &cw, &chunks);
    const ChunkArgs ca{a.scores, a.ctx_len, cand_key, cand_idx, a.rows, a.hkv, a.width, a.k, cw,
                       chunks};
    hipError_t e = cw > kWideRowMinWidth ? wide::launch_chunk_select(ca, stream)
                                         : launch_chunk_select(ca, stream);
    if (e != hipSuccess) return e;
    const int ncand = chunks * a.k;
    const size_t shared = ncand > kWideRowMinWidth ? wide::row_shared_bytes() : sizeof(RowShared);
    const bool fused = mode == 3 && (size_t)(12 * plan_pad(a.k) + ncand) * 4 + shared <= 65536;
    const int m = fused ? 3 : 1;
    // the stop event goes with the last launch: the merge, or the plan after it
    LaunchStop *merge_stop = (mode == 1 || fused) ? stop : nullptr;
    e = ncand > kWideRowMinWidth
            ? wide::launch_merge_select_plan(a, m, cand_key, cand_idx, ncand, stream, merge_stop)
            : launch_merge_select_plan(a, m, cand_key, cand_idx, ncand, stream, merge_stop);
    if (e != hipSuccess || mode == 1 || fused) return e;
    return launch_row_select_plan(a, 2, stream, stop);
}
#endif

hipError_t launch_row_select_plan(const SelectPlanArgs &a, int mode, hipStream_t stream,
                                  LaunchStop *stop) {
    if (a.rows == 0) return hipSuccess;
#ifndef OASIS_ROW_WIDE
    if ((mode & 1) && a.width > kWideRowMinWidth)
        return wide::launch_row_select_plan(a, mode, stream, stop);
#endif
    const int Kp = plan_pad(a.k);
    const size_t w = (size_t)(a.width > 0 ? a.width : 1);
    const dim3 grid(a.rows), block(kRowThreads);
    if (mode == 1) {
        launch_k(row_select_plan_kernel<1>, grid, block, (Kp + w) * 4, stream, stop, a);
    } else if (mode == 2) {
        launch_k(row_select_plan_kernel<2>, grid, block, (size_t)12 * Kp * 4, stream, stop, a);
    } else {
        launch_k(row_select_plan_kernel<3>, grid, block, (12 * Kp + w + (w + 31) / 32) * 4, stream, stop, a);
    }
    return hipGetLastError();
}

#ifdef OASIS_ROW_WIDE
}  // namespace wide
#endif
}  // namespace oasis
