// select_plan_impl.h -- the select, plan and fused select + plan kernels and
// their launcher: one workgroup per (sequence, KV head) row
// (row_select_plan.h).  Included by select_plan.hip (256 threads per row) and
// by select_plan_wide.hip (OASIS_ROW_WIDE: 1024 threads per row, namespace
// oasis::wide, for rows of more than kWideRowMinWidth blocks).
//
// The fused kernel keeps the row's keys, its selection and its slot table in
// LDS from start to end: the selection never goes back to HBM before it is
// planned, the slot table is read while the selection runs, and the launch
// between the two steps disappears.
#pragma once
#include "row_select_plan.h"

namespace oasis {
#ifdef OASIS_ROW_WIDE
namespace wide {
#endif


__device__ __forceinline__ float key_to_score(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

// MODE 1 = select, 2 = plan (selection read from a.sel), 3 = select then plan.
template <int MODE>
__global__ __launch_bounds__(kRowThreads) void row_select_plan_kernel(SelectPlanArgs a) {
    extern __shared__ int dyn[];
    __shared__ RowShared sh;
    const int tid = threadIdx.x;
    const int row = blockIdx.x;
    const int K = a.k;
    const int Kp = plan_pad(K);
    int *sel = dyn;                                               // Kp
    int *pl = sel + Kp;                                           // 9 Kp (plan)
    uint32_t *keys = reinterpret_cast<uint32_t *>(MODE & 2 ? pl + 9 * Kp : pl);   // width
    const float *srow = a.scores + (size_t)row * a.width;
    const size_t rk = (size_t)row * K;

    PlanPrefetch pf;
    if (MODE & 2) plan_prefetch(a.slot_block + rk, a.last_use + rk, K, pf);   // in flight during the select
    if (MODE & 1) {
        const int nb = load_row_keys(srow, a.width, a.ctx_len + row / a.hkv, keys);
        __syncthreads();
        row_select(keys, nb, K, sel, sh);
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
        const int step = a.step + (a.step_dev ? *a.step_dev : 0);
        int32_t *fb = a.fetch_block + (size_t)row * a.cap;
        int32_t *fs = a.fetch_slot + (size_t)row * a.cap;
        if (MODE & 1)
            row_plan(sel, [&](int s) { return key_to_score(keys[s]); }, K, a.cap, step, pf,
                     a.slot_block + rk, a.last_use + rk, fb, fs, a.fetch_count + row, pl, sh);
        else
            row_plan(sel, [&](int s) { return srow[s]; }, K, a.cap, step, pf, a.slot_block + rk,
                     a.last_use + rk, fb, fs, a.fetch_count + row, pl, sh);
    }
}

bool row_select_plan_fits(int width, int k, int mode) {
    if (k > kMaxKBlocks) return false;
    if (mode == 1) return width <= kRowSelectMaxWidth;
    if (mode == 2) return true;
    return width <= kFusedMaxWidth && k <= kFusedMaxK;
}

hipError_t launch_row_select_plan(const SelectPlanArgs &a, int mode, hipStream_t stream) {
    if (a.rows == 0) return hipSuccess;
#ifndef OASIS_ROW_WIDE
    if ((mode & 1) && a.width > kWideRowMinWidth) return wide::launch_row_select_plan(a, mode, stream);
#endif
    const int Kp = plan_pad(a.k);
    const size_t w = (size_t)(a.width > 0 ? a.width : 1);
    const dim3 grid(a.rows), block(kRowThreads);
    if (mode == 1) {
        hipLaunchKernelGGL(row_select_plan_kernel<1>, grid, block, (Kp + w) * 4, stream, a);
    } else if (mode == 2) {
        hipLaunchKernelGGL(row_select_plan_kernel<2>, grid, block, (size_t)10 * Kp * 4, stream, a);
    } else {
        hipLaunchKernelGGL(row_select_plan_kernel<3>, grid, block, (10 * Kp + w) * 4, stream, a);
    }
    return hipGetLastError();
}

#ifdef OASIS_ROW_WIDE
}  // namespace wide
#endif
}  // namespace oasis
