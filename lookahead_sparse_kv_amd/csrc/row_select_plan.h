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
// a radix select over digits of at most 11 bits of u - kmin (the row's own key
// range): an LDS histogram of the keys that still match the prefix, a
// workgroup scan over the bins from the top, and the bin where the count
// crosses the remaining K.  Keys above tau are taken, and copies of tau fill
// the rest in ascending block order (ordered scans: over the ballots of the
// keys a thread holds in registers, or over index-contiguous chunks), so ties
// go to the lower index and the set comes out ascending.
//
// Plan: each thread owns contiguous chunks of the selection and of the slot
// table, so positions are exclusive scans; hits are binary searches in the
// ascending selection; only misses (among misses) and eviction candidates
// (among candidates) are ranked by counting.  When the selection is a
// threshold (every key at or above the K-th is taken) the fused launch plans
// straight from the keys instead, without compacting the selection first
// (row_threshold_plan).  Exact and deterministic.
#pragma once

#include "oasis_device.h"
#include "oasis_launch.h"

namespace oasis {
#ifdef OASIS_ROW_WIDE
// Compiled a second time for wide rows (select_plan_wide.hip): the same code
// with four times the threads per row, in a namespace of its own.
namespace wide {
#ifndef OASIS_ROW_WIDE_THREADS
#define OASIS_ROW_WIDE_THREADS 1024
#endif
constexpr int kRowThreads = OASIS_ROW_WIDE_THREADS;
#else
constexpr int kRowThreads = 256;
#endif
constexpr int kRowWaves = kRowThreads / kWave;
constexpr int kHistBins = 2048;          // widest radix digit: 11 bits
constexpr int kPlanPadding = 16;

__device__ __forceinline__ uint32_t score_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;            // -0.0 == +0.0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_to_score(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

// Scores of one row into LDS as keys, for the row's valid blocks n < nb;
// returns nb.  A thread's loads (8 per round of 8 * kRowThreads blocks) are all issued
// before the first is used, from indices clamped into the row (always in
// bounds of the [B][Hkv][W] scores, with no branch around the loads), so the
// first round does not wait for the context length, which is loaded beside it
// and applied when the keys are written.
// keys a thread holds in registers, n = u * kRowThreads + tid: rows of up to
// 2,048 blocks at 256 threads, 8,192 at 512 or 1,024
constexpr int kKeyRegs = kRowThreads == 512 ? 16 : 8;
static_assert(kKeyRegs % 4 == 0, "a thread's chunk is read 16 bytes at a time");


__device__ __forceinline__ int load_row_keys(const float *srow, int width, const int32_t *ctx_p,
                                             uint32_t *keys, uint32_t (&kr)[kKeyRegs]) {
    constexpr int U = kKeyRegs;
    constexpr int kRound = kRowThreads * U;
    if (width <= 0) return 0;
    const int ctx_raw = *ctx_p;
    const int last = width - 1;
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int n = u * kRowThreads + (int)threadIdx.x;
        v[u] = srow[n < width ? n : last];
    }
    const int ctx = ctx_raw < 0 ? 0 : ctx_raw;
    const int c = ctx / kBlockTokens + (ctx % kBlockTokens != 0);   // ceil, no overflow
    const int nb = c > width ? width : c;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int n = u * kRowThreads + (int)threadIdx.x;
        kr[u] = score_key(v[u]);
        if (n < nb) keys[n] = kr[u];
    }
    for (int n0 = kRound; n0 < nb; n0 += kRound) {      // rows longer than one round
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int n = n0 + u * kRowThreads + (int)threadIdx.x;
            v[u] = srow[n < width ? n : last];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int n = n0 + u * kRowThreads + (int)threadIdx.x;
            if (n < nb) keys[n] = score_key(v[u]);
        }
    }
    return nb;
}

// Inclusive scan of one int per thread over the workgroup.  trailing: end
// with a barrier, so that wave_sums may be written again at once; a caller
// that reaches another barrier before the next scan passes false.
__device__ __forceinline__ int row_inclusive_scan(int v, int *wave_sums, bool trailing = true) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    v = wave_inclusive_scan(v);
    if (lane == kWave - 1) wave_sums[wave] = v;
    __syncthreads();
    int off = 0;
#pragma unroll
    for (int w = 0; w < kRowWaves; ++w) off += (w < wave) ? wave_sums[w] : 0;
    if (trailing) __syncthreads();
    return v + off;
}

constexpr int kRankMax = 64;             // threshold bins this small are ranked directly

struct RowShared {
    int hist[kHistBins];
    int wave_sums[kRowWaves];
    uint32_t wave_min[kRowWaves], wave_max[kRowWaves];
    int digit, above, count;
    alignas(16) uint32_t gkey[kRankMax];    // keys of a small threshold bin
    int rank_acc[kRankMax];                 // per gathered key: (keys above) | (keys at or above) << 16
    int ngather, gt_in_bin, ge_in_bin;
    uint32_t tau;
    int reg_cnt[kKeyRegs * kRowWaves];      // per (register, wave): taken keys | copies of tau << 16
};

// Lanes below this one whose bit is set in a wave-wide mask.
__device__ __forceinline__ int lanes_below(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Where the K-th largest key lies: the keys taken are those above tau and,
// unless whole, the first krem copies of tau in index order (whole: every key
// >= tau, exactly K of them).  all_ties: every copy of tau is taken as well,
// so the keys taken are exactly the keys >= tau.
struct RowCut {
    uint32_t tau;
    int krem;
    bool whole;
    bool all_ties;
};

// Hooks of row_find_cut for work that needs the same two barriers:
// clear() runs before the first, mark() before the second.
struct NoMarks {
    __device__ void clear() const {}
    __device__ void mark() const {}
};

// The cut of `nb` > K keys (keys[0..nb) in LDS; REGS: in registers instead,
// as row_select takes them).
//
// The radix digits are taken from u - kmin over the row's own key range
// [kmin, kmax], the first one being the top 11 bits of that span: block scores
// share one or two exponents, so digits taken from the raw keys would put
// nearly every key in a handful of bins and serialise the LDS atomics.  A pass
// that finds the threshold bin holding exactly the keys still to take ends the
// search: every key from that bin's base up is taken, with no tie to split.
// A threshold bin of at most kRankMax keys ends it too: those keys are
// gathered and counted against each other, which gives the K-th largest key
// exactly (the key tau with fewer than krem keys above it in the bin and at
// least krem at or above it).
template <bool REGS, class Marks = NoMarks>
__device__ __forceinline__ RowCut row_find_cut(const uint32_t *keys, int nb, int K, RowShared &sh,
                                               const uint32_t (&kr)[kKeyRegs],
                                               const Marks &marks = Marks()) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    // f(u, n) over every key u = keys[n], n < nb, of this thread
    const auto each_key = [&](auto &&f) {
        if constexpr (REGS) {
#pragma unroll
            for (int u = 0; u < kKeyRegs; ++u) {
                const int n = u * kRowThreads + tid;
                if (n < nb) f(kr[u], n);
            }
        } else {
            for (int n = tid; n < nb; n += kRowThreads) f(keys[n], n);
        }
    };
    // the row's key range (and the first histogram cleared)
    uint32_t kmn = 0xffffffffu, kmx = 0u;
    each_key([&](uint32_t u, int) {
        kmn = u < kmn ? u : kmn;
        kmx = u > kmx ? u : kmx;
    });
    kmn = wave_min_u32(kmn);
    kmx = wave_max_u32(kmx);
    if (lane == 0) { sh.wave_min[wave] = kmn; sh.wave_max[wave] = kmx; }
    for (int i = tid; i < kHistBins; i += kRowThreads) sh.hist[i] = 0;
    marks.clear();
    __syncthreads();
    uint32_t kmin = sh.wave_min[0], kmax = sh.wave_max[0];
#pragma unroll
    for (int w = 1; w < kRowWaves; ++w) {
        kmin = sh.wave_min[w] < kmin ? sh.wave_min[w] : kmin;
        kmax = sh.wave_max[w] > kmax ? sh.wave_max[w] : kmax;
    }
    const uint32_t span = kmax - kmin;
    const int span_bits = span ? 32 - __builtin_clz(span) : 0;
    int width = span_bits < 11 ? (span_bits > 0 ? span_bits : 1) : 11;   // bits of this digit
    int shift = span_bits > 11 ? span_bits - 11 : 0;                     // its lowest bit
    uint32_t prefix = 0, pmask = 0;               // over u - kmin
    int krem = K;                                 // still to take among keys matching the prefix
    bool whole = false;                           // the threshold bin is taken whole
#pragma unroll 1
    for (int pass = 0;; ++pass) {
        const int nbins = 1 << width;
        const int sbins = nbins > kRowThreads ? nbins : kRowThreads;   // bins scanned (rest zero)
        if (pass > 0) {
            for (int i = tid; i < sbins; i += kRowThreads) sh.hist[i] = 0;
            __syncthreads();
        }
        each_key([&](uint32_t u, int) {
            const uint32_t d = u - kmin;
            if ((d & pmask) == prefix) atomicAdd(&sh.hist[(d >> shift) & (uint32_t)(nbins - 1)], 1);
        });
        if (pass == 0) marks.mark();
        __syncthreads();
        // thread t owns `per` bins counted from the top: bins hi, hi-1, .., lo
        // (its counts held in registers for the search below)
        const int per = sbins / kRowThreads;
        const int hi = sbins - 1 - tid * per;
        int h[kHistBins / kRowThreads];
        int local = 0;
#pragma unroll
        for (int j = 0; j < kHistBins / kRowThreads; ++j) {
            h[j] = j < per ? sh.hist[hi - j >= 0 ? hi - j : 0] : 0;
            local += h[j];
        }
        const int incl = row_inclusive_scan(local, sh.wave_sums, false);   // a barrier follows
        int acc = incl - local;                   // keys in bins above hi
        if (acc < krem && krem <= incl) {
            bool found = false;
#pragma unroll
            for (int j = 0; j < kHistBins / kRowThreads; ++j) {
                const int c = h[j];
                if (!found && j < per && acc + c >= krem) {
                    sh.digit = hi - j; sh.above = acc; sh.count = c;
                    found = true;
                }
                acc += c;
            }
        }
        if (tid == 0) sh.ngather = 0;
        __syncthreads();
        prefix |= (uint32_t)sh.digit << shift;
        pmask |= (uint32_t)(nbins - 1) << shift;
        krem -= sh.above;
        whole = sh.count == krem;
        const int cnt = sh.count;
        __syncthreads();                          // digit / above / count are rewritten next pass
        if (whole || shift == 0) break;
        if (cnt <= kRankMax) {
            // the cnt keys left in the threshold bin, gathered: a ballot of
            // the matching lanes per round, one slot reservation per wave
            if (tid < kRankMax) sh.rank_acc[tid] = 0;
            if constexpr (REGS) {
                uint64_t bal[kKeyRegs];
                int total = 0;
#pragma unroll
                for (int u = 0; u < kKeyRegs; ++u) {
                    const int n = u * kRowThreads + tid;
                    bal[u] = __ballot(n < nb && ((kr[u] - kmin) & pmask) == prefix);
                    total += __popcll(bal[u]);
                }
                if (total) {
                    int base = 0;
                    if (lane == 0) base = atomicAdd(&sh.ngather, total);
                    base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
                    for (int u = 0; u < kKeyRegs; ++u) {
                        if ((bal[u] >> lane) & 1) sh.gkey[base + lanes_below(bal[u])] = kr[u];
                        base += __popcll(bal[u]);
                    }
                }
            } else {
                for (int n0 = 0; n0 < nb; n0 += kRowThreads) {     // uniform trip count
                    const int n = n0 + tid;
                    const uint32_t u = n < nb ? keys[n] : 0u;
                    const bool m = n < nb && ((u - kmin) & pmask) == prefix;
                    const uint64_t bal = __ballot(m);
                    if (bal) {
                        int base = 0;
                        if (lane == 0) base = atomicAdd(&sh.ngather, __popcll(bal));
                        base = __builtin_amdgcn_readfirstlane(base);
                        if (m) sh.gkey[base + lanes_below(bal)] = u;
                    }
                }
            }
            __syncthreads();
            // the bin's keys counted against each other, the comparisons
            // spread over every wave: wave w compares key j (lane j) with
            // keys [w * S, w * S + S) and adds (above, at or above) to key j's
            // tally.  Key j is tau when fewer than krem keys lie above it
            // and at least krem at or above it (every copy of tau agrees).
            constexpr int S = kRankMax / kRowWaves;
            if (lane < cnt) {
                const uint32_t kj = sh.gkey[lane];
                int gt = 0, ge = 0;
#pragma unroll
                for (int c0 = 0; c0 < S; c0 += 4) {
                    const int i0 = wave * S + c0;
                    if (i0 >= cnt) break;
                    const uint4 k4 = *reinterpret_cast<const uint4 *>(&sh.gkey[i0]);
                    const uint32_t kk[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const bool in = i0 + c < cnt;
                        gt += in && kk[c] > kj;
                        ge += in && kk[c] >= kj;
                    }
                }
                if (gt | ge) atomicAdd(&sh.rank_acc[lane], gt | (ge << 16));
            }
            __syncthreads();
            if (tid < cnt) {
                const int t = sh.rank_acc[tid];
                const int gt = t & 0xffff, ge = t >> 16;
                if (gt < krem && krem <= ge) {
                    sh.tau = sh.gkey[tid]; sh.gt_in_bin = gt; sh.ge_in_bin = ge;
                }
            }
            __syncthreads();
            krem -= sh.gt_in_bin;                  // copies of tau still to take
            return RowCut{sh.tau, krem, false, sh.ge_in_bin - sh.gt_in_bin == krem};
        }
        width = shift < 11 ? shift : 11;
        shift -= width;
    }
    // whole: every key >= tau is taken (exactly K); otherwise the last digit
    // was resolved (the bin holds the copies of tau alone) and its first krem
    // copies are taken.
    return RowCut{kmin + prefix, krem, whole, whole};
}

// The K keys of a cut into sel[0..K), ascending.  Ends with a barrier.
template <bool REGS>
__device__ __forceinline__ void row_compact(const uint32_t *keys, int nb, int *sel, RowShared &sh,
                                            const uint32_t (&kr)[kKeyRegs], const RowCut &cut) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const uint32_t tau = cut.tau;
    const int krem = cut.krem;
    const bool whole = cut.whole;
    if constexpr (REGS) {
        // Ordered compaction from the registers: key n = u * kRowThreads + tid,
        // so index order is (u, wave, lane).  Per register, a ballot of the
        // keys taken outright (above tau; at or above it when whole) and one
        // of the copies of tau; their counts per (u, wave) slot, scanned in
        // slot order, give each taken key its position: the taken keys before
        // it plus the copies of tau before it, at most krem.
        constexpr int NS = kKeyRegs * kRowWaves;
        static_assert(NS <= 2 * kWave && kRowWaves % 2 == 0, "two (register, wave) slots per lane");
        uint64_t bg[kKeyRegs], be[kKeyRegs];
        int mine = 0;
#pragma unroll
        for (int u = 0; u < kKeyRegs; ++u) {
            // bitwise, not short-circuit, so that no compare is branched around
            const bool in = u * kRowThreads + tid < nb;
            const bool eq = kr[u] == tau;
            bg[u] = __ballot(in & ((kr[u] > tau) | (whole & eq)));
            be[u] = __ballot(in & !whole & eq);
            const int packed = __popcll(bg[u]) | (__popcll(be[u]) << 16);
            mine = lane == u ? packed : mine;
        }
        if (lane < kKeyRegs) sh.reg_cnt[lane * kRowWaves + wave] = mine;
        __syncthreads();
        // every wave scans the slots itself, lane l holding slots 2l and 2l + 1;
        // slot u * kRowWaves + wave has this wave's parity (kRowWaves is even)
        const int c0 = 2 * lane < NS ? sh.reg_cnt[2 * lane] : 0;
        const int c1 = 2 * lane + 1 < NS ? sh.reg_cnt[2 * lane + 1] : 0;
        const int ex0 = wave_inclusive_scan(c0 + c1) - c0 - c1;
        const int wv = __builtin_amdgcn_readfirstlane(wave);
        const int ex = (wv & 1) ? ex0 + c0 : ex0;
#pragma unroll
        for (int u = 0; u < kKeyRegs; ++u) {
            const int before = __builtin_amdgcn_readlane(ex, (u * kRowWaves + wv) >> 1);
            const int gt_b = (before & 0xffff) + lanes_below(bg[u]);
            const int eq_b = (before >> 16) + lanes_below(be[u]);
            const bool take = (bool)((bg[u] >> lane) & 1) | ((bool)((be[u] >> lane) & 1) & (eq_b < krem));
            if (take) sel[gt_b + (eq_b < krem ? eq_b : krem)] = u * kRowThreads + tid;
        }
        __syncthreads();
        return;
    }
    const int E = (nb + kRowThreads - 1) / kRowThreads;
    const int lo = tid * E;
    const int hi = lo + E < nb ? lo + E : nb;
    int c_gt = 0, c_eq = 0;
    uint32_t ck[kKeyRegs];                        // this thread's chunk, when it fits
    if (E <= kKeyRegs) {
        if (E == kKeyRegs && lo + kKeyRegs <= nb) {       // 16-byte aligned chunk: 16-byte reads
#pragma unroll
            for (int i = 0; i < kKeyRegs; i += 4) {
                const uint4 a = *reinterpret_cast<const uint4 *>(keys + lo + i);
                ck[i] = a.x; ck[i + 1] = a.y; ck[i + 2] = a.z; ck[i + 3] = a.w;
            }
        } else {                                          // read together, indices clamped (nb > K >= 1)
#pragma unroll
            for (int i = 0; i < kKeyRegs; ++i) ck[i] = keys[lo + i < nb ? lo + i : nb - 1];
        }
#pragma unroll
        for (int i = 0; i < kKeyRegs; ++i) {
            const bool in = lo + i < hi;
            c_gt += in && (whole ? ck[i] >= tau : ck[i] > tau);
            c_eq += in && !whole && ck[i] == tau;
        }
    } else {
        for (int n = lo; n < hi; ++n) {
            const uint32_t u = keys[n];
            c_gt += whole ? u >= tau : u > tau;
            c_eq += !whole && u == tau;
        }
    }
    // one scan of both counts (each < 2^16): the keys taken before this
    // thread's chunk are all the larger ones and the first krem copies of tau
    const int packed = (c_eq << 16) | c_gt;
    const int before = row_inclusive_scan(packed, sh.wave_sums, false) - packed;   // (barrier at the end)
    const int gt_before = before & 0xffff;
    const int eq_before = before >> 16;
    int pos = gt_before + (eq_before < krem ? eq_before : krem);
    int er = eq_before;
    if (E <= kKeyRegs) {
#pragma unroll
        for (int i = 0; i < kKeyRegs; ++i) {
            if (lo + i >= hi) break;
            const uint32_t u = ck[i];
            bool take = whole ? u >= tau : u > tau;
            if (!whole && u == tau) { take = er < krem; ++er; }
            if (take) sel[pos++] = lo + i;
        }
    } else {
        for (int n = lo; n < hi; ++n) {
            const uint32_t u = keys[n];
            bool take = whole ? u >= tau : u > tau;
            if (!whole && u == tau) { take = er < krem; ++er; }
            if (take) sel[pos++] = n;
        }
    }
    __syncthreads();
}

// Top-K of `nb` keys (keys[0..nb), already in LDS) into sel[0..K): ascending,
// -1 padded.  Ends with a barrier; sel may then be read by every thread.
// REGS: every key of the row is in the calling thread's registers instead,
// kr[u] = key u * kRowThreads + tid (nb <= kKeyRegs * kRowThreads); the
// passes over all keys read those registers, and `keys` is not read.
template <bool REGS>
__device__ __forceinline__ void row_select(const uint32_t *keys, int nb, int K, int *sel,
                                           RowShared &sh, const uint32_t (&kr)[kKeyRegs]) {
    if (nb <= K) {
        for (int i = threadIdx.x; i < K; i += kRowThreads) sel[i] = i < nb ? i : -1;
        __syncthreads();
        return;
    }
    row_compact<REGS>(keys, nb, sel, sh, kr, row_find_cut<REGS>(keys, nb, K, sh, kr));
}

// Without the keys in registers.
__device__ __forceinline__ void row_select(const uint32_t *keys, int nb, int K, int *sel,
                                           RowShared &sh) {
    const uint32_t none[kKeyRegs] = {};
    row_select<false>(keys, nb, K, sel, sh, none);
}

__device__ __forceinline__ int4 ld_i4(const int *p) { return *reinterpret_cast<const int4 *>(p); }
__device__ __forceinline__ float4 ld_f4(const float *p) { return *reinterpret_cast<const float4 *>(p); }

// LDS of the plan: 9 arrays of Kp = roundup(K, 16) ints after `sel` (Kp ints).
__host__ __device__ __forceinline__ int plan_pad(int K) {
    return (K + kPlanPadding - 1) / kPlanPadding * kPlanPadding;
}

// Exclusive scan of one int per thread; `total` gets the workgroup sum.
// trailing as in row_inclusive_scan.
__device__ __forceinline__ int row_exclusive_scan(int v, int *wave_sums, int &total,
                                                  bool trailing = true) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int x = wave_inclusive_scan(v);
    if (lane == kWave - 1) wave_sums[wave] = x;
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kRowWaves; ++w) {
        const int ws = wave_sums[w];
        off += (w < wave) ? ws : 0;
        tot += ws;
    }
    if (trailing) __syncthreads();
    total = tot;
    return x - v + off;
}

constexpr int kPlanMaxPer = kMaxKBlocks / kRowThreads;   // entries per thread, at most

// Entries of the row's slot table this thread plans: [tid * E, tid * E + E),
// E = ceil(K / kRowThreads), read before the selection runs.  The loads are
// unconditional, from indices clamped into the row (K >= 1), and nothing here
// uses them, so they stay in flight through the selection; the plan reads
// only the entries with u < E and tid * E + u < K.
struct PlanPrefetch {
    int sb[kPlanMaxPer];
    int lu[kPlanMaxPer];
};

__device__ __forceinline__ void plan_prefetch(const int32_t *slot_block, const int32_t *last_use,
                                              int K, PlanPrefetch &pf) {
    const int E = (K + kRowThreads - 1) / kRowThreads;
    const int lo = threadIdx.x * E;
#pragma unroll
    for (int u = 0; u < kPlanMaxPer; ++u) {
        const int j = lo + u;
        const int jc = j < K ? j : K - 1;
        pf.sb[u] = slot_block[jc];
        pf.lu[u] = last_use[jc];
    }
}

// Ranks of the compacted misses by (score desc, block asc) when more than
// cap of them, and of the compacted eviction candidates by (last use asc,
// block asc) when any is evicted, into m_rank / c_rank (zeroed by the
// caller).  Candidates with equal keys (one block resident in two slots: a
// table no plan produces, but one a caller may pass) go by compacted
// position, i.e. slot order, so that every victim rank is distinct; misses
// are distinct blocks.  Each rank is a tally of the entries ahead of it, the comparisons
// spread over the workgroup: wave w compares entry i (lane i, i + 64, ...)
// with a slice of the others, four per 16-byte LDS read, and adds its count
// to i's tally.  The caller's barrier follows.
__device__ __forceinline__ void plan_ranks(const float *m_score, const int *m_block, int *m_rank,
                                           int M, int cap, const int *c_lu, const int *c_block,
                                           int *c_rank, int C, int n_victims) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    if (M > cap) {
        const int S = ((M + kRowWaves - 1) / kRowWaves + 3) & ~3;
        const int q_lo = wave * S, q_hi = q_lo + S < M ? q_lo + S : M;
        for (int i = lane; i < M && q_lo < q_hi; i += kWave) {
            const float sc = m_score[i];
            const int blk = m_block[i];
            int r = 0;
            for (int q0 = q_lo; q0 < q_hi; q0 += 4) {
                const float4 s4 = ld_f4(m_score + q0);
                const int4 b4 = ld_i4(m_block + q0);
                const float ss[4] = {s4.x, s4.y, s4.z, s4.w};
                const int bb[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    r += (q0 + c < q_hi) & ((ss[c] > sc) | ((ss[c] == sc) & (bb[c] < blk)));
            }
            if (r) atomicAdd(&m_rank[i], r);
        }
    }
    if (n_victims > 0) {
        const int S = ((C + kRowWaves - 1) / kRowWaves + 3) & ~3;
        const int q_lo = wave * S, q_hi = q_lo + S < C ? q_lo + S : C;
        for (int i = lane; i < C && q_lo < q_hi; i += kWave) {
            const int l0 = c_lu[i], b0 = c_block[i];
            int r = 0;
            for (int q0 = q_lo; q0 < q_hi; q0 += 4) {
                const int4 l4 = ld_i4(c_lu + q0);
                const int4 b4 = ld_i4(c_block + q0);
                const int ll[4] = {l4.x, l4.y, l4.z, l4.w};
                const int bb[4] = {b4.x, b4.y, b4.z, b4.w};
                // (block, position) below (b0, i): a block below b0, or b0
                // itself at an earlier position (blocks are >= 0, so the
                // subtraction cannot wrap)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    r += (q0 + c < q_hi) &
                         ((ll[c] < l0) | ((ll[c] == l0) & (bb[c] - (int)(q0 + c < i) < b0)));
            }
            if (r) atomicAdd(&c_rank[i], r);
        }
    }
}

// Fetched misses before compacted miss i (those ranked below cap).
__device__ __forceinline__ int fetched_before(const int *m_rank, int i, int cap) {
    int f = 0;
#pragma unroll 2
    for (int q0 = 0; q0 < i; q0 += 4) {
        const int4 r4 = ld_i4(m_rank + q0);
        const int rr[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) f += (q0 + c < i) & (rr[c] < cap);
    }
    return f;
}

// The plan of one row.  sel[0..K) (LDS) holds the selection; sel_score_of(s)
// gives the fp32 score of block s; pf holds this thread's part of the slot
// table (plan_prefetch); slot_block / last_use / fetch_* point at this row's
// part of the global arrays.  `pl` is 11 * Kp ints of LDS.
//
// Each thread owns a contiguous chunk of selection entries and of slots, so
// every position (the p-th miss or fetched block in ascending order, the p-th
// free slot or eviction candidate) comes from an exclusive scan; counts that
// do not depend on each other share one scan, packed as two 16-bit fields.
// Hits are found by binary search in the ascending selection (a selection
// that is not ascending is sorted first); only the misses are ranked against
// each other by (score desc, block asc), and only the eviction candidates by
// (last use asc, block asc).  min(misses, cap) misses are fetched, so the
// number of victims is known as soon as the misses are counted.
template <class ScoreOf>
__device__ __forceinline__ void row_plan(int *sel, ScoreOf sel_score_of, int K, int cap, int step,
                                         const PlanPrefetch &pf,
                                         int32_t *slot_block, int32_t *last_use,
                                         int32_t *fetch_block, int32_t *fetch_slot,
                                         int32_t *fetch_count, int *pl, RowShared &sh,
                                         bool ascending = false, int *map = nullptr,
                                         int map_len = 0) {
    const int tid = threadIdx.x;
    const int Kp = plan_pad(K);
    const int E = (K + kRowThreads - 1) / kRowThreads;
    const int lo = tid * E;
    float *sel_score = reinterpret_cast<float *>(pl);
    int *sb = pl + Kp;             // slot -> block as read (-1 = empty)
    int *lu = pl + 2 * Kp;
    int *hit_sel = pl + 3 * Kp;    // per selection entry: resident
    int *fill = pl + 4 * Kp;       // per slot: block fetched into it, -1
    int *dest = pl + 5 * Kp;       // destination slot of the p-th fetched block
    float *m_score = reinterpret_cast<float *>(pl + 6 * Kp);   // misses, compacted
    int *m_block = pl + 7 * Kp;
    int *c_lu = pl + 8 * Kp;       // eviction candidates, compacted: last use
    int *c_block = hit_sel;        //   ... and block (hit_sel is dead by then)
    int *m_rank = pl + 9 * Kp;     // per compacted miss: its rank (a tally)
    int *c_rank = pl + 10 * Kp;    // per compacted eviction candidate: its rank (a tally)

    for (int i = tid; i < Kp; i += kRowThreads) {
        if (i >= K) sel[i] = -1;
        hit_sel[i] = 0;
        fill[i] = -1;
        dest[i] = -1;
        m_rank[i] = 0;
        c_rank[i] = 0;
    }
    bool unsorted = false;
#pragma unroll
    for (int u = 0; u < kPlanMaxPer; ++u) {
        const int j = lo + u;
        if (u < E && j < K) {
            sb[j] = pf.sb[u] < 0 ? -1 : pf.sb[u];
            lu[j] = pf.lu[u];
            if (!ascending && j + 1 < K) {
                const int x = sel[j], y = sel[j + 1];
                unsorted |= (x < 0 && y >= 0) || (x >= 0 && y >= 0 && x >= y);
            }
        }
    }
    // a selection from the row select is ascending by construction
    if (!ascending && __syncthreads_or(unsorted)) {
        // not ascending: order by (valid first, block, entry) into fill / dest, then back
        int key_s[kPlanMaxPer];
#pragma unroll
        for (int u = 0; u < kPlanMaxPer; ++u) {
            const int i = lo + u;
            key_s[u] = -1;
            if (u < E && i < K) {
                const int x = sel[i];
                // valid entries by (block, entry), then the invalid ones (blocks < 2^31,
                // entries < 2^11)
                const long long kx = x < 0 ? (1LL << 50) + i : ((long long)x << 11) + i;
                int r = 0;
                for (int j = 0; j < K; ++j) {
                    const int y = sel[j];
                    const long long ky = y < 0 ? (1LL << 50) + j : ((long long)y << 11) + j;
                    r += ky < kx;
                }
                key_s[u] = r;
            }
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kPlanMaxPer; ++u)
            if (key_s[u] >= 0) fill[key_s[u]] = sel[lo + u];
        __syncthreads();
        for (int i = tid; i < K; i += kRowThreads) { sel[i] = fill[i]; fill[i] = -1; }
        __syncthreads();
    }
    for (int i = tid; i < Kp; i += kRowThreads) {
        const int x = sel[i];
        sel_score[i] = (i < K && x >= 0) ? sel_score_of(x) : 0.f;
        // map (where given): block -> selection entry, over the row's keys,
        // which are dead once read here (a block's key is read and its map
        // entry written by the thread of the one entry selecting it)
        if (map && i < K && x >= 0 && x < map_len) map[x] = i;
    }
    // one scan: valid selection entries (an ascending prefix) | empty slots
    bool empty[kPlanMaxPer];
    int my_valid = 0, my_empty = 0;
#pragma unroll
    for (int u = 0; u < kPlanMaxPer; ++u) {
        const int j = lo + u;
        my_valid += (u < E && j < K && sel[j] >= 0) ? 1 : 0;
        empty[u] = u < E && j < K && pf.sb[u] < 0;
        my_empty += empty[u];
    }
    int tot_a;
    const int pos_a = row_exclusive_scan(my_valid | (my_empty << 16), sh.wave_sums, tot_a);
    const int m_valid = tot_a & 0xffff;                    // (ends with a barrier: sb, lu visible)
    const int nfree = tot_a >> 16;
    int epos = pos_a >> 16;

    // hits: every resident block is looked up in the selection
    bool hit[kPlanMaxPer], cand[kPlanMaxPer];
#pragma unroll
    for (int u = 0; u < kPlanMaxPer; ++u) {
        const int j = lo + u;
        hit[u] = cand[u] = false;
        if (u < E && j < K) {
            const int blk = sb[j];
            if (blk >= 0) {
                int l;
                if (map) {
                    // the map entry of an unselected block holds anything:
                    // it is a hit only if the entry it names selects blk
                    l = blk < map_len ? map[blk] : -1;
                    if ((unsigned)l >= (unsigned)m_valid) l = m_valid;
                } else {
                    int h = m_valid;                       // first entry >= blk
                    l = 0;
                    while (l < h) {
                        const int mid = (l + h) >> 1;
                        if (sel[mid] < blk) l = mid + 1; else h = mid;
                    }
                }
                if (l < m_valid && sel[l] == blk) { hit[u] = true; hit_sel[l] = 1; }
                cand[u] = !hit[u];
            }
        }
    }
    __syncthreads();
    // one scan: misses (in ascending block order) | eviction candidates
    bool miss[kPlanMaxPer];
    int my_miss = 0, my_cand = 0;
#pragma unroll
    for (int u = 0; u < kPlanMaxPer; ++u) {
        const int i = lo + u;
        miss[u] = u < E && i < K && sel[i] >= 0 && !hit_sel[i];
        my_miss += miss[u];
        my_cand += cand[u];
    }
    int tot_b;
    const int pos_b = row_exclusive_scan(my_miss | (my_cand << 16), sh.wave_sums, tot_b,
                                         false);                 // a barrier follows the compaction
    const int M = tot_b & 0xffff;
    const int C = tot_b >> 16;
    const int nF = M < cap ? M : cap;                      // the first min(M, cap) misses are fetched
    const int n_victims = nF > nfree ? nF - nfree : 0;     // (C >= n_victims always)
    int mpos = pos_b & 0xffff, cpos = pos_b >> 16;
    int mp[kPlanMaxPer], cp[kPlanMaxPer];
#pragma unroll
    for (int u = 0; u < kPlanMaxPer; ++u) {
        mp[u] = cp[u] = -1;
        if (miss[u]) {
            mp[u] = mpos;
            m_score[mpos] = sel_score[lo + u];
            m_block[mpos] = sel[lo + u];
            ++mpos;
        }
        if (cand[u] && n_victims > 0) {
            cp[u] = cpos;
            c_lu[cpos] = lu[lo + u];
            c_block[cpos] = sb[lo + u];
            ++cpos;
        }
    }
    __syncthreads();
    // ranks: the first cap misses are fetched; the first n_victims candidates
    // are evicted in rank order, after the free slots (ascending)
    plan_ranks(m_score, m_block, m_rank, M, cap, c_lu, c_block, c_rank, C, n_victims);
    __syncthreads();
    bool fetched[kPlanMaxPer];
#pragma unroll
    for (int u = 0; u < kPlanMaxPer; ++u) {
        fetched[u] = miss[u] && (M <= cap || m_rank[mp[u]] < cap);
        if (empty[u]) {
            if (epos < nF) dest[epos] = lo + u;
            ++epos;
        }
        if (cp[u] >= 0) {
            const int rank = c_rank[cp[u]];
            if (rank < n_victims) dest[nfree + rank] = lo + u;
        }
    }
    __syncthreads();
    // the p-th fetched block (ascending) goes to dest[p]; p counts the fetched
    // misses before this one in block order
#pragma unroll
    for (int u = 0; u < kPlanMaxPer; ++u) {
        if (fetched[u]) {
            const int fpos = M > cap ? fetched_before(m_rank, mp[u], cap) : mp[u];
            if (fpos >= nF) continue;   // only a selection with repeated blocks gets here
            const int blk = sel[lo + u];
            const int d = dest[fpos];
            fetch_block[fpos] = blk;
            fetch_slot[fpos] = d;
            if (d >= 0) fill[d] = blk;
        }
    }
    for (int p = nF + tid; p < cap; p += kRowThreads) {
        fetch_block[p] = -1;
        fetch_slot[p] = -1;
    }
    if (tid == 0) *fetch_count = nF;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kPlanMaxPer; ++u) {
        const int j = lo + u;
        if (u < E && j < K) {
            const int f = fill[j];
            slot_block[j] = f >= 0 ? f : sb[j];
            last_use[j] = (f >= 0 || hit[u]) ? step : lu[j];
        }
    }
}

// Resident marks of the threshold plan: one bit per block of the row, cleared
// while the selection starts and set from this thread's prefetched slots in
// its first histogram pass (row_find_cut's hooks), so the barriers the
// selection takes anyway order both.
struct ResidentMarks {
    uint32_t *bits;          // (width + 31) / 32 words of LDS
    int width;
    int K;
    const PlanPrefetch *pf;
    __device__ void clear() const {
        for (int i = threadIdx.x; i < (width + 31) / 32; i += kRowThreads) bits[i] = 0u;
    }
    __device__ void mark() const {
        const int E = (K + kRowThreads - 1) / kRowThreads;
        const int lo = threadIdx.x * E;
#pragma unroll
        for (int u = 0; u < kPlanMaxPer; ++u) {
            const int blk = pf->sb[u];
            if (u < E && lo + u < K && blk >= 0 && blk < width)
                atomicOr(&bits[blk >> 5], 1u << (blk & 31));
        }
    }
};

// The plan of a row whose selection is a threshold: the blocks taken are
// exactly the valid ones with key >= T (K of them), every key in this
// thread's registers (kr[u] = key of block u * kRowThreads + tid, n < nb), the
// resident blocks marked in res_bits (ResidentMarks).  The selection is never
// compacted on its own: one exchange of counts places the selected blocks
// (staged in `sel`, Kp ints of LDS, for sel_out when given), the misses
// (selected, not resident: block order), the eviction candidates (resident,
// not selected: slot order) and the free slots, and a slot's block is a hit
// when its key is at or above T.
// The rest is row_plan's: ranks, the first cap misses fetched into the free
// slots and then the least recently used candidates, the table rewritten.
// The same result as row_select followed by row_plan.  `pl` is 8 * Kp ints.
__device__ __forceinline__ void row_threshold_plan(
        const uint32_t (&kr)[kKeyRegs], int nb, uint32_t T, const uint32_t *keys,
        const uint32_t *res_bits, int K, int cap, int step, const PlanPrefetch &pf,
        int32_t *sel_out, int *sel, int32_t *slot_block, int32_t *last_use, int32_t *fetch_block,
        int32_t *fetch_slot, int32_t *fetch_count, int *pl, RowShared &sh) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int Kp = plan_pad(K);
    const int E = (K + kRowThreads - 1) / kRowThreads;
    const int lo = tid * E;
    float *m_score = reinterpret_cast<float *>(pl);   // misses, compacted
    int *m_block = pl + Kp;
    int *m_rank = pl + 2 * Kp;
    int *c_lu = pl + 3 * Kp;                          // eviction candidates, compacted
    int *c_block = pl + 4 * Kp;
    int *c_rank = pl + 5 * Kp;
    int *dest = pl + 6 * Kp;                          // destination slot of the p-th fetched block
    int *fill = pl + 7 * Kp;                          // per slot: block fetched into it, -1
    for (int i = tid; i < Kp; i += kRowThreads) {
        m_rank[i] = 0;
        c_rank[i] = 0;
        dest[i] = -1;
        fill[i] = -1;
    }
    // blocks: selected, and selected but not resident, one ballot each per
    // register; counts per (register, wave) slot
    constexpr int NS = kKeyRegs * kRowWaves;
    static_assert(NS <= 2 * kWave && kRowWaves % 2 == 0, "two (register, wave) slots per lane");
    uint64_t bt[kKeyRegs], bm[kKeyRegs];
    int mine = 0;
#pragma unroll
    for (int u = 0; u < kKeyRegs; ++u) {
        const int n = u * kRowThreads + tid;
        const bool in = n < nb;
        const uint32_t word = res_bits[in ? n >> 5 : 0];
        const bool taken = in & (kr[u] >= T);
        bt[u] = __ballot(taken);
        bm[u] = __ballot(taken & !((word >> (n & 31)) & 1u));
        const int packed = __popcll(bt[u]) | (__popcll(bm[u]) << 16);
        mine = lane == u ? packed : mine;
    }
    if (lane < kKeyRegs) sh.reg_cnt[lane * kRowWaves + wave] = mine;
    // slots (this thread's contiguous chunk): hits, eviction candidates, free
    bool hit[kPlanMaxPer], cand[kPlanMaxPer], empty[kPlanMaxPer];
    int my_ce = 0;
#pragma unroll
    for (int u = 0; u < kPlanMaxPer; ++u) {
        const int blk = pf.sb[u];
        const bool ok = u < E && lo + u < K;
        hit[u] = ok && blk >= 0 && blk < nb && keys[blk] >= T;
        cand[u] = ok && blk >= 0 && !hit[u];
        empty[u] = ok && blk < 0;
        my_ce += (int)cand[u] | ((int)empty[u] << 16);
    }
    const int ce_incl = wave_inclusive_scan(my_ce);
    if (lane == kWave - 1) sh.wave_sums[wave] = ce_incl;
    __syncthreads();
    // block slots scanned by every wave, lane l holding slots 2l and 2l + 1;
    // slot u * kRowWaves + wave has this wave's parity (kRowWaves is even)
    const int c0 = 2 * lane < NS ? sh.reg_cnt[2 * lane] : 0;
    const int c1 = 2 * lane + 1 < NS ? sh.reg_cnt[2 * lane + 1] : 0;
    const int incl = wave_inclusive_scan(c0 + c1);
    const int tm_total = __builtin_amdgcn_readlane(incl, kWave - 1);
    const int n_taken = tm_total & 0xffff;
    const int M = tm_total >> 16;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int ex = (wv & 1) ? incl - c1 : incl - c0 - c1;
    int off = 0, ce_total = 0;
#pragma unroll
    for (int w = 0; w < kRowWaves; ++w) {
        const int ws = sh.wave_sums[w];
        off += (w < wv) ? ws : 0;
        ce_total += ws;
    }
    const int C = ce_total & 0xffff;
    const int nfree = ce_total >> 16;
    const int nF = M < cap ? M : cap;                      // the first min(M, cap) misses are fetched
    const int n_victims = nF > nfree ? nF - nfree : 0;     // (C >= n_victims always)
    int mp[kKeyRegs];
#pragma unroll
    for (int u = 0; u < kKeyRegs; ++u) {
        const int before = __builtin_amdgcn_readlane(ex, (u * kRowWaves + wv) >> 1);
        const int n = u * kRowThreads + tid;
        mp[u] = -1;
        if ((bt[u] >> lane) & 1) {
            if (sel_out) sel[(before & 0xffff) + lanes_below(bt[u])] = n;
            if ((bm[u] >> lane) & 1) {
                const int q = (before >> 16) + lanes_below(bm[u]);
                m_score[q] = key_to_score(kr[u]);
                m_block[q] = n;
                mp[u] = q;
            }
        }
    }
    const int ce_before = ce_incl - my_ce + off;
    int cpos = ce_before & 0xffff, epos = ce_before >> 16;
    int cp[kPlanMaxPer];
#pragma unroll
    for (int u = 0; u < kPlanMaxPer; ++u) {
        cp[u] = -1;
        if (empty[u]) {
            if (epos < nF) dest[epos] = lo + u;
            ++epos;
        }
        if (cand[u] && n_victims > 0) {
            cp[u] = cpos;
            c_lu[cpos] = pf.lu[u];
            c_block[cpos] = pf.sb[u];
            ++cpos;
        }
    }
    __syncthreads();
    // the selection leaves in one coalesced pass (scattered stores from the
    // registers would issue a store per register and wave)
    if (sel_out)
        for (int i = tid; i < K; i += kRowThreads) sel_out[i] = i < n_taken ? sel[i] : -1;
    plan_ranks(m_score, m_block, m_rank, M, cap, c_lu, c_block, c_rank, C, n_victims);
    __syncthreads();
    bool fetched[kKeyRegs];
#pragma unroll
    for (int u = 0; u < kKeyRegs; ++u) fetched[u] = mp[u] >= 0 && (M <= cap || m_rank[mp[u]] < cap);
#pragma unroll
    for (int u = 0; u < kPlanMaxPer; ++u) {
        if (cp[u] >= 0) {
            const int rank = c_rank[cp[u]];
            if (rank < n_victims) dest[nfree + rank] = lo + u;
        }
    }
    __syncthreads();
    // the p-th fetched block (ascending) goes to dest[p]
#pragma unroll
    for (int u = 0; u < kKeyRegs; ++u) {
        if (fetched[u]) {
            const int fpos = M > cap ? fetched_before(m_rank, mp[u], cap) : mp[u];
            if (fpos >= nF) continue;   // (cannot happen: the ranks of distinct blocks are distinct)
            const int blk = u * kRowThreads + tid;
            const int d = dest[fpos];
            fetch_block[fpos] = blk;
            fetch_slot[fpos] = d;
            if (d >= 0) fill[d] = blk;
        }
    }
    for (int p = nF + tid; p < cap; p += kRowThreads) {
        fetch_block[p] = -1;
        fetch_slot[p] = -1;
    }
    if (tid == 0) *fetch_count = nF;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kPlanMaxPer; ++u) {
        const int j = lo + u;
        if (u < E && j < K) {
            const int f = fill[j];
            slot_block[j] = f >= 0 ? f : (pf.sb[u] < 0 ? -1 : pf.sb[u]);
            last_use[j] = (f >= 0 || hit[u]) ? step : pf.lu[u];
        }
    }
}

#ifdef OASIS_ROW_WIDE
}  // namespace wide
#endif
}  // namespace oasis
