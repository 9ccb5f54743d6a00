// sparse_attn.hip -- split-K sparse paged decode attention over the working set.
//
// OasisKV (metalmedia.ai summary), Figure 7 caption: attention runs over the
// sparse KV working set.  For each query row i, head h of KV head g:
//   out = sum_t softmax_t(scale * q . k_t) v_t over the valid tokens of the
//   row's listed blocks.
//
// Design (gfx950): one wave per (sequence, KV head, split) walks its share of
// the row's block list.  Per 16-token block:
//   S (16 tokens x 16 query rows) = 16x16x32 bf16 MFMAs, A = key tile
//     (stored in 8-dimension slices: 16 B per lane, 1 KiB contiguous per
//     load), B = the group's query rows;
//   online softmax per query row in fp32 (exp2 with a folded log2(e));
//   O^T (D x 16 query rows) += V^T (D x 32 tokens) * P (32 tokens x 16 rows)
//     for two blocks at a time: 16x16x32 bf16 MFMAs whose B operand is P
//     exactly as the two S tiles left it in registers, and whose A operand is
//     read straight from the dim-major value tiles (8 B per lane per block,
//     512 contiguous bytes per load).
// The gather is HBM-bound (each selected K and V byte is read once), and the
// next pair of blocks is loaded before the current pair is computed.  With
// 128 rows or more (and at most 16 query rows) one 8-wave workgroup per row
// walks the list and merges its waves in LDS; with fewer rows split-K spreads
// rows over enough waves to fill 256 CUs and a second kernel merges the
// (max, sum, O) partials of the splits.
#include "oasis_device.h"
#include "oasis_launch.h"

namespace oasis {

constexpr int kAttnWaves = 4;
#ifndef OASIS_ATTN_STAGES
#define OASIS_ATTN_STAGES 2          // block pairs in flight per wave
#endif
constexpr int kAttnStages = OASIS_ATTN_STAGES;
#ifndef OASIS_ATTN_CPOL
#define OASIS_ATTN_CPOL 2        // K/V tile loads: non-temporal (each byte is read once)
#endif
#ifndef OASIS_ATTN_TARGET_WAVES
#define OASIS_ATTN_TARGET_WAVES 1024
#endif
constexpr int kAttnTargetWaves = OASIS_ATTN_TARGET_WAVES;   // enough to give every CU several waves
constexpr int kAttnMinPerSplit = 4;
constexpr int kAttnMaxPerSplit = 64;     // one list entry per lane

void attn_split_plan(int rows, int n_blk, int *splits, int *per_split) {
    int s = rows > 0 ? (kAttnTargetWaves + rows - 1) / rows : 1;
    const int s_max = (n_blk + kAttnMinPerSplit - 1) / kAttnMinPerSplit;
    if (s > s_max) s = s_max;
    const int s_min = (n_blk + kAttnMaxPerSplit - 1) / kAttnMaxPerSplit;
    if (s < s_min) s = s_min;
    if (s < 1) s = 1;
    const int per = (n_blk + s - 1) / s;
    *per_split = per;
    *splits = (n_blk + per - 1) / per;
}

template <int D>
struct BlockRegs {
    u32x4 k[D / 32];   // key tile: token r16, dims 32*kk + 8*j4 .. +8
    u32x2 v[D / 16];   // value tile (dim-major): dim 16*mt + r16, tokens 4*j4 .. +4
};

// Load one block's key and value tiles.  An absent block has zero-byte
// resources: every lane reads zeros and no memory is touched, so the load
// instructions are issued unconditionally and the compiler can count the
// loads in flight exactly.
template <int D>
__device__ __forceinline__ void load_block(BlockRegs<D> &r, rsrc_t kr, rsrc_t vr, uint32_t koff,
                                           uint32_t voff) {
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) r.k[kk] = buf_load16<OASIS_ATTN_CPOL>(kr, koff, 1024 * kk);
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt)
        r.v[mt] = __builtin_amdgcn_raw_buffer_load_b64(vr, voff, 16 * kBlockTokens * 2 * mt, OASIS_ATTN_CPOL);
}

// Masks of the two bf16 values of tokens (t0, t0 + 1) that are valid (< nt).
__device__ __forceinline__ uint32_t pair_mask(int t0, int nt) {
    return (t0 < nt ? 0x0000ffffu : 0u) | (t0 + 1 < nt ? 0xffff0000u : 0u);
}

// Running softmax state of a wave, per 16-column tile nt of query rows.
template <int D, int NT>
struct WaveAcc {
    float m_run[NT];          // running max of column r16 (log2 units)
    float l_run[NT];          // this lane's share of the column's running sum
    f32x4 o[NT][D / 16];      // O^T rows 16*mt + 4*j4 + i of column r16
};

// B operand of QK^T, tile nt: query row c = 16*nt + r16 = (query i, head
// g*G + hr), dims 32*kk + 8*j4 .. +8; rows past n_rows_q are zero.
template <int D, int NT>
__device__ __forceinline__ void load_query(const AttnArgs &a, int b, int g,
                                           bf16x8 (&qv)[NT][D / 32]) {
    const int lane = threadIdx.x & (kWave - 1);
    const int r16 = lane & 15;
    const int j4 = lane >> 4;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int c = 16 * nt + r16;
        if (c < a.n_rows_q) {
            const int iq = c / a.group;
            const int hr = c - iq * a.group;
            const uint16_t *qp =
                a.q + (((size_t)b * a.n_q + iq) * a.hq + (size_t)g * a.group + hr) * D + 8 * j4;
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk) qv[nt][kk] = as_bf16x8(load_u32x4(qp + 32 * kk));
        } else {
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk) qv[nt][kk] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
        }
    }
}

// Entry e0 + lane of row (b, g) (lane < ne <= 64): its page and number of
// valid tokens (page -1 = skip).
struct WaveEntries {
    int page, ntok;
};

__device__ __forceinline__ WaveEntries load_entries(const AttnArgs &a, int row, int b, int e0,
                                                    int ne) {
    const int lane = threadIdx.x & (kWave - 1);
    WaveEntries w{-1, 0};
    if (lane < ne) {
        const int ctx = a.ctx_len[b];
        const size_t e = (size_t)row * a.n_blk + e0 + lane;
        const int ent = a.blk ? a.blk[e] : e0 + lane;
        const int lg = a.blk_logical ? a.blk_logical[e] : ent;
        if (ent >= 0 && ent < a.width && lg >= 0) {
            const int p = a.page_table[(size_t)b * a.width + ent];
            long long nt = (long long)ctx - (long long)lg * kBlockTokens;
            nt = nt > kBlockTokens ? kBlockTokens : nt;
            if (p >= 0 && p < a.num_pages && nt > 0) { w.page = p; w.ntok = (int)nt; }
        }
    }
    return w;
}

// Accumulate list entries [e0, e0 + ne) (ne <= 64) of row (b, g), whose pages
// `ent` holds (load_entries), into acc.  NE > 0: ne == NE is known at compile
// time, so the walk over the pairs is fully unrolled and the loads and waits
// of consecutive pairs are scheduled together (the common case: 128 listed
// blocks over 8 waves).
template <int D, int NT, int NE = 0>
__device__ __forceinline__ void attn_wave_range(const AttnArgs &a, int g, int ne_arg,
                                                WaveEntries ent, const bf16x8 (&qv)[NT][D / 32],
                                                WaveAcc<D, NT> &acc) {
    const int ne = NE > 0 ? NE : ne_arg;
    constexpr int KK = D / 32;
    constexpr int MT = D / 16;
    const int lane = threadIdx.x & (kWave - 1);
    const int r16 = lane & 15;
    const int j4 = lane >> 4;
    const float NEG_INF = -__builtin_inff();
    const int my_page = ent.page, my_ntok = ent.ntok;

    const size_t page_stride = (size_t)a.hkv * kBlockTokens * D;
    const size_t head_off = (size_t)g * kBlockTokens * D;       // same for K and V tiles
    constexpr uint32_t kTileBytes = kBlockTokens * D * 2;
    // key tiles in 8-dimension slices: token r16, dims 32*kk + 8*j4 .. +8 at
    // lane * 16 + kk * 1 KiB (1 KiB contiguous per load)
    const uint32_t koff = (uint32_t)lane * 16;
    const uint32_t voff = (uint32_t)(r16 * kBlockTokens + 4 * j4) * 2;  // + 512 B per mt
    auto tile = [&](const uint16_t *pool, int e) {
        const int p = e < ne ? readlane_i(my_page, e) : -1;
        return p >= 0 ? make_rsrc(pool + (size_t)p * page_stride + head_off, kTileBytes)
                      : make_rsrc(pool, 0u);
    };

    // Entries go in pairs, kStages pairs in flight: the pair kStages - 1 ahead
    // of the current one is loaded before the current one is computed.
    constexpr int S = kAttnStages;
    BlockRegs<D> stage[S][2];
#pragma unroll
    for (int st = 0; st < S - 1; ++st)
#pragma unroll
        for (int u = 0; u < 2; ++u)
            load_block<D>(stage[st][u], tile(a.k_pool, 2 * st + u), tile(a.v_pool, 2 * st + u), koff, voff);
    constexpr int kPairUnroll = NE > 0 ? NE / 2 : 1;
#pragma unroll kPairUnroll
    for (int i = 0; i < ne; i += 2) {
        int ntok[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            ntok[u] = (i + u < ne && readlane_i(my_page, i + u) >= 0) ? readlane_i(my_ntok, i + u) : 0;
            const int e = i + 2 * (S - 1) + u;
            load_block<D>(stage[S - 1][u], tile(a.k_pool, e), tile(a.v_pool, e), koff, voff);
        }
        BlockRegs<D> (&cur)[2] = stage[0];
        if (ntok[0] + ntok[1] > 0) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                if (ntok[u] < kBlockTokens) {
                    // zero the values of tokens past the context so that whatever the
                    // page holds there cannot reach O (0 * NaN would)
                    const uint32_t k01 = pair_mask(4 * j4, ntok[u]);
                    const uint32_t k23 = pair_mask(4 * j4 + 2, ntok[u]);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) { cur[u].v[mt].x &= k01; cur[u].v[mt].y &= k23; }
                }
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                float x[2][4];
                float mb = NEG_INF;
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < KK; ++kk) s = mfma16x16x32(as_bf16x8(cur[u].k[kk]), qv[t][kk], s);
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        x[u][q4] = (4 * j4 + q4 < ntok[u]) ? s[q4] * a.scale_log2 : NEG_INF;
                        mb = fmaxf(mb, x[u][q4]);
                    }
                }
                mb = max_xor32(max_xor16(mb));
                const float m_new = fmaxf(acc.m_run[t], mb);   // finite: the pair has a valid token
                const float alpha = exp2f(acc.m_run[t] - m_new);
                uint32_t pw[2][2];
                float psum = 0.f;
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    pw[u][0] = pack_bf16x2(exp2f(x[u][0] - m_new), exp2f(x[u][1] - m_new));
                    pw[u][1] = pack_bf16x2(exp2f(x[u][2] - m_new), exp2f(x[u][3] - m_new));
                    // the normaliser sums the same bf16-rounded weights the MFMA uses
                    psum += bf16_bits_to_float(pw[u][0] & 0xffffu) + bf16_bits_to_float(pw[u][0] >> 16) +
                            bf16_bits_to_float(pw[u][1] & 0xffffu) + bf16_bits_to_float(pw[u][1] >> 16);
                }
                acc.l_run[t] = acc.l_run[t] * alpha + psum;
                acc.m_run[t] = m_new;
                // O^T += V^T P over the pair's 32 tokens: reduction index 8*j4 + i is
                // token 4*j4 + i of the first block (i < 4) or of the second (i >= 4).
                const bf16x8 pb = as_bf16x8(u32x4{pw[0][0], pw[0][1], pw[1][0], pw[1][1]});
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    acc.o[t][mt] *= alpha;
                    const u32x4 va = {cur[0].v[mt].x, cur[0].v[mt].y, cur[1].v[mt].x, cur[1].v[mt].y};
                    acc.o[t][mt] = mfma16x16x32(as_bf16x8(va), pb, acc.o[t][mt]);
                }
            }
        }
#pragma unroll
        for (int st = 0; st < S - 1; ++st) {
            stage[st][0] = stage[st + 1][0];
            stage[st][1] = stage[st + 1][1];
        }
    }
}

// Output element (c, d) of row `row` from the partials of its splits, taken
// kChunk splits at a time: the loads of a chunk are unconditional (indices
// past the last split repeat it, with weight 0), so they are all in flight at
// once.  The launcher picks kChunk >= splits where it can (up to 32), so that
// one round of loads covers the row.
template <int D, int kChunk>
__device__ __forceinline__ void merge_one(const AttnArgs &a, int row, int c, int d) {
    const int b = row / a.hkv;
    const int g = row - b * a.hkv;
    const float NEG_INF = -__builtin_inff();
    const size_t slot0 = (size_t)row * a.splits * a.n_rows_q + c;
    float M = NEG_INF, L = 0.f, O = 0.f;
    for (int s0 = 0; s0 < a.splits; s0 += kChunk) {
        float m[kChunk], l[kChunk], o[kChunk];
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
            const int s = s0 + u < a.splits ? s0 + u : a.splits - 1;
            const size_t slot = slot0 + (size_t)s * a.n_rows_q;
            m[u] = a.part_ml[2 * slot];
            l[u] = a.part_ml[2 * slot + 1];
            o[u] = a.part_o[slot * D + d];
        }
        float mc = NEG_INF;
#pragma unroll
        for (int u = 0; u < kChunk; ++u)
            if (s0 + u < a.splits) mc = fmaxf(mc, m[u]);
        const float Mn = fmaxf(M, mc);
        if (Mn == NEG_INF) continue;              // no valid token so far
        const float r = M == NEG_INF ? 0.f : exp2f(M - Mn);
        L *= r;
        O *= r;
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
            const float w = (s0 + u < a.splits && m[u] != NEG_INF) ? exp2f(m[u] - Mn) : 0.f;
            L += w * l[u];
            O += w * o[u];
        }
        M = Mn;
    }
    const float res = L > 0.f ? O / L : 0.f;
    const int iq = c / a.group;
    const int hr = c - iq * a.group;
    a.out[(((size_t)b * a.n_q + iq) * a.hq + (size_t)g * a.group + hr) * D + d] =
        (uint16_t)float_to_bf16_bits(res);
}

// NT = 1: up to 16 query rows per KV head; NT = 2: up to 32 (the normal and
// the draft queries together), at one wave per SIMD for the registers.
template <int D, int NT>
__global__ __launch_bounds__(kAttnWaves * kWave, NT == 1 && kAttnStages == 2 ? 2 : 1) void attn_partial_kernel(AttnArgs a) {
    constexpr int MT = D / 16;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // uniform: keeps row indices scalar
    const int gw = blockIdx.x * kAttnWaves + wave;
    const int rows = a.batch * a.hkv;
    const int row = gw / a.splits;
    if (row >= rows) return;
    const int split = gw - row * a.splits;
    const int b = row / a.hkv;
    const int g = row - b * a.hkv;
    const int r16 = lane & 15;
    const int j4 = lane >> 4;
    const int e0 = split * a.per_split;
    int ne = a.n_blk - e0;
    ne = ne < a.per_split ? ne : a.per_split;
    // the list and page-table loads first: a wait for them then does not
    // wait for the query load behind them
    const WaveEntries ent = load_entries(a, row, b, e0, ne);
    bf16x8 qv[NT][D / 32];
    load_query<D, NT>(a, b, g, qv);
    WaveAcc<D, NT> acc;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        acc.m_run[t] = -__builtin_inff();
        acc.l_run[t] = 0.f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc.o[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (ne == 16)
        attn_wave_range<D, NT, 16>(a, g, 16, ent, qv, acc);
    else
        attn_wave_range<D, NT>(a, g, ne, ent, qv, acc);

#pragma unroll
    for (int t = 0; t < NT; ++t) {
        // Column totals of the normaliser live in lanes r16, r16+16, r16+32, r16+48.
        float l_run = acc.l_run[t];
        l_run = add_xor32(add_xor16(l_run));
        const int c = 16 * t + r16;
        if (c < a.n_rows_q) {
            const size_t slot = ((size_t)row * a.splits + split) * a.n_rows_q + c;
            float *po = a.part_o + slot * D + 4 * j4;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) *reinterpret_cast<f32x4 *>(po + 16 * mt) = acc.o[t][mt];
            if (j4 == 0) {
                a.part_ml[2 * slot] = acc.m_run[t];
                a.part_ml[2 * slot + 1] = l_run;
            }
        }
    }
}

// From kAttnRowFillRows rows (one per CU) attention runs as one 8-wave
// workgroup per row, merged in LDS.  From OASIS_ATTN_ROWSPLIT_MIN_ROWS up to
// that, a row takes several such workgroups (enough to give every CU one) that
// merge across workgroups through the workspace; below it, split-K over more
// waves fills the CUs and a second launch merges.
#ifndef OASIS_ATTN_ROW_MIN_ROWS
#define OASIS_ATTN_ROW_MIN_ROWS 256
#endif
constexpr int kAttnRowFillRows = OASIS_ATTN_ROW_MIN_ROWS;
#ifndef OASIS_ATTN_ROWSPLIT_MIN_ROWS
#define OASIS_ATTN_ROWSPLIT_MIN_ROWS 128
#endif
#ifndef OASIS_ATTN_ROW_WAVES
#define OASIS_ATTN_ROW_WAVES 8
#endif
constexpr int kRowAttnWaves = OASIS_ATTN_ROW_WAVES;   // waves of the one-workgroup-per-row kernel
#ifndef OASIS_ATTN_ROWSPLIT_WAVES
#define OASIS_ATTN_ROWSPLIT_WAVES 8
#endif
constexpr int kRowSplitWaves = OASIS_ATTN_ROWSPLIT_WAVES;
#ifndef OASIS_ATTN_ROWSPLIT_WGS
#define OASIS_ATTN_ROWSPLIT_WGS 256     // workgroups the row-split launch aims for
#endif

// Workgroups per row (two: the hand-over is a pairwise token exchange) and
// list entries per workgroup for the row-split kernel; false where it does
// not apply (too few rows, or fewer than two entries per wave, which would
// leave waves without a block pair).
inline bool rowsplit_plan(int rows, int n_blk, int *splits, int *per) {
    if (rows < OASIS_ATTN_ROWSPLIT_MIN_ROWS || rows >= kAttnRowFillRows || rows < 1) return false;
    const int s = (OASIS_ATTN_ROWSPLIT_WGS + rows - 1) / rows;
    const int p = (n_blk + s - 1) / s;
    if (s != 2 || p < 2 * kRowSplitWaves) return false;
    *splits = (n_blk + p - 1) / p;
    *per = p;
    return *splits == 2;
}

__host__ __device__ inline int row_attn_wave_floats(int n_rows_q, int head_dim) {
    return (n_rows_q * (head_dim + 2) + 3) & ~3;
}

// The 8 waves of a workgroup walk entries [w_begin, w_end) of row `row`,
// each a contiguous eighth (NE > 0: an eighth of exactly NE entries takes the
// fully unrolled walk), and leave their (O, max, sum) in the workgroup's LDS.
template <int D, int NE, int NW = kRowAttnWaves, int NT = 1>
__device__ __forceinline__ void row_waves_to_lds(const AttnArgs &a, int row, int w_begin, int w_end,
                                                 float *red) {
    constexpr int MT = D / 16;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int b = row / a.hkv;
    const int g = row - b * a.hkv;
    const int r16 = lane & 15;
    const int j4 = lane >> 4;
    const int nrq = a.n_rows_q;
    const int per = (w_end - w_begin + NW - 1) / NW;
    const int e_begin = w_begin + wave * per < w_end ? w_begin + wave * per : w_end;
    const int e_end = e_begin + per < w_end ? e_begin + per : w_end;
    // the first chunk's list and page-table loads first: a wait for them
    // then does not wait for the query load behind them
    const int ne0 = e_end - e_begin < kWave ? e_end - e_begin : kWave;
    const WaveEntries ent0 = load_entries(a, row, b, e_begin, ne0);
    bf16x8 qv[NT][D / 32];
    load_query<D, NT>(a, b, g, qv);
    WaveAcc<D, NT> acc;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        acc.m_run[t] = -__builtin_inff();
        acc.l_run[t] = 0.f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc.o[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (NE > 0 && e_end - e_begin == NE) {
        attn_wave_range<D, NT, NE>(a, g, NE, ent0, qv, acc);
    } else {
        for (int e0 = e_begin; e0 < e_end; e0 += kWave) {
            const int ne = e_end - e0 < kWave ? e_end - e0 : kWave;
            attn_wave_range<D, NT>(a, g, ne, e0 == e_begin ? ent0 : load_entries(a, row, b, e0, ne),
                                   qv, acc);
        }
    }
    const int wstride = row_attn_wave_floats(nrq, D);
    float *wo = red + (size_t)wave * wstride;
    float *wm = wo + (size_t)nrq * D;
    float *wl = wm + nrq;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        float l_run = acc.l_run[t];
        l_run = add_xor32(add_xor16(l_run));
        const int c = 16 * t + r16;                 // query row of this column
        if (c < nrq) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                *reinterpret_cast<f32x4 *>(wo + (size_t)c * D + 16 * mt + 4 * j4) = acc.o[t][mt];
            if (j4 == 0) { wm[c] = acc.m_run[t]; wl[c] = l_run; }
        }
    }
}

// (max, sum, O) of query row c, dim d, over the NW waves' LDS partials.
template <int D, int NW = kRowAttnWaves>
__device__ __forceinline__ void lds_merge_waves(const float *red, int nrq, int c, int d, float &M,
                                                float &L, float &O) {
    const float NEG_INF = -__builtin_inff();
    const int wstride = row_attn_wave_floats(nrq, D);
    M = NEG_INF;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, red[(size_t)w * wstride + (size_t)nrq * D + c]);
    L = 0.f;
    O = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const float *base = red + (size_t)w * wstride;
        const float m = base[(size_t)nrq * D + c];
        const float wgt = (m == NEG_INF) ? 0.f : exp2f(m - M);
        L += wgt * base[(size_t)nrq * D + nrq + c];
        O += wgt * base[(size_t)c * D + d];
    }
}

__device__ __forceinline__ void store_out(const AttnArgs &a, int row, int c, int d, int D, float res) {
    const int b = row / a.hkv;
    const int g = row - b * a.hkv;
    const int iq = c / a.group;
    const int hr = c - iq * a.group;
    a.out[(((size_t)b * a.n_q + iq) * a.hq + (size_t)g * a.group + hr) * D + d] =
        (uint16_t)float_to_bf16_bits(res);
}

// One workgroup per row: wave w walks a contiguous eighth of the row's list,
// 64 entries at a time; the waves' (max, sum, O) are merged in LDS.  With
// 128 rows it runs at the speed of split-K alone, and beside a concurrent
// scoring launch the step is faster: it occupies one CU per row and needs no
// merge launch.
template <int D>
__global__ __launch_bounds__(kRowAttnWaves * kWave) void attn_row_kernel(AttnArgs a) {
    extern __shared__ float red[];
    const int row = blockIdx.x;
    const int nrq = a.n_rows_q;
    row_waves_to_lds<D, 128 / kRowAttnWaves>(a, row, 0, a.n_blk, red);   // 128 listed blocks: unrolled
    __syncthreads();
    for (int idx = threadIdx.x; idx < nrq * D; idx += kRowAttnWaves * kWave) {
        const int c = idx / D;
        const int d = idx - c * D;
        float M, L, O;
        lds_merge_waves<D>(red, nrq, c, d, M, L, O);
        store_out(a, row, c, d, D, L > 0.f ? O / L : 0.f);
    }
}

#ifndef OASIS_ATTN_TAGGED
#define OASIS_ATTN_TAGGED 1
#endif

// A partial value and the call's token in one 64-bit word, written and read
// with single-copy-atomic device-scope accesses: a reader that finds this
// call's token in the word has this call's value, in whatever order the
// writer's stores landed, so no store needs to be waited for before another
// workgroup may look.
__device__ __forceinline__ void store_tagged(uint64_t *p, float v, uint32_t token) {
    const uint64_t w = ((uint64_t)token << 32) | __float_as_uint(v);
    __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_tagged(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool has_token(uint64_t w, uint32_t token) {
    return (uint32_t)(w >> 32) == token;
}
__device__ __forceinline__ float tagged_value(uint64_t w) { return __uint_as_float((uint32_t)w); }

// (max, sum, O) of the row's two shares merged in share order, then O / sum.
__device__ __forceinline__ float merge_two(float m0, float l0, float o0, float m1, float l1, float o1) {
    const float NEG_INF = -__builtin_inff();
    float M = NEG_INF, L = 0.f, O = 0.f;
    if (m0 != NEG_INF) { M = m0; L = l0; O = o0; }
    if (m1 != NEG_INF) {
        const float Mn = fmaxf(M, m1);
        const float r_old = M == NEG_INF ? 0.f : exp2f(M - Mn);
        const float r_new = exp2f(m1 - Mn);
        L = L * r_old + l1 * r_new;
        O = O * r_old + o1 * r_new;
    }
    return L > 0.f ? O / L : 0.f;
}

// Waits on another workgroup's published partial end after this many polls
// (about 4 ms): that workgroup issued its stores before the swap this one has
// seen, so they land within microseconds; the bound only guarantees that
// every wave exits.  A row whose partner's words never showed up is written
// as NaN.
constexpr int kTaggedPolls = 1 << 16;

// Two workgroups per row, hand-over by tagged partials: each workgroup merges
// its 8 waves in LDS and publishes its (max, sum, O) as tagged words without
// waiting for the stores to land, then swaps the tag into the row's flag.
// The one that gets the tag back arrived second: its partner published
// before swapping, so it polls the partner's words until every one carries
// the tag, merges the two in share order and writes the output.  The other
// leaves.  A workgroup waits only for a partner that has already swapped, so
// nothing assumes that both are on the GPU at once.
//
// The tag of a call's words is its token mixed with the row's epoch, a word
// of the workspace that each workgroup reads before it publishes and that the
// merging workgroup advances after it has read both partials.  So the tag
// changes from call to call even where the token does not (a call replayed
// from a captured graph keeps the token it was captured with), and words an
// earlier call or another shape left in the workspace do not carry it.  If a
// flag happens to hold the tag already, both workgroups take themselves for
// the second, and both merge the same two partials into the same bits.
template <int D, int NE, int NW>
__device__ __forceinline__ void rowsplit_tagged_tail(const AttnArgs &a, int row, int part,
                                                     const float *red, uint32_t epoch) {
    constexpr int EPT = (16 * D + NW * kWave - 1) / (NW * kWave);   // elements per thread, at most
    __shared__ int is_last;
    const int nrq = a.n_rows_q;
    const uint32_t tag = a.token + epoch * 0x9E3779B1u;
    uint64_t *po = reinterpret_cast<uint64_t *>(a.part_o);      // [rows][2][nrq][D]
    uint64_t *pml = reinterpret_cast<uint64_t *>(a.part_ml);    // [rows][2][nrq][2]
    const int other = 1 - part;
    float myM[EPT], myL[EPT], myO[EPT];
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
        const int idx = threadIdx.x + k * NW * kWave;
        if (idx < nrq * D) {
            const int c = idx / D;
            const int d = idx - c * D;
            lds_merge_waves<D, NW>(red, nrq, c, d, myM[k], myL[k], myO[k]);
            const size_t slot = ((size_t)row * 2 + part) * nrq + c;
            store_tagged(po + slot * D + d, myO[k], tag);
            if (d == 0) {
                store_tagged(pml + 2 * slot, myM[k], tag);
                store_tagged(pml + 2 * slot + 1, myL[k], tag);
            }
        }
    }
    __syncthreads();                        // every thread's stores are issued
    if (threadIdx.x == 0) {
        const uint32_t seen = __hip_atomic_exchange(a.row_flag + row, tag, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        is_last = seen == tag;
    }
    __syncthreads();
    if (!is_last) return;
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
        const int idx = threadIdx.x + k * NW * kWave;
        if (idx < nrq * D) {
            const int c = idx / D;
            const int d = idx - c * D;
            const size_t slot = ((size_t)row * 2 + other) * nrq + c;
            uint64_t oO = 0, oM = 0, oL = 0;
            bool ok = false;
            for (int poll = 0; poll < kTaggedPolls && !ok; ++poll) {
                if (poll) __builtin_amdgcn_s_sleep(2);
                oO = load_tagged(po + slot * D + d);
                oM = load_tagged(pml + 2 * slot);
                oL = load_tagged(pml + 2 * slot + 1);
                ok = has_token(oO, tag) && has_token(oM, tag) && has_token(oL, tag);
            }
            const float m1 = tagged_value(oM), l1 = tagged_value(oL), o1 = tagged_value(oO);
            const float res = !ok ? __builtin_nanf("")
                              : part == 0 ? merge_two(myM[k], myL[k], myO[k], m1, l1, o1)
                                          : merge_two(m1, l1, o1, myM[k], myL[k], myO[k]);
            store_out(a, row, c, d, D, res);
        }
    }
    if (threadIdx.x == 0) {
        // the row's next call gets another tag; its flag no longer matters
        __hip_atomic_fetch_add(a.row_epoch + row, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Two workgroups per row (rows too few to fill the CUs one per row):
// workgroup s walks entries [s * per_split, (s + 1) * per_split) with 8 waves
// merged in LDS, and publishes its (max, sum, O) partial with device-scope
// stores, which write through to the point where every XCD's L2 sees them.
// Each then swaps the call's token into the row's flag with one device-scope
// atomic exchange: the first gets back whatever the flag held (0 after any
// earlier call, or anything in a fresh workspace: never this call's token),
// the second gets the token, reads both partials with device-scope loads,
// merges them, writes the output and sets the flag back to 0.  No L2-wide
// write-back or invalidate is needed: the only data that crosses workgroups
// is written and read at device scope, and each workgroup's stores have
// completed before its exchange is issued.
template <int D, int NE, int NT = 1, int NW = kRowSplitWaves>
__global__ __launch_bounds__(NW * kWave) void attn_rowsplit_kernel(AttnArgs a) {
    extern __shared__ float red[];
    __shared__ int is_last;
    const int S = a.splits;
    const int row = blockIdx.x / S;
    const int part = blockIdx.x - row * S;
    const int nrq = a.n_rows_q;
    const float NEG_INF = -__builtin_inff();
    const int w_begin = part * a.per_split < a.n_blk ? part * a.per_split : a.n_blk;
    const int w_end = w_begin + a.per_split < a.n_blk ? w_begin + a.per_split : a.n_blk;
    __shared__ uint32_t epoch;
    if constexpr (OASIS_ATTN_TAGGED && NT == 1) {
        if (threadIdx.x == 0)
            epoch = __hip_atomic_load(a.row_epoch + row, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    row_waves_to_lds<D, NE, NW, NT>(a, row, w_begin, w_end, red);
    __syncthreads();
    if constexpr (OASIS_ATTN_TAGGED && NT == 1) {
        rowsplit_tagged_tail<D, NE, NW>(a, row, part, red, epoch);
        return;
    }
    for (int idx = threadIdx.x; idx < nrq * D; idx += NW * kWave) {
        const int c = idx / D;
        const int d = idx - c * D;
        float M, L, O;
        lds_merge_waves<D, NW>(red, nrq, c, d, M, L, O);
        const size_t slot = ((size_t)row * S + part) * nrq + c;
        __hip_atomic_store(a.part_o + slot * D + d, O, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (d == 0) {
            __hip_atomic_store(a.part_ml + 2 * slot, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.part_ml + 2 * slot + 1, L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);          // this thread's partial stores have completed
    __syncthreads();                        // ... and every thread's
    if (threadIdx.x == 0) {
        const uint32_t seen = __hip_atomic_exchange(a.row_flag + row, a.token, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        const int last = seen == a.token;
        if (last) __hip_atomic_store(a.row_flag + row, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        is_last = last;
    }
    __syncthreads();
    if (!is_last) return;
    for (int idx = threadIdx.x; idx < nrq * D; idx += NW * kWave) {
        const int c = idx / D;
        const int d = idx - c * D;
        float M = NEG_INF, L = 0.f, O = 0.f;
        for (int s = 0; s < S; ++s) {
            const size_t slot = ((size_t)row * S + s) * nrq + c;
            const float m = __hip_atomic_load(a.part_ml + 2 * slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const float l = __hip_atomic_load(a.part_ml + 2 * slot + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const float o = __hip_atomic_load(a.part_o + slot * D + d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (m == NEG_INF) continue;             // no valid token in that share
            const float Mn = fmaxf(M, m);
            const float r_old = M == NEG_INF ? 0.f : exp2f(M - Mn);
            const float r_new = exp2f(m - Mn);
            L = L * r_old + l * r_new;
            O = O * r_old + o * r_new;
            M = Mn;
        }
        store_out(a, row, c, d, D, L > 0.f ? O / L : 0.f);
    }
}

// Merge the splits of one (row, query row) pair: thread d owns head dim d.
template <int D, int kChunk>
__global__ __launch_bounds__(D) void attn_merge_kernel(AttnArgs a) {
    const int pair = blockIdx.x;                 // row * n_rows_q + c
    const int row = pair / a.n_rows_q;
    merge_one<D, kChunk>(a, row, pair - row * a.n_rows_q, threadIdx.x);
}

template <int D>
void launch_merge(const AttnArgs &a, int rows, hipStream_t stream, LaunchStop *stop) {
    const dim3 grid(rows * a.n_rows_q), block(D);
    if (a.splits <= 8)
        launch_k(attn_merge_kernel<D, 8>, grid, block, 0, stream, stop, a);
    else if (a.splits <= 16)
        launch_k(attn_merge_kernel<D, 16>, grid, block, 0, stream, stop, a);
    else
        launch_k(attn_merge_kernel<D, 32>, grid, block, 0, stream, stop, a);
}

hipError_t launch_sparse_decode_attn(const AttnArgs &a, int head_dim, bool share_gpu, hipStream_t stream,
                                     LaunchStop *stop) {
    const int rows = a.batch * a.hkv;
    if (rows == 0) return hipSuccess;
    const long long waves = (long long)rows * a.splits;
    dim3 grid((unsigned)((waves + kAttnWaves - 1) / kAttnWaves));
    dim3 block(kAttnWaves * kWave);
    const size_t row_lds = (size_t)kRowAttnWaves * row_attn_wave_floats(a.n_rows_q, head_dim) * 4;
    const bool row_fits = a.n_rows_q <= 16 && row_lds <= 65536;
    // sharing the GPU with a concurrent launch: one CU per row from the
    // row-split range up, which leaves the other CUs to that launch
    const int row_min = share_gpu ? OASIS_ATTN_ROWSPLIT_MIN_ROWS : kAttnRowFillRows;
    if (rows >= row_min && row_fits) {
        const size_t lds = row_lds;
        if (head_dim == 128)
            launch_k(attn_row_kernel<128>, dim3(rows), dim3(kRowAttnWaves * kWave), lds, stream, stop, a);
        else
            launch_k(attn_row_kernel<64>, dim3(rows), dim3(kRowAttnWaves * kWave), lds, stream, stop, a);
        return hipGetLastError();
    }
    int wg_splits = 0, wg_per = 0;
    if (row_fits && rowsplit_plan(rows, a.n_blk, &wg_splits, &wg_per) &&
        wg_splits * (OASIS_ATTN_TAGGED ? 2 : 1) <= a.splits) {
        // the workspace holds room for a.splits partials per row of 4-byte
        // words; the tagged hand-over stores 8-byte words for its two shares
        AttnArgs r = a;
        r.splits = wg_splits;
        r.per_split = wg_per;
        const dim3 grid2((unsigned)(rows * wg_splits)), block2(kRowSplitWaves * kWave);
        const size_t lds2 = (size_t)kRowSplitWaves * row_attn_wave_floats(a.n_rows_q, head_dim) * 4;
        // a wave share of exactly 8 or 16 entries takes the fully unrolled walk
        const int share = wg_per % kRowSplitWaves == 0 ? wg_per / kRowSplitWaves : 0;
        if (head_dim == 128) {
            if (share == 8) launch_k(attn_rowsplit_kernel<128, 8>, grid2, block2, lds2, stream, stop, r);
            else if (share == 16) launch_k(attn_rowsplit_kernel<128, 16>, grid2, block2, lds2, stream, stop, r);
            else launch_k(attn_rowsplit_kernel<128, 0>, grid2, block2, lds2, stream, stop, r);
        } else {
            if (share == 8) launch_k(attn_rowsplit_kernel<64, 8>, grid2, block2, lds2, stream, stop, r);
            else if (share == 16) launch_k(attn_rowsplit_kernel<64, 16>, grid2, block2, lds2, stream, stop, r);
            else launch_k(attn_rowsplit_kernel<64, 0>, grid2, block2, lds2, stream, stop, r);
        }
        return hipGetLastError();
    }
    // 17..32 query rows (the normal and the draft queries together): the same
    // two-workgroup split with two 16-column tiles, 4 waves per workgroup (one
    // per SIMD: the two tiles' accumulators need the registers)
    constexpr int kSplit2Waves = 4;
    const size_t lds_t2 = (size_t)kSplit2Waves * row_attn_wave_floats(a.n_rows_q, head_dim) * 4;
    if (a.n_rows_q > 16 && a.n_rows_q <= 32 && lds_t2 <= 65536 &&
        rowsplit_plan(rows, a.n_blk, &wg_splits, &wg_per) && wg_splits <= a.splits) {
        AttnArgs r = a;
        r.splits = wg_splits;
        r.per_split = wg_per;
        const dim3 grid2((unsigned)(rows * wg_splits)), block2(kSplit2Waves * kWave);
        const bool share16 = wg_per == 16 * kSplit2Waves;     // 16 entries per wave: unrolled
        if (head_dim == 128) {
            if (share16) launch_k(attn_rowsplit_kernel<128, 16, 2, kSplit2Waves>, grid2, block2, lds_t2, stream, stop, r);
            else launch_k(attn_rowsplit_kernel<128, 0, 2, kSplit2Waves>, grid2, block2, lds_t2, stream, stop, r);
        } else {
            if (share16) launch_k(attn_rowsplit_kernel<64, 16, 2, kSplit2Waves>, grid2, block2, lds_t2, stream, stop, r);
            else launch_k(attn_rowsplit_kernel<64, 0, 2, kSplit2Waves>, grid2, block2, lds_t2, stream, stop, r);
        }
        return hipGetLastError();
    }
    const bool two = a.n_rows_q > 16;
    if (head_dim == 128) {
        if (two) hipLaunchKernelGGL((attn_partial_kernel<128, 2>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((attn_partial_kernel<128, 1>), grid, block, 0, stream, a);
        launch_merge<128>(a, rows, stream, stop);
    } else {
        if (two) hipLaunchKernelGGL((attn_partial_kernel<64, 2>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((attn_partial_kernel<64, 1>), grid, block, 0, stream, a);
        launch_merge<64>(a, rows, stream, stop);
    }
    return hipGetLastError();
}

}  // namespace oasis
