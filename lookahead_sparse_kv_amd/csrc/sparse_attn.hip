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
//     (token-major, 16 B per lane), B = the group's query rows;
//   online softmax per query row in fp32 (exp2 with a folded log2(e));
//   O^T (D x 16 query rows) += V^T (D x 16 tokens) * P (16 tokens x 16 rows):
//     16x16x16 bf16 MFMAs whose B operand is P exactly as the S tile left it
//     in registers, and whose A operand is read straight from the dim-major
//     value tile (8 B per lane, 512 contiguous bytes per load).
// The gather is HBM-bound (each selected K and V byte is read once); split-K
// spreads rows over enough waves to fill 256 CUs, and the next block's loads
// are issued before the current block is computed.  A second kernel merges
// the (max, sum, O) partials of the splits.
#include "oasis_device.h"
#include "oasis_launch.h"

namespace oasis {

constexpr int kAttnWaves = 4;
constexpr int kAttnTargetWaves = 2048;   // enough to give every CU several waves
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
    u32x4 k[D / 32];
    u32x2 v[D / 16];
};

template <int D>
__device__ __forceinline__ void load_block(BlockRegs<D> &r, const uint16_t *kp, const uint16_t *vp) {
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) r.k[kk] = load_u32x4(kp + 32 * kk);
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) r.v[mt] = load_u32x2(vp + 16 * kBlockTokens * mt);
}

template <int D>
__global__ __launch_bounds__(kAttnWaves * kWave) void attn_partial_kernel(AttnArgs a) {
    constexpr int KK = D / 32;
    constexpr int MT = D / 16;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
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
    const int ctx = a.ctx_len[b];
    const float NEG_INF = -__builtin_inff();

    // B operand of QK^T: query row r16 = (query i, head g*G + hr), dims 32*kk + 8*j4 .. +8.
    bf16x8 qv[KK];
    const bool col_ok = r16 < a.n_rows_q;
    if (col_ok) {
        const int iq = r16 / a.group;
        const int hr = r16 - iq * a.group;
        const uint16_t *qp =
            a.q + (((size_t)b * a.n_q + iq) * a.hq + (size_t)g * a.group + hr) * D + 8 * j4;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qv[kk] = as_bf16x8(load_u32x4(qp + 32 * kk));
    } else {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qv[kk] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
    }

    // Entry e0 + lane: its page and number of valid tokens (0 = skip).
    int my_page = -1, my_ntok = 0;
    if (lane < ne) {
        const size_t e = (size_t)row * a.n_blk + e0 + lane;
        const int ent = a.blk ? a.blk[e] : e0 + lane;
        const int lg = a.blk_logical ? a.blk_logical[e] : ent;
        if (ent >= 0 && ent < a.width && lg >= 0) {
            const int p = a.page_table[(size_t)b * a.width + ent];
            long long nt = (long long)ctx - (long long)lg * kBlockTokens;
            nt = nt > kBlockTokens ? kBlockTokens : nt;
            if (p >= 0 && p < a.num_pages && nt > 0) { my_page = p; my_ntok = (int)nt; }
        }
    }

    const size_t page_stride = (size_t)a.hkv * kBlockTokens * D;
    const uint16_t *kbase = a.k_pool + (size_t)g * kBlockTokens * D + (size_t)r16 * D + 8 * j4;
    const uint16_t *vbase = a.v_pool + (size_t)g * D * kBlockTokens + (size_t)r16 * kBlockTokens + 4 * j4;

    float m_run = NEG_INF;      // running max of column r16 (log2 units)
    float l_run = 0.f;          // this lane's share of the column's running sum
    f32x4 o[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Find the first valid entry and prefetch it.
    int i = 0;
    while (i < ne && readlane_i(my_page, i) < 0) ++i;
    BlockRegs<D> cur;
    if (i < ne) {
        const size_t off = (size_t)readlane_i(my_page, i) * page_stride;
        load_block<D>(cur, kbase + off, vbase + off);
    }
    while (i < ne) {
        const int nt = readlane_i(my_ntok, i);
        int nx = i + 1;
        while (nx < ne && readlane_i(my_page, nx) < 0) ++nx;
        BlockRegs<D> nxt;
        if (nx < ne) {
            const size_t off = (size_t)readlane_i(my_page, nx) * page_stride;
            load_block<D>(nxt, kbase + off, vbase + off);
        }

        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) s = mfma16x16x32(as_bf16x8(cur.k[kk]), qv[kk], s);
        float x[4];
        float mb = NEG_INF;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            x[t] = (4 * j4 + t < nt) ? s[t] * a.scale_log2 : NEG_INF;
            mb = fmaxf(mb, x[t]);
        }
        mb = fmaxf(mb, shfl_xor_f(mb, 16));
        mb = fmaxf(mb, shfl_xor_f(mb, 32));
        const float m_new = fmaxf(m_run, mb);    // finite: every block has a valid token
        const float alpha = exp2f(m_run - m_new);
        const uint32_t p01 = pack_bf16x2(exp2f(x[0] - m_new), exp2f(x[1] - m_new));
        const uint32_t p23 = pack_bf16x2(exp2f(x[2] - m_new), exp2f(x[3] - m_new));
        // the normaliser sums the same bf16-rounded weights the MFMA uses
        const float psum = bf16_bits_to_float(p01 & 0xffffu) + bf16_bits_to_float(p01 >> 16) +
                           bf16_bits_to_float(p23 & 0xffffu) + bf16_bits_to_float(p23 >> 16);
        l_run = l_run * alpha + psum;
        m_run = m_new;
        if (nt < kBlockTokens) {
            // zero the values of masked tokens so that garbage cannot reach O
            const int base_t = 4 * j4;
            const uint32_t k01 = (base_t + 0 < nt ? 0x0000ffffu : 0u) | (base_t + 1 < nt ? 0xffff0000u : 0u);
            const uint32_t k23 = (base_t + 2 < nt ? 0x0000ffffu : 0u) | (base_t + 3 < nt ? 0xffff0000u : 0u);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) { cur.v[mt].x &= k01; cur.v[mt].y &= k23; }
        }
        const s16x4 pb = as_s16x4(u32x2{p01, p23});
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            o[mt] *= alpha;
            o[mt] = mfma16x16x16(as_s16x4(cur.v[mt]), pb, o[mt]);
        }
        cur = nxt;
        i = nx;
    }

    // Column totals of the normaliser live in lanes r16, r16+16, r16+32, r16+48.
    l_run += shfl_xor_f(l_run, 16);
    l_run += shfl_xor_f(l_run, 32);
    if (col_ok) {
        const size_t slot = ((size_t)row * a.splits + split) * a.n_rows_q + r16;
        float *po = a.part_o + slot * D + 4 * j4;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) *reinterpret_cast<f32x4 *>(po + 16 * mt) = o[mt];
        if (j4 == 0) {
            a.part_ml[2 * slot] = m_run;
            a.part_ml[2 * slot + 1] = l_run;
        }
    }
}

// Merge the splits of one (row, query row) pair: thread d owns head dim d.
template <int D>
__global__ __launch_bounds__(D) void attn_merge_kernel(AttnArgs a) {
    const int pair = blockIdx.x;                 // row * n_rows_q + c
    const int row = pair / a.n_rows_q;
    const int c = pair - row * a.n_rows_q;
    const int b = row / a.hkv;
    const int g = row - b * a.hkv;
    const int d = threadIdx.x;
    float M = -__builtin_inff();
    for (int s = 0; s < a.splits; ++s) {
        const size_t slot = ((size_t)row * a.splits + s) * a.n_rows_q + c;
        M = fmaxf(M, a.part_ml[2 * slot]);
    }
    float L = 0.f, O = 0.f;
    if (M != -__builtin_inff()) {
        for (int s = 0; s < a.splits; ++s) {
            const size_t slot = ((size_t)row * a.splits + s) * a.n_rows_q + c;
            const float m = a.part_ml[2 * slot];
            if (m == -__builtin_inff()) continue;
            const float w = exp2f(m - M);
            L += w * a.part_ml[2 * slot + 1];
            O += w * a.part_o[slot * D + d];
        }
    }
    const float res = L > 0.f ? O / L : 0.f;
    const int iq = c / a.group;
    const int hr = c - iq * a.group;
    a.out[(((size_t)b * a.n_q + iq) * a.hq + (size_t)g * a.group + hr) * D + d] =
        (uint16_t)float_to_bf16_bits(res);
}

hipError_t launch_sparse_decode_attn(const AttnArgs &a, int head_dim, hipStream_t stream) {
    const int rows = a.batch * a.hkv;
    if (rows == 0) return hipSuccess;
    const long long waves = (long long)rows * a.splits;
    dim3 grid((unsigned)((waves + kAttnWaves - 1) / kAttnWaves));
    dim3 block(kAttnWaves * kWave);
    if (head_dim == 128) {
        hipLaunchKernelGGL(attn_partial_kernel<128>, grid, block, 0, stream, a);
        hipLaunchKernelGGL(attn_merge_kernel<128>, dim3(rows * a.n_rows_q), dim3(128), 0, stream, a);
    } else {
        hipLaunchKernelGGL(attn_partial_kernel<64>, grid, block, 0, stream, a);
        hipLaunchKernelGGL(attn_merge_kernel<64>, dim3(rows * a.n_rows_q), dim3(64), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace oasis
