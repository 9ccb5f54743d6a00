// pool_block.h -- min/max pooling of one 16-token key tile, shared by the
// pooling kernel and the compressed scorer's refresh of a sequence's last block.
//
// OasisKV (metalmedia.ai summary), Figure 7 caption: the GPU keeps the keys
// compressed by per-block min/max pooling.  For one block and one dimension d
// the pooled pair is (min, max) of k_t[d] over the block's valid tokens; both
// are bf16 key values, so the pooling is exact.
//
// A key tile is stored in 8-dimension slices ([D/8][16][8], 256 B per slice).
// kLanes lanes share a slice: lane l reads tokens (l % kLanes) + kLanes * i of
// slice l / kLanes, so one load instruction reads runs of kLanes * 16
// contiguous bytes, each lane takes the min/max over its own tokens in
// registers, and the group of kLanes lanes is folded with DPP lane moves
// (quad exchanges, then the half-row mirror for groups of eight).
#pragma once
#include "oasis_device.h"

namespace oasis {

template <int D>
struct PoolGeom {
    static constexpr int kSlices = D / 8;                       // 8-dimension slices per tile
    static constexpr int kLanes = kWave / kSlices;              // lanes per slice: 4 (D 128), 8 (D 64)
    static constexpr int kLoads = kBlockTokens / kLanes;        // 16-byte loads per lane per tile
    static_assert(kLanes == 4 || kLanes == 8, "DPP fold covers groups of 4 or 8 lanes");
};

// Byte offset, inside the tile, of lane `lane`'s first token; load i adds
// i * kLanes * 16 bytes.
template <int D>
__device__ __forceinline__ uint32_t pool_lane_offset(int lane) {
    using G = PoolGeom<D>;
    return (uint32_t)((lane / G::kLanes) * kBlockTokens + lane % G::kLanes) * 16u;
}

template <int D, int CPOL>
__device__ __forceinline__ void pool_load(rsrc_t r, uint32_t lane_off,
                                          u32x4 (&v)[PoolGeom<D>::kLoads]) {
#pragma unroll
    for (int i = 0; i < PoolGeom<D>::kLoads; ++i)
        v[i] = buf_load16<CPOL>(r, lane_off, i * PoolGeom<D>::kLanes * 16);
}

// One token group (16 bytes: eight dimensions of one token) into the lane's
// running min/max, if `ok`.
__device__ __forceinline__ void pool_fold_tokens(const u32x4 &v, bool ok, float (&mn)[8],
                                                 float (&mx)[8]) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float lo = bf16_bits_to_float(v[w] & 0xffffu);
        const float hi = bf16_bits_to_float(v[w] >> 16);
        mn[2 * w] = ok ? fminf(mn[2 * w], lo) : mn[2 * w];
        mx[2 * w] = ok ? fmaxf(mx[2 * w], lo) : mx[2 * w];
        mn[2 * w + 1] = ok ? fminf(mn[2 * w + 1], hi) : mn[2 * w + 1];
        mx[2 * w + 1] = ok ? fmaxf(mx[2 * w + 1], hi) : mx[2 * w + 1];
    }
}

// The lanes of a slice's group folded together: every lane of the group ends
// with the group's min/max.
template <int D>
__device__ __forceinline__ void pool_fold_lanes(float (&mn)[8], float (&mx)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        mn[e] = fminf(mn[e], dpp_f<kDppQuadXor1>(mn[e]));
        mx[e] = fmaxf(mx[e], dpp_f<kDppQuadXor1>(mx[e]));
        mn[e] = fminf(mn[e], dpp_f<kDppQuadXor2>(mn[e]));
        mx[e] = fmaxf(mx[e], dpp_f<kDppQuadXor2>(mx[e]));
        if (PoolGeom<D>::kLanes == 8) {
            mn[e] = fminf(mn[e], dpp_f<kDppHalfMirror>(mn[e]));
            mx[e] = fmaxf(mx[e], dpp_f<kDppHalfMirror>(mx[e]));
        }
    }
}

template <int D, bool FULL>
__device__ __forceinline__ void pool_slice_tokens(const u32x4 (&v)[PoolGeom<D>::kLoads], int nt,
                                                  int t0, float (&mn)[8], float (&mx)[8]) {
    using G = PoolGeom<D>;
#pragma unroll
    for (int i = 0; i < G::kLoads; ++i) pool_fold_tokens(v[i], FULL || t0 + G::kLanes * i < nt, mn, mx);
}

// (mn, mx) of slice lane / kLanes over its tokens t < nt (1 <= nt <= 16), in
// every lane of the slice's group.
template <int D>
__device__ __forceinline__ void pool_slice(const u32x4 (&v)[PoolGeom<D>::kLoads], int nt, int lane,
                                           float (&mn)[8], float (&mx)[8]) {
    using G = PoolGeom<D>;
    const int t0 = lane % G::kLanes;
    const float INF = __builtin_inff();
#pragma unroll
    for (int e = 0; e < 8; ++e) { mn[e] = INF; mx[e] = -INF; }
    if (nt >= kBlockTokens)
        pool_slice_tokens<D, true>(v, nt, t0, mn, mx);
    else
        pool_slice_tokens<D, false>(v, nt, t0, mn, mx);
    pool_fold_lanes<D>(mn, mx);
}

// Eight widened bf16 values back to their bit patterns (exact: each one is a
// bf16 key element, or +-inf).
__device__ __forceinline__ u32x4 pack_exact_bf16x8(const float (&x)[8]) {
    u32x4 p;
#pragma unroll
    for (int w = 0; w < 4; ++w)
        p[w] = (__builtin_bit_cast(uint32_t, x[2 * w]) >> 16) |
               (__builtin_bit_cast(uint32_t, x[2 * w + 1]) & 0xffff0000u);
    return p;
}

// The empty box of a block outside the pool: min = +inf, max = -inf.
constexpr uint32_t kBf16PosInfPair = 0x7f807f80u;
constexpr uint32_t kBf16NegInfPair = 0xff80ff80u;

}  // namespace oasis
