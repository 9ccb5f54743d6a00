// oasis_device.h -- device-side helpers shared by the gfx950 kernels:
// vector types for MFMA operands, bf16 bit conversions, wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace oasis {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 with round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return float_to_bf16_bits(lo) | (float_to_bf16_bits(hi) << 16);
}

// 16-byte and 8-byte global loads (non-temporal hint off: keys are streamed
// once per step, but the working set may be re-read by attention next step).
__device__ __forceinline__ u32x4 load_u32x4(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}
__device__ __forceinline__ u32x2 load_u32x2(const void *p) {
    return *reinterpret_cast<const u32x2 *>(p);
}

// Buffer resource over one tile: loads at byte offsets >= `bytes` return zero
// and touch no memory, so a block that is absent is "loaded" with bytes = 0
// without a branch around the load instruction.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;   // raw (untyped) 32-bit data, gfx9 family

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kRsrcWord3);
}
// byte offset = lane part (VGPR) + constant part (scalar offset, no extra VGPR);
// CPOL is the cache-policy operand of the load.
template <int CPOL = 0>
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t lane_off, int const_off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, lane_off, const_off, CPOL);
}
__device__ __forceinline__ u32x2 buf_load8(rsrc_t r, uint32_t lane_off, int const_off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, lane_off, const_off, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ s16x4 as_s16x4(u32x2 v) { return __builtin_bit_cast(s16x4, v); }

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16).
// Lane l supplies A row (l % 16), B column (l % 16), and the same eight
// reduction indices in both (lane group l / 16); it receives D rows
// 4 * (l / 16) + i, i < 4, of column l % 16.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D(16x16, fp32) += A(16x16, bf16) * B(16x16, bf16), four reduction indices
// per lane, same lane roles as above.
__device__ __forceinline__ f32x4 mfma16x16x16(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
    return __shfl_xor(v, mask, kWave);
}
__device__ __forceinline__ int shfl_xor_i(int v, int mask) {
    return __shfl_xor(v, mask, kWave);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor_f(v, m));
    return v;
}

__device__ __forceinline__ int readlane_i(int v, int lane) {
    return __builtin_amdgcn_readlane(v, lane);
}

// DPP lane moves (register-only, no LDS traffic).  mov_dpp<CTRL>(v) is v of
// the lane that CTRL selects, 0 where that lane is outside the row.
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2, 3, 0, 1]
constexpr int kDppRowShr1 = 0x111;     // row_shr:k = 0x110 + k
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppRowMirror = 0x140;   // lane i <- lane 15 - i within each 16 lanes
constexpr int kDppHalfMirror = 0x141;  // lane i <- lane 7 - i within each 8 lanes
constexpr int kDppRowBcast15 = 0x142;  // lane 15 of each row into the next row
constexpr int kDppRowBcast31 = 0x143;  // lane 31 into rows 2 and 3

template <int CTRL>
__device__ __forceinline__ int mov_dpp(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, mov_dpp<CTRL>(__builtin_bit_cast(int, v)));
}

// v combined (max or sum) with v of lane ^ 16 / lane ^ 32, through the gfx950
// row swaps (v_permlane16_swap / v_permlane32_swap on two copies of v): the
// two results hold v and its partner's v in every lane, so a commutative
// combine of them is the exchange-and-combine, with no LDS traffic.
__device__ __forceinline__ float max_xor16(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float add_xor16(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}
__device__ __forceinline__ float add_xor32(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// Inclusive prefix sum over the 64 lanes of a wave: Hillis-Steele within each
// 16-lane row (row shifts by 1, 2, 4, 8 with zero fill), then the row totals
// carried across rows by the two row broadcasts.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
    x += mov_dpp<kDppRowShr1>(x);
    x += mov_dpp<kDppRowShr2>(x);
    x += mov_dpp<kDppRowShr4>(x);
    x += mov_dpp<kDppRowShr8>(x);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowBcast15, 0xa, 0xf, false);   // rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowBcast31, 0xc, 0xf, false);   // rows 2, 3
    return x;
}

// Minimum / maximum over the wave (every lane gets it): a fold within each
// 16-lane row by quad exchanges and mirrors, then the four rows' results.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    uint32_t t;
    t = (uint32_t)mov_dpp<kDppQuadXor1>((int)v); v = t < v ? t : v;
    t = (uint32_t)mov_dpp<kDppQuadXor2>((int)v); v = t < v ? t : v;
    t = (uint32_t)mov_dpp<kDppHalfMirror>((int)v); v = t < v ? t : v;
    t = (uint32_t)mov_dpp<kDppRowMirror>((int)v); v = t < v ? t : v;
    const uint32_t a = (uint32_t)readlane_i((int)v, 0), b = (uint32_t)readlane_i((int)v, 16);
    const uint32_t c = (uint32_t)readlane_i((int)v, 32), d = (uint32_t)readlane_i((int)v, 48);
    const uint32_t ab = a < b ? a : b, cd = c < d ? c : d;
    return ab < cd ? ab : cd;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    uint32_t t;
    t = (uint32_t)mov_dpp<kDppQuadXor1>((int)v); v = t > v ? t : v;
    t = (uint32_t)mov_dpp<kDppQuadXor2>((int)v); v = t > v ? t : v;
    t = (uint32_t)mov_dpp<kDppHalfMirror>((int)v); v = t > v ? t : v;
    t = (uint32_t)mov_dpp<kDppRowMirror>((int)v); v = t > v ? t : v;
    const uint32_t a = (uint32_t)readlane_i((int)v, 0), b = (uint32_t)readlane_i((int)v, 16);
    const uint32_t c = (uint32_t)readlane_i((int)v, 32), d = (uint32_t)readlane_i((int)v, 48);
    const uint32_t ab = a > b ? a : b, cd = c > d ? c : d;
    return ab > cd ? ab : cd;
}

}  // namespace oasis
