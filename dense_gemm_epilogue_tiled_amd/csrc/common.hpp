// Shared device-side types and helpers for the gfx950 GEMM + ReLU kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gr {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Byte selectors for v_perm_b32 (result byte i = selector byte i, where 0-3
// pick bytes of the second operand and 4-7 bytes of the first): join the low
// halves, or the high halves, of two dwords into one (second.half, first.half).
constexpr uint32_t kPermLoHalves = 0x05040100u;
constexpr uint32_t kPermHiHalves = 0x07060302u;

// Two fp16 values taken from the same half-slot of two dwords:
// result = (lo_src.half[h], hi_src.half[h]).
__device__ __forceinline__ uint32_t pair_halves(uint32_t lo_src, uint32_t hi_src, int h) {
    return __builtin_amdgcn_perm(hi_src, lo_src, h ? kPermHiHalves : kPermLoHalves);
}

// The fused epilogue on one fp32 accumulator: ReLU (negative, -0 and NaN all
// give +0), then round to nearest even fp16 (v_cvt_f16_f32 under the default
// rounding mode).  Returns the fp16 bit pattern.
__device__ __forceinline__ uint16_t relu_to_f16(float x) {
    float r = (x > 0.0f) ? x : 0.0f;
    _Float16 h = (_Float16)r;
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t relu_pack2(float x0, float x1) {
    return (uint32_t)relu_to_f16(x0) | ((uint32_t)relu_to_f16(x1) << 16);
}

// Map a 1-D workgroup id to a tile (tm, tn).
//  1. Workgroups are handed to the 8 XCDs round-robin (id % 8), each XCD
//     with its own L2.  Renumber so that each XCD receives a contiguous range
//     of logical ids: neighbouring tiles, which share A row panels and B
//     column panels, then run on the same XCD.
//  2. Logical ids walk the tile grid in groups of `group_m` tile rows, column
//     by column inside a group, so tiles running at the same time reuse the
//     same panels from L2 (the grid-level swizzle of the TileLang tutorial,
//     chapter "Layout and bank conflicts").
// Both steps are bijections on [0, tiles_m * tiles_n): they change only when
// a tile runs, never what it computes.
__device__ __forceinline__ void tile_of_workgroup(uint32_t wg, uint32_t n_wg, uint32_t tiles_m,
                                                  uint32_t tiles_n, uint32_t group_m,
                                                  uint32_t& tm, uint32_t& tn) {
    const uint32_t kXcds = 8;
    uint32_t x = wg % kXcds, s = wg / kXcds;
    uint32_t q = n_wg / kXcds, r = n_wg % kXcds;
    uint32_t lid = x * q + (x < r ? x : r) + s;
    uint32_t per_group = group_m * tiles_n;
    uint32_t g = lid / per_group;
    uint32_t first_m = g * group_m;
    uint32_t gm = tiles_m - first_m < group_m ? tiles_m - first_m : group_m;
    uint32_t in_g = lid - g * per_group;
    tm = first_m + in_g % gm;
    tn = in_g / gm;
}

}  // namespace gr
