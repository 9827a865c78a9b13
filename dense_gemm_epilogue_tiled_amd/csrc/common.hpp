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

// The same epilogue for bfloat16 output: ReLU, then round to nearest even
// bf16 (the upper 16 bits of the fp32 pattern after adding 0x7FFF plus the
// lowest kept bit; exact for every non-negative fp32, +Inf included, and
// values above the largest bf16 round to +Inf).
__device__ __forceinline__ uint16_t relu_to_bf16(float x) {
    const float r = (x > 0.0f) ? x : 0.0f;
    const uint32_t u = __builtin_bit_cast(uint32_t, r);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Element types of A, B and C.  Operands travel as 16-bit patterns (f16x8
// registers); only the matrix-core instruction and the output rounding
// depend on the type.  Accumulation is fp32 for both.
struct ElemF16 {
    static constexpr bool kIsF16 = true;
    static __device__ __forceinline__ f32x16 mfma32(f16x8 b, f16x8 a, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(b, a, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mfma16(f16x8 b, f16x8 a, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(b, a, c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint16_t relu_round(float x) { return relu_to_f16(x); }
};

struct ElemBF16 {
    static constexpr bool kIsF16 = false;
    static __device__ __forceinline__ f32x16 mfma32(f16x8 b, f16x8 a, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, b), __builtin_bit_cast(bf16x8, a),
                                                        c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mfma16(f16x8 b, f16x8 a, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b), __builtin_bit_cast(bf16x8, a),
                                                        c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint16_t relu_round(float x) { return relu_to_bf16(x); }
};

template <typename E>
__device__ __forceinline__ uint32_t relu_pack2_e(float x0, float x1) {
    return (uint32_t)E::relu_round(x0) | ((uint32_t)E::relu_round(x1) << 16);
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

// Edges for the pipelined whole-tile kernels on matrices whose size is not a
// multiple of the tile (their rows must still be 16-byte aligned and K a
// multiple of the strip depth, so every copy stays a whole 16-byte chunk):
//   * rows: the last tile row is moved up to end at row M (M >= BM), so every
//     row a tile copies exists; the rows it shares with the tile row above are
//     computed twice and stored once, by the tile that owns them.
//   * columns: a copy of a chunk past the last chunk that holds a column < N
//     reads that last chunk instead.  The chunk holds real bytes of the row
//     (the pitch is a multiple of 8 elements, so it never runs past the
//     16-byte block of element N-1); the columns >= N it brings in only
//     reach outputs that are never stored.
//   * stores: an output is written only if its row is owned by the tile and
//     its column is < N (epi::store_wave_tile below).
namespace edge {

__device__ __forceinline__ int64_t shifted_row0(int64_t m_tile, int64_t M, int64_t bm) {
    return m_tile + bm <= M ? m_tile : M - bm;
}

// Chunk (8 columns) `c` of the tile starting at column n0, clamped to the
// last chunk holding a column < N.
__device__ __forceinline__ uint32_t clamp_chunk(uint32_t c, int64_t n0, int64_t N) {
    const uint32_t last = (uint32_t)((N - 1) / 8 - n0 / 8);
    return c < last ? c : last;
}

}  // namespace edge

// Write-back of one wave's tile of C (FM x FN blocks of 32 x 32) through LDS.
//
// The MFMA accumulators hold C^T blocks: a lane owns 4 consecutive columns of
// one row, and one store instruction of the whole wave would touch 32 rows.
// Instead the wave first writes its ReLU'd fp16 tile to LDS (row-major,
// 64*FN bytes per row; the 16-byte chunk c of row r sits at slot c XOR (r mod
// CHUNKS), CHUNKS = 4*FN chunks per row, with its two 8-byte halves swapped
// when (r / CHUNKS) is odd, so that the 8-byte writes of 32 rows and the
// read-back below avoid bank conflicts), then reads it back so that
// consecutive lanes hold consecutive columns of C:
//   vec_c == 8: 16-byte chunks, CHUNKS lanes per row segment;
//   vec_c == 4: the same chunks stored as two 8-byte halves;
//   vec_c == 1: one element per lane, 64 consecutive columns per store.
// Every store instruction then covers whole row segments of C.  The caller's
// LDS must be free: the routine starts with a workgroup barrier (all waves
// call it), and the wave's region (32*FM x 32*FN fp16) is its own.
// EDGE: only rows in [row_min, M) and columns < N are stored.
namespace epi {

template <int FM, int FN>
struct WaveTile {
    static constexpr int ROWS = 32 * FM;
    static constexpr int COLS = 32 * FN;
    static constexpr uint32_t ROW_BYTES = 2 * COLS;
    static constexpr uint32_t CHUNKS = COLS / 8;  // 16-byte chunks per row
    static constexpr uint32_t REGION_BYTES = ROWS * ROW_BYTES;
    static constexpr uint32_t SHIFT = CHUNKS == 16 ? 4 : (CHUNKS == 8 ? 3 : 2);
    static_assert((1u << SHIFT) == CHUNKS, "CHUNKS is 4, 8 or 16");

    static __device__ __forceinline__ uint32_t off(uint32_t row, uint32_t chunk) {
        return row * ROW_BYTES + ((chunk ^ (row & (CHUNKS - 1))) << 4);
    }
    // Which 8-byte half of its slot the half `h` of a chunk of row `row` uses.
    static __device__ __forceinline__ uint32_t half_slot(uint32_t row, uint32_t h) {
        return h ^ ((row >> SHIFT) & 1u);
    }
};

constexpr uint32_t REGION_BYTES = WaveTile<4, 4>::REGION_BYTES;  // 32 KiB for a 128 x 128 wave tile

template <bool EDGE, typename E = ElemF16, int FM, int FN>
__device__ __forceinline__ void store_wave_tile(const f32x16 (&acc)[FM][FN], uint8_t* region, uint32_t lane,
                                                uint16_t* __restrict__ C, int64_t ldc, int64_t row0, int64_t col0,
                                                int64_t row_min, int64_t M, int64_t N, int vec_c) {
    using T = WaveTile<FM, FN>;
    __syncthreads();
    const uint32_t r_lane = lane & 31u, half = lane >> 5;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const uint32_t row = 32u * i + r_lane;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                u32x2 p;
                p[0] = relu_pack2_e<E>(acc[i][j][4 * q + 0], acc[i][j][4 * q + 1]);
                p[1] = relu_pack2_e<E>(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
                *reinterpret_cast<u32x2*>(region + T::off(row, 4u * j + q) + 8u * T::half_slot(row, half)) = p;
            }
        }
    }
    __syncthreads();
    if (vec_c >= 4) {
        constexpr uint32_t ROWS_PER = 64u / T::CHUNKS;  // rows per wave instruction
        const uint32_t ch = lane & (T::CHUNKS - 1);
#pragma unroll 8
        for (uint32_t k = 0; k < T::ROWS / ROWS_PER; ++k) {
            const uint32_t row = ROWS_PER * k + (lane >> T::SHIFT);
            u32x4 v = *reinterpret_cast<const u32x4*>(region + T::off(row, ch));
            if ((row >> T::SHIFT) & 1u) v = u32x4{v[2], v[3], v[0], v[1]};
            const int64_t m = row0 + row;
            const int64_t n = col0 + 8 * ch;
            uint16_t* dst = C + m * ldc + n;
            if (EDGE && (m < row_min || m >= M)) continue;
            if (!EDGE || n + 8 <= N) {
                // C is written once and never read back here: nontemporal
                // stores keep it from displacing the A and B panels in L2.
                if (vec_c == 8) {
                    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst));
                } else {
                    __builtin_nontemporal_store(u32x2{v[0], v[1]}, reinterpret_cast<u32x2*>(dst));
                    __builtin_nontemporal_store(u32x2{v[2], v[3]}, reinterpret_cast<u32x2*>(dst + 4));
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (n + e < N) dst[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
            }
        }
    } else {
#pragma unroll 8
        for (uint32_t k = 0; k < (uint32_t)(T::ROWS * T::COLS / 64); ++k) {
            const uint32_t idx = 64u * k + lane;
            const uint32_t row = idx / T::COLS;
            const uint32_t col = idx % T::COLS;
            const uint32_t e = col & 7u;
            const uint16_t h = *reinterpret_cast<const uint16_t*>(region + T::off(row, col >> 3) +
                                                                  8u * T::half_slot(row, e >> 2) + 2u * (e & 3u));
            const int64_t m = row0 + row;
            const int64_t n = col0 + col;
            if (EDGE && (m < row_min || m >= M || n >= N)) continue;
            C[m * ldc + n] = h;
        }
    }
}

}  // namespace epi

}  // namespace gr
