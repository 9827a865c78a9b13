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

// Round to nearest even bfloat16 with no ReLU (NaN stays a quiet NaN; the
// carry of the rounding bias moves into the exponent, so the largest values
// round to +-Inf).
__device__ __forceinline__ uint16_t to_bf16(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Element types of A, B and C.  Operands travel as 16-bit patterns (f16x8
// registers); only the matrix-core instruction and the output rounding
// depend on the type.  Accumulation is fp32 for both.  kGeneral selects the
// epilogue: false is the fused ReLU; true (the Epi<> wrapper below) is bias
// plus a run-time activation.
struct ElemF16 {
    static constexpr bool kIsF16 = true;
    static constexpr bool kGeneral = false;
    static __device__ __forceinline__ float widen(uint16_t h) {
        return (float)__builtin_bit_cast(_Float16, h);
    }
    static __device__ __forceinline__ uint16_t round(float x) {
        return __builtin_bit_cast(uint16_t, (_Float16)x);
    }
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
    static constexpr bool kGeneral = false;
    static __device__ __forceinline__ float widen(uint16_t h) {
        return __builtin_bit_cast(float, (uint32_t)h << 16);
    }
    static __device__ __forceinline__ uint16_t round(float x) { return to_bf16(x); }
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

// ---- epilogues beyond ReLU ------------------------------------------------------
//
// out[m][n] = round(act(scale * acc[m][n] + bias[n])): a bias broadcast along the
// rows and one of the activations the elementwise pattern lists (relu,
// sigmoid, tanh, gelu; "Tilelang Cuda Patterns", section 1), plus SiLU and
// the tanh form of GELU.  The activation is evaluated in fp32 on the biased
// accumulator, then rounded once to the output type.

// Activation codes (equal to the GR_ACT_* values of the C ABI).
enum : int {
    kActNone = 0,
    kActRelu = 1,
    kActGelu = 2,      // x * Phi(x) = x/2 * (1 + erf(x / sqrt 2))
    kActGeluTanh = 3,  // x/2 * (1 + tanh(sqrt(2/pi) * (x + 0.044715 x^3)))
    kActSilu = 4,      // x / (1 + e^-x)
    kActSigmoid = 5,   // 1 / (1 + e^-x)
    kActTanh = 6,
    kActCount = 7
};

// Run-time arguments of the general epilogue, passed by value to every
// kernel (ignored by the ReLU instantiations).
struct EpiArgs {
    const uint16_t* bias;  // N values of C's element type, or nullptr for none
    int act;               // kAct*
    float scale;           // multiplies the accumulator first (1 except for the fp8 calls)
};

// The activations in fp32, in forms built from the hardware exp2 and
// reciprocal (v_exp_f32, v_rcp_f32: about 1 ulp each) and a few FMAs, so
// the epilogue's vector work stays small next to the tile's matrix work:
//   sigmoid(x) = 1 / (1 + e^-x), SiLU(x) = x sigmoid(x);
//   tanh form of GELU: x/2 (1 + tanh u) = x / (1 + e^(-2u)) (exact identity,
//     no cancellation for x << 0);
//   GELU = x Phi(x) with Phi(-|x|) = erfc(|x|/sqrt 2) / 2 from the rational
//     approximation of Abramowitz and Stegun, formula 7.1.26 (erfc(z) =
//     t P(t) e^(-z^2), t = 1/(1 + p z), |error in erf| <= 1.5e-7), and
//     Phi(|x|) = 1 - Phi(-|x|);
//   tanh(a) = (1 - e^(-2a)) / (1 + e^(-2a)) for a = |x| >= 1/16, and its
//     odd Taylor polynomial to a^5 below (relative error < 4e-9), sign
//     restored.
// Each is within about 2e-7 * max(1, |x|) of the exact function in absolute
// terms, far below half an ulp of the fp16 or bfloat16 result at the sizes
// that matter.
namespace act {

__device__ __forceinline__ float ex(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896341f); }
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }

template <int A>
__device__ __forceinline__ float apply(float x) {
    if constexpr (A == kActRelu) {
        return x > 0.0f ? x : 0.0f;
    } else if constexpr (A == kActGelu) {
        const float z = __builtin_fabsf(x) * 0.70710678118654752f;
        const float t = rcp(1.0f + 0.3275911f * z);
        const float poly =
            t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
        const float q = 0.5f * poly * ex(-z * z);  // Phi(-|x|)
        return x * (x >= 0.0f ? 1.0f - q : q);
    } else if constexpr (A == kActGeluTanh) {
        const float u = 0.79788456080286536f * x * (1.0f + 0.044715f * x * x);
        return x * rcp(1.0f + ex(-2.0f * u));
    } else if constexpr (A == kActSilu) {
        return x * rcp(1.0f + ex(-x));
    } else if constexpr (A == kActSigmoid) {
        return rcp(1.0f + ex(-x));
    } else if constexpr (A == kActTanh) {
        const float a = __builtin_fabsf(x);
        const float e = ex(-2.0f * a);
        const float big = (1.0f - e) * rcp(1.0f + e);
        const float a2 = a * a;
        const float small = a * (1.0f + a2 * (-0.333333333f + a2 * 0.133333333f));
        return __builtin_copysignf(a < 0.0625f ? small : big, x);
    } else {
        return x;
    }
}

template <int A>
struct Tag {
    static constexpr int value = A;
};

// Call f(Tag<act>{}) with the activation as a compile-time constant, so the
// per-element code has no branch on it.
template <typename F>
__device__ __forceinline__ void dispatch(int a, F&& f) {
    switch (a) {
        case kActRelu: f(Tag<kActRelu>{}); break;
        case kActGelu: f(Tag<kActGelu>{}); break;
        case kActGeluTanh: f(Tag<kActGeluTanh>{}); break;
        case kActSilu: f(Tag<kActSilu>{}); break;
        case kActSigmoid: f(Tag<kActSigmoid>{}); break;
        case kActTanh: f(Tag<kActTanh>{}); break;
        default: f(Tag<kActNone>{}); break;
    }
}

}  // namespace act

__device__ __forceinline__ float activate(float x, int a) {
    switch (a) {
        case kActRelu: return act::apply<kActRelu>(x);
        case kActGelu: return act::apply<kActGelu>(x);
        case kActGeluTanh: return act::apply<kActGeluTanh>(x);
        case kActSilu: return act::apply<kActSilu>(x);
        case kActSigmoid: return act::apply<kActSigmoid>(x);
        case kActTanh: return act::apply<kActTanh>(x);
        default: return x;
    }
}

// The general-epilogue form of an element type.
template <typename Base>
struct Epi : Base {
    static constexpr bool kGeneral = true;
};

// One output value: the fused ReLU, or bias + activation.  n is the output
// column; a bias is read only for n < N.
template <typename E>
__device__ __forceinline__ uint16_t epi_value(float acc, int64_t n, int64_t N, const EpiArgs& ep) {
    if constexpr (E::kGeneral) {
        float x = __fmul_rn(acc, ep.scale);
        if (ep.bias != nullptr && n < N) x = __fadd_rn(x, E::widen(ep.bias[n]));
        return E::round(activate(x, ep.act));
    } else {
        return E::relu_round(acc);
    }
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
// a tile runs, never what it computes.  group_m with kNoXcdRemap set skips
// step 1 (logical id = workgroup id): a test hook that checks exactly that.
constexpr uint32_t kNoXcdRemap = 0x80000000u;
__device__ __forceinline__ void tile_of_workgroup(uint32_t wg, uint32_t n_wg, uint32_t tiles_m,
                                                  uint32_t tiles_n, uint32_t group_m,
                                                  uint32_t& tm, uint32_t& tn) {
    const uint32_t kXcds = 8;
    const bool remap = (group_m & kNoXcdRemap) == 0;
    group_m &= ~kNoXcdRemap;
    uint32_t x = wg % kXcds, s = wg / kXcds;
    uint32_t q = n_wg / kXcds, r = n_wg % kXcds;
    uint32_t lid = remap ? x * q + (x < r ? x : r) + s : wg;
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
// The same move for a last tile column (N >= bn): it ends at column N.
__device__ __forceinline__ int64_t shifted_col0(int64_t n_tile, int64_t N, int64_t bn) {
    return n_tile + bn <= N ? n_tile : N - bn;
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

// Accumulator layouts of a wave tile of 32*FM x 32*FN, both from MFMAs
// issued with B as the first operand, so every block holds C^T:
//   f32x16 [FM][FN] (v_mfma_f32_32x32x16): lane l, register 4q + t of block
//     (i, j) is row 32i + l%32, column 32j + 8q + 4(l/32) + t;
//   f32x4 [2FM][2FN] (v_mfma_f32_16x16x32): lane l, register t of block
//     (i, j) is row 16i + l%16, column 16j + 4(l/16) + t.
// Either way a lane holds runs of 4 consecutive columns of one row.
template <typename Acc>
struct AccTile;
template <int BM, int BN>
struct AccTile<f32x16[BM][BN]> {
    static constexpr int FM = BM, FN = BN;
};
template <int BM, int BN>
struct AccTile<f32x4[BM][BN]> {
    static_assert(BM % 2 == 0 && BN % 2 == 0, "16 x 16 blocks pair up into 32 x 32 ones");
    static constexpr int FM = BM / 2, FN = BN / 2;
};

// fp32 values of the next 32-row block of a wave tile into LDS: element
// (r, c) of the block is word c%4 of 16-byte chunk off(r, c/4).  Called for
// the blocks in order from a rolled loop: each call writes the first block
// and moves the others up, so that no register is selected by the caller's
// loop counter (which makes the compiler keep the accumulators in scratch
// memory).
template <int FM, int FN, typename Off>
__device__ __forceinline__ void stage_fp32_rows(f32x16 (&acc)[FM][FN], uint8_t* region, uint32_t lane, Off off) {
    const uint32_t r_lane = lane & 31u, half = lane >> 5;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *reinterpret_cast<f32x4*>(region + off(r_lane, 8u * j + 2u * q + half)) =
                f32x4{acc[0][j][4 * q + 0], acc[0][j][4 * q + 1], acc[0][j][4 * q + 2], acc[0][j][4 * q + 3]};
#pragma unroll
    for (int ii = 0; ii + 1 < FM; ++ii)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[ii][j] = acc[ii + 1][j];
}
// 16 x 16 blocks: the first two block rows, then the others move up by two.
template <int BM, int BN, typename Off>
__device__ __forceinline__ void stage_fp32_rows(f32x4 (&acc)[BM][BN], uint8_t* region, uint32_t lane, Off off) {
    const uint32_t r = lane & 15u, g = lane >> 4;
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
        for (int j = 0; j < BN; ++j) *reinterpret_cast<f32x4*>(region + off(16u * ii + r, 4u * j + g)) = acc[ii][j];
#pragma unroll
    for (int ii = 0; ii + 2 < BM; ++ii)
#pragma unroll
        for (int j = 0; j < BN; ++j) acc[ii][j] = acc[ii + 2][j];
}

// General epilogue (bias + activation) for one wave's tile, one 32-row block
// at a time: the wave writes the block's fp32 accumulators to its LDS region
// (32 rows x 32*FN columns, 16-byte chunk c of row r at slot c XOR (r mod
// chunks per row)), then reads it back with each lane on 4 consecutive
// columns, so the bias is loaded once per lane and every store covers whole
// row segments (8-byte stores when C's rows allow, else 2-byte ones).  Needs
// 16 KiB (FN = 4) or 8 KiB (FN = 2) of LDS per wave; all waves call it.
// acc may be overwritten.
template <bool EDGE, typename E, typename Acc>
__device__ __forceinline__ void store_wave_tile_general(Acc& acc, uint8_t* region, uint32_t lane,
                                                        uint16_t* __restrict__ C, int64_t ldc, int64_t row0,
                                                        int64_t col0, int64_t row_min, int64_t M, int64_t N,
                                                        int vec_c, const EpiArgs& ep, int64_t col_min = 0) {
    constexpr int FM = AccTile<Acc>::FM, FN = AccTile<Acc>::FN;
    constexpr uint32_t COLS = 32 * FN;
    constexpr uint32_t CHUNKS = COLS / 4;  // 16-byte fp32 chunks per row, also lanes per row on the way back
    constexpr uint32_t ROW_BYTES = 4 * COLS;
    constexpr uint32_t RPI = 64 / CHUNKS;  // rows per read-back instruction
    auto off = [](uint32_t row, uint32_t chunk) -> uint32_t {
        return row * ROW_BYTES + ((chunk ^ (row & (CHUNKS - 1))) << 4);
    };
    const uint32_t ch = lane & (CHUNKS - 1);  // this lane's chunk on the way back
    const int64_t n = col0 + 4 * ch;
    const bool has_bias = ep.bias != nullptr;
    float b[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (has_bias) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
            if (n + t < N) b[t] = E::widen(ep.bias[n + t]);
    }
    const bool wide = vec_c >= 4;
    // The block loop and the read-back loop stay rolled, so the activation
    // code exists once per kernel; only the register-indexed write of block
    // i is unrolled (one branch per block).
#pragma unroll 1
    for (int i = 0; i < FM; ++i) {
        __syncthreads();
        stage_fp32_rows(acc, region, lane, off);
        __syncthreads();
        // One copy of the read-back per activation; two rows in flight.
        act::dispatch(ep.act, [&](auto tag) {
            constexpr int A = decltype(tag)::value;
#pragma unroll 2
            for (uint32_t k = 0; k < 32u / RPI; ++k) {
                const uint32_t row = RPI * k + lane / CHUNKS;
                const int64_t m = row0 + 32 * i + row;
                const f32x4 v = *reinterpret_cast<const f32x4*>(region + off(row, ch));
                if (EDGE && (m < row_min || m >= M)) continue;
                uint16_t o[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    // scale, then bias: two roundings, never fused into one
                    const float x = __fmul_rn(v[t], ep.scale);
                    o[t] = E::round(act::apply<A>(has_bias ? __fadd_rn(x, b[t]) : x));
                }
                uint16_t* dst = C + m * ldc + n;
                if (wide && (!EDGE || (n + 4 <= N && n >= col_min))) {
                    __builtin_nontemporal_store(u32x2{(uint32_t)o[0] | ((uint32_t)o[1] << 16),
                                                      (uint32_t)o[2] | ((uint32_t)o[3] << 16)},
                                                reinterpret_cast<u32x2*>(dst));
                } else {
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        if (!EDGE || (n + t < N && n + t >= col_min)) dst[t] = o[t];
                }
            }
        });
    }
}

// fp32 partial sums of a wave tile (split-K): block (i, j) of the
// accumulators holds C^T, so lane l register r is row row0 + 32i + l%32,
// column col0 + 32j + 8(r/4) + 4(l/32) + r%4.  part is the split's M x N
// array (pitch N); only rows < M and columns < N are written (EDGE).
template <bool EDGE, int FM, int FN>
__device__ __forceinline__ void store_partials(const f32x16 (&acc)[FM][FN], float* __restrict__ part,
                                               uint32_t lane, int64_t row0, int64_t col0, int64_t M, int64_t N) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int64_t m = row0 + 32 * i + (lane & 31u);
        const bool row_ok = !EDGE || m < M;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t n = col0 + 32 * j + 8 * q + 4 * (lane >> 5);
                float* dst = part + m * N + n;
                if (!EDGE || (row_ok && n + 4 <= N && (N & 3) == 0)) {
                    *reinterpret_cast<f32x4*>(dst) = f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1],
                                                           acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                } else if (row_ok) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < N) dst[e] = acc[i][j][4 * q + e];
                }
            }
        }
    }
}

// ReLU'd fp16 values of a whole wave tile into LDS (layout of WaveTile T).
template <typename T, typename E, int FM, int FN>
__device__ __forceinline__ void stage_relu_tile(const f32x16 (&acc)[FM][FN], uint8_t* region, uint32_t lane) {
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
}
// 16 x 16 blocks: the 4 columns of lane l in block (i, j) are half (l/16)%2
// of 16-byte chunk 2j + l/32 of row 16i + l%16.
template <typename T, typename E, int BM, int BN>
__device__ __forceinline__ void stage_relu_tile(const f32x4 (&acc)[BM][BN], uint8_t* region, uint32_t lane) {
    const uint32_t r = lane & 15u, g = lane >> 4;
#pragma unroll
    for (int i = 0; i < BM; ++i) {
        const uint32_t row = 16u * i + r;
#pragma unroll
        for (int j = 0; j < BN; ++j) {
            u32x2 p;
            p[0] = relu_pack2_e<E>(acc[i][j][0], acc[i][j][1]);
            p[1] = relu_pack2_e<E>(acc[i][j][2], acc[i][j][3]);
            *reinterpret_cast<u32x2*>(region + T::off(row, 2u * j + (g >> 1)) + 8u * T::half_slot(row, g & 1u)) = p;
        }
    }
}

// Elements [s, s + L) (s >= 0, L >= 1, s + L <= 8) of the eight 16-bit
// values in v, to dst[s], ..., dst[s + L - 1]: at most two stores of 4, 2 or
// 1 elements, overlapping when L is not 4, 2 or 1 (the lane then writes the
// shared elements twice, with the same bits).  Replaces up to eight 2-byte
// stores per partial row segment of C.  The stores may be misaligned: the
// memory system of this part splits a misaligned access itself (the
// direct-to-LDS copies read from any 2-byte address on the same footing).
__device__ __forceinline__ void store_run(uint16_t* dst, const u32x4& v, int s, int L) {
    const uint64_t lo = (uint64_t)v[1] << 32 | v[0];
    const uint64_t hi = (uint64_t)v[3] << 32 | v[2];
    // elements j, j + 1, ... in the low bits (0 <= j <= 7; zeros past 7)
    auto from = [&](int j) -> uint64_t {
        if (j == 0) return lo;
        if (j < 4) return (lo >> (16 * j)) | (hi << (64 - 16 * j));
        return hi >> (16 * (j - 4));
    };
    if (L >= 4) {
        *reinterpret_cast<uint64_t*>(dst + s) = from(s);
        *reinterpret_cast<uint64_t*>(dst + s + L - 4) = from(s + L - 4);
    } else if (L >= 2) {
        *reinterpret_cast<uint32_t*>(dst + s) = (uint32_t)from(s);
        *reinterpret_cast<uint32_t*>(dst + s + L - 2) = (uint32_t)from(s + L - 2);
    } else {
        dst[s] = (uint16_t)from(s);
    }
}

// acc may be overwritten.
// col_min: with EDGE, columns below it belong to the tile on the left (a last
// tile column moved left to end at column N) and are not stored either.
template <bool EDGE, typename E = ElemF16, typename Acc>
__device__ __forceinline__ void store_wave_tile(Acc& acc, uint8_t* region, uint32_t lane,
                                                uint16_t* __restrict__ C, int64_t ldc, int64_t row0, int64_t col0,
                                                int64_t row_min, int64_t M, int64_t N, int vec_c,
                                                const EpiArgs& ep, int64_t col_min = 0) {
    constexpr int FM = AccTile<Acc>::FM, FN = AccTile<Acc>::FN;
    using T = WaveTile<FM, FN>;
    if constexpr (E::kGeneral) {
        static_assert(32 * 32 * FN * 4 <= T::REGION_BYTES, "the fp32 block fits the wave's region");
        store_wave_tile_general<EDGE, E>(acc, region, lane, C, ldc, row0, col0, row_min, M, N, vec_c, ep, col_min);
        return;
    }
    __syncthreads();
    stage_relu_tile<T, E>(acc, region, lane);
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
            if (!EDGE || (n + 8 <= N && n >= col_min)) {
                // C is written once and never read back here: nontemporal
                // stores keep it from displacing the A and B panels in L2.
                if (vec_c == 8) {
                    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst));
                } else {
                    __builtin_nontemporal_store(u32x2{v[0], v[1]}, reinterpret_cast<u32x2*>(dst));
                    __builtin_nontemporal_store(u32x2{v[2], v[3]}, reinterpret_cast<u32x2*>(dst + 4));
                }
            } else {
                // a partial row segment: the columns in [col_min, N)
                const int64_t first = n < col_min ? col_min - n : 0;
                const int64_t end = N - n < 8 ? N - n : 8;
                if (end > first) store_run(dst, v, (int)first, (int)(end - first));
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
            if (EDGE && (m < row_min || m >= M || n >= N || n < col_min)) continue;
            C[m * ldc + n] = h;
        }
    }
}

// ReLU(acc) of a 128 x 128 wave tile (8 x 8 blocks of 16 x 16) stored 32
// rows at a time through an 8 KiB LDS region of the wave's own, for the
// persistent tile loop, which keeps the rest of LDS for the next tile's
// copies.  Whole tiles, 16-byte aligned rows of C.  Each round: block rows
// 2r and 2r+1 packed to fp16 into the region (layout of a 32 x 128 wave
// tile), read back as 16-byte row segments, four rows per instruction, and
// written with nontemporal stores.  The region is the wave's alone and a
// wave's LDS operations complete in order, so no barrier is needed.
constexpr uint32_t ROWS32_BYTES = WaveTile<1, 4>::REGION_BYTES;  // 8 KiB

template <typename E, int BM, int BN>
__device__ __forceinline__ void store_wave_tile_rows32(const f32x4 (&acc)[BM][BN], uint8_t* region,
                                                       uint16_t* __restrict__ C, int64_t ldc, int64_t row0,
                                                       int64_t col0) {
    static_assert(BM == 8 && BN == 8, "a 128 x 128 wave tile of 16 x 16 blocks");
    using T = WaveTile<1, 4>;
    constexpr uint32_t ROWS_PER = 64u / T::CHUNKS;  // 4
    // Called once per tile of a loop: the lane id is recomputed here (from
    // the exec mask count), so neither it nor the addresses derived from it
    // live, or spill, through the main loop; a reload of a spill would wait
    // for every copy of the next tile already in flight.
    // (volatile: a plain mbcnt is loop-invariant, and the compiler hoists it)
    uint32_t lane;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
    const uint32_t r = lane & 15u, g = lane >> 4;
    const uint32_t ch = lane & (T::CHUNKS - 1);
#pragma unroll
    for (int round = 0; round < BM / 2; ++round) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
            const uint32_t row = 16u * ii + r;
#pragma unroll
            for (int j = 0; j < BN; ++j) {
                const f32x4& a = acc[2 * round + ii][j];
                u32x2 p;
                p[0] = relu_pack2_e<E>(a[0], a[1]);
                p[1] = relu_pack2_e<E>(a[2], a[3]);
                *reinterpret_cast<u32x2*>(region + T::off(row, 2u * j + (g >> 1)) + 8u * T::half_slot(row, g & 1u)) =
                    p;
            }
        }
#pragma unroll
        for (uint32_t k = 0; k < 32u / ROWS_PER; ++k) {
            const uint32_t row = ROWS_PER * k + (lane >> T::SHIFT);
            u32x4 v = *reinterpret_cast<const u32x4*>(region + T::off(row, ch));
            if ((row >> T::SHIFT) & 1u) v = u32x4{v[2], v[3], v[0], v[1]};
            uint16_t* dst = C + (row0 + 32 * round + row) * ldc + col0 + 8 * ch;
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst));
        }
    }
}

}  // namespace epi

}  // namespace gr
