// MFMA tile kernel: C = ReLU(A * B), fp16 operands, fp32 accumulators, fp16 out.
//
// The structure follows the output-stationary tiled GEMM of the TileLang
// tutorial, chapter "GEMM walkthrough and parameter derivation": every
// workgroup owns one BM x BN tile of C, clears an fp32 accumulator, walks K in
// BK-wide strips (copy the A strip and the B strip to shared memory, multiply,
// accumulate), and writes the tile back once.  The ReLU and the fp16 cast run
// on the fp32 accumulators right before that write, as in the blog "TileLang
// programming basics", section 2 (the FP16 GEMM + ReLU listing).  The chapter
// "Software pipelining" motivates overlapping the next strip's copy with the
// current strip's math; here that is a register-staged double buffer.
//
// gfx950 design (the pages' A100 tiling is prior art, not the blueprint):
//   * 256 x 256 x 64 tile, 4 wave64s in a 2 x 2 grid, 128 x 128 per wave,
//     v_mfma_f32_32x32x16_f16 (16 blocks of 32 x 32 per wave, 256 fp32
//     accumulators per lane, which the compiler keeps in AGPRs).
//   * A and B both live in LDS "k-contiguous": 8 consecutive k of one row (of
//     A) or one column (of B) form a 16-byte chunk, which is exactly the
//     operand a lane feeds to the MFMA, read with one ds_read_b128.  A arrives
//     k-contiguous; B (row-major K x N) is transposed in registers: each
//     thread loads an 8 x 8 block with eight 16-byte loads and reorders it
//     with v_perm_b32 before writing eight chunks.
//   * The MFMA is issued with the operands swapped (B chunk as the first
//     operand), so it produces C^T blocks: each lane then holds 4 consecutive
//     columns of one row of C and the epilogue writes 8-byte vectors.
//   * LDS rows are paired into 256-byte lines and the 16-byte chunk index is
//     XOR-swizzled so that the 16 lanes of every ds_read_b128 / ds_write_b128
//     quarter-wave touch 16 distinct chunk slots (all banks once), for the A
//     writes, the transposed B writes and the fragment reads alike (the
//     shared-memory swizzle of the chapter "Layout and bank conflicts",
//     re-derived for this access pattern).
//   * Edge guards (GUARD=true): any element outside [0,M) x [0,K) of A or
//     [0,K) x [0,N) of B is loaded as 0 in both operands, so the K tail adds
//     exact zeros; outputs outside [0,M) x [0,N) are computed but not stored.
//     VA / VB give the widest legal load (8, 2 or 1 fp16 elements) for rows
//     that are not 16-byte aligned.
#pragma once

#include "common.hpp"

namespace gr {

namespace tile {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int THREADS = 256;
constexpr int WAVE_TM = 128;  // rows of C per wave
constexpr int WAVE_TN = 128;  // columns of C per wave
constexpr int FM = WAVE_TM / 32;
constexpr int FN = WAVE_TN / 32;
constexpr int STAGE_BYTES = (BM + BN) * BK * 2;  // A tile then B tile
constexpr int B_OFFSET = BM * BK * 2;
constexpr int LDS_BYTES = 2 * STAGE_BYTES;       // double buffer: 128 KiB

// Byte offset of the 16-byte chunk `c` (k = 8c .. 8c+7) of LDS row `row`.
// Two rows share a 256-byte line; the chunk slot is XOR-swizzled with a
// function of the line index chosen so that (a) 16 consecutive rows reading
// the same chunk, (b) two consecutive rows writing all 8 chunks and (c) rows
// 8 apart writing the same chunk all land on 16 distinct slots.
__device__ __forceinline__ uint32_t lds_chunk(uint32_t row, uint32_t c) {
    uint32_t p = row >> 1;
    uint32_t g = ((p & 7u) ^ ((p >> 3) & 7u)) | (((p >> 2) & 1u) << 3);
    uint32_t e = ((row & 1u) << 3) | c;
    return (p << 8) | ((e ^ g) << 4);
}

// Load `V` consecutive fp16 elements starting at element `idx` of `base`
// (element-aligned to V) into 16-bit lanes of `out` starting at slot `slot`.
template <int V>
__device__ __forceinline__ void load_vec(const uint16_t* base, int64_t idx, uint16_t* out) {
    if constexpr (V == 8) {
        *reinterpret_cast<u32x4*>(out) = *reinterpret_cast<const u32x4*>(base + idx);
    } else if constexpr (V == 4) {
        *reinterpret_cast<u32x2*>(out) = *reinterpret_cast<const u32x2*>(base + idx);
    } else if constexpr (V == 2) {
        *reinterpret_cast<uint32_t*>(out) = *reinterpret_cast<const uint32_t*>(base + idx);
    } else {
        out[0] = base[idx];
    }
}

// Eight consecutive elements [col, col+8) of row `row` of a row-major matrix
// with pitch `ld`, zero outside [0, rows) x [0, cols).  V = widest legal load.
template <bool GUARD, int V>
__device__ __forceinline__ u32x4 load8(const uint16_t* base, int64_t ld, int64_t row, int64_t col,
                                       int64_t rows, int64_t cols) {
    if constexpr (!GUARD) {
        return *reinterpret_cast<const u32x4*>(base + row * ld + col);
    } else {
        union {
            u32x4 v;
            uint16_t h[8];
        } u;
        u.v = u32x4{0u, 0u, 0u, 0u};
        if (row < rows) {
            const int64_t rbase = row * ld;
            if (col + 8 <= cols) {
#pragma unroll
                for (int s = 0; s < 8; s += V) load_vec<V>(base, rbase + col + s, &u.h[s]);
            } else {
#pragma unroll
                for (int s = 0; s < 8; ++s)
                    if (col + s < cols) u.h[s] = base[rbase + col + s];
            }
        }
        return u.v;
    }
}

// BT=true: B is given transposed (Bt, N x K row-major, pitch ldb); its
// chunks are loaded like A's (rows n, 8 consecutive k) and stored as they
// are, since the LDS B tile is k-contiguous already.
// AT=true: A is given transposed (At, K x M row-major, pitch lda); it is
// loaded like row-major B (8 x 8 blocks of k rows x m columns) and transposed
// in registers into the k-contiguous LDS A tile.
// E: element type (ElemF16 or ElemBF16; only the MFMA and the rounding differ).
template <bool GUARD, int VA, int VB, bool BT = false, typename E = ElemF16, bool AT = false>
__global__ __launch_bounds__(THREADS, 1) void gemm_relu_tile_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, uint16_t* __restrict__ C,
    int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
    uint32_t tiles_m, uint32_t tiles_n, uint32_t group_m, int vec_c, EpiArgs ep) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wave = tid >> 6;
    const uint32_t wm = wave >> 1;  // wave row in the 2 x 2 wave grid
    const uint32_t wn = wave & 1u;  // wave column

    uint32_t tm, tn;
    tile_of_workgroup(blockIdx.x, gridDim.x, tiles_m, tiles_n, group_m, tm, tn);
    const int64_t m0 = (int64_t)tm * BM;
    const int64_t n0 = (int64_t)tn * BN;

    // Global -> register staging.  A: 8 chunks per thread, rows tid/8 + 32j,
    // chunk tid%8 (8 lanes cover one 128-byte row strip).  B: one 8 x 8 block
    // per thread: k rows 8*(tid/32) .. +7, columns 8*(tid%32) .. +7 (32 lanes
    // cover one 512-byte row strip).
    const uint32_t a_row = tid >> 3, a_chunk = tid & 7u;
    const uint32_t b_kb = tid >> 5, b_ng = tid & 31u;
    u32x4 ra[8], rb[8];

    const int64_t KT = (K + BK - 1) / BK;

    auto load_tiles = [&](int64_t kt) {
        const int64_t k0 = kt * BK;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if constexpr (AT) ra[j] = load8<GUARD, VA>(A, lda, k0 + 8 * b_kb + j, m0 + 8 * b_ng, K, M);
            else ra[j] = load8<GUARD, VA>(A, lda, m0 + a_row + 32 * j, k0 + 8 * a_chunk, M, K);
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            if constexpr (BT) rb[r] = load8<GUARD, VB>(B, ldb, n0 + a_row + 32 * r, k0 + 8 * a_chunk, N, K);
            else rb[r] = load8<GUARD, VB>(B, ldb, k0 + 8 * b_kb + r, n0 + 8 * b_ng, K, N);
        }
    };

    auto store_tiles = [&](uint32_t stage) {
        uint8_t* sa = lds + stage * STAGE_BYTES;
        uint8_t* sb = sa + B_OFFSET;
        if constexpr (AT) {
            // Transpose the 8 (k) x 8 (m) block: column c becomes one k-chunk.
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                u32x4 o;
#pragma unroll
                for (int d = 0; d < 4; ++d) o[d] = pair_halves(ra[2 * d][c >> 1], ra[2 * d + 1][c >> 1], c & 1);
                *reinterpret_cast<u32x4*>(sa + lds_chunk(8 * b_ng + c, b_kb)) = o;
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                *reinterpret_cast<u32x4*>(sa + lds_chunk(a_row + 32 * j, a_chunk)) = ra[j];
        }
        if constexpr (BT) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                *reinterpret_cast<u32x4*>(sb + lds_chunk(a_row + 32 * j, a_chunk)) = rb[j];
        } else {
            // Transpose the 8 (k) x 8 (n) block: column c becomes one k-chunk.
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                u32x4 o;
#pragma unroll
                for (int d = 0; d < 4; ++d) o[d] = pair_halves(rb[2 * d][c >> 1], rb[2 * d + 1][c >> 1], c & 1);
                *reinterpret_cast<u32x4*>(sb + lds_chunk(8 * b_ng + c, b_kb)) = o;
            }
        }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    if (KT > 0) {
        load_tiles(0);
        store_tiles(0);
        __syncthreads();
    }

    const uint32_t frag_row = lane & 31u;  // row (A) / column (B) inside a 32-block
    const uint32_t frag_half = lane >> 5;  // which 8-wide half of a 16-wide k step

    for (int64_t kt = 0; kt < KT; ++kt) {
        const uint32_t stage = (uint32_t)(kt & 1);
        if (kt + 1 < KT) load_tiles(kt + 1);

        const uint8_t* sa = lds + stage * STAGE_BYTES;
        const uint8_t* sb = sa + B_OFFSET;
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            const uint32_t chunk = 2 * s + frag_half;
            f16x8 af[FM], bf[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = *reinterpret_cast<const f16x8*>(sa + lds_chunk(wm * WAVE_TM + 32 * i + frag_row, chunk));
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bf[j] = *reinterpret_cast<const f16x8*>(sb + lds_chunk(wn * WAVE_TN + 32 * j + frag_row, chunk));
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = E::mfma32(bf[j], af[i], acc[i][j]);
        }

        if (kt + 1 < KT) store_tiles(stage ^ 1u);
        __syncthreads();
    }

    if constexpr (E::kGeneral) {
        // Bias + activation through LDS (the operand stages are free now:
        // the K loop ends with a barrier).
        static_assert(4 * 16384 <= LDS_BYTES, "four 16 KiB wave regions");
        epi::store_wave_tile_general<GUARD, E>(acc, lds + wave * 16384u, lane, C, ldc, m0 + wm * WAVE_TM,
                                               n0 + wn * WAVE_TN, 0, M, N, vec_c, ep);
        return;
    }

    // Epilogue.  Block (i, j) holds C^T: lane l, register r is
    // C[m][n] with m = 32i + l%32 and n = 32j + 8(r/4) + 4(l/32) + r%4.
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int64_t m = m0 + wm * WAVE_TM + 32 * i + frag_row;
        if (GUARD && m >= M) continue;
        uint16_t* crow = C + m * ldc;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t n = n0 + wn * WAVE_TN + 32 * j + 8 * q + 4 * frag_half;
                const float v[4] = {acc[i][j][4 * q + 0], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                    acc[i][j][4 * q + 3]};
                if (!GUARD || (vec_c >= 4 && n + 4 <= N)) {
                    u32x2 p;
                    p[0] = relu_pack2_e<E>(v[0], v[1]);
                    p[1] = relu_pack2_e<E>(v[2], v[3]);
                    *reinterpret_cast<u32x2*>(crow + n) = p;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < N) crow[n + e] = E::relu_round(v[e]);
                }
            }
        }
    }
}

}  // namespace tile
}  // namespace gr
