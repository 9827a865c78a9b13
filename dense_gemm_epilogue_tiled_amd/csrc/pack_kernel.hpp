// Operand packing for the pipelined tile kernels.
//
// The pipelined kernels copy whole, 16-byte aligned chunks of A and B straight
// into LDS and walk K in whole 32-deep strips.  An operand whose rows are not
// 16-byte aligned, or a K that is not a multiple of 32, rules that out.  With
// a caller-provided workspace the library instead copies such an operand once
// into an aligned buffer whose K extent is padded with zeros (the edge rule
// that out-of-range elements enter the product as 0 in both operands, which
// makes the padded K steps add exact zeros), then runs the pipelined kernel
// on the copy.  The copy costs one extra read and write of the operand, small
// against the product for the shapes this is used for.
//
// One launch packs up to two operands: workgroups [0, blocks_first) serve the
// first job, the rest the second.  Every thread writes 16-byte groups of the
// destination (8 fp16), UNROLL of them at a time (all loads first, then the
// stores), each read with 2-byte loads so that any source alignment and pitch
// works; the eight loads of a wave together cover 1 KiB of contiguous source.
// Only groups at a row's end test each element against the row length.
// (Reading each group as the aligned 16-byte blocks that hold it and shifting
// it into place was measured slower.)  Destination rows and pitch are 16-byte
// aligned.
#pragma once

#include "common.hpp"

namespace gr {

namespace pack {

constexpr int THREADS = 256;

// dst[r][c] = src[r][c] for r < rows, c < cols; 0 for the rest of the
// rows_d x ldd destination.
struct Job {
    const uint16_t* src;
    uint16_t* dst;
    int64_t lds;     // source pitch (elements)
    int64_t ldd;     // destination pitch (elements, multiple of 8)
    int64_t rows;    // source rows
    int64_t cols;    // source columns
    int64_t rows_d;  // destination rows (>= rows)
};

constexpr int UNROLL = 2;

// Value of destination group g (8 fp16) and its element offset in dst.
__device__ __forceinline__ u32x4 group_value(const Job& j, int64_t g, int64_t& off) {
    const int64_t gpr = j.ldd / 8;  // 16-byte groups per destination row
    const int64_t r = g / gpr;
    const int64_t c0 = (g - r * gpr) * 8;
    off = r * j.ldd + c0;
    uint32_t h[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    if (r < j.rows) {
        const uint16_t* s = j.src + r * j.lds + c0;
        if (c0 + 8 <= j.cols) {
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = s[e];
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (c0 + e < j.cols) h[e] = s[e];
        }
    }
    u32x4 v;
#pragma unroll
    for (int d = 0; d < 4; ++d) v[d] = h[2 * d] | (h[2 * d + 1] << 16);
    return v;
}

// Grid: blocks_first workgroups stride over the first job's groups, the
// remaining ones over the second job's (an empty job has rows_d == 0).
__global__ __launch_bounds__(THREADS) void pack_kernel(Job first, Job second, uint32_t blocks_first) {
    const bool is_first = blockIdx.x < blocks_first;
    const Job& j = is_first ? first : second;
    const int64_t blk = is_first ? blockIdx.x : blockIdx.x - blocks_first;
    const int64_t nblk = is_first ? blocks_first : gridDim.x - blocks_first;
    const int64_t groups = j.rows_d * (j.ldd / 8);
    for (int64_t g0 = blk * THREADS * UNROLL + threadIdx.x; g0 < groups; g0 += nblk * THREADS * UNROLL) {
        u32x4 v[UNROLL];
        int64_t off[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int64_t g = g0 + (int64_t)u * THREADS;
            if (g < groups) v[u] = group_value(j, g, off[u]);
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int64_t g = g0 + (int64_t)u * THREADS;
            if (g < groups) *reinterpret_cast<u32x4*>(j.dst + off[u]) = v[u];
        }
    }
}

}  // namespace pack
}  // namespace gr
