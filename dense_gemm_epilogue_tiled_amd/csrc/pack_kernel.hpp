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
// destination (8 fp16), each built from element loads of the source, so any
// source alignment and pitch works; destination rows and pitch are 16-byte
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

__device__ __forceinline__ void pack_group(const Job& j, int64_t g) {
    const int64_t gpr = j.ldd / 8;  // 16-byte groups per destination row
    const int64_t r = g / gpr;
    const int64_t c0 = (g - r * gpr) * 8;
    uint32_t h[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    if (r < j.rows) {
        const uint16_t* s = j.src + r * j.lds;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (c0 + e < j.cols) h[e] = s[c0 + e];
    }
    u32x4 v;
#pragma unroll
    for (int d = 0; d < 4; ++d) v[d] = h[2 * d] | (h[2 * d + 1] << 16);
    *reinterpret_cast<u32x4*>(j.dst + r * j.ldd + c0) = v;
}

// Grid: blocks_first workgroups stride over the first job's groups, the
// remaining ones over the second job's (an empty job has rows_d == 0).
__global__ __launch_bounds__(THREADS) void pack_kernel(Job first, Job second, uint32_t blocks_first) {
    const bool is_first = blockIdx.x < blocks_first;
    const Job& j = is_first ? first : second;
    const int64_t blk = is_first ? blockIdx.x : blockIdx.x - blocks_first;
    const int64_t nblk = is_first ? blocks_first : gridDim.x - blocks_first;
    const int64_t groups = j.rows_d * (j.ldd / 8);
    for (int64_t g = blk * THREADS + threadIdx.x; g < groups; g += nblk * THREADS) pack_group(j, g);
}

}  // namespace pack
}  // namespace gr
