// Read-bandwidth probe (a measurement aid, not part of the operation): the
// HBM read ceiling the bandwidth-bound small-M path is judged against.
//
// The roofline of a streaming kernel is the bandwidth the memory system can
// actually deliver to such a read pattern, which the published 8 TB/s
// exceeds; the TileLang tutorial's chapter "性能取证" (performance forensics)
// attributes a slow kernel layer by layer against such ceilings.  256
// workgroups of 512 threads read the buffer once with nontemporal 16-byte
// loads, four per thread in flight (32 KiB per workgroup, the depth that
// measured fastest on this part), in one of two patterns:
//   CONTIGUOUS: workgroup g streams the g-th 1/256 of the buffer;
//   ROW_PIECES: the buffer as rows of 32 KiB (an fp16 matrix 16384 wide),
//     workgroup g reads the 256-byte piece g % 128 of every row in half
//     g / 128 of the rows: the pattern of the small-M split's first pass.
// The words each workgroup reads are XOR-folded into one 64-bit value, so
// the loads cannot be optimised away and a test can check that every byte
// was read.
#pragma once

#include "common.hpp"

namespace gr {

namespace probe {

constexpr int WGS = 256;
constexpr int THREADS = 512;
constexpr int UNROLL = 4;
constexpr int64_t GRANULE = int64_t(WGS) * THREADS * UNROLL * 16;  // 8 MiB: bytes must be a multiple
constexpr int64_t ROW_BYTES = 32768;
constexpr int PIECE_BYTES = 256;
enum Pattern { CONTIGUOUS = 0, ROW_PIECES = 1 };

template <int PATTERN>
__global__ __launch_bounds__(THREADS) void stream_read_kernel(const u32x4* __restrict__ src, int64_t bytes,
                                                              uint64_t* __restrict__ sink) {
    u32x4 acc = u32x4{0u, 0u, 0u, 0u};
    if constexpr (PATTERN == CONTIGUOUS) {
        const int64_t vec_per_wg = bytes / 16 / WGS;
        const u32x4* p = src + (int64_t)blockIdx.x * vec_per_wg;
        for (int64_t i = threadIdx.x; i < vec_per_wg; i += (int64_t)THREADS * UNROLL) {
            u32x4 v[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) v[u] = __builtin_nontemporal_load(p + i + (int64_t)u * THREADS);
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) acc ^= v[u];
        }
    } else {
        constexpr int64_t ROW_VEC = ROW_BYTES / 16;
        constexpr int CHUNKS = PIECE_BYTES / 16;            // 16 lanes per row piece
        constexpr int ROWS_PER_PASS = THREADS / CHUNKS;     // 32
        const int64_t rows_half = bytes / ROW_BYTES / 2;    // a multiple of 128
        const uint32_t piece = blockIdx.x % (WGS / 2), half = blockIdx.x / (WGS / 2);
        const u32x4* p = src + (int64_t)half * rows_half * ROW_VEC + (int64_t)piece * CHUNKS +
                         (threadIdx.x % CHUNKS);
        const int64_t r0 = threadIdx.x / CHUNKS;
        for (int64_t r = r0; r < rows_half; r += (int64_t)ROWS_PER_PASS * UNROLL) {
            u32x4 v[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u)
                v[u] = __builtin_nontemporal_load(p + (r + (int64_t)u * ROWS_PER_PASS) * ROW_VEC);
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) acc ^= v[u];
        }
    }
    // fold: every lane's words, then one store per workgroup
    const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    __shared__ uint32_t fold[THREADS];
    fold[threadIdx.x] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t f = 0;
        for (int t = 0; t < THREADS; ++t) f ^= fold[t];
        sink[blockIdx.x] = f;
    }
}

}  // namespace probe
}  // namespace gr
