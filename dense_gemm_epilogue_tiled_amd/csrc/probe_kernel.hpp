// Read-bandwidth probe (a measurement aid, not part of the operation): the
// HBM read ceiling the bandwidth-bound small-M path is judged against.
//
// The roofline of a streaming kernel is the bandwidth the memory system can
// actually deliver to such a read pattern, which the published 8 TB/s
// exceeds; the TileLang tutorial's chapter "性能取证" (performance forensics)
// attributes a slow kernel layer by layer against such ceilings.  Here 256
// workgroups of 512 threads each stream one contiguous 1/256 of the buffer
// with nontemporal 16-byte loads, four in flight per thread (32 KiB per
// workgroup), the fastest pattern measured on this part; the words are
// XOR-folded into one 64-bit value per workgroup so the loads are not
// optimised away.
#pragma once

#include "common.hpp"

namespace gr {

namespace probe {

constexpr int WGS = 256;
constexpr int THREADS = 512;
constexpr int UNROLL = 4;
constexpr int64_t GRANULE = int64_t(WGS) * THREADS * UNROLL * 16;  // 8 MiB: bytes must be a multiple

__global__ __launch_bounds__(THREADS) void stream_read_kernel(const u32x4* __restrict__ src, int64_t vec_per_wg,
                                                              uint64_t* __restrict__ sink) {
    const u32x4* p = src + (int64_t)blockIdx.x * vec_per_wg;
    u32x4 acc = u32x4{0u, 0u, 0u, 0u};
    for (int64_t i = threadIdx.x; i < vec_per_wg; i += (int64_t)THREADS * UNROLL) {
        u32x4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) v[u] = __builtin_nontemporal_load(p + i + (int64_t)u * THREADS);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) acc ^= v[u];
    }
    // fold: every lane's words, then one store per workgroup
    uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
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
