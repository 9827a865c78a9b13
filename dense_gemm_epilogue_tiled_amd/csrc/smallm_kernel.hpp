// Small-M kernel: C = ReLU(A * B) when A has at most 16 rows (GEMV-like).
//
// With so few rows the product is bound by reading B once from HBM (about 8
// FLOP per byte), so the kernel is organised around streaming B: the GEMV
// pattern of "Tilelang Cuda Patterns", section 4 (threads spread over N, a
// serial walk over K, an fp32 register accumulator per thread, one cast at the
// end), re-thought for gfx950:
//   * One workgroup owns a 64-column strip of C (all rows) and the whole of
//     K, so no partial sums ever leave the workgroup and ReLU is applied once,
//     after the complete K sum (ReLU of a sum is not the sum of ReLUs).
//   * Its W waves take interleaved 32-deep K steps.  In one step a lane reads
//     8 rows x 4 columns of B (eight 8-byte loads; 16 lanes cover 128
//     contiguous bytes of each row) and 8 k of one row of A (one 16-byte load,
//     A is tiny and stays in cache).
//   * The 8 x 4 block is transposed in registers (v_perm_b32) into four
//     8-element k-vectors, which are MFMA operands as they stand: four
//     v_mfma_f32_16x16x32_f16 per step, with the B vectors as the first
//     operand (16 "rows" = 16 lanes x 4 columns) and A as the second (16
//     columns = the 16 rows of A; rows >= M are zero).  The matrix cores do
//     the multiply-adds, so the vector ALUs only move data.
//   * At the end each wave's fp32 partials go to LDS, the W partials of every
//     output are added, then ReLU, the fp16 cast and the store.
//   * GUARD=true adds the edge checks: k >= K, n >= N and m >= M read as 0.
#pragma once

#include "common.hpp"

namespace gr {

namespace smallm {

constexpr int MAX_M = 16;
constexpr int NB = 64;      // columns of C per workgroup
constexpr int KSTEP = 32;   // K per MFMA step

template <int W>
struct Shape {
    static constexpr int THREADS = 64 * W;
    static constexpr int RED_BYTES = W * MAX_M * NB * 4;
};

// B is read exactly once, so its loads are marked nontemporal: they then
// stream past the caches instead of evicting other lines (on this part a
// plain streaming read of 256 MiB reaches about 5.7 TB/s, a nontemporal one
// about 6.5 TB/s).
__device__ __forceinline__ u32x2 stream_load8(const uint16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}

// Four consecutive fp16 of row `k` starting at column `n`; zero outside.
template <bool GUARD>
__device__ __forceinline__ u32x2 load_b4(const uint16_t* B, int64_t ldb, int64_t k, int64_t n, int64_t K,
                                         int64_t N) {
    if constexpr (!GUARD) {
        return stream_load8(B + k * ldb + n);
    } else {
        u32x2 v = u32x2{0u, 0u};
        if (k < K) {
            const uint16_t* p = B + k * ldb + n;
            if (n + 4 <= N) {
                v = stream_load8(p);
            } else {
                uint32_t h[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (n + e < N) h[e] = p[e];
                v[0] = h[0] | (h[1] << 16);
                v[1] = h[2] | (h[3] << 16);
            }
        }
        return v;
    }
}

// Eight consecutive fp16 of row `m` of A starting at column `k`; zero outside.
template <bool GUARD>
__device__ __forceinline__ u32x4 load_a8(const uint16_t* A, int64_t lda, int64_t m, int64_t k, int64_t M,
                                         int64_t K) {
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (m < M) {
        const uint16_t* p = A + m * lda + k;
        if (!GUARD || k + 8 <= K) {
            v = *reinterpret_cast<const u32x4*>(p);
        } else {
            uint32_t h[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (k + e < K) h[e] = p[e];
            v[0] = h[0] | (h[1] << 16);
            v[1] = h[2] | (h[3] << 16);
            v[2] = h[4] | (h[5] << 16);
            v[3] = h[6] | (h[7] << 16);
        }
    }
    return v;
}

template <int W, int U, bool GUARD>
__global__ __launch_bounds__(64 * W, 1) void gemm_relu_smallm_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, uint16_t* __restrict__ C,
    int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc) {
    __shared__ __attribute__((aligned(16))) float red[W][MAX_M][NB];

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wave = tid >> 6;
    const uint32_t li = lane & 15u;  // MFMA row slot (4 columns of B) / column slot (row of A)
    const uint32_t lg = lane >> 4;   // which 8-deep k group of the 32-deep step

    const int64_t n_base = (int64_t)blockIdx.x * NB;
    const int64_t n_lane = n_base + 4 * li;
    const int64_t steps = (K + KSTEP - 1) / KSTEP;

    f32x4 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = f32x4{};

    // Loads of one group of U steps (this wave's steps s0, s0+W, ...).
    auto load_group = [&](int64_t s0, u32x2 (&rb)[U][8], u32x4 (&ra)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t s = s0 + (int64_t)u * W;
            const int64_t k = s * KSTEP + 8 * lg;
            if (s < steps) {
#pragma unroll
                for (int r = 0; r < 8; ++r) rb[u][r] = load_b4<GUARD>(B, ldb, k + r, n_lane, K, N);
                ra[u] = load_a8<GUARD>(A, lda, li, k, M, K);
            } else {
#pragma unroll
                for (int r = 0; r < 8; ++r) rb[u][r] = u32x2{0u, 0u};
                ra[u] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    auto compute_group = [&](const u32x2 (&rb)[U][8], const u32x4 (&ra)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const f16x8 a = __builtin_bit_cast(f16x8, ra[u]);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                u32x4 o;
#pragma unroll
                for (int d = 0; d < 4; ++d) o[d] = pair_halves(rb[u][2 * d][c >> 1], rb[u][2 * d + 1][c >> 1], c & 1);
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, o), a, acc[c], 0, 0, 0);
            }
        }
    };

    // Two register sets: the loads of group g+1 are in flight while group g
    // is transposed and multiplied, so each wave keeps U*8 loads outstanding.
    const int64_t stride = (int64_t)W * U;
    u32x2 rb0[U][8], rb1[U][8];
    u32x4 ra0[U], ra1[U];
    int64_t s0 = wave;
    if (s0 < steps) load_group(s0, rb0, ra0);
    for (; s0 < steps; s0 += 2 * stride) {
        if (s0 + stride < steps) load_group(s0 + stride, rb1, ra1);
        compute_group(rb0, ra0);
        if (s0 + stride >= steps) break;
        if (s0 + 2 * stride < steps) load_group(s0 + 2 * stride, rb0, ra0);
        compute_group(rb1, ra1);
    }

    // acc[c] holds C^T: lane l, register r is the partial sum for row
    // m = l%16 and column n = n_base + 4(4(l/16) + r) + c.
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][li][4 * (4 * lg + r) + c] = acc[c][r];
    __syncthreads();

    for (uint32_t o = tid; o < (uint32_t)(MAX_M * NB); o += 64 * W) {
        const uint32_t m = o / NB, nl = o % NB;
        const int64_t n = n_base + nl;
        if ((int64_t)m < M && n < N) {
            float sum = 0.0f;
#pragma unroll
            for (int w = 0; w < W; ++w) sum += red[w][m][nl];
            C[(int64_t)m * ldc + n] = relu_to_f16(sum);
        }
    }
}

}  // namespace smallm
}  // namespace gr
