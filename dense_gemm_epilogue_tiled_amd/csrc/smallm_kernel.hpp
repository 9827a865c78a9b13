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

// ---- split-K variant (needs a workspace) -------------------------------------
//
// A 64-column strip over all of K reads each row of B as one 128-byte piece,
// 32 KiB away from the next: measured on this part, that pattern streams at
// about 5.5 TB/s, while blocks of 256 columns over a quarter of K (512-byte
// pieces) reach about 6.2 TB/s.  With scratch memory the small-M product is
// therefore split in K, the split-K of the TileLang tutorial's chapter on
// performance forensics (work for idle CUs when M x N is small), here with a
// second pass because ReLU must see the complete sum:
//   pass 1: workgroup (cb, s) owns columns [256 cb, 256 cb + 256) and the K
//           range of split s; its 4 waves are 2 column halves x 2 interleaved
//           32-deep K phases; 16-byte nontemporal loads of B (8 columns per
//           lane, an 8 x 8 block per step transposed in registers into 8
//           operands of v_mfma_f32_16x16x32_f16); the two K phases are summed
//           in LDS and the fp32 partial sums of rows m < M written to
//           part[s][m][n].
//   pass 2: every output sums its S partials in split order, then ReLU and
//           the fp16 rounding, then the store.
// Both passes are deterministic; the result differs from the single-pass
// kernel only by fp32 summation order.
constexpr int SPLIT_NB = 256;
constexpr int SPLIT_THREADS = 256;
constexpr int SPLIT_U = 2;  // 32-deep steps per load group

// Eight consecutive fp16 of row k from column n; zero outside [0,kend) x [0,N).
template <bool GUARD>
__device__ __forceinline__ u32x4 load_b8(const uint16_t* B, int64_t ldb, int64_t k, int64_t n, int64_t kend,
                                         int64_t N) {
    if constexpr (!GUARD) {
        return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(B + k * ldb + n));
    } else {
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (k < kend) {
            const uint16_t* p = B + k * ldb + n;
            if (n + 8 <= N) {
                v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
            } else {
                uint32_t h[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (n + e < N) h[e] = p[e];
#pragma unroll
                for (int d = 0; d < 4; ++d) v[d] = h[2 * d] | (h[2 * d + 1] << 16);
            }
        }
        return v;
    }
}

template <bool GUARD>
__global__ __launch_bounds__(SPLIT_THREADS, 1) void gemm_relu_smallm_split_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, float* __restrict__ part, int64_t M, int64_t N,
    int64_t K, int64_t lda, int64_t ldb, int64_t k_per_split, uint32_t n_blocks) {
    __shared__ __attribute__((aligned(16))) float red[2][MAX_M][SPLIT_NB];

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wave = tid >> 6;
    const uint32_t ch = wave & 1u;   // column half (128 columns)
    const uint32_t kp = wave >> 1;   // K phase: steps kp, kp + 2, ...
    const uint32_t li = lane & 15u;  // 8 columns of B / row of A
    const uint32_t lg = lane >> 4;   // 8-deep k group of the 32-deep step

    const uint32_t cb = blockIdx.x % n_blocks;
    const int64_t s = blockIdx.x / n_blocks;
    const int64_t n_base = (int64_t)cb * SPLIT_NB + 128 * ch;
    const int64_t n_lane = n_base + 8 * li;
    const int64_t k_begin = s * k_per_split;
    const int64_t k_end = k_begin + k_per_split < K ? k_begin + k_per_split : K;
    const int64_t steps = k_end > k_begin ? (k_end - k_begin + KSTEP - 1) / KSTEP : 0;

    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{};

    auto load_group = [&](int64_t t0, u32x4 (&rb)[SPLIT_U][8], u32x4 (&ra)[SPLIT_U]) {
#pragma unroll
        for (int u = 0; u < SPLIT_U; ++u) {
            const int64_t t = t0 + 2 * u;
            const int64_t k = k_begin + t * KSTEP + 8 * lg;
            if (t < steps) {
#pragma unroll
                for (int r = 0; r < 8; ++r) rb[u][r] = load_b8<GUARD>(B, ldb, k + r, n_lane, k_end, N);
                ra[u] = load_a8<true>(A, lda, li, k, M, k_end);
            } else {
#pragma unroll
                for (int r = 0; r < 8; ++r) rb[u][r] = u32x4{0u, 0u, 0u, 0u};
                ra[u] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    auto compute_group = [&](const u32x4 (&rb)[SPLIT_U][8], const u32x4 (&ra)[SPLIT_U]) {
#pragma unroll
        for (int u = 0; u < SPLIT_U; ++u) {
            const f16x8 a = __builtin_bit_cast(f16x8, ra[u]);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                u32x4 o;
#pragma unroll
                for (int d = 0; d < 4; ++d) o[d] = pair_halves(rb[u][2 * d][j >> 1], rb[u][2 * d + 1][j >> 1], j & 1);
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, o), a, acc[j], 0, 0, 0);
            }
        }
    };

    // Two register sets: the loads of group g+1 are in flight while group g
    // is transposed and multiplied.
    const int64_t stride = 2 * SPLIT_U;
    u32x4 rb0[SPLIT_U][8], rb1[SPLIT_U][8];
    u32x4 ra0[SPLIT_U], ra1[SPLIT_U];
    int64_t t0 = kp;
    if (t0 < steps) load_group(t0, rb0, ra0);
    for (; t0 < steps; t0 += 2 * stride) {
        if (t0 + stride < steps) load_group(t0 + stride, rb1, ra1);
        compute_group(rb0, ra0);
        if (t0 + stride >= steps) break;
        if (t0 + 2 * stride < steps) load_group(t0 + 2 * stride, rb0, ra0);
        compute_group(rb1, ra1);
    }

    // acc[j] holds C^T: lane l, register r is the partial sum for row
    // m = l%16 and column n = n_base + 8(4(l/16) + r) + j.
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[kp][li][128 * ch + 8 * (4 * lg + r) + j] = acc[j][r];
    __syncthreads();

    const int64_t n0 = (int64_t)cb * SPLIT_NB;
    for (uint32_t o = tid; o < (uint32_t)(MAX_M * SPLIT_NB); o += SPLIT_THREADS) {
        const uint32_t m = o / SPLIT_NB, nl = o % SPLIT_NB;
        const int64_t n = n0 + nl;
        if ((int64_t)m < M && n < N) part[(s * M + m) * N + n] = red[0][m][nl] + red[1][m][nl];
    }
}

// Pass 2: C[m][n] = ReLU(sum over s of part[s][m][n]), rounded to fp16.
__global__ __launch_bounds__(256) void gemm_relu_smallm_reduce_kernel(const float* __restrict__ part,
                                                                      uint16_t* __restrict__ C, int64_t M,
                                                                      int64_t N, int64_t ldc, int splits) {
    const int64_t total = M * N;
    for (int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x; o < total; o += (int64_t)gridDim.x * 256) {
        float sum = 0.0f;
        for (int s = 0; s < splits; ++s) sum += part[(int64_t)s * total + o];
        const int64_t m = o / N, n = o - m * N;
        C[m * ldc + n] = relu_to_f16(sum);
    }
}

}  // namespace smallm
}  // namespace gr
