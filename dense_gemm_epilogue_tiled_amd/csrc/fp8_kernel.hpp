// fp8 (OCP e4m3) GEMM with the fused epilogue: C = act(scale * A * Bt^T + bias),
// A M x K and Bt N x K, both k-contiguous bytes, fp32 accumulation, fp16 or
// bfloat16 output.  gfx950's v_mfma_f32_32x32x64_f8f6f4 multiplies a 32 x 64
// block of e4m3 values by a 64 x 32 one per instruction, twice the rate of the
// fp16 instruction.
//
// Operand layout.  Each lane supplies 32 bytes (8 VGPRs) per operand: the 32
// rows of a block are the lanes mod 32, and the two lane halves split the 64
// k of the step.  Which k a given byte position stands for inside the
// instruction does not matter here: A and B use the same positions for the
// same k, so filling both operands by one rule -- lane half h gets the two
// 16-byte chunks h and 2 + h (chunk 2s + h, s = 0, 1) of its row's 64-byte k
// strip -- pairs every A[m][k] with B[k][n] exactly once.  The output block follows the usual
// 32 x 32 MFMA layout; B goes in as the first operand, so each lane ends with
// 4 consecutive columns of one row of C (as in the fp16 kernels).
//
// gemm_fp8_tile_kernel: the 32-deep pipelined kernel's scheme for a given-
// transposed B (tile2_kernel.hpp) with one 64-byte fp8 strip in place of one
// 32-deep fp16 strip -- a strip row is 64 bytes either way, so the 4-slot
// ring, the direct-to-LDS copies, the swizzle and the fragment reads are the
// same; per strip each wave issues 16 MFMAs (4 x 4 blocks) instead of 32.
// Rows of A and Bt past M and N read row M-1 and N-1 (their results are never
// stored), so any M and N work; K must be a multiple of 64 and rows 16-byte
// aligned.
// gemm_fp8_guarded_kernel: every other shape (any K, any alignment), operands
// loaded straight into registers with bounds checks, out-of-range bytes 0.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "tile2_kernel.hpp"

namespace gr {

namespace fp8 {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// One 32 x 32 x 64 block product, both operands OCP e4m3 (format code 0),
// no block scales.
__device__ __forceinline__ f32x16 mfma(const u32x4& b0, const u32x4& b1, const u32x4& a0, const u32x4& a1,
                                        f32x16 c) {
    const i32x8 bo = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
    const i32x8 ao = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bo, ao, c, 0, 0, 0, 0, 0, 0);
}

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;  // k per strip (bytes)
constexpr int STAGES = 4;
constexpr int THREADS = 256;
constexpr int WAVE_TM = 128;
constexpr int WAVE_TN = 128;
constexpr int FM = WAVE_TM / 32;
constexpr int FN = WAVE_TN / 32;
constexpr int A_BYTES = BM * BK;  // 16 KiB
constexpr int B_BYTES = BN * BK;  // 16 KiB
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
constexpr int LDS_BYTES = STAGES * STAGE_BYTES;  // 128 KiB
static_assert(LDS_BYTES >= 4 * epi::REGION_BYTES, "the epilogue stages four wave tiles in LDS");
constexpr int COPIES = A_BYTES / (THREADS * 16);  // 16-byte copies per thread per operand: 4
// Largest row pitch (bytes) for which the per-lane copy offsets of a tile's
// 256 rows fit in 32 bits.
constexpr int64_t MAX_LD = (int64_t(1) << 31) / BM;

#define GR_LDS __attribute__((address_space(3)))

// Fragments of one strip: chunk 2s + lane/32 of the A rows (blocks i) and of
// the Bt rows (blocks j), one ds_read_b128 each.
struct Frags {
    u32x4 a[2][FM];
    u32x4 b[2][FN];
};

__device__ __forceinline__ u32x4 read16(const GR_LDS uint8_t* p) { return *(const GR_LDS u32x4*)p; }

// E: output element type with the general epilogue (Epi<ElemF16> or
// Epi<ElemBF16>); ep.scale carries scale_a * scale_b.
template <bool EDGE, typename E>
__global__ __launch_bounds__(THREADS, 1) void gemm_fp8_tile_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ Bt, uint16_t* __restrict__ C, int64_t M, int64_t N,
    int64_t K, int64_t lda, int64_t ldb, int64_t ldc, uint32_t tiles_m, uint32_t tiles_n, uint32_t group_m,
    int vec_c, EpiArgs ep) {
    static_assert(E::kGeneral, "the fp8 kernels use the general epilogue");
    using tile2::a_off;
    using tile2::barrier;
    using tile2::dma16;
    using tile2::pin;
    using tile2::wait_vmcnt;

    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t wm = wave >> 1;
    const uint32_t wn = wave & 1u;

    uint32_t tm, tn;
    tile_of_workgroup(blockIdx.x, gridDim.x, tiles_m, tiles_n, group_m, tm, tn);
    const int64_t m0 = (int64_t)tm * BM;
    const int64_t n0 = (int64_t)tn * BN;

    // ---- copies: copy i of this wave fills LDS block 4*wave + i of a slot ----
    // block = 16 rows x 64 bytes; lane -> row lane/4, slot lane%4 (chunk slot
    // XOR (row/4)%4).  Rows past M (N) read row M-1 (N-1).
    const uint8_t* base_a = A + m0 * lda;
    const uint8_t* base_b = Bt + n0 * ldb;
    uint32_t off_a[COPIES], off_b[COPIES];
#pragma unroll
    for (int i = 0; i < COPIES; ++i) {
        const uint32_t blk = 4u * wave + (uint32_t)i;
        const uint32_t r = 16u * blk + (lane >> 2);
        const uint32_t c = (lane & 3u) ^ ((r >> 2) & 3u);
        uint32_t ra = r, rb = r;
        if constexpr (EDGE) {
            ra = m0 + r < M ? r : (uint32_t)(M - 1 - m0);
            rb = n0 + r < N ? r : (uint32_t)(N - 1 - n0);
        }
        off_a[i] = (uint32_t)(ra * lda + 16u * c);
        off_b[i] = (uint32_t)(rb * ldb + 16u * c);
    }
    const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(GR_LDS uint8_t*)lds);

    // Copy c (0..7) of strip `kt` into `slot`: c even -> A copy c/2, odd -> B.
    auto dma_one = [&](uint32_t slot, uint32_t kt, int c) {
        const int i = c >> 1;
        const uint32_t blk = 4u * wave + (uint32_t)i;
        if ((c & 1) == 0)
            dma16(base_a + (int64_t)kt * BK, off_a[i], lds_base + slot * STAGE_BYTES + blk * 1024u);
        else
            dma16(base_b + (int64_t)kt * BK, off_b[i], lds_base + slot * STAGE_BYTES + A_BYTES + blk * 1024u);
    };
    auto issue = [&](uint32_t slot, uint32_t kt) {
#pragma unroll
        for (int c = 0; c < 2 * COPIES; ++c) dma_one(slot, kt, c);
    };

    // ---- fragment addresses: row wm*128 + 32i + lane%32 (A) or
    // wn*128 + 32j + lane%32 (Bt), chunk 2s + lane/32; block i or j is 2 KiB on.
    const GR_LDS uint8_t* lds_p = (const GR_LDS uint8_t*)lds;
    const uint32_t ar = wm * WAVE_TM + (lane & 31u);
    const uint32_t br = wn * WAVE_TN + (lane & 31u);
    const GR_LDS uint8_t* a_ptr[2];
    const GR_LDS uint8_t* b_ptr[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        a_ptr[s] = lds_p + a_off(ar, 2u * s + (lane >> 5));
        b_ptr[s] = lds_p + A_BYTES + a_off(br, 2u * s + (lane >> 5));
    }

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    // The 16 fragment reads of one strip, in the order the next step's MFMAs
    // (block row i, then column j) first need them: A0, B0..B3, A1..A3, each
    // as its two chunks.
    auto read_one = [&](Frags& f, uint32_t slot, int r) {
        const int q = r >> 1, s = r & 1;
        const uint32_t so = slot * STAGE_BYTES;
        if (q == 0) f.a[s][0] = read16(a_ptr[s] + so);
        else if (q <= 4) f.b[s][q - 1] = read16(b_ptr[s] + so + 2048u * (q - 1));
        else f.a[s][q - 4] = read16(a_ptr[s] + so + 2048u * (q - 4));
    };
    auto mfma_one = [&](const Frags& f, int t) {
        const int i = t >> 2, j = t & 3;
        acc[i][j] = mfma(f.b[0][j], f.b[1][j], f.a[0][i], f.a[1][i], acc[i][j]);
    };

    const uint32_t KT = (uint32_t)(K / BK);  // >= 1, whole strips only

    // Prologue: strips 0, 1, 2 in flight; strip 0 landed and read.
    issue(0, 0);
    if (KT > 1) issue(1, 1);
    if (KT > 2) issue(2, 2);
    if (KT > 2) wait_vmcnt<2 * 2 * COPIES>();
    else if (KT > 1) wait_vmcnt<2 * COPIES>();
    else wait_vmcnt<0>();
    barrier();

    Frags f0, f1;
#pragma unroll
    for (int r = 0; r < 16; ++r) read_one(f0, 0, r);

    // Steady step on strip kt (slot SLOT = kt % 4), fragments in `cur`: 2
    // MFMAs; wait for this wave's copies of strip kt+1; barrier (all copies of
    // kt+1 landed, every wave done with the slot of kt-1); then 14 MFMAs with
    // two memory operations after each of the first 12: the 16 reads of strip
    // kt+1 and the 8 copies of strip kt+3 (every third operation).
    auto step = [&](auto slot_c, uint32_t kt, Frags& cur, Frags& nxt) {
        constexpr uint32_t SLOT = decltype(slot_c)::value;
#pragma unroll
        for (int t = 0; t < 2; ++t) mfma_one(cur, t);
        pin();
        wait_vmcnt<2 * COPIES>();
        barrier();
        pin();
        int rd = 0, cp = 0;
#pragma unroll
        for (int t = 2; t < 16; ++t) {
            mfma_one(cur, t);
            pin();
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int k = 2 * (t - 2) + u;
                if (k < 24) {
                    if (k % 3 == 1) {
                        dma_one((SLOT + 3) % STAGES, kt + 3, cp);
                        ++cp;
                    } else {
                        read_one(nxt, (SLOT + 1) % STAGES, rd);
                        ++rd;
                    }
                }
            }
            pin();
        }
    };
    using S0 = std::integral_constant<uint32_t, 0>;
    using S1 = std::integral_constant<uint32_t, 1>;
    using S2 = std::integral_constant<uint32_t, 2>;
    using S3 = std::integral_constant<uint32_t, 3>;

    // The same step with its decisions taken at run time (last strips).
    auto step_tail = [&](uint32_t kt, Frags& cur, Frags& nxt) {
        if (kt >= KT) return;
        const bool more = kt + 1 < KT;
#pragma unroll
        for (int t = 0; t < 2; ++t) mfma_one(cur, t);
        pin();
        if (more) {
            if (kt + 2 < KT) wait_vmcnt<2 * COPIES>();
            else wait_vmcnt<0>();
            barrier();
        }
        pin();
        if (kt + 3 < KT) issue((kt + 3) % STAGES, kt + 3);
        pin();
        if (more) {
#pragma unroll
            for (int r = 0; r < 16; ++r) read_one(nxt, (kt + 1) % STAGES, r);
        }
        pin();
#pragma unroll
        for (int t = 2; t < 16; ++t) mfma_one(cur, t);
        pin();
    };

    const uint32_t steady = KT > 3 ? ((KT - 3) & ~3u) : 0;
    uint32_t kt = 0;
    for (; kt < steady; kt += 4) {
        step(S0{}, kt, f0, f1);
        step(S1{}, kt + 1, f1, f0);
        step(S2{}, kt + 2, f0, f1);
        step(S3{}, kt + 3, f1, f0);
    }
    step_tail(kt, f0, f1);
    step_tail(kt + 1, f1, f0);
    step_tail(kt + 2, f0, f1);
    step_tail(kt + 3, f1, f0);
    step_tail(kt + 4, f0, f1);
    step_tail(kt + 5, f1, f0);

    // Epilogue (scale, bias, activation, rounding), staged through LDS.
    epi::store_wave_tile<EDGE, E>(acc, lds + wave * epi::REGION_BYTES, lane, C, ldc, m0 + wm * WAVE_TM,
                                  n0 + wn * WAVE_TN, m0, M, N, vec_c, ep);
}

// ---- guarded kernel: any K, any alignment ------------------------------------

constexpr int G_BM = 128;  // 2 x 2 waves of 64 x 64
constexpr int G_BN = 128;

// 16 bytes of row `row` starting at byte k: one 16-byte load when the row is
// in range, the run lies inside [0, K) and the address is 16-byte aligned;
// else byte by byte, 0 outside [0, rows) x [0, K).
__device__ __forceinline__ u32x4 load16(const uint8_t* __restrict__ base, int64_t ld, int64_t row, int64_t rows,
                                        int64_t k, int64_t K) {
    if (row >= rows || k >= K) return u32x4{0u, 0u, 0u, 0u};
    const uint8_t* p = base + row * ld + k;
    if (k + 16 <= K && ((uintptr_t)p & 15u) == 0) return *reinterpret_cast<const u32x4*>(p);
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 16; ++e)
        if (k + e < K) w[e >> 2] |= (uint32_t)p[e] << (8 * (e & 3));
    return u32x4{w[0], w[1], w[2], w[3]};
}

template <typename E>
__global__ __launch_bounds__(256) void gemm_fp8_guarded_kernel(const uint8_t* __restrict__ A,
                                                              const uint8_t* __restrict__ Bt,
                                                              uint16_t* __restrict__ C, int64_t M, int64_t N,
                                                              int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                                                              uint32_t tiles_n, int vec_c, EpiArgs ep) {
    static_assert(E::kGeneral, "the fp8 kernels use the general epilogue");
    // The epilogue stages each wave's fp32 blocks here (8 KiB per wave).
    __shared__ __attribute__((aligned(1024))) uint8_t lds[4 * epi::WaveTile<2, 2>::REGION_BYTES];
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = threadIdx.x >> 6;
    const int64_t m0 = (int64_t)(blockIdx.x / tiles_n) * G_BM + 64 * (wave >> 1);
    const int64_t n0 = (int64_t)(blockIdx.x % tiles_n) * G_BN + 64 * (wave & 1u);
    const uint32_t r = lane & 31u, h = lane >> 5;

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

    // Lane half h takes chunks h and 2 + h (16 bytes each) of each 64-byte k
    // step, for both operands: the assignment of the pipelined kernel, so the
    // two kernels feed the matrix cores identical operands.
    for (int64_t k0 = 0; k0 < K; k0 += BK) {
        u32x4 a[2][2], b[2][2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
            for (int i = 0; i < 2; ++i) a[i][s] = load16(A, lda, m0 + 32 * i + r, M, k0 + 32 * s + 16 * h, K);
#pragma unroll
            for (int j = 0; j < 2; ++j) b[j][s] = load16(Bt, ldb, n0 + 32 * j + r, N, k0 + 32 * s + 16 * h, K);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = mfma(b[j][0], b[j][1], a[i][0], a[i][1], acc[i][j]);
    }

    // The same write-back as the pipelined kernels (scale, bias, activation
    // and rounding by one piece of code), for rows [m0, M) and columns < N.
    epi::store_wave_tile<true, E>(acc, lds + wave * epi::WaveTile<2, 2>::REGION_BYTES, lane, C, ldc, m0, n0, m0, M,
                                  N, vec_c, ep);
}

#undef GR_LDS

}  // namespace fp8
}  // namespace gr
