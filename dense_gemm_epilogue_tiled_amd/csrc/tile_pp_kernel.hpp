// Ping-pong MFMA tile kernel for whole tiles: C = ReLU(A * B), fp16 in, fp32
// accumulate, fp16 out.
//
// Same tile, LDS ring and operand layouts as the pipelined kernel (256 x 256
// output tile, 32-deep K strips, 4-slot direct-to-LDS ring, A read with
// ds_read_b128, B with ds_read_b64_tr_b16, MFMA issued with B first so lanes
// end with 4 consecutive columns of C), but with 8 waves split into two
// groups of 4 that take turns:
//   * waves w and w+4 of a workgroup run on the same SIMD, so each SIMD has
//     one wave of group 0 (rows 0..127 of the tile) and one of group 1 (rows
//     128..255); each wave owns 128 x 64 of C (128 fp32 accumulators/lane);
//   * time is cut into phases separated by workgroup barriers.  In every
//     phase one group only issues MFMAs (16 per wave, back to back) while the
//     other group only moves data: it reads its fragments of the next strip
//     from LDS and issues its half of a future strip's copies.  The next
//     phase swaps the roles.  The matrix core of each SIMD therefore always
//     has one wave feeding it, and no wave mixes memory instructions into its
//     MFMA stream (the decoupling of copies and math the chapter "Software
//     pipelining" of the TileLang tutorial describes, done here with two
//     waves per SIMD instead of asynchronous copies within one).
//   * strip d is copied in two halves: by group 0 in phase 2d-7 and by group
//     1 in phase 2d-6; it is read by group 0 in phase 2d-1 and by group 1 in
//     phase 2d; its slot (d % 4) is next written in phase 2d+1.  Before the
//     barrier ending each even phase 2k every wave waits for its own copy of
//     strip k+1 (up to two later strips may stay in flight); memory-phase
//     waves wait for their LDS reads before every barrier.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "tile2_kernel.hpp"

namespace gr {

namespace pp {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 32;
constexpr int STAGES = 4;
constexpr int THREADS = 512;
constexpr int WAVE_TM = 128;
constexpr int WAVE_TN = 64;
constexpr int FM = WAVE_TM / 32;  // 4
constexpr int FN = WAVE_TN / 32;  // 2
constexpr int KSUB = BK / 16;     // 2
constexpr int A_BYTES = BM * BK * 2;
constexpr int STAGE_BYTES = A_BYTES + BK * BN * 2;
constexpr int LDS_BYTES = STAGES * STAGE_BYTES;  // 128 KiB
constexpr int COPIES = 2;                         // per operand, per wave, per strip
constexpr int64_t MAX_LDA = tile2::MAX_LDA;
constexpr int64_t MAX_LDB = tile2::MAX_LDB;

#define GR_LDS __attribute__((address_space(3)))

struct Frags {
    f16x8 a[KSUB][FM];
    f16x8 b[KSUB][FN];
};

__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__global__ __launch_bounds__(THREADS) void gemm_relu_pp_kernel(const uint16_t* __restrict__ A,
                                                               const uint16_t* __restrict__ B,
                                                               uint16_t* __restrict__ C, int64_t M, int64_t N,
                                                               int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                                                               uint32_t tiles_m, uint32_t tiles_n, uint32_t group_m) {
    using tile2::a_off;
    using tile2::b_off;
    using tile2::barrier;
    using tile2::dma16;
    using tile2::pin;
    using tile2::read_a_operand;
    using tile2::read_b_operand;
    using tile2::wait_vmcnt;

    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];

    // With two waves per SIMD (256 registers each) the compiler would
    // otherwise keep the MFMA accumulators in ordinary VGPRs and spill; a
    // reference to an accumulation register makes it use the AGPR form.
    {
        uint32_t agpr;
        asm volatile("v_accvgpr_write_b32 %0, 0" : "=a"(agpr));
        (void)agpr;
    }

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t grp = wave >> 2;  // 0: rows 0..127, 1: rows 128..255
    const uint32_t wq = wave & 3u;   // column quarter

    uint32_t tm, tn;
    tile_of_workgroup(blockIdx.x, gridDim.x, tiles_m, tiles_n, group_m, tm, tn);
    const int64_t m0 = (int64_t)tm * BM;
    const int64_t n0 = (int64_t)tn * BN;

    // ---- copies: this wave fills A blocks 2w, 2w+1 and B blocks 2w, 2w+1 ----
    const uint8_t* base_a = reinterpret_cast<const uint8_t*>(A + m0 * lda);
    const uint8_t* base_b = reinterpret_cast<const uint8_t*>(B + n0);
    const int64_t step_a = BK * 2;
    const int64_t step_b = (int64_t)BK * ldb * 2;
    uint32_t off_a[COPIES], off_b[COPIES];
#pragma unroll
    for (int i = 0; i < COPIES; ++i) {
        const uint32_t blk = 2u * wave + (uint32_t)i;
        const uint32_t ra = 16u * blk + (lane >> 2);
        const uint32_t ca = (lane & 3u) ^ ((ra >> 2) & 3u);
        off_a[i] = (uint32_t)((ra * lda + 8u * ca) * 2);
        const uint32_t rb = 2u * blk + (lane >> 5);
        const uint32_t cb = (lane & 31u) ^ ((rb & 3u) << 2);
        off_b[i] = (uint32_t)((rb * ldb + 8u * cb) * 2);
    }
    const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(GR_LDS uint8_t*)lds);

    // This wave's copies of strip `d` into ring slot d % 4.
    auto issue = [&](uint32_t d) {
        const uint32_t slot = d % STAGES;
#pragma unroll
        for (int i = 0; i < COPIES; ++i) {
            const uint32_t blk = 2u * wave + (uint32_t)i;
            dma16(base_a + (int64_t)d * step_a, off_a[i], lds_base + slot * STAGE_BYTES + blk * 1024u);
            dma16(base_b + (int64_t)d * step_b, off_b[i], lds_base + slot * STAGE_BYTES + A_BYTES + blk * 1024u);
        }
    };

    // ---- fragment addresses (see the pipelined kernel for the derivation) ---
    const GR_LDS uint8_t* lds_p = (const GR_LDS uint8_t*)lds;
    const uint32_t ar = grp * WAVE_TM + (lane & 31u);
    const GR_LDS uint8_t* a_ptr[KSUB];
#pragma unroll
    for (int s = 0; s < KSUB; ++s) a_ptr[s] = lds_p + a_off(ar, 2u * s + (lane >> 5));
    const uint32_t bk = 8u * (lane >> 5) + ((lane & 15u) >> 2);
    const GR_LDS uint8_t* b_ptr[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const uint32_t n = wq * WAVE_TN + 32u * j + 16u * ((lane >> 4) & 1u) + 4u * (lane & 3u);
        b_ptr[j] = lds_p + A_BYTES + b_off(bk, n >> 3) + 2u * (n & 7u);
    }

    auto read_frags = [&](Frags& f, uint32_t slot) {
        const uint32_t so = slot * STAGE_BYTES;
#pragma unroll
        for (int s = 0; s < KSUB; ++s) {
#pragma unroll
            for (int j = 0; j < FN; ++j) f.b[s][j] = read_b_operand(b_ptr[j] + so + 8192u * s);
#pragma unroll
            for (int i = 0; i < FM; ++i) f.a[s][i] = read_a_operand(a_ptr[s] + so + 2048u * i);
        }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    auto compute = [&](const Frags& f) {
#pragma unroll
        for (int s = 0; s < KSUB; ++s)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.b[s][j], f.a[s][i], acc[i][j], 0, 0, 0);
    };

    const uint32_t KT = (uint32_t)(K / BK);  // >= 1, whole strips only
    Frags f;

    // Wait for this wave's copy of strip k+1, letting the copies of strips
    // k+2 and k+3 (where they exist) stay in flight.
    auto wait_strip_after = [&](uint32_t k) {
        const uint32_t later = (k + 2 < KT) + (k + 3 < KT);
        if (later == 2) wait_vmcnt<4 * COPIES>();
        else if (later == 1) wait_vmcnt<2 * COPIES>();
        else wait_vmcnt<0>();
    };

    // Prologue.  Each memory phase M(j) reads strip j and copies strip j+3, so
    // group 0 (first M is M(1)) starts by copying strips 0..3 and group 1
    // (first M is M(0)) strips 0..2.  Then strip 0 has to land everywhere.
    const uint32_t pre = grp == 0 ? 4u : 3u;
    for (uint32_t d = 0; d < pre && d < KT; ++d) issue(d);
    {
        const uint32_t n_issued = pre < KT ? pre : KT;
        if (n_issued == 4) wait_vmcnt<6 * COPIES>();
        else if (n_issued == 3) wait_vmcnt<4 * COPIES>();
        else if (n_issued == 2) wait_vmcnt<2 * COPIES>();
        else wait_vmcnt<0>();
    }
    barrier();
    pin();
    read_frags(f, 0);
    wait_lgkm0();
    if (grp == 1) {
        // M(0) of group 1 (phase 0, while group 0 computes strip 0).
        if (3 < KT) issue(3);
        if (1 < KT) wait_strip_after(0);
        barrier();
    }
    pin();

    // Both groups run the same rounds, group 1 one phase behind group 0:
    //   C(k): 16 MFMAs on strip k | barrier | M(k+1): read strip k+1, copy
    //   strip k+4 | barrier.
    // Group 0's compute phases are the even ones, so it certifies strip k+1
    // after C(k); group 1 does so after M(k+1) (for strip k+2).
    for (uint32_t k = 0; k < KT; ++k) {
        compute(f);
        pin();
        if (grp == 0 && k + 1 < KT) wait_strip_after(k);
        barrier();
        pin();
        if (k + 1 < KT) {
            read_frags(f, (k + 1) % STAGES);
            if (k + 4 < KT) issue(k + 4);
        }
        wait_lgkm0();
        if (grp == 1 && k + 2 < KT) wait_strip_after(k + 1);
        barrier();
        pin();
    }
    if (grp == 0) barrier();  // group 1 passed one more barrier in its prologue

    // Epilogue: block (i, j) holds C^T; lane l, register r is C[m][n] with
    // m = 32i + l%32, n = 32j + 8(r/4) + 4(l/32) + r%4.
    const uint32_t frag_row = lane & 31u;
    const uint32_t frag_half = lane >> 5;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int64_t m = m0 + grp * WAVE_TM + 32 * i + frag_row;
        uint16_t* crow = C + m * ldc;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t n = n0 + wq * WAVE_TN + 32 * j + 8 * q + 4 * frag_half;
                u32x2 p;
                p[0] = relu_pack2(acc[i][j][4 * q + 0], acc[i][j][4 * q + 1]);
                p[1] = relu_pack2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
                *reinterpret_cast<u32x2*>(crow + n) = p;
            }
        }
    }
    (void)M;
    (void)N;
}

#undef GR_LDS

}  // namespace pp
}  // namespace gr
