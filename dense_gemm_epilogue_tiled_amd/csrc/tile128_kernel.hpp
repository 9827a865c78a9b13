// Pipelined MFMA tile kernel with 128 x 128 tiles, for problems too small to
// fill the chip with 256 x 256 tiles (fewer than half a wave of them: e.g.
// 1024^3 has 16 large tiles for 256 CUs, 2048^3 has 64).
//
// Same output-stationary tiling and fused epilogue as the large-tile kernels
// (TileLang tutorial, chapter "GEMM walkthrough and parameter derivation";
// software pipelining as in its chapter "Software pipelining"), sized down:
//   * 128 x 128 tile, 4 waves (2 x 2) of 64 x 64, v_mfma_f32_32x32x16_f16
//     (2 x 2 blocks, 64 fp32 accumulators per lane), B as first operand.
//   * A strip [128 m][32 k] (64-byte rows, chunk XOR (m/4)%4) and B strip
//     [32 k][128 n] (256-byte rows, chunk XOR 4*(k%4)) per step, 16 KiB,
//     copied with global_load_lds_dwordx4 into a 4-slot ring three strips
//     ahead (64 KiB), so two workgroups share a CU: one computes while the
//     other waits on LDS or a barrier.
//   * Per step: wait for this wave's copies of the strip, barrier (all copies
//     landed, every wave done with the slot about to be refilled), issue the
//     copies of strip kt+3, read the strip's fragments (ds_read_b128 for A,
//     ds_read_b64_tr_b16 for B), 8 MFMAs.
//   * Edges (EDGE=true): a copy of a row past M reads row M-1 instead (the
//     per-lane copy offsets are clamped once), so any M >= 1 works; B copies
//     past N read the last chunk (edge:: in common.hpp); the rows and columns
//     they feed are never stored, and the LDS-staged store of C is guarded.
//   * SPLIT=true (split-K, with a workspace): workgroup g covers tile
//     g % tiles of the K range of split g / tiles, and writes its fp32 sums
//     for the outputs it owns to part[split][m][n]; a second pass
//     (smallm::gemm_relu_smallm_reduce_kernel) adds the splits in order and
//     applies ReLU, so ReLU still sees the complete sum.
// Rows of A and B must be 16-byte aligned and K a positive multiple of 32.
#pragma once

#include "common.hpp"
#include "tile2_kernel.hpp"

namespace gr {

namespace tile128 {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 32;
constexpr int STAGES = 4;
constexpr int THREADS = 256;
constexpr int WAVE_TM = 64;
constexpr int WAVE_TN = 64;
constexpr int FM = WAVE_TM / 32;
constexpr int FN = WAVE_TN / 32;
constexpr int KSUB = BK / 16;
constexpr int A_BYTES = BM * BK * 2;  // 8 KiB
constexpr int B_BYTES = BK * BN * 2;  // 8 KiB
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
constexpr int LDS_BYTES = STAGES * STAGE_BYTES;  // 64 KiB
constexpr int COPIES = A_BYTES / (THREADS * 16);  // 16-byte copies per thread per operand: 2
static_assert(LDS_BYTES >= 4 * (int)epi::WaveTile<FM, FN>::REGION_BYTES, "epilogue staging fits");
constexpr int64_t MAX_LDA = (int64_t(1) << 31) / (BM * 2);
constexpr int64_t MAX_LDB = (int64_t(1) << 31) / (BK * 2);

#define GR_LDS __attribute__((address_space(3)))

__device__ __forceinline__ uint32_t a_off(uint32_t m, uint32_t c) { return m * 64u + ((c ^ ((m >> 2) & 3u)) << 4); }
__device__ __forceinline__ uint32_t b_off(uint32_t k, uint32_t c) { return k * 256u + ((c ^ ((k & 3u) << 2)) << 4); }

// B operand (8 consecutive k of one column per lane) from two transposing
// reads 4 rows apart.
__device__ __forceinline__ f16x8 read_b_operand(const GR_LDS uint8_t* p) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GR_LDS s16x4*)p);
    s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GR_LDS s16x4*)(p + 4 * 256));
    return __builtin_bit_cast(f16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// BT=true: B given transposed (Bt, N x K row-major, pitch ldb), staged and
// read like A (rows of Bt past N clamped to row N-1).
// E: element type (ElemF16 or ElemBF16; only the MFMA and the rounding differ).
template <bool EDGE, bool SPLIT, bool BT = false, typename E = ElemF16>
__global__ __launch_bounds__(THREADS, 2) void gemm_relu_tile128_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, uint16_t* __restrict__ C, int64_t M, int64_t N,
    int64_t K, int64_t lda, int64_t ldb, int64_t ldc, uint32_t tiles_m, uint32_t tiles_n, uint32_t group_m,
    int vec_c, float* __restrict__ part, int64_t k_per_split, EpiArgs ep) {
    using tile2::barrier;
    using tile2::dma16;
    using tile2::read_a_operand;
    using tile2::wait_vmcnt;

    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t wm = wave >> 1;
    const uint32_t wn = wave & 1u;

    const uint32_t tiles = tiles_m * tiles_n;
    const uint32_t wg = SPLIT ? blockIdx.x % tiles : blockIdx.x;
    const int64_t split = SPLIT ? blockIdx.x / tiles : 0;
    uint32_t tm, tn;
    tile_of_workgroup(wg, SPLIT ? tiles : gridDim.x, tiles_m, tiles_n, group_m, tm, tn);
    const int64_t m0 = (int64_t)tm * BM;
    const int64_t n0 = (int64_t)tn * BN;
    // K range of this workgroup (all of K unless split).
    const int64_t k_begin = SPLIT ? split * k_per_split : 0;
    const int64_t k_rest = K - k_begin > 0 ? K - k_begin : 0;
    const int64_t k_len = SPLIT ? (k_rest < k_per_split ? k_rest : k_per_split) : K;

    // ---- copies: copy i of this wave fills LDS block 2*wave + i of a slot ---
    // A block = 16 rows x 64 bytes; lane -> row lane/4, slot lane%4.
    // B block = 4 rows x 256 bytes; lane -> row lane/16, slot lane%16.
    const uint8_t* base_a = reinterpret_cast<const uint8_t*>(A + m0 * lda + k_begin);
    const uint8_t* base_b = reinterpret_cast<const uint8_t*>(BT ? B + n0 * ldb + k_begin : B + k_begin * ldb + n0);
    const int64_t step_a = BK * 2;
    const int64_t step_b = BT ? (int64_t)BK * 2 : (int64_t)BK * ldb * 2;
    uint32_t off_a[COPIES], off_b[COPIES];
#pragma unroll
    for (int i = 0; i < COPIES; ++i) {
        const uint32_t blk = 2u * wave + (uint32_t)i;
        const uint32_t ra = 16u * blk + (lane >> 2);
        const uint32_t ca = (lane & 3u) ^ ((ra >> 2) & 3u);
        uint32_t ra_src = ra;  // row of A this lane copies into LDS row ra
        if constexpr (EDGE) ra_src = m0 + ra < M ? ra : (uint32_t)(M - 1 - m0);
        off_a[i] = (uint32_t)((ra_src * lda + 8u * ca) * 2);
        if constexpr (BT) {
            uint32_t rb_src = ra;  // row n0 + ra of Bt, clamped to N-1
            if constexpr (EDGE) rb_src = n0 + ra < N ? ra : (uint32_t)(N - 1 - n0);
            off_b[i] = (uint32_t)((rb_src * ldb + 8u * ca) * 2);
        } else {
            const uint32_t rb = 4u * blk + (lane >> 4);
            uint32_t cb = (lane & 15u) ^ ((rb & 3u) << 2);
            if constexpr (EDGE) cb = edge::clamp_chunk(cb, n0, N);
            off_b[i] = (uint32_t)((rb * ldb + 8u * cb) * 2);
        }
    }
    const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(GR_LDS uint8_t*)lds);
    auto issue = [&](uint32_t kt) {
        const uint32_t slot = kt % STAGES;
#pragma unroll
        for (int i = 0; i < COPIES; ++i) {
            const uint32_t blk = 2u * wave + (uint32_t)i;
            dma16(base_a + (int64_t)kt * step_a, off_a[i], lds_base + slot * STAGE_BYTES + blk * 1024u);
            dma16(base_b + (int64_t)kt * step_b, off_b[i], lds_base + slot * STAGE_BYTES + A_BYTES + blk * 1024u);
        }
    };

    // ---- fragment addresses --------------------------------------------------
    // A operand of MFMA step s, block i: row wm*64 + 32i + lane%32, chunk
    // 2s + lane/32 (block i is 2 KiB further on).  B operand of step s,
    // block j: rows 16s + 8(lane/32) + (lane%16)/4 (+4 for the second read),
    // column wn*64 + 32j + 16((lane/16)%2) + 4(lane%4).
    const GR_LDS uint8_t* lds_p = (const GR_LDS uint8_t*)lds;
    const uint32_t ar = wm * WAVE_TM + (lane & 31u);
    const GR_LDS uint8_t* a_ptr[KSUB];
#pragma unroll
    for (int s = 0; s < KSUB; ++s) a_ptr[s] = lds_p + a_off(ar, 2u * s + (lane >> 5));
    const uint32_t bk = 8u * (lane >> 5) + ((lane & 15u) >> 2);
    const GR_LDS uint8_t* b_ptr[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const uint32_t n = wn * WAVE_TN + 32u * j + 16u * ((lane >> 4) & 1u) + 4u * (lane & 3u);
        b_ptr[j] = lds_p + A_BYTES + b_off(bk, n >> 3) + 2u * (n & 7u);
    }
    // BT: B operand of step s, block j: row wn*64 + 32j + lane%32 of the Bt
    // strip, chunk 2s + lane/32 (A's layout; block j is 2 KiB further on).
    const uint32_t br = wn * WAVE_TN + (lane & 31u);
    const GR_LDS uint8_t* bt_ptr[KSUB];
#pragma unroll
    for (int s = 0; s < KSUB; ++s) bt_ptr[s] = lds_p + A_BYTES + a_off(br, 2u * s + (lane >> 5));

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    const uint32_t KT = (uint32_t)(k_len / BK);  // whole strips only (>= 1 unless an empty split)
    if (KT > 0) issue(0);
    if (KT > 1) issue(1);
    if (KT > 2) issue(2);

    for (uint32_t kt = 0; kt < KT; ++kt) {
        // Strip kt must have landed; strips kt+1 and kt+2 may stay in flight.
        const uint32_t ahead = (KT - 1 - kt) < 2u ? (KT - 1 - kt) : 2u;
        if (ahead == 2) wait_vmcnt<4 * COPIES>();
        else if (ahead == 1) wait_vmcnt<2 * COPIES>();
        else wait_vmcnt<0>();
        barrier();
        if (kt + 3 < KT) issue(kt + 3);
        const uint32_t so = (kt % STAGES) * STAGE_BYTES;
        f16x8 fa[KSUB][FM], fb[KSUB][FN];
#pragma unroll
        for (int s = 0; s < KSUB; ++s) {
#pragma unroll
            for (int i = 0; i < FM; ++i) fa[s][i] = read_a_operand(a_ptr[s] + so + 2048u * i);
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                if constexpr (BT) fb[s][j] = read_a_operand(bt_ptr[s] + so + 2048u * j);
                else fb[s][j] = read_b_operand(b_ptr[j] + so + 16u * 256u * s);
            }
        }
#pragma unroll
        for (int s = 0; s < KSUB; ++s)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = E::mfma32(fb[s][j], fa[s][i], acc[i][j]);
    }

    if constexpr (SPLIT) {
        epi::store_partials<EDGE>(acc, part + split * M * N, lane, m0 + wm * WAVE_TM, n0 + wn * WAVE_TN, M, N);
        (void)C;
        (void)ldc;
        (void)vec_c;
    } else {
        // Epilogue: ReLU, fp16 and the store of C, staged through LDS.
        epi::store_wave_tile<EDGE, E>(acc, lds + wave * epi::WaveTile<FM, FN>::REGION_BYTES, lane, C, ldc,
                                   m0 + wm * WAVE_TM, n0 + wn * WAVE_TN, m0, M, N, vec_c, ep);
        (void)part;
    }
}

#undef GR_LDS

}  // namespace tile128
}  // namespace gr
