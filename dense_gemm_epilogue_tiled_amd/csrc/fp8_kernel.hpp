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
// gemm_fp8_tile_kernel<BMT>: the 32-deep pipelined kernel's scheme for a
// given-transposed B (tile2_kernel.hpp) with one 64-byte fp8 strip in place
// of one 32-deep fp16 strip -- a strip row is 64 bytes either way, so the
// 4-slot ring, the direct-to-LDS copies, the swizzle and the fragment reads
// are the same; 256 x 256 tiles (16 MFMAs per strip per wave) or, when those
// would leave CUs idle, 128 x 128 tiles with two workgroups per CU.  Rows of
// A and Bt past M and N read row M-1 and N-1 (their results are never
// stored), so any M and N work; K must be a multiple of 64 and rows 16-byte
// aligned.
// gemm_fp8_smallm_kernel: M <= 16, a bandwidth-bound stream over Bt.
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

constexpr int BK = 64;  // k per strip (bytes)
constexpr int STAGES = 4;
constexpr int THREADS = 256;
// Largest row pitch (bytes) for which the per-lane copy offsets of a 256-row
// tile fit in 32 bits.
constexpr int64_t MAX_LD = (int64_t(1) << 31) / 256;

#define GR_LDS __attribute__((address_space(3)))

// Geometry of the pipelined kernel for BMT x BMT tiles (256 or 128): 2 x 2
// waves of BMT/2 x BMT/2, FM x FN blocks of 32 x 32 per wave.
template <int BMT>
struct Tile {
    static constexpr int BM = BMT;
    static constexpr int BN = BMT;
    static constexpr int WAVE_T = BMT / 2;
    static constexpr int FM = WAVE_T / 32;
    static constexpr int FN = WAVE_T / 32;
    static constexpr int A_BYTES = BM * BK;  // 16 or 8 KiB
    static constexpr int B_BYTES = BN * BK;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;     // 128 or 64 KiB
    static constexpr int COPIES = A_BYTES / (THREADS * 16);   // 16-byte copies per thread per operand
    static constexpr int REGION = epi::WaveTile<FM, FN>::REGION_BYTES;
    static constexpr int MIN_WAVES = BMT == 256 ? 1 : 2;       // workgroups per CU
    static_assert(LDS_BYTES >= 4 * REGION, "the epilogue stages four wave tiles in LDS");
};

__device__ __forceinline__ u32x4 read16(const GR_LDS uint8_t* p) { return *(const GR_LDS u32x4*)p; }

// E: output element type with the general epilogue (Epi<ElemF16> or
// Epi<ElemBF16>); ep.scale carries scale_a * scale_b.
// SPLIT=true (split-K, with a workspace): workgroup g covers tile g % tiles
// over the K range of split g / tiles (k_per_split bytes, a multiple of 64;
// no split is empty) and writes its unscaled fp32 sums to part[split][m][n];
// a second pass adds the splits in order and applies the epilogue.
template <int BMT, bool EDGE, typename E, bool SPLIT = false>
__global__ __launch_bounds__(THREADS, Tile<BMT>::MIN_WAVES) void gemm_fp8_tile_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ Bt, uint16_t* __restrict__ C, int64_t M, int64_t N,
    int64_t K, int64_t lda, int64_t ldb, int64_t ldc, uint32_t tiles_m, uint32_t tiles_n, uint32_t group_m,
    int vec_c, float* __restrict__ part, int64_t k_per_split, EpiArgs ep) {
    static_assert(E::kGeneral, "the fp8 kernels use the general epilogue");
    using T = Tile<BMT>;
    constexpr int FM = T::FM, FN = T::FN, COPIES = T::COPIES;
    using tile2::a_off;
    using tile2::barrier;
    using tile2::dma16;
    using tile2::pin;
    using tile2::wait_vmcnt;

    __shared__ __attribute__((aligned(1024))) uint8_t lds[T::LDS_BYTES];

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
    const int64_t m0 = (int64_t)tm * T::BM;
    const int64_t n0 = (int64_t)tn * T::BN;
    // K range of this workgroup (all of K unless split).
    const int64_t k_begin = SPLIT ? split * k_per_split : 0;
    const int64_t k_rest = K - k_begin > 0 ? K - k_begin : 0;
    const int64_t k_len = SPLIT ? (k_rest < k_per_split ? k_rest : k_per_split) : K;

    // ---- copies: copy i of this wave fills LDS block COPIES*wave + i of a
    // slot; block = 16 rows x 64 bytes; lane -> row lane/4, slot lane%4 (chunk
    // slot XOR (row/4)%4).  Rows past M (N) read row M-1 (N-1).
    const uint8_t* base_a = A + m0 * lda + k_begin;
    const uint8_t* base_b = Bt + n0 * ldb + k_begin;
    uint32_t off_a[COPIES], off_b[COPIES];
#pragma unroll
    for (int i = 0; i < COPIES; ++i) {
        const uint32_t blk = (uint32_t)COPIES * wave + (uint32_t)i;
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

    // Copy c (0 .. 2*COPIES-1) of strip `kt` into `slot`: c even -> A copy
    // c/2, odd -> B.
    auto dma_one = [&](uint32_t slot, uint32_t kt, int c) {
        const int i = c >> 1;
        const uint32_t blk = (uint32_t)COPIES * wave + (uint32_t)i;
        if ((c & 1) == 0)
            dma16(base_a + (int64_t)kt * BK, off_a[i], lds_base + slot * T::STAGE_BYTES + blk * 1024u);
        else
            dma16(base_b + (int64_t)kt * BK, off_b[i],
                  lds_base + slot * T::STAGE_BYTES + T::A_BYTES + blk * 1024u);
    };
    auto issue = [&](uint32_t slot, uint32_t kt) {
#pragma unroll
        for (int c = 0; c < 2 * COPIES; ++c) dma_one(slot, kt, c);
    };

    // ---- fragment addresses: row wm*WAVE_T + 32i + lane%32 (A) or
    // wn*WAVE_T + 32j + lane%32 (Bt), chunk 2s + lane/32; block i or j is 2 KiB on.
    const GR_LDS uint8_t* lds_p = (const GR_LDS uint8_t*)lds;
    const uint32_t ar = wm * T::WAVE_T + (lane & 31u);
    const uint32_t br = wn * T::WAVE_T + (lane & 31u);
    const GR_LDS uint8_t* a_ptr[2];
    const GR_LDS uint8_t* b_ptr[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        a_ptr[s] = lds_p + a_off(ar, 2u * s + (lane >> 5));
        b_ptr[s] = lds_p + T::A_BYTES + a_off(br, 2u * s + (lane >> 5));
    }

    struct Frags {
        u32x4 a[2][FM];
        u32x4 b[2][FN];
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    // The 2 (FM + FN) fragment reads of one strip, in the order the next
    // step's MFMAs (block row i, then column j) first need them: A0, B0 ..,
    // A1 .., each as its two chunks.
    constexpr int READS = 2 * (FM + FN);
    auto read_one = [&](Frags& f, uint32_t slot, int r) {
        const int q = r >> 1, s = r & 1;
        const uint32_t so = slot * T::STAGE_BYTES;
        if (q == 0) f.a[s][0] = read16(a_ptr[s] + so);
        else if (q <= FN) f.b[s][q - 1] = read16(b_ptr[s] + so + 2048u * (q - 1));
        else f.a[s][q - FN] = read16(a_ptr[s] + so + 2048u * (q - FN));
    };
    constexpr int MFMAS = FM * FN;
    auto mfma_one = [&](const Frags& f, int t) {
        const int i = t / FN, j = t % FN;
        acc[i][j] = mfma(f.b[0][j], f.b[1][j], f.a[0][i], f.a[1][i], acc[i][j]);
    };

    const uint32_t KT = (uint32_t)(k_len / BK);  // >= 1, whole strips only

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
    for (int r = 0; r < READS; ++r) read_one(f0, 0, r);

    // Steady step on strip kt (slot SLOT = kt % 4), fragments in `cur`: PRE
    // MFMAs; wait for this wave's copies of strip kt+1; barrier (all copies of
    // kt+1 landed, every wave done with the slot of kt-1); then the other
    // MFMAs with the READS reads of strip kt+1 and the 2*COPIES copies of
    // strip kt+3 (every third operation) spread evenly behind them.
    constexpr int PRE = 2;
    constexpr int OPS = READS + 2 * COPIES;
    constexpr int PER = (OPS + (MFMAS - PRE) - 1) / (MFMAS - PRE);
    auto step = [&](auto slot_c, uint32_t kt, Frags& cur, Frags& nxt) {
        constexpr uint32_t SLOT = decltype(slot_c)::value;
#pragma unroll
        for (int t = 0; t < PRE; ++t) mfma_one(cur, t);
        pin();
        wait_vmcnt<2 * COPIES>();
        barrier();
        pin();
        int rd = 0, cp = 0;
#pragma unroll
        for (int t = PRE; t < MFMAS; ++t) {
            mfma_one(cur, t);
            pin();
#pragma unroll
            for (int u = 0; u < PER; ++u) {
                const int k = PER * (t - PRE) + u;
                if (k < OPS) {
                    if (k % 3 == 1 && cp < 2 * COPIES) {
                        dma_one((SLOT + 3) % STAGES, kt + 3, cp);
                        ++cp;
                    } else if (rd < READS) {
                        read_one(nxt, (SLOT + 1) % STAGES, rd);
                        ++rd;
                    } else {
                        dma_one((SLOT + 3) % STAGES, kt + 3, cp);
                        ++cp;
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
        for (int t = 0; t < PRE; ++t) mfma_one(cur, t);
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
            for (int r = 0; r < READS; ++r) read_one(nxt, (kt + 1) % STAGES, r);
        }
        pin();
#pragma unroll
        for (int t = PRE; t < MFMAS; ++t) mfma_one(cur, t);
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

    if constexpr (SPLIT) {
        epi::store_partials<EDGE>(acc, part + split * M * N, lane, m0 + wm * T::WAVE_T, n0 + wn * T::WAVE_T, M,
                                  N);
        (void)C;
        (void)ldc;
        (void)vec_c;
    } else {
        // Epilogue (scale, bias, activation, rounding), staged through LDS.
        epi::store_wave_tile<EDGE, E>(acc, lds + wave * T::REGION, lane, C, ldc, m0 + wm * T::WAVE_T,
                                      n0 + wn * T::WAVE_T, m0, M, N, vec_c, ep);
        (void)part;
    }
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

// ---- small M (M <= 16): streaming Bt ---------------------------------------------
//
// The fp16 small-M kernel for a given-transposed B (smallm_kernel.hpp), with
// bytes for elements: a workgroup of 4 waves owns 64 columns of C (64 rows of
// Bt); K moves in 512-deep chunks (512 bytes of each row) through a 4-slot
// LDS ring, three chunks ahead; each wave copies its 16 Bt rows and 4 of the
// 16 rows of the A chunk (rows past M read row M-1; their outputs are never
// stored), then runs 4 v_mfma_f32_16x16x128_f8f6f4 per chunk (lane group
// l/16 takes chunks 8s + 2(l/16) and 8s + 2(l/16) + 1 of step s, for both
// operands).  Needs K a multiple of 512 and 16-byte aligned rows.
constexpr int SM_KC = 512;                       // k (bytes) per chunk
constexpr int SM_NB = 64;                        // columns per workgroup
constexpr int SM_MAX_M = 16;
constexpr int SM_BT_BYTES = SM_NB * SM_KC;       // 32 KiB
constexpr int SM_A_BYTES = SM_MAX_M * SM_KC;     // 8 KiB
constexpr int SM_SLOT = SM_BT_BYTES + SM_A_BYTES;
constexpr int SM_SLOTS = 4;
constexpr int SM_COPIES = 10;                    // copies per wave per chunk: 8 (Bt) + 2 (A)
constexpr int64_t SM_MAX_LD = (int64_t(1) << 32) / SM_NB - SM_KC;

__device__ __forceinline__ f32x4 mfma16(const u32x4& b0, const u32x4& b1, const u32x4& a0, const u32x4& a1,
                                        f32x4 c) {
    const i32x8 bo = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
    const i32x8 ao = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bo, ao, c, 0, 0, 0, 0, 0, 0);
}

template <bool GUARD, typename E>
__global__ __launch_bounds__(256, 1) void gemm_fp8_smallm_kernel(const uint8_t* __restrict__ A,
                                                                const uint8_t* __restrict__ Bt,
                                                                uint16_t* __restrict__ C, int64_t M, int64_t N,
                                                                int64_t K, int64_t lda, int64_t ldbt, int64_t ldc,
                                                                EpiArgs ep) {
    static_assert(E::kGeneral, "the fp8 kernels use the general epilogue");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[SM_SLOTS * SM_SLOT];

    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t n_wg = (int64_t)blockIdx.x * SM_NB;

    // Copy i of a chunk: LDS rows 2i, 2i+1 of the Bt block (this wave: rows
    // 16w .. 16w+15) or of the A block (rows 4w .. 4w+3); lane -> row
    // 2i + lane/32, slot lane%32, which holds global chunk slot ^ (row % 16).
    uint32_t off_bt[8], off_a[2];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t row = 16u * wave + 2u * i + (lane >> 5);
        const uint32_t chunk = (lane & 31u) ^ (row & 15u);
        int64_t n = n_wg + row;
        if (GUARD && n >= N) n = N - 1;
        off_bt[i] = (uint32_t)((n - n_wg) * ldbt + chunk * 16);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint32_t row = 4u * wave + 2u * i + (lane >> 5);
        const uint32_t chunk = (lane & 31u) ^ (row & 15u);
        const int64_t m = (int64_t)row < M ? (int64_t)row : M - 1;
        off_a[i] = (uint32_t)(m * lda + chunk * 16);
    }
    const uint8_t* base_bt = Bt + n_wg * ldbt;
    const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(GR_LDS uint8_t*)lds);
    auto issue = [&](int64_t kc) {
        const uint32_t slot = lds_base + (uint32_t)(kc % SM_SLOTS) * SM_SLOT;
        const int64_t kb = kc * SM_KC;
#pragma unroll
        for (int i = 0; i < 8; ++i) tile2::dma16(base_bt + kb, off_bt[i], slot + (16u * wave + 2u * i) * 512u);
#pragma unroll
        for (int i = 0; i < 2; ++i) tile2::dma16(A + kb, off_a[i], slot + SM_BT_BYTES + (4u * wave + 2u * i) * 512u);
    };

    // Fragments of step s: Bt row 16w + l%16 and A row l%16, chunks
    // 8s + 2(l/16) and 8s + 2(l/16) + 1.
    const uint32_t li = lane & 15u, lg = lane >> 4;
    const uint32_t bt_row = 16u * wave + li;
    f32x4 acc0 = f32x4{}, acc1 = f32x4{};

    const int64_t chunks = K / SM_KC;
    for (int64_t c = 0; c < SM_SLOTS - 1 && c < chunks; ++c) issue(c);
    for (int64_t kc = 0; kc < chunks; ++kc) {
        // chunk kc landed; the (up to SM_SLOTS - 2) chunks after it may still be in flight
        const int64_t ahead = chunks - 1 - kc < SM_SLOTS - 2 ? chunks - 1 - kc : SM_SLOTS - 2;
        if (ahead >= 2) tile2::wait_vmcnt<2 * SM_COPIES>();
        else if (ahead == 1) tile2::wait_vmcnt<SM_COPIES>();
        else tile2::wait_vmcnt<0>();
        tile2::barrier();
        if (kc + SM_SLOTS - 1 < chunks) issue(kc + SM_SLOTS - 1);
        const uint8_t* slot = lds + (kc % SM_SLOTS) * SM_SLOT;
#pragma unroll
        for (int st = 0; st < SM_KC / 128; ++st) {
            const uint32_t c0 = 8u * st + 2u * lg;
            const uint8_t* brow = slot + bt_row * 512u;
            const uint8_t* arow = slot + SM_BT_BYTES + li * 512u;
            const u32x4 b0 = *reinterpret_cast<const u32x4*>(brow + ((c0 ^ (bt_row & 15u)) << 4));
            const u32x4 b1 = *reinterpret_cast<const u32x4*>(brow + (((c0 + 1u) ^ (bt_row & 15u)) << 4));
            const u32x4 a0 = *reinterpret_cast<const u32x4*>(arow + ((c0 ^ li) << 4));
            const u32x4 a1 = *reinterpret_cast<const u32x4*>(arow + (((c0 + 1u) ^ li) << 4));
            if (st & 1) acc1 = mfma16(b0, b1, a0, a1, acc1);
            else acc0 = mfma16(b0, b1, a0, a1, acc0);
        }
    }

    // acc holds C^T: lane l, register r is C[m][n] with m = l%16 and
    // n = n_wg + 16w + 4(l/16) + r.
    const int64_t m = li;
    if (m < M) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t n = n_wg + 16 * wave + 4 * lg + r;
            if (!GUARD || n < N) C[m * ldc + n] = epi_value<E>(acc0[r] + acc1[r], n, N, ep);
        }
    }
}

#undef GR_LDS

}  // namespace fp8
}  // namespace gr
