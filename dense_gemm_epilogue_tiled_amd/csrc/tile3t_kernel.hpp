// Pipelined MFMA tile kernel for B given transposed (Bt, N x K row-major) and
// K a multiple of 64 (16-byte aligned rows of A and Bt; EDGE=true for M >= 256
// and N that do not fill whole tiles).
//
// With both operands k-contiguous, both can move in 64-deep strips whose row
// segments are whole 128-byte cache lines (the 256 x 256 tile kernel with B
// row-major can do this for A only).  A strip is [256 rows][64 k], 32 KiB, in
// the layout of the 64-deep A strips of that kernel (128-byte rows, chunk
// index XOR (row/2)%8), for A and for Bt alike.
//
// The strips form one sequence A0, Bt0, A1, Bt1, ... (strip t: A strip t/2 or
// Bt strip t/2) in a ring of 5 slots of 32 KiB (160 KiB): strip t lives in slot
// t % 5.  Step kt (32 MFMAs per wave) uses half kt%2 of the pair of strips
// 2(kt/2), 2(kt/2)+1; the fragments for step kt+1 are read while step kt runs.
// Step s copies strip s+4 (8 copies per wave), which overwrites strip s-1.
//
// Only odd steps 2p-1, whose reads start on pair p, wait for copies and meet
// at a barrier; the reads of an even step 2p use the pair made visible one
// step before.  Before that barrier every wave waits for its own fragment
// reads as well (lgkmcnt 0; the last one was issued 8 MFMAs before).  After
// the barrier of step 2p-1 every read of pair p-1 (issued in steps 2p-3 and
// 2p-2) has completed in every wave, so the copies of steps 2p-1 and 2p
// (strips 2p+3 and 2p+4, over strips 2p-2 and 2p-1 of pair p-1) may start.
// Pair p+1 must have landed by the wait of step 2p+1: its A strip was copied
// three steps before, its Bt strip two, and the wait lets the previous step's
// 8 copies stay in flight.
//
// Each wave owns 128 x 128 of C as 8 x 8 blocks of 16 x 16
// (v_mfma_f32_16x16x32, 64 per step, each taking all 32 k of the step; with
// the same reads and copies this measured 5-8% faster than 16 blocks of
// 32 x 32 with two v_mfma_f32_32x32x16 per step).  Fragments: ds_read_b128
// of 8 consecutive k of one row, 16 rows per read.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "tile2_kernel.hpp"
#include "tile3_kernel.hpp"

namespace gr {

namespace tile3t {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 32;      // K per step
constexpr int BKS = 64;     // K per strip
constexpr int SLOTS = 5;
constexpr int THREADS = 256;
constexpr int WAVE_TM = 128;
constexpr int WAVE_TN = 128;
constexpr int FM = WAVE_TM / 16;  // 16-row blocks of A per wave
constexpr int FN = WAVE_TN / 16;  // 16-row blocks of Bt per wave
constexpr int SLOT_BYTES = BM * BKS * 2;   // 32 KiB (BM == BN)
constexpr int LDS_BYTES = SLOTS * SLOT_BYTES;  // 160 KiB

#define GR_LDS __attribute__((address_space(3)))

static_assert(BM == BN, "A and Bt strips share one slot size");
static_assert(LDS_BYTES >= 4 * epi::REGION_BYTES, "the epilogue stages four wave tiles in LDS");

__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Operands of one 32-deep step.
struct Frags {
    f16x8 a[FM];
    f16x8 b[FN];
};

// E: element type (ElemF16 or ElemBF16) or Epi<...> for bias + activation.
template <bool EDGE, typename E = ElemF16>
__global__ __launch_bounds__(THREADS, 1) void gemm_relu_tile3t_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ Bt, uint16_t* __restrict__ C, int64_t M, int64_t N,
    int64_t K, int64_t lda, int64_t ldb, int64_t ldc, uint32_t tiles_m, uint32_t tiles_n, uint32_t group_m,
    int vec_c, EpiArgs ep) {
    using tile2::barrier;
    using tile2::dma16;
    using tile2::pin;
    using tile2::read_a_operand;
    using tile2::wait_vmcnt;
    using tile3::a64_off;

    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t wm = wave >> 1;
    const uint32_t wn = wave & 1u;

    uint32_t tm, tn;
    tile_of_workgroup(blockIdx.x, gridDim.x, tiles_m, tiles_n, group_m, tm, tn);
    const int64_t m_tile = (int64_t)tm * BM;
    const int64_t m0 = EDGE ? edge::shifted_row0(m_tile, M, BM) : m_tile;
    const int64_t n0 = (int64_t)tn * BN;

    // ---- copies -------------------------------------------------------------
    // A strip = 32 blocks of 8 rows x 128 bytes; this wave fills blocks
    // 8w .. 8w+7 (rows 64w .. 64w+63).  lane -> row lane/8, slot lane%8 (chunk
    // slot XOR (row/2)%8).  Copies 4..7 are copies 0..3 moved down 32 rows,
    // which leaves the XOR term unchanged: for A that is a wave-uniform base
    // offset; rows of Bt past N are clamped to row N-1, so Bt keeps 8 offsets.
    const uint8_t* base_a = reinterpret_cast<const uint8_t*>(A + m0 * lda);
    const uint8_t* base_b = reinterpret_cast<const uint8_t*>(Bt + n0 * ldb);
    constexpr int64_t step_k = BKS * 2;  // bytes per strip along a row
    uint32_t off_a[4], off_b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t r = 64u * wave + 8u * (uint32_t)i + (lane >> 3);
        const uint32_t c = (lane & 7u) ^ ((r >> 1) & 7u);
        if (i < 4) off_a[i] = (uint32_t)((r * lda + 8u * c) * 2);
        uint32_t rn = r;
        if constexpr (EDGE) rn = n0 + r < N ? r : (uint32_t)(N - 1 - n0);
        off_b[i] = (uint32_t)((rn * ldb + 8u * c) * 2);
    }
    const int64_t half_a = 32 * lda * 2;
    const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(GR_LDS uint8_t*)lds);

    const uint32_t KT = (uint32_t)(K / BK);  // even, >= 2
    const uint32_t NS = KT;                  // strips: 2 per 64 k

    // Copy c (0..7) of strip t.
    auto dma_strip = [&](uint32_t t, int c) {
        const uint32_t j = t >> 1;
        const uint32_t dst = lds_base + (t % SLOTS) * SLOT_BYTES + (8u * wave + (uint32_t)c) * 1024u;
        if (t & 1u) dma16(base_b + (int64_t)j * step_k, off_b[c], dst);
        else dma16(base_a + (int64_t)j * step_k + (c >= 4 ? half_a : 0), off_a[c & 3], dst);
    };
    auto copy_strip = [&](uint32_t t) {
        if (t < NS) {
#pragma unroll
            for (int c = 0; c < 8; ++c) dma_strip(t, c);
        }
    };

    // ---- fragment addresses --------------------------------------------------
    // Operand for half h, block i: row 128*wm (A) or 128*wn (Bt) + 16i +
    // lane%16, chunk 4h + lane/16 (the 16-row block moves the row swizzle
    // term (row/2)%8 by a multiple of 8: none).  Block i is +2 KiB, and half 1
    // is half 0 XOR 64 (chunks of half 0 are below 4; slot offsets are
    // multiples of 1 KiB).
    const GR_LDS uint8_t* lds_p = (const GR_LDS uint8_t*)lds;
    const uint32_t a_addr = (uint32_t)(uintptr_t)(lds_p + a64_off(wm * WAVE_TM + (lane & 15u), lane >> 4));
    const uint32_t b_addr = (uint32_t)(uintptr_t)(lds_p + a64_off(wn * WAVE_TN + (lane & 15u), lane >> 4));

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{};

    // Read r (0..15) of the fragments of a step using half H of the pair in
    // slots at byte offsets ao (A) and bo (Bt), in the order the MFMAs consume
    // them: A0, B0 .. B7, A1 .. A7.
    auto read_one = [&](auto h_c, Frags& f, uint32_t ao, uint32_t bo, int r) {
        constexpr uint32_t H = decltype(h_c)::value;
        if (r == 0 || r > FN) {
            const int i = r == 0 ? 0 : r - FN;
            const uint32_t addr = ((a_addr + ao) ^ (64u * H)) + 2048u * i;
            f.a[i] = read_a_operand((const GR_LDS uint8_t*)(uintptr_t)addr);
        } else {
            const int j = r - 1;
            const uint32_t addr = ((b_addr + bo) ^ (64u * H)) + 2048u * j;
            f.b[j] = read_a_operand((const GR_LDS uint8_t*)(uintptr_t)addr);
        }
    };
    auto a_slot = [&](uint32_t kt) { return ((kt & ~1u) % SLOTS) * SLOT_BYTES; };
    auto b_slot = [&](uint32_t kt) { return ((kt | 1u) % SLOTS) * SLOT_BYTES; };
    using H0 = std::integral_constant<uint32_t, 0>;
    using H1 = std::integral_constant<uint32_t, 1>;

    // MFMA t (0..63) of a step: block row t/8, block column t%8.
    auto mfma_one = [&](const Frags& f, int t) {
        const int i = t >> 3, j = t & 7;
        acc[i][j] = E::mfma16(f.b[j], f.a[i], acc[i][j]);
    };

    // Prologue: strips 0 .. 3 (A0, Bt0, A1, Bt1); wait for the first pair.
    copy_strip(0);
    copy_strip(1);
    copy_strip(2);
    copy_strip(3);
    if (NS >= 4) wait_vmcnt<16>();
    else wait_vmcnt<0>();
    barrier();

    Frags f0, f1;
#pragma unroll
    for (int r = 0; r < 16; ++r) read_one(H0{}, f0, a_slot(0), b_slot(0), r);

    // Steady step: strip kt+4 exists and strips up to kt+3 were issued before
    // it.  8 MFMAs, the waits and the barrier (odd kt only), then one memory
    // operation after every second of the next 48 MFMAs (a copy after every
    // third of those).
    // NH = half used by step kt+1 (kt odd: NH = 0, the next pair's strips
    // were copied by step kt-2 at the latest and step kt-1's 8 copies may
    // remain; kt even: NH = 1, no wait).
    auto step = [&](auto nh_c, uint32_t kt, Frags& cur, Frags& nxt) {
        constexpr uint32_t NH = decltype(nh_c)::value;
#pragma unroll
        for (int t = 0; t < 8; ++t) mfma_one(cur, t);
        pin();
        if constexpr (NH == 0) {
            wait_vmcnt<8>();
            wait_lgkm0();
            barrier();
        }
        pin();
        const uint32_t ao = a_slot(kt + 1), bo = b_slot(kt + 1);
        const uint32_t t_copy = kt + 4;
        int rd = 0, cp = 0;
#pragma unroll
        for (int t = 8; t < 64; ++t) {
            mfma_one(cur, t);
            pin();
            const int k = t - 8;
            if (k < 48 && (k & 1) == 0) {
                if ((k >> 1) % 3 == 1) {
                    dma_strip(t_copy, cp);
                    ++cp;
                } else {
                    read_one(nh_c, nxt, ao, bo, rd);
                    ++rd;
                }
            }
            pin();
        }
    };

    // Generic step with its decisions taken at run time (first step and the
    // last few): for odd kt, before the reads for step kt+1, every strip up to
    // that step's pair (2p+1, p = (kt+1)/2) must have landed; issued so far
    // are the strips up to min(kt+3, NS-1).  Even kt: no wait (step 0 reads
    // pair 0, which the prologue waited for).
    auto step_any = [&](uint32_t kt, Frags& cur, Frags& nxt) {
        if (kt >= KT) return;
        const bool more = kt + 1 < KT;
#pragma unroll
        for (int t = 0; t < 8; ++t) mfma_one(cur, t);
        pin();
        if (more && (kt & 1u)) {
            const uint32_t need = 2u * ((kt + 1) >> 1) + 1u;
            const uint32_t issued = kt + 3 < NS - 1 ? kt + 3 : NS - 1;
            const uint32_t allowed = issued > need ? 8u * (issued - need) : 0u;
            if (allowed >= 16) wait_vmcnt<16>();
            else if (allowed == 8) wait_vmcnt<8>();
            else wait_vmcnt<0>();
            wait_lgkm0();
            barrier();
        }
        pin();
        copy_strip(kt + 4);
        pin();
        if (more) {
            const uint32_t ao = a_slot(kt + 1), bo = b_slot(kt + 1);
            if ((kt + 1) & 1u) {
#pragma unroll
                for (int r = 0; r < 16; ++r) read_one(H1{}, nxt, ao, bo, r);
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) read_one(H0{}, nxt, ao, bo, r);
            }
        }
        pin();
#pragma unroll
        for (int t = 8; t < 64; ++t) mfma_one(cur, t);
        pin();
    };

    // Step 0 generic; steady steps 1 .. KT-5 in (odd, even) pairs; then up to
    // five generic steps.
    step_any(0, f0, f1);
    uint32_t kt = 1;
    const uint32_t last_steady = KT > 5 ? KT - 5 : 0;
    for (; kt + 1 <= last_steady; kt += 2) {
        step(H0{}, kt, f1, f0);
        step(H1{}, kt + 1, f0, f1);
    }
    step_any(kt, f1, f0);
    step_any(kt + 1, f0, f1);
    step_any(kt + 2, f1, f0);
    step_any(kt + 3, f0, f1);
    step_any(kt + 4, f1, f0);
    step_any(kt + 5, f0, f1);

    // Epilogue: activation, rounding and the store of C, staged through LDS.
    // Whole tiles with 16-byte rows of C (the fp16/bf16 ReLU): after one
    // barrier (no copy is in flight any more, so all of LDS is free) each
    // wave stores its tile 32 rows at a time through 8 KiB of its own, with
    // no further barrier.  Otherwise the whole wave tile is staged; the lane
    // index is then marked as redefined so the epilogue's lane addresses are
    // computed here, not kept from before the main loop (a spilled register
    // otherwise).
    if constexpr (!EDGE && !E::kGeneral) {
        if (vec_c == 8) {
            barrier();
            epi::store_wave_tile_rows32<E>(acc, lds + wave * epi::ROWS32_BYTES, C, ldc, m0 + wm * WAVE_TM,
                                           n0 + wn * WAVE_TN);
            return;
        }
    }
    uint32_t elane = lane;
    asm volatile("" : "+v"(elane));
    epi::store_wave_tile<EDGE, E>(acc, lds + wave * epi::REGION_BYTES, elane, C, ldc, m0 + wm * WAVE_TM,
                                  n0 + wn * WAVE_TN, m_tile, M, N, vec_c, ep);
}

#undef GR_LDS

}  // namespace tile3t
}  // namespace gr
