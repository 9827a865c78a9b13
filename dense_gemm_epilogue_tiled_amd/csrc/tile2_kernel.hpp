// Pipelined MFMA tile kernel for whole tiles: C = ReLU(A * B), fp16 in, fp32
// accumulate, fp16 out.  Same output-stationary tiling as the guarded kernel
// (TileLang tutorial, chapter "GEMM walkthrough and parameter derivation"),
// with the K loop software-pipelined over a 4-deep LDS ring (the num_stages
// idea of the chapter "Software pipelining": while the matrix cores work on
// strip k, the copies of strips k+1 .. k+3 are in flight).
//
// gfx950 mechanics:
//   * Copies are direct-to-LDS (global_load_lds_dwordx4): each lane moves 16
//     bytes from HBM/L2 straight into LDS, no VGPR staging and no VALU work.
//     A wave's instruction fills 1 KiB of LDS contiguously, so the LDS
//     swizzle is applied on the global side: every lane fetches the chunk
//     that belongs at its LDS slot.
//   * A tile [256 m][32 k]: 64-byte rows, 16-byte chunk index XOR (m/4)%4.
//     Fragment reads (ds_read_b128, one MFMA operand per lane) touch 16
//     distinct bank groups per quarter-wave.
//   * B tile [32 k][256 n] stays row-major (n contiguous, 512-byte rows),
//     chunk index XOR 4*(k%4).  The MFMA wants 8 consecutive k of one column
//     per lane; ds_read_b64_tr_b16 gives exactly that: each 16-lane group
//     reads a 4 (k) x 16 (n) block as 16 row pieces of 8 bytes, and the
//     hardware hands lane j the 4 k values of column j.  Two such reads make
//     one 8-k operand.  The XOR puts the 4 rows of a block in 4 distinct
//     bank groups.
//   * 256 x 256 tile, 4 waves (2 x 2), 128 x 128 per wave, 256 fp32
//     accumulators per lane in AGPRs, v_mfma_f32_32x32x16_f16 issued with B
//     as the first operand so each lane ends with 4 consecutive columns of a
//     row of C.
//   * Fragments of strip k+1 are read from LDS while the MFMAs of strip k
//     run (two register sets).  One barrier per strip.  The waits on the
//     direct-to-LDS copies (vmcnt) and on the transposing reads (lgkmcnt)
//     are placed by hand: the compiler cannot see which LDS slot an
//     in-flight copy writes and would otherwise wait for all of them.
//   * C is written through LDS once the K loop is done (epi::store_wave_tile).
// Rows of A and B must be 16-byte aligned and K a multiple of 32 (the planner
// checks).  EDGE=true serves M >= 256 and any N that do not fill whole tiles
// (edge:: in common.hpp); the guarded register-staged kernel takes the rest.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace gr {

namespace tile2 {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 32;
constexpr int STAGES = 4;
constexpr int THREADS = 256;
constexpr int WAVE_TM = 128;
constexpr int WAVE_TN = 128;
constexpr int FM = WAVE_TM / 32;
constexpr int FN = WAVE_TN / 32;
constexpr int KSUB = BK / 16;                 // MFMA k-steps per strip
constexpr int A_BYTES = BM * BK * 2;          // 16 KiB
constexpr int B_BYTES = BK * BN * 2;          // 16 KiB
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
constexpr int LDS_BYTES = STAGES * STAGE_BYTES;  // 128 KiB
static_assert(LDS_BYTES >= 4 * epi::REGION_BYTES, "the epilogue stages four wave tiles in LDS");
constexpr int COPIES = A_BYTES / (THREADS * 16);  // 16-byte copies per thread per operand: 4

#define GR_LDS __attribute__((address_space(3)))

// Byte offset of chunk c (8 fp16) of A-tile row m / B-tile row k.
__device__ __forceinline__ uint32_t a_off(uint32_t m, uint32_t c) { return m * 64u + ((c ^ ((m >> 2) & 3u)) << 4); }
__device__ __forceinline__ uint32_t b_off(uint32_t k, uint32_t c) { return k * 512u + ((c ^ ((k & 3u) << 2)) << 4); }

// One 16-byte direct-to-LDS copy per lane: LDS[m0 + 16 * lane] =
// *(base + voff).  Issued through inline assembly so that the compiler does
// not track it: otherwise it would make every later LDS read wait for all
// copies in flight.  The kernel itself waits for them (wait_vmcnt + barrier)
// before reading.  base is wave-uniform (SGPRs), voff a per-lane byte offset.
// The LDS address travels in M0 as an explicit operand, so the compiler
// writes M0 itself and knows the statement reads it; the s_nop covers the
// wait state between an M0 write and an LDS DMA that reads it.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds_addr) {
    asm volatile(
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(voff), "s"(base), "{m0}"(lds_addr)
        : "memory");
}

// The same copy marked nontemporal (a stream read once: the lines are not
// kept in the caches for reuse).
__device__ __forceinline__ void dma16_nt(const void* base, uint32_t voff, uint32_t lds_addr) {
    asm volatile(
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1 nt"
        :
        : "v"(voff), "s"(base), "{m0}"(lds_addr)
        : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Fragments of one strip: A operands (one ds_read_b128 each) and B operands
// (two ds_read_b64_tr_b16 each).  These are ordinary loads: the compiler
// places their lgkmcnt waits.
struct Frags {
    f16x8 a[KSUB][FM];
    f16x8 b[KSUB][FN];
};

__device__ __forceinline__ f16x8 read_b_operand(const GR_LDS uint8_t* p) {
    s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GR_LDS s16x4*)p);
    s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GR_LDS s16x4*)(p + 2048));
    return __builtin_bit_cast(f16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ f16x8 read_a_operand(const GR_LDS uint8_t* p) { return *(const GR_LDS f16x8*)p; }

// Pin the instruction order: nothing is scheduled across this point.
__device__ __forceinline__ void pin() { __builtin_amdgcn_sched_barrier(0); }

// Largest row pitches for which the per-lane copy offsets of one tile fit in
// 32 bits (A: 256 rows of the tile, B: 32 rows of a strip).
constexpr int64_t MAX_LDA = (int64_t(1) << 31) / (BM * 2);
constexpr int64_t MAX_LDB = (int64_t(1) << 31) / (BK * 2);

// BT=true: B is given transposed (Bt, N x K row-major, pitch ldb): its strips
// [256 n][32 k] are staged exactly like A's (64-byte rows, chunk XOR (n/4)%4)
// and its fragments are read like A's (ds_read_b128); rows of Bt past N are
// clamped to row N-1 (their columns are never stored).
// E: element type (ElemF16 or ElemBF16; only the MFMA and the rounding differ).
// AT=true: A is given transposed (At, K x M row-major, pitch lda): its strips
// [32 k][256 m] are staged exactly like B's (512-byte rows, chunk XOR
// 4(k%4)) and its fragments are read like B's (ds_read_b64_tr_b16); with
// EDGE the last tile row moves up to end at row M as usual (M >= 256), so
// every copied column of At is < M.
template <bool EDGE, bool BT = false, typename E = ElemF16, bool AT = false>
__global__ __launch_bounds__(THREADS, 1) void gemm_relu_tile2_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, uint16_t* __restrict__ C, int64_t M, int64_t N,
    int64_t K, int64_t lda, int64_t ldb, int64_t ldc, uint32_t tiles_m, uint32_t tiles_n, uint32_t group_m,
    int vec_c, EpiArgs ep) {
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

    // ---- copies: copy i of this wave fills LDS block 4*wave + i of a slot ---
    // A block = 16 rows x 64 bytes; lane -> row lane/4, slot lane%4.
    // B block = 2 rows x 512 bytes; lane -> row lane/32, slot lane%32.
    // Wave-uniform bases (advanced one strip per step) + per-lane offsets.
    static_assert(!(AT && BT), "one transposed operand at a time");
    const uint8_t* base_a = reinterpret_cast<const uint8_t*>(AT ? A + m0 : A + m0 * lda);
    const uint8_t* base_b = reinterpret_cast<const uint8_t*>(BT ? B + n0 * ldb : B + n0);
    const int64_t step_a = AT ? (int64_t)BK * lda * 2 : BK * 2;
    const int64_t step_b = BT ? (int64_t)BK * 2 : (int64_t)BK * ldb * 2;
    uint32_t off_a[COPIES], off_b[COPIES];
#pragma unroll
    for (int i = 0; i < COPIES; ++i) {
        const uint32_t blk = 4u * wave + (uint32_t)i;
        const uint32_t ra = 16u * blk + (lane >> 2);
        const uint32_t ca = (lane & 3u) ^ ((ra >> 2) & 3u);
        if constexpr (AT) {
            // At strip row k = 2 blk + lane/32, chunk slot lane%32 (the B layout)
            const uint32_t rk = 2u * blk + (lane >> 5);
            const uint32_t cm = (lane & 31u) ^ ((rk & 3u) << 2);
            off_a[i] = (uint32_t)((rk * lda + 8u * cm) * 2);
        } else {
            off_a[i] = (uint32_t)((ra * lda + 8u * ca) * 2);
        }
        if constexpr (BT) {
            uint32_t rb_src = ra;  // row n0 + ra of Bt, clamped to N-1
            if constexpr (EDGE) rb_src = n0 + ra < N ? ra : (uint32_t)(N - 1 - n0);
            off_b[i] = (uint32_t)((rb_src * ldb + 8u * ca) * 2);
        } else {
            const uint32_t rb = 2u * blk + (lane >> 5);
            uint32_t cb = (lane & 31u) ^ ((rb & 3u) << 2);
            if constexpr (EDGE) cb = edge::clamp_chunk(cb, n0, N);
            off_b[i] = (uint32_t)((rb * ldb + 8u * cb) * 2);
        }
    }
    const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(GR_LDS uint8_t*)lds);

    // Copy c (0..7) of strip `kt` into `slot`: c even -> A copy c/2, odd -> B.
    auto dma_one = [&](uint32_t slot, uint32_t kt, int c) {
        const int i = c >> 1;
        const uint32_t blk = 4u * wave + (uint32_t)i;
        if ((c & 1) == 0)
            dma16(base_a + (int64_t)kt * step_a, off_a[i], lds_base + slot * STAGE_BYTES + blk * 1024u);
        else
            dma16(base_b + (int64_t)kt * step_b, off_b[i], lds_base + slot * STAGE_BYTES + A_BYTES + blk * 1024u);
    };
    auto issue = [&](uint32_t slot, uint32_t kt) {
#pragma unroll
        for (int c = 0; c < 2 * COPIES; ++c) dma_one(slot, kt, c);
    };

    // ---- fragment addresses --------------------------------------------------
    // A operand of MFMA step s, block i: row wm*128 + 32i + lane%32, chunk
    // 2s + lane/32 (the XOR term depends on the lane only, so block i is a
    // constant 2 KiB further on).
    const GR_LDS uint8_t* lds_p = (const GR_LDS uint8_t*)lds;
    const uint32_t ar = wm * WAVE_TM + (lane & 31u);
    const GR_LDS uint8_t* a_ptr[KSUB];
#pragma unroll
    for (int s = 0; s < KSUB; ++s) a_ptr[s] = lds_p + a_off(ar, 2u * s + (lane >> 5));
    // AT: A operand of step s, block i, read like a B operand (row 16s +
    // 8(lane/32) + 4h + (lane%16)/4 of the At strip, column wm*128 + 32i +
    // 16((lane/16)%2) + 4(lane%4)).
    const uint32_t ak = 8u * (lane >> 5) + ((lane & 15u) >> 2);
    const GR_LDS uint8_t* at_ptr[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const uint32_t m = wm * WAVE_TM + 32u * i + 16u * ((lane >> 4) & 1u) + 4u * (lane & 3u);
        at_ptr[i] = lds_p + b_off(ak, m >> 3) + 2u * (m & 7u);
    }
    // B operand of step s, block j, half h: row 16s + 8(lane/32) + 4h +
    // (lane%16)/4, column wn*128 + 32j + 16((lane/16)%2) + 4(lane%4); the XOR
    // term depends on j, so each j has its own base; s and h are constant
    // row offsets (8 KiB and 2 KiB).
    const uint32_t bk = 8u * (lane >> 5) + ((lane & 15u) >> 2);
    const GR_LDS uint8_t* b_ptr[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const uint32_t n = wn * WAVE_TN + 32u * j + 16u * ((lane >> 4) & 1u) + 4u * (lane & 3u);
        b_ptr[j] = lds_p + A_BYTES + b_off(bk, n >> 3) + 2u * (n & 7u);
    }
    // BT: B operand of step s, block j is row wn*128 + 32j + lane%32 of the
    // Bt strip, chunk 2s + lane/32 (block j is 2 KiB further on).
    const uint32_t br = wn * WAVE_TN + (lane & 31u);
    const GR_LDS uint8_t* bt_ptr[KSUB];
#pragma unroll
    for (int s = 0; s < KSUB; ++s) bt_ptr[s] = lds_p + A_BYTES + a_off(br, 2u * s + (lane >> 5));

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    // The 16 fragment reads of one strip (from `slot`), in the order the next
    // step's MFMAs consume them: A(0,0), B(0,0..3), A(0,1..3), A(1,0),
    // B(1,0..3), A(1,1..3).
    auto read_one = [&](Frags& f, uint32_t slot, int r) {
        const int s = r >> 3, q = r & 7;
        const uint32_t so = slot * STAGE_BYTES;
        if (q == 0 || q > 4) {
            const int i = q == 0 ? 0 : q - 4;
            if constexpr (AT) f.a[s][i] = read_b_operand(at_ptr[i] + so + 8192u * s);
            else f.a[s][i] = read_a_operand(a_ptr[s] + so + 2048u * i);
        } else {
            const int j = q - 1;
            if constexpr (BT) f.b[s][j] = read_a_operand(bt_ptr[s] + so + 2048u * j);
            else f.b[s][j] = read_b_operand(b_ptr[j] + so + 8192u * s);
        }
    };

    // MFMA t of a step: s = t/16, i = (t/4)%4, j = t%4.
    auto mfma_one = [&](const Frags& f, int t) {
        const int s = t >> 4, i = (t >> 2) & 3, j = t & 3;
        acc[i][j] = E::mfma32(f.b[s][j], f.a[s][i], acc[i][j]);
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

    // Steady-state step on strip kt (ring slot SLOT = kt % 4), whose
    // fragments are in `cur` (read one step earlier; the compiler waits for
    // them at their first use):
    //   4 MFMAs; wait for this wave's copy of strip kt+1; barrier (all copies
    //   of kt+1 landed, every wave done with the slot of kt-1); then 28 MFMAs
    //   with 24 memory operations between the first 24 of them: the 16 reads
    //   of strip kt+1 into `nxt` (in consumption order) and the 8 copies of
    //   strip kt+3 into the slot of kt-1, one operation after each MFMA.
    // Op k (0..23): every third op (k % 3 == 1) is a copy, the rest reads.
    auto step = [&](auto slot_c, uint32_t kt, Frags& cur, Frags& nxt) {
        constexpr uint32_t SLOT = decltype(slot_c)::value;
#pragma unroll
        for (int t = 0; t < 4; ++t) mfma_one(cur, t);
        pin();
        wait_vmcnt<2 * COPIES>();
        barrier();
        pin();
        int rd = 0, cp = 0;
#pragma unroll
        for (int t = 4; t < 32; ++t) {
            mfma_one(cur, t);
            pin();
            const int k = t - 4;
            if (k < 24) {
                if (k % 3 == 1) {
                    dma_one((SLOT + 3) % STAGES, kt + 3, cp);
                    ++cp;
                } else {
                    read_one(nxt, (SLOT + 1) % STAGES, rd);
                    ++rd;
                }
            }
            pin();
        }
    };
    using S0 = std::integral_constant<uint32_t, 0>;
    using S1 = std::integral_constant<uint32_t, 1>;
    using S2 = std::integral_constant<uint32_t, 2>;
    using S3 = std::integral_constant<uint32_t, 3>;

    // The same step with its three decisions taken at run time; used for the
    // last few strips only.
    auto step_tail = [&](uint32_t kt, Frags& cur, Frags& nxt) {
        if (kt >= KT) return;
        const bool more = kt + 1 < KT;
#pragma unroll
        for (int t = 0; t < 4; ++t) mfma_one(cur, t);
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
        for (int t = 4; t < 32; ++t) mfma_one(cur, t);
        pin();
    };

    // Steady state, a multiple of 4 strips (one pass round the ring): every
    // step copies strip kt+3 and reads strip kt+1.  Then at most six steps
    // finish the K loop.
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

    // Epilogue: ReLU, fp16 and the store of C, staged through LDS (the
    // operand ring is no longer needed).
    // The lane index is marked as redefined so the epilogue's lane addresses
    // are computed here, not kept from before the main loop (a spilled
    // register otherwise).
    uint32_t elane = lane;
    asm volatile("" : "+v"(elane));
    epi::store_wave_tile<EDGE, E>(acc, lds + wave * epi::REGION_BYTES, elane, C, ldc, m0 + wm * WAVE_TM,
                               n0 + wn * WAVE_TN, m_tile, M, N, vec_c, ep);
}

#undef GR_LDS

}  // namespace tile2
}  // namespace gr
