// Pipelined MFMA tile kernel for K a multiple of 64 (16-byte aligned rows;
// EDGE=true for M >= 256 and N that do not fill whole tiles).
//
// The 32-deep pipelined kernel (see tile2_kernel.hpp) with one change in
// how A is staged: A moves in 64-deep strips (128-byte row segments, one
// full cache line per row) through a 3-slot ring, while B keeps its 32-deep
// strips (512-byte row segments) in a 4-slot ring.  With 32-deep A strips
// every A row segment is half a cache line, and A alone produces two thirds
// of all L2 requests; full-line segments halve that.  LDS: 4 x 16 KiB (B) +
// 3 x 32 KiB (A) = 160 KiB, all of it.
//
// One step still covers one 32-deep B strip kt (32 MFMAs per wave).  Step kt
// uses half kt%2 of A strip kt/2.  Every step issues 8 copies per wave: half
// of A strip kt/2 + 2 and the whole of B strip kt+3, so "everything issued
// two or more steps ago has landed" is one vmcnt wait in the steady state.
//   A strip j lives in slot j % 3; it is last read while step 2j runs (the
//   reads for step 2j+1), so strip j+3 may be copied from step 2j+2 on; the
//   two halves of strip a+2 are copied in steps 2a and 2a+1.
//   A tile layout [256 m][64 k]: 128-byte rows, chunk index XOR (m/2)%8, so
//   16 consecutive rows reading one chunk hit 16 distinct bank groups.
//
// Each wave owns 128 x 128 of C as 8 x 8 blocks of 16 x 16
// (v_mfma_f32_16x16x32, 64 per step, each taking all 32 k of the step):
// measured 7% faster than 4 x 4 blocks of 32 x 32 (v_mfma_f32_32x32x16, two
// per block and step) with the same copies and fragment bytes.  A fragments:
// ds_read_b128 of 8 consecutive k of one row, 16 rows per read; B fragments:
// two ds_read_b64_tr_b16, each 16-lane group taking a 4 k x 16 n block.
#pragma once


#include <type_traits>

#include "common.hpp"
#include "tile2_kernel.hpp"

namespace gr {

namespace tile3 {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 32;      // K per step (B strip)
constexpr int BKA = 64;     // K per A strip
constexpr int B_SLOTS = 4;
constexpr int A_SLOTS = 3;
constexpr int THREADS = 256;
constexpr int WAVE_TM = 128;
constexpr int WAVE_TN = 128;
constexpr int FM = WAVE_TM / 16;
constexpr int FN = WAVE_TN / 16;
constexpr int B_SLOT_BYTES = BK * BN * 2;     // 16 KiB
constexpr int A_SLOT_BYTES = BM * BKA * 2;    // 32 KiB
constexpr int A_BASE = B_SLOTS * B_SLOT_BYTES;  // 64 KiB
constexpr int LDS_BYTES = A_BASE + A_SLOTS * A_SLOT_BYTES;  // 160 KiB
constexpr int64_t MAX_LDA = tile2::MAX_LDA;
constexpr int64_t MAX_LDB = tile2::MAX_LDB;

#define GR_LDS __attribute__((address_space(3)))

static_assert(LDS_BYTES >= 4 * epi::REGION_BYTES, "the epilogue stages four wave tiles in LDS");

// Byte offset of chunk c (8 fp16) of row m of an A slot (128-byte rows).
__device__ __forceinline__ uint32_t a64_off(uint32_t m, uint32_t c) { return m * 128u + ((c ^ ((m >> 1) & 7u)) << 4); }

struct Frags {
    f16x8 a[FM];
    f16x8 b[FN];
};

// E: element type (ElemF16 or ElemBF16; only the MFMA and the rounding
// differ) or Epi<...> for bias + activation.
// UA (with EDGE, M >= 256, N >= 256, K > 128): rows of A and B need not be
// 16-byte aligned and K need not be a multiple of 64.  The direct-to-LDS
// copies read any 2-byte aligned address (measured on this part: every
// offset gives the bytes of the offset address); the last T = (K - 1) % 64 +
// 1 steps of k are copied like a strip from k = K - 64 and multiplied, with
// the elements at k < K - T zeroed in both operands' fragments, before the
// pipeline starts, and the pipeline then runs over [0, K - T) (a multiple of
// 64).  The last tile column is moved left to end at
// column N, like the last tile row, so every copy reads inside [0, M) x
// [T, K) of A and [T, K) x [0, N) of B: nothing outside the operands is ever
// read, whatever their alignment.  Tail first means a different k order
// than the aligned kernels (a different fp32 rounding order, equally valid).
//
// PERSIST (whole tiles, 16-byte rows of C, the fp16/bf16 ReLU epilogue): a
// persistent tile loop, the TileLang tutorial's "Persistent kernel": the
// grid holds at most one workgroup per CU and workgroup g takes the tiles
// of the logical ids g, g + grid, g + 2 grid, ... (the XCD renumbering and
// tile-row groups of tile_of_workgroup apply to the logical ids).  When a
// tile's last step is done, the workgroup issues the next tile's first
// copies (A strips 0 and 1, B strips 0 to 2: every slot but A slot 2) before
// it stores the finished tile, 32 rows at a time through an 8 KiB region per
// wave in A slot 2; the copies' latency, the launch of a new workgroup and
// the stores overlap.  The copy waits stay those of the first tile: the
// copies complete in order among themselves, so "at most n operations
// outstanding" still means "all but the last n copies landed" when stores
// are outstanding as well (it then waits a little longer).
template <bool EDGE, typename E = ElemF16, bool UA = false, bool PERSIST = false>
__global__ __launch_bounds__(THREADS, 1) void gemm_relu_tile3_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, uint16_t* __restrict__ C, int64_t M, int64_t N,
    int64_t K, int64_t lda, int64_t ldb, int64_t ldc, uint32_t tiles_m, uint32_t tiles_n, uint32_t group_m,
    int vec_c, EpiArgs ep) {
    using tile2::b_off;
    using tile2::barrier;
    using tile2::dma16;
    using tile2::pin;
    using tile2::read_a_operand;
    using tile2::read_b_operand;
    using tile2::wait_vmcnt;

    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t wm = wave >> 1;
    const uint32_t wn = wave & 1u;

    static_assert(!UA || EDGE, "the unaligned variant moves edge tiles");
    static_assert(!PERSIST || (!EDGE && !UA && !E::kGeneral), "the persistent loop takes whole tiles, ReLU");
    const uint32_t n_tiles = tiles_m * tiles_n;
    uint32_t vt = blockIdx.x;  // logical workgroup id (PERSIST: of the current tile)
    uint32_t tm, tn;
    tile_of_workgroup(vt, PERSIST ? n_tiles : gridDim.x, tiles_m, tiles_n, group_m, tm, tn);
    const int64_t m_tile = (int64_t)tm * BM;
    int64_t m0 = EDGE ? edge::shifted_row0(m_tile, M, BM) : m_tile;
    const int64_t n_tile = (int64_t)tn * BN;
    int64_t n0 = UA ? edge::shifted_col0(n_tile, N, BN) : n_tile;
    // UA: the last T = 1..64 steps of k handled first; the pipeline covers
    // [0, K - T).
    const int64_t T = UA ? (K - 1) % BKA + 1 : 0;

    // ---- copies -------------------------------------------------------------
    // A strip (32 KiB) = 32 blocks of 8 rows x 128 bytes; this wave fills
    // blocks 8w .. 8w+7, the first four in the even step, the rest in the odd
    // one.  lane -> row lane/8, slot lane%8 (chunk slot XOR (row/2)%8).
    // B strip (16 KiB) = 16 blocks of 2 rows x 512 bytes; this wave fills
    // blocks 4w .. 4w+3.  lane -> row lane/32, slot lane%32.
    const uint8_t* base_a = reinterpret_cast<const uint8_t*>(A + m0 * lda);
    const uint8_t* base_b = reinterpret_cast<const uint8_t*>(B + n0);  // PERSIST: next tile's later
    const int64_t step_a = BKA * 2;
    const int64_t step_b = (int64_t)BK * ldb * 2;
    // The odd-step half (blocks +4, rows +32) only adds a wave-uniform
    // 32-row offset: the chunk XOR term, (row/2)%8, is unchanged by it.
    uint32_t off_a[4], off_b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t blk = 8u * wave + (uint32_t)i;
        const uint32_t ra = 8u * blk + (lane >> 3);
        const uint32_t ca = (lane & 7u) ^ ((ra >> 1) & 7u);
        off_a[i] = (uint32_t)((ra * lda + 8u * ca) * 2);
    }
    const int64_t half_a = 32 * lda * 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t blk = 4u * wave + (uint32_t)i;
        const uint32_t rb = 2u * blk + (lane >> 5);
        uint32_t cb = (lane & 31u) ^ ((rb & 3u) << 2);
        if constexpr (EDGE && !UA) cb = edge::clamp_chunk(cb, n0, N);
        off_b[i] = (uint32_t)((rb * ldb + 8u * cb) * 2);
    }
    const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(GR_LDS uint8_t*)lds);

    // Copy c (0..3) of half `h` of A strip j, or copy c of B strip d.
    auto dma_a = [&](uint32_t j, uint32_t h, int c) {
        const uint32_t blk = 8u * wave + 4u * h + (uint32_t)c;
        dma16(base_a + (int64_t)j * step_a + (int64_t)h * half_a, off_a[c],
              lds_base + A_BASE + (j % A_SLOTS) * A_SLOT_BYTES + blk * 1024u);
    };
    auto dma_b = [&](uint32_t d, int c) {
        const uint32_t blk = 4u * wave + (uint32_t)c;
        dma16(base_b + (int64_t)d * step_b, off_b[c], lds_base + (d % B_SLOTS) * B_SLOT_BYTES + blk * 1024u);
    };

    // ---- fragment addresses --------------------------------------------------
    // A operand for half h, block i: row wm*128 + 16i + lane%16, chunk
    // 4h + lane/16 of the 64-deep strip (16 rows move the swizzle term
    // (row/2)%8 by a multiple of 8: none); block i is +2 KiB.  The chunk of
    // half 1 is the chunk of half 0 plus 4, i.e. XOR 4 (chunks of half 0 are
    // below 4), and XOR commutes with the row swizzle: half 1's address is
    // half 0's address XOR 64 (slot and block offsets are multiples of 1 KiB
    // and leave that bit alone).
    // B operand, block j: lane l gets column wn*128 + 16j + l%16, k 8(l/16)
    // .. +7 of the 32-deep strip.  Each 16-lane group reads a 4 k x 16 n block
    // with ds_read_b64_tr_b16 (lane address: row 8(l/16) + (l%16)/4, columns
    // 4(l%4) .. +3), then the one 4 rows further on.  Block j adds 2j to the
    // 16-byte chunk index, which the swizzle (chunk XOR 4(k%4)) leaves on
    // address bits 5-7 together with the XOR term: block j's address is
    // block 0's XOR 32j.
    const GR_LDS uint8_t* lds_p = (const GR_LDS uint8_t*)lds;
    uint32_t a_addr = (uint32_t)(uintptr_t)(lds_p + A_BASE + a64_off(wm * WAVE_TM + (lane & 15u), lane >> 4));
    const uint32_t bk = 8u * (lane >> 4) + ((lane & 15u) >> 2);
    const uint32_t bn = wn * WAVE_TN + 4u * (lane & 3u);
    uint32_t b_addr = (uint32_t)(uintptr_t)(lds_p + b_off(bk, bn >> 3) + 2u * (bn & 7u));

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{};

    // Read r (0..15) of the fragments of a step using half H of the A strip in
    // slot byte offset `ao` and the B strip at `bo`, in the order the MFMAs
    // consume them: A0, B0 .. B7, A1 .. A7.
    auto read_one = [&](auto h_c, Frags& f, uint32_t ao, uint32_t bo, int r) {
        constexpr uint32_t H = decltype(h_c)::value;
        if (r == 0 || r > FN) {
            const int i = r == 0 ? 0 : r - FN;
            const uint32_t addr = ((a_addr + ao) ^ (64u * H)) + 2048u * i;
            f.a[i] = read_a_operand((const GR_LDS uint8_t*)(uintptr_t)addr);
        } else {
            const int j = r - 1;
            f.b[j] = read_b_operand((const GR_LDS uint8_t*)(uintptr_t)((b_addr + bo) ^ (32u * j)));
        }
    };
    auto a_slot = [&](uint32_t kt) { return ((kt >> 1) % A_SLOTS) * A_SLOT_BYTES; };
    auto b_slot = [&](uint32_t kt) { return (kt % B_SLOTS) * B_SLOT_BYTES; };
    using H0 = std::integral_constant<uint32_t, 0>;
    using H1 = std::integral_constant<uint32_t, 1>;

    // MFMA t (0..63) of a step: block row t/8, block column t%8.
    auto mfma_one = [&](const Frags& f, int t) {
        const int i = t >> 3, j = t & 7;
        acc[i][j] = E::mfma16(f.b[j], f.a[i], acc[i][j]);
    };

    uint32_t KT = (uint32_t)((K - T) / BK);  // even, >= 2 (UA: >= 4)
    uint32_t KTA = KT / 2;

    // UA: the tail strip, k in [K - 64, K) (inside the operands, as K >
    // 128), is copied first into the slots the prologue leaves free: A slot
    // 2, and B slots 3 (k < K - 32, needed only when T > 32) and 2 (k >= K -
    // 32).  Its elements at k < K - T belong to the pipeline's last strip:
    // they are zeroed in the fragments of both operands after the reads, so
    // they add nothing, whatever their values.  The pipeline then starts at
    // k = 0, where the rows start: on rows aligned to 128 bytes its copies
    // read whole cache lines, whatever K.
    if constexpr (UA) {
        const uint8_t* tail_a = reinterpret_cast<const uint8_t*>(A + m0 * lda + (K - BKA));
        const uint8_t* tail_b = reinterpret_cast<const uint8_t*>(B + (K - BKA) * ldb + n0);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                dma16(tail_a + h * half_a, off_a[c],
                      lds_base + A_BASE + 2 * A_SLOT_BYTES + (8u * wave + 4u * h + (uint32_t)c) * 1024u);
        if (T > BK) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                dma16(tail_b, off_b[c], lds_base + 3 * B_SLOT_BYTES + (4u * wave + (uint32_t)c) * 1024u);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c)
            dma16(tail_b + step_b, off_b[c], lds_base + 2 * B_SLOT_BYTES + (4u * wave + (uint32_t)c) * 1024u);
    }

    // Prologue copies, in this order: A0, B0, B1, A1, B2.
    auto prologue_a0_b0_b1_a1 = [&]() {
#pragma unroll
        for (int c = 0; c < 4; ++c) dma_a(0, 0, c);
#pragma unroll
        for (int c = 0; c < 4; ++c) dma_a(0, 1, c);
#pragma unroll
        for (int c = 0; c < 4; ++c) dma_b(0, c);
        if (KT > 1) {
#pragma unroll
            for (int c = 0; c < 4; ++c) dma_b(1, c);
        }
        if (KTA > 1) {
#pragma unroll
            for (int c = 0; c < 4; ++c) dma_a(1, 0, c);
#pragma unroll
            for (int c = 0; c < 4; ++c) dma_a(1, 1, c);
        }
    };
    auto prologue_b2 = [&]() {
        if (KT > 2) {
#pragma unroll
            for (int c = 0; c < 4; ++c) dma_b(2, c);
        }
    };
    prologue_a0_b0_b1_a1();
    if constexpr (UA) {
        // The tail's copies, issued before the 24 above (A0, B0, B1, A1),
        // have landed once at most those 24 remain; the barrier makes every
        // wave's part visible.
        wait_vmcnt<24>();
        __syncthreads();
        // In half H of the strip, both operands of this lane hold k = K - 64
        // + 32 H + 8 (lane / 16) + e, e = 0..7: keep the elements with k >=
        // K - T, i.e. e >= v below.
        auto tail_half = [&](auto h_c, uint32_t bo) {
            constexpr uint32_t H = decltype(h_c)::value;
            const int v = (int)(BKA - T) - (int)(32u * H + 8u * (lane >> 4));
            u32x4 keep;
#pragma unroll
            for (int d = 0; d < 4; ++d)
                keep[d] = (2 * d >= v ? 0x0000FFFFu : 0u) | (2 * d + 1 >= v ? 0xFFFF0000u : 0u);
            Frags ft;
#pragma unroll
            for (int r = 0; r < 16; ++r) read_one(h_c, ft, 2 * A_SLOT_BYTES, bo, r);
#pragma unroll
            for (int i = 0; i < FM; ++i) ft.a[i] = __builtin_bit_cast(f16x8, __builtin_bit_cast(u32x4, ft.a[i]) & keep);
#pragma unroll
            for (int j = 0; j < FN; ++j) ft.b[j] = __builtin_bit_cast(f16x8, __builtin_bit_cast(u32x4, ft.b[j]) & keep);
#pragma unroll
            for (int t = 0; t < 64; ++t) mfma_one(ft, t);
        };
        if (T > BK) tail_half(H0{}, 3 * B_SLOT_BYTES);
        tail_half(H1{}, 2 * B_SLOT_BYTES);
        // every wave is done with the tail's slots before strips are copied into them
        __syncthreads();
    }
    prologue_b2();

    // Copies issued in step s (the A half, then the B strip).
    auto issue_step = [&](uint32_t s) {
        const uint32_t ja = (s >> 1) + 2;
        if (ja < KTA) {
#pragma unroll
            for (int c = 0; c < 4; ++c) dma_a(ja, s & 1u, c);
        }
        if (s + 3 < KT) {
#pragma unroll
            for (int c = 0; c < 4; ++c) dma_b(s + 3, c);
        }
    };
    auto n_issued = [&](uint32_t s) -> uint32_t { return 4u * ((s >> 1) + 2 < KTA) + 4u * (s + 3 < KT); };

    for (;;) {  // one tile per pass; only PERSIST comes back
    if constexpr (PERSIST) {
        // The per-lane copy offsets and fragment addresses are the same for
        // every tile.  Marking them as redefined here keeps the compiler from
        // hoisting the many addresses it derives from them out of the tile
        // loop, where they would stay live through the epilogue and spill.
#pragma unroll
        for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(off_a[i]), "+v"(off_b[i]));
        asm volatile("" : "+v"(a_addr), "+v"(b_addr));
        // likewise the step counts, or the conditions derived from them are
        // kept (as vector registers, spilled) across the tile loop
        asm volatile("" : "+s"(KT), "+s"(KTA));
    }
    // A0 and B0 landed: the copies after them may stay in flight.
    {
        const uint32_t after = 4u * (KT > 1) + 8u * (KTA > 1) + 4u * (KT > 2);
        if (after == 16) wait_vmcnt<16>();
        else if (after == 12) wait_vmcnt<12>();
        else if (after == 4) wait_vmcnt<4>();
        else wait_vmcnt<0>();
    }
    barrier();

    Frags f0, f1;
#pragma unroll
    for (int r = 0; r < 16; ++r) read_one(H0{}, f0, a_slot(0), b_slot(0), r);

    // Steady step: every copy of step kt exists and the wait is "only the
    // previous step's 8 copies may remain".  8 MFMAs, wait + barrier, then
    // one memory operation after every second of the next 48 MFMAs (a copy
    // after every third of those).  NH = half of A used by step kt+1.
    auto step = [&](auto nh_c, uint32_t kt, Frags& cur, Frags& nxt) {
#pragma unroll
        for (int t = 0; t < 8; ++t) mfma_one(cur, t);
        pin();
        wait_vmcnt<8>();
        barrier();
        pin();
        const uint32_t ja = (kt >> 1) + 2;
        const uint32_t ao = a_slot(kt + 1), bo = b_slot(kt + 1);
        int rd = 0, cp = 0;
#pragma unroll
        for (int t = 8; t < 64; ++t) {
            mfma_one(cur, t);
            pin();
            const int k = t - 8;
            if (k < 48 && (k & 1) == 0) {
                if ((k >> 1) % 3 == 1) {
                    if (cp < 4) dma_a(ja, kt & 1u, cp);
                    else dma_b(kt + 3, cp - 4);
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
    // last few).
    auto step_any = [&](uint32_t kt, Frags& cur, Frags& nxt) {
        if (kt >= KT) return;
        const bool more = kt + 1 < KT;
#pragma unroll
        for (int t = 0; t < 8; ++t) mfma_one(cur, t);
        pin();
        if (more) {
            uint32_t allowed;
            if (kt == 0) allowed = 8u * (KTA > 1) + 4u * (KT > 2);
            else if (kt == 1) allowed = n_issued(0);
            else allowed = n_issued(kt - 1);
            if (allowed >= 12) wait_vmcnt<12>();
            else if (allowed == 8) wait_vmcnt<8>();
            else if (allowed == 4) wait_vmcnt<4>();
            else wait_vmcnt<0>();
            barrier();
        }
        pin();
        issue_step(kt);
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

    // Step 0 generic; steady steps 1 .. S-1 (an even count, all copies
    // present: kt < KT - 4); then up to five generic steps.
    step_any(0, f0, f1);
    uint32_t kt = 1;
    const uint32_t last_steady = KT > 5 ? KT - 5 : 0;  // steady steps are kt <= last_steady
    for (; kt + 1 <= last_steady; kt += 2) {  // kt odd: step kt+1 uses half 0, step kt+2 half 1
        step(H0{}, kt, f1, f0);
        step(H1{}, kt + 1, f0, f1);
    }
    step_any(kt, f1, f0);
    step_any(kt + 1, f0, f1);
    step_any(kt + 2, f1, f0);
    step_any(kt + 3, f0, f1);
    step_any(kt + 4, f1, f0);
    step_any(kt + 5, f0, f1);

    if constexpr (PERSIST) {
        // Every wave is done with the operand slots (its last fragment reads
        // were consumed by its MFMAs): the next tile's first copies may go
        // out, then this tile is stored through A slot 2, which they leave
        // alone (the next tile's step 0 copies into it after its barrier).
        const int64_t c_row = m0 + wm * WAVE_TM, c_col = n0 + wn * WAVE_TN;
        barrier();
        const uint32_t next = vt + gridDim.x;
        if (next < n_tiles) {
            vt = next;
            tile_of_workgroup(vt, n_tiles, tiles_m, tiles_n, group_m, tm, tn);
            m0 = (int64_t)tm * BM;
            n0 = (int64_t)tn * BN;
            base_a = reinterpret_cast<const uint8_t*>(A + m0 * lda);
            base_b = reinterpret_cast<const uint8_t*>(B + n0);
            prologue_a0_b0_b1_a1();
            prologue_b2();
        }
        epi::store_wave_tile_rows32<E>(acc, lds + A_BASE + 2 * A_SLOT_BYTES + wave * epi::ROWS32_BYTES, C, ldc,
                                       c_row, c_col);
        if (next >= n_tiles) break;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{};
    } else {
        // Epilogue: ReLU, fp16 and the store of C, staged through LDS (the
        // operand ring is no longer needed).  Whole tiles with 16-byte rows
        // of C (the fp16/bf16 ReLU): after one barrier each wave stores its
        // tile 32 rows at a time through 8 KiB of its own, with no further
        // barrier (measured about 1% faster at 4096^3 than staging the whole
        // tile between two barriers).  Otherwise the whole tile is staged.
        if (!EDGE && !E::kGeneral && vec_c == 8) {
            barrier();
            epi::store_wave_tile_rows32<E>(acc, lds + A_BASE + 2 * A_SLOT_BYTES + wave * epi::ROWS32_BYTES, C, ldc,
                                           m0 + wm * WAVE_TM, n0 + wn * WAVE_TN);
        } else {
            // The lane index is marked as redefined so the epilogue's lane
            // addresses are computed here, not kept from before the main
            // loop (one spilled register otherwise).
            uint32_t elane = lane;
            asm volatile("" : "+v"(elane));
            epi::store_wave_tile<EDGE, E>(acc, lds + wave * epi::REGION_BYTES, elane, C, ldc, m0 + wm * WAVE_TM,
                                       n0 + wn * WAVE_TN, m_tile, M, N, vec_c, ep, n_tile);
        }
        break;
    }
    }  // tile loop
}

#undef GR_LDS

}  // namespace tile3
}  // namespace gr
