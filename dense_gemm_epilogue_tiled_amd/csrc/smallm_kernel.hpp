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
#include "tile2_kernel.hpp"

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

// E: element type (ElemF16 or ElemBF16; only the MFMA and the rounding differ).
// MB: blocks of 16 rows of A (M <= 16 * MB).  Each transposed B operand feeds
// MB MFMAs, one per block of A rows, so up to 64 rows still read B once.
template <int W, int U, bool GUARD, typename E = ElemF16, int MB = 1>
__global__ __launch_bounds__(64 * W, 1) void gemm_relu_smallm_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, uint16_t* __restrict__ C,
    int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, EpiArgs ep) {
    constexpr int ROWS = MAX_M * MB;
    __shared__ __attribute__((aligned(16))) float red[W][ROWS][NB];

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wave = tid >> 6;
    const uint32_t li = lane & 15u;  // MFMA row slot (4 columns of B) / column slot (row of A)
    const uint32_t lg = lane >> 4;   // which 8-deep k group of the 32-deep step

    const int64_t n_base = (int64_t)blockIdx.x * NB;
    const int64_t n_lane = n_base + 4 * li;
    const int64_t steps = (K + KSTEP - 1) / KSTEP;

    f32x4 acc[MB][4];
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[b][c] = f32x4{};

    // Loads of one group of U steps (this wave's steps s0, s0+W, ...).
    auto load_group = [&](int64_t s0, u32x2 (&rb)[U][8], u32x4 (&ra)[U][MB]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t s = s0 + (int64_t)u * W;
            const int64_t k = s * KSTEP + 8 * lg;
            if (s < steps) {
#pragma unroll
                for (int r = 0; r < 8; ++r) rb[u][r] = load_b4<GUARD>(B, ldb, k + r, n_lane, K, N);
#pragma unroll
                for (int b = 0; b < MB; ++b) ra[u][b] = load_a8<GUARD>(A, lda, li + 16 * b, k, M, K);
            } else {
#pragma unroll
                for (int r = 0; r < 8; ++r) rb[u][r] = u32x2{0u, 0u};
#pragma unroll
                for (int b = 0; b < MB; ++b) ra[u][b] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    auto compute_group = [&](const u32x2 (&rb)[U][8], const u32x4 (&ra)[U][MB]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                u32x4 o;
#pragma unroll
                for (int d = 0; d < 4; ++d) o[d] = pair_halves(rb[u][2 * d][c >> 1], rb[u][2 * d + 1][c >> 1], c & 1);
#pragma unroll
                for (int b = 0; b < MB; ++b)
                    acc[b][c] = E::mfma16(__builtin_bit_cast(f16x8, o), __builtin_bit_cast(f16x8, ra[u][b]), acc[b][c]);
            }
        }
    };

    // Two register sets: the loads of group g+1 are in flight while group g
    // is transposed and multiplied, so each wave keeps U*8 loads outstanding.
    const int64_t stride = (int64_t)W * U;
    u32x2 rb0[U][8], rb1[U][8];
    u32x4 ra0[U][MB], ra1[U][MB];
    int64_t s0 = wave;
    if (s0 < steps) load_group(s0, rb0, ra0);
    for (; s0 < steps; s0 += 2 * stride) {
        if (s0 + stride < steps) load_group(s0 + stride, rb1, ra1);
        compute_group(rb0, ra0);
        if (s0 + stride >= steps) break;
        if (s0 + 2 * stride < steps) load_group(s0 + 2 * stride, rb0, ra0);
        compute_group(rb1, ra1);
    }

    // acc[b][c] holds C^T: lane l, register r is the partial sum for row
    // m = 16b + l%16 and column n = n_base + 4(4(l/16) + r) + c.
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][16 * b + li][4 * (4 * lg + r) + c] = acc[b][c][r];
    __syncthreads();

    for (uint32_t o = tid; o < (uint32_t)(ROWS * NB); o += 64 * W) {
        const uint32_t m = o / NB, nl = o % NB;
        const int64_t n = n_base + nl;
        if ((int64_t)m < M && n < N) {
            float sum = 0.0f;
#pragma unroll
            for (int w = 0; w < W; ++w) sum += red[w][m][nl];
            C[(int64_t)m * ldc + n] = epi_value<E>(sum, n, N, ep);
        }
    }
}

// ---- streaming variant: B copied straight into LDS ----------------------------
//
// The kernel above holds B in registers and reads it in 128-byte row pieces
// (64-column strips).  Measured on this part, streaming reads are fastest
// with 256-byte row pieces and 32 KiB in flight per workgroup (a plain read
// of the small-M workload's B in that pattern: 39.2-39.9 us, 6.7-6.9 TB/s;
// 512-byte to 4 KiB pieces were slower), and the in-flight bytes should stay
// there: when each wave waits for its own slot and then computes, the
// workgroup's copies in flight dip while it computes.  This variant moves B
// (and A) with direct-to-LDS copies (global_load_lds_dwordx4, nontemporal):
//   * workgroup (cb, s): columns [NB cb, NB cb + NB) and the K range of split
//     s (all of K without a split); its W waves take the range's 32-row slots
//     in turn (wave w: slots w, w + W, ...) through a ring of R slots of its
//     own: slot q + R - 1 is copied before slot q is waited for, so every
//     wave keeps R - 1 to R slots in flight and the workgroup W (R - 1) to
//     W R; a wave reads back only what it copied itself, so no barrier is
//     needed.  Measured first pass of the small-M split (8 x 16384 x 8192, two
//     splits, NB = 128): 2 waves x ring of 2 40.0-40.5 us, 4 waves x 1 slot
//     41.9-42.2 us, 4 waves x 2 slots 47.2 us, 8 waves x 1 slot 45.1 us;
//     single pass (NB = 64): 4 waves x 2 slots 47.1-47.5 us, 8 waves x 1
//     slot 48.8 us;
//   * copies: a slot is 32 rows of 2 NB bytes of B, then (when A is given
//     row-major) 16 rows x 32 k of A; one copy instruction moves 1 KiB
//     (1024 / 2NB whole rows of B); 16-byte chunk c of row r of B sits at
//     chunk slot c XOR 2(r mod 4), chunk c of row r of A at c XOR (r/4) mod 4
//     (the rows one 16-lane group reads land in distinct banks);
//   * compute: per slot and 16-column block j, the B operand of
//     v_mfma_f32_16x16x32 (16 columns x 32 k) comes from two
//     ds_read_b64_tr_b16, the A operand (16 rows of A x 32 k; rows >= M copy
//     row M - 1, whose outputs are never stored) from one 16-byte LDS read;
//   * B may have any 2-byte alignment (the copies read any address); the
//     last column block moves left to end at column N (N >= NB), so every
//     copy reads inside [0, K) x [0, N) and only the block's own columns
//     are stored;
//   * at the end the W waves' partial sums are added in LDS in wave order;
//     without a split the epilogue (ReLU, rounding) follows; with a split
//     the fp32 sum of the range goes to part[s][m][n] for the ordered second
//     pass (gemm_relu_smallm_reduce_kernel below).  Adding two splits in the
//     same launch instead (the second workgroup of a column block to finish
//     reads the other's agent-scope partial sums after an exchange on a
//     per-block flag) measured 0.7 us slower: the stores, the exchange and
//     the reloads sit one after another at the end of every workgroup.
// Needs M <= 16, K % 32 == 0 (whole slots), 16-byte rows of A.
// AT=true: A is given transposed (At, K x M row-major, pitch lda, any
// alignment): each lane gathers its 8 consecutive k of one column of At with
// 2-byte loads (A is small and stays in the caches), one slot per wave.
namespace stream {

constexpr int SLOT_ROWS = 32;

// What a workgroup does with its range sum: store C (no split), or store
// the fp32 partial sum for the ordered second pass.
enum Mode { WHOLE = 0, PARTIAL = 1 };

__device__ __forceinline__ uint32_t chunk_slot(uint32_t row, uint32_t c) { return c ^ ((row & 3u) << 1); }

}  // namespace stream

template <int NB, int W, int R, int MODE, typename E = ElemF16, bool AT = false, int MB = 1, bool RBLK = false,
          bool BT = false>
__global__ __launch_bounds__(64 * W, 1) void gemm_relu_smallm_stream_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, uint16_t* __restrict__ C,
    float* __restrict__ part, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
    int64_t k_per_split, uint32_t n_blocks, uint32_t order, EpiArgs ep) {
    // RBLK: blocks of 16 MB rows over all of M, all of K, the copies cached
    // (every operand block is read by several workgroups).  The grid is
    // ceil(M / 16 MB) row blocks x n_blocks column blocks; the workgroup's
    // block comes from tile_of_workgroup with the order word `order` (groups
    // of row blocks, XCD renumbering unless bit 31 is set; group 1 with bit
    // 31 is plain row-major order).  The other modes ignore `order`.
    // BT (row blocks only): B is given transposed, N x K with pitch ldb; a
    // slot's B is NB / 16 blocks of 16 rows of Bt x 32 k, copied and read
    // like the blocks of A (the MFMA's B operand wants 8 consecutive k of one
    // column per lane, which is a row piece of Bt).
    static_assert(!RBLK || (MODE == stream::WHOLE && !AT), "row blocks: one pass, A row-major");
    static_assert(!BT || RBLK, "B transposed: row blocks only");
    auto copy16 = [](const void* base, uint32_t voff, uint32_t lds_addr) {
        if constexpr (RBLK) tile2::dma16(base, voff, lds_addr);
        else tile2::dma16_nt(base, voff, lds_addr);
    };
    constexpr bool ADMA = !AT;                           // A copied into the slot beside B
    constexpr int ROWB = 2 * NB;                         // bytes of one row piece
    constexpr int CH = NB / 8;                           // 16-byte chunks per row piece
    constexpr int ROWS = MAX_M * MB;                     // rows of A: MB blocks of 16
    constexpr int BSLOT = stream::SLOT_ROWS * ROWB;      // bytes of B per slot
    constexpr int SLOT = BSLOT + (ADMA ? 1024 * MB : 0); // + MB x 16 rows x 32 k of A
    constexpr int DPS = BSLOT / 1024;                    // copy instructions of B per slot
    constexpr int OPS = DPS + (ADMA ? MB : 0);           // memory operations per slot
    constexpr int RPI = 1024 / ROWB;                     // rows per copy instruction
    constexpr int NBLK = NB / 16;                        // MFMA column blocks per slot
    constexpr int T = 64 * W;
    static_assert(BT || (CH >= 8 && DPS * RPI == stream::SLOT_ROWS), "whole rows per copy instruction");
    static_assert(!BT || DPS == NB / 16, "one copy instruction per 16 rows of Bt");
    static_assert(ROWS * NB * 4 <= R * SLOT, "the cross-wave sum fits a wave's slots");
    static_assert(NB % 64 == 0, "the sum's column-group XOR (up to 15) stays inside a row");
    static_assert(!AT || (R == 1 && MB == 1), "A gathered into registers: one slot per wave, 16 rows");
    static_assert(MB == 1 || MB == 2 || MB == 4, "1, 2 or 4 blocks of 16 rows");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[W * R * SLOT];

    const uint32_t tid = threadIdx.x, lane = tid & 63u;
    const uint32_t w = __builtin_amdgcn_readfirstlane(tid >> 6);
    uint32_t cb;
    int64_t s;
    if (RBLK && order != (kNoXcdRemap | 1u)) {
        uint32_t rb, nb;
        tile_of_workgroup(blockIdx.x, gridDim.x, gridDim.x / n_blocks, n_blocks, order, rb, nb);
        cb = nb;
        s = rb;
    } else {
        // plain row-major order without the general mapping's divisions
        // (they delay the first copies: 1024^3 8.70 -> 8.60 us)
        cb = blockIdx.x % n_blocks;
        s = blockIdx.x / n_blocks;
    }
    if constexpr (RBLK) {
        A += s * ROWS * lda;
        C += s * ROWS * ldc;
        M = M - s * ROWS < ROWS ? M - s * ROWS : ROWS;
        s = 0;
    }
    const int64_t n_own = (int64_t)cb * NB;
    const int64_t n0 = n_own + NB <= N ? n_own : N - NB;  // the last block ends at column N
    const int64_t k_begin = s * k_per_split;
    const int64_t k_end = k_begin + k_per_split < K ? k_begin + k_per_split : K;
    const int64_t slots = (k_end - k_begin) / stream::SLOT_ROWS;
    const int64_t nw = slots > (int64_t)w ? (slots - w + W - 1) / W : 0;  // this wave's slots
    const uint32_t ring = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds + w * R * SLOT;

    // copy instruction i of a slot: lane -> row i RPI + lane / CH, chunk slot
    // lane % CH, which holds chunk (lane % CH) XOR 2 (row mod 4)
    // A copy of a slot (ADMA), one per block of 16 rows: lane -> row 16 mb +
    // lane / 4 (rows >= M read row M - 1; their outputs are never stored),
    // chunk slot lane % 4 holding chunk (lane % 4) XOR (row / 4) % 4 of the
    // row's 32 k.  BT: the blocks of Bt (rows n0 + 16 i + lane / 4, all < N)
    // the same way.
    const uint32_t arow = lane >> 2, apos = lane & 3u;
    uint32_t voff[DPS];
#pragma unroll
    for (int i = 0; i < DPS; ++i) {
        if constexpr (BT) {
            voff[i] = (uint32_t)(((16 * i + arow) * ldb + 8 * (apos ^ ((arow >> 2) & 3u))) * 2);
        } else {
            const uint32_t row = i * RPI + lane / CH;
            voff[i] = (uint32_t)((row * ldb + 8 * stream::chunk_slot(row, lane % CH)) * 2);
        }
    }
    const uint16_t* b_range = BT ? B + n0 * ldb + k_begin : B + k_begin * ldb + n0;
    uint32_t aoff[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int64_t r = 16 * mb + arow;
        const uint32_t asrc = r < M ? (uint32_t)r : (uint32_t)(M - 1);
        aoff[mb] = (uint32_t)((asrc * lda + 8 * (apos ^ ((arow >> 2) & 3u))) * 2);
    }
    const uint32_t am = lane & 15u, ag = lane >> 4;

    // B operand of column block j: lane l (group g = l/16, i = l%16) reads
    // row 8g + i/4 (then + 4), columns 16j + 4(i%4) .. +3.
    const uint32_t fi = lane & 15u, fg = lane >> 4;
    const uint32_t frow = 8 * fg + (fi >> 2);
    f32x4 acc[MB][NBLK];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < NBLK; ++j) acc[mb][j] = f32x4{};

    // Slot q of this wave is slot t = w + W q of the range, in ring entry q % R.
    u32x4 areg = u32x4{0u, 0u, 0u, 0u};
    auto issue = [&](int64_t q) {
        const int64_t t = (int64_t)w + (int64_t)W * q;
        const uint32_t dst = ring + (uint32_t)(q % R) * SLOT;
        const uint8_t* src = reinterpret_cast<const uint8_t*>(b_range + t * stream::SLOT_ROWS * (BT ? 1 : ldb));
#pragma unroll
        for (int i = 0; i < DPS; ++i) copy16(src, voff[i], dst + i * 1024);
        if constexpr (ADMA) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                copy16(reinterpret_cast<const uint8_t*>(A + k_begin + t * stream::SLOT_ROWS), aoff[mb],
                       dst + BSLOT + 1024 * mb);
        } else {
            const int64_t k = k_begin + t * stream::SLOT_ROWS + 8 * ag;
            uint32_t h[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = (int64_t)am < M ? (uint32_t)A[(k + e) * lda + am] : 0u;
            areg = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
        }
    };

    // R - 1 slots ahead: slot q + R - 1 goes out (into the entry slot q - 1
    // used, whose reads its MFMAs consumed) before slot q is waited for.
    const int64_t ahead = nw < R - 1 ? nw : R - 1;
    for (int64_t q = 0; q < ahead; ++q) issue(q);
    for (int64_t q = 0; q < nw; ++q) {
        const bool more = q + R - 1 < nw;
        if (more) issue(q + R - 1);
        if (more) tile2::wait_vmcnt<(R - 1) * OPS>();  // slot q's copies have landed
        else tile2::wait_vmcnt<0>();
        const uint32_t base = ring + (uint32_t)(q % R) * SLOT;
        f16x8 a[MB];
        if constexpr (ADMA) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                a[mb] = *reinterpret_cast<const __attribute__((address_space(3))) f16x8*>(
                    (uintptr_t)(base + BSLOT + 1024 * mb + am * 64 + ((ag ^ ((am >> 2) & 3u)) << 4)));
        } else {
            a[0] = __builtin_bit_cast(f16x8, areg);
        }
#pragma unroll
        for (int j = 0; j < NBLK; ++j) {
            f16x8 b;
            if constexpr (BT) {
                b = *reinterpret_cast<const __attribute__((address_space(3))) f16x8*>(
                    (uintptr_t)(base + 1024 * j + am * 64 + ((ag ^ ((am >> 2) & 3u)) << 4)));
            } else {
                const uint32_t c = 2 * j + ((fi >> 1) & 1u);
                const uint32_t p0 = base + frow * ROWB + (stream::chunk_slot(frow, c) << 4) + 8 * (fi & 1u);
                const uint32_t p1 = base + (frow + 4) * ROWB + (stream::chunk_slot(frow + 4, c) << 4) + 8 * (fi & 1u);
                typedef short s16x4 __attribute__((ext_vector_type(4)));
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4*)(uintptr_t)p0);
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4*)(uintptr_t)p1);
                b = __builtin_bit_cast(f16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) acc[mb][j] = E::mfma16(b, a[mb], acc[mb][j]);
        }
    }

    // acc[j] holds C^T: lane l, register r is row m = l%16, column 16j +
    // 4(l/16) + r of the block.  Sum the waves in order through LDS (each
    // wave's partials in its own slot, [ROWS][NB] fp32).  Column group c (4
    // floats) of row m sits at group c XOR (m mod 16): the 16 lanes that
    // store one register group hold 16 rows, which without the XOR all fall
    // in the same 4 of the 64 banks (rows are NB floats apart); with it they
    // cover all 64.
    __syncthreads();
    float* red = reinterpret_cast<float*>(lds);  // wave w at w * R * SLOT
    auto red_at = [](uint32_t m, uint32_t c) { return m * NB + (c ^ ((m & 15u) << 2)); };
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < NBLK; ++j)
            *reinterpret_cast<f32x4*>(red + w * (R * SLOT / 4) +
                                      red_at(16 * mb + (lane & 15u), 16 * j + 4 * (lane >> 4))) = acc[mb][j];
    __syncthreads();
    for (uint32_t o = tid; o < (uint32_t)(ROWS * NB); o += T) {
        const uint32_t m = o / NB, nl = o % NB;
        const int64_t n = n0 + nl;
        if ((int64_t)m >= M || n < n_own) continue;
        float v = 0.0f;
#pragma unroll
        for (int ww = 0; ww < W; ++ww) v += red[ww * (R * SLOT / 4) + red_at(m, nl)];
        if constexpr (MODE == stream::WHOLE) C[(int64_t)m * ldc + n] = epi_value<E>(v, n, N, ep);
        else part[(s * M + m) * N + n] = v;
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

// E: element type of A and B (only its MFMA is used here; pass 2 rounds).
template <bool GUARD, typename E = ElemF16>
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
                acc[j] = E::mfma16(__builtin_bit_cast(f16x8, o), a, acc[j]);
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

// Pass 2: C[m][n] = epilogue(sum over s of part[s][m][n]) -- the fused ReLU
// and rounding, or (E = Epi<...>) scale, bias, activation and rounding.  The
// sum starts from +0 and adds the splits in order, whatever the variant.
// VEC4 (N % 4 == 0): each thread owns four consecutive outputs of one row,
// reads them with 16-byte loads and (vec_c >= 4) stores them with one 8-byte
// store.
template <typename E = ElemF16, bool VEC4 = false>
__global__ __launch_bounds__(256) void gemm_relu_smallm_reduce_kernel(const float* __restrict__ part,
                                                                      uint16_t* __restrict__ C, int64_t M,
                                                                      int64_t N, int64_t ldc, int splits,
                                                                      int vec_c, EpiArgs ep) {
    const int64_t total = M * N;
    if constexpr (VEC4) {
        for (int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x; 4 * o < total; o += (int64_t)gridDim.x * 256) {
            f32x4 sum = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
            for (int s = 0; s < splits; ++s) {
                const f32x4* src = reinterpret_cast<const f32x4*>(part + (int64_t)s * total) + o;
                const f32x4 v = __builtin_nontemporal_load(src);
                sum = f32x4{sum[0] + v[0], sum[1] + v[1], sum[2] + v[2], sum[3] + v[3]};
            }
            const int64_t m = 4 * o / N, n = 4 * o - m * N;
            uint16_t r[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) r[e] = epi_value<E>(sum[e], n + e, N, ep);
            uint16_t* dst = C + m * ldc + n;
            if (vec_c >= 4) {
                *reinterpret_cast<u32x2*>(dst) =
                    u32x2{(uint32_t)r[0] | ((uint32_t)r[1] << 16), (uint32_t)r[2] | ((uint32_t)r[3] << 16)};
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) dst[e] = r[e];
            }
        }
    } else {
        (void)vec_c;
        for (int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x; o < total; o += (int64_t)gridDim.x * 256) {
            float sum = 0.0f;
            for (int s = 0; s < splits; ++s) sum += part[(int64_t)s * total + o];
            const int64_t m = o / N, n = o - m * N;
            C[m * ldc + n] = epi_value<E>(sum, n, N, ep);
        }
    }
}

// ---- B given transposed (Bt, N x K row-major): the GEMV pattern proper ------
//
// With B stored as N x K (a weight matrix in the layout of the GEMV pattern of
// "Tilelang Cuda Patterns", section 4), every column of C is a dot product of
// two contiguous rows.  A workgroup owns 64 columns (64 rows of Bt): its 8
// waves are 4 column groups of 16 x 2 interleaved K phases (groups of BT_U
// 32-deep steps alternate between the phases), so that 8 waves per CU keep
// loads in flight.  Per step a lane loads 16 bytes of one Bt row (row l%16,
// k group l/16) and 16 bytes of one row of A, and both are
// v_mfma_f32_16x16x32_f16 operands as they stand -- no transpose.  Two
// register sets of BT_U steps; at the end the two K phases are added in LDS,
// then ReLU, fp16 and the store.
constexpr int BT_COLS = 16;    // columns of C per column group
constexpr int BT_GROUPS = 4;   // column groups per workgroup
constexpr int BT_PHASES = 2;   // interleaved K phases per column group
constexpr int BT_WAVES = BT_GROUPS * BT_PHASES;
constexpr int BT_NB = BT_COLS * BT_GROUPS;  // columns per workgroup
constexpr int BT_U = 8;

// Eight consecutive fp16 of Bt row n from column k; zero outside [0,N) x [0,K).
template <bool GUARD>
__device__ __forceinline__ u32x4 load_bt8(const uint16_t* Bt, int64_t ldbt, int64_t n, int64_t k, int64_t N,
                                          int64_t K) {
    if constexpr (!GUARD) {
        return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Bt + n * ldbt + k));
    } else {
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (n < N && k < K) {
            const uint16_t* p = Bt + n * ldbt + k;
            if (k + 8 <= K) {
                v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
            } else {
                uint32_t h[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (k + e < K) h[e] = p[e];
#pragma unroll
                for (int d = 0; d < 4; ++d) v[d] = h[2 * d] | (h[2 * d + 1] << 16);
            }
        }
        return v;
    }
}

// E: element type and epilogue (ElemF16, ElemBF16, or Epi<...> for bias +
// activation with ep).
template <bool GUARD, typename E = ElemF16>
__global__ __launch_bounds__(64 * BT_WAVES) void gemm_relu_smallm_bt_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ Bt, uint16_t* __restrict__ C, int64_t M, int64_t N,
    int64_t K, int64_t lda, int64_t ldbt, int64_t ldc, EpiArgs ep) {
    __shared__ __attribute__((aligned(16))) float red[BT_PHASES][MAX_M][BT_NB];

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wave = tid >> 6;
    const uint32_t cg = wave % BT_GROUPS;  // column group
    const uint32_t kp = wave / BT_GROUPS;  // K phase
    const uint32_t li = lane & 15u;        // row of Bt (column of C) / row of A
    const uint32_t lg = lane >> 4;         // 8-deep k group of the 32-deep step

    const int64_t n_wg = (int64_t)blockIdx.x * BT_NB;
    const int64_t n_base = n_wg + BT_COLS * cg;
    const int64_t n_row = n_base + li;
    const int64_t steps = (K + KSTEP - 1) / KSTEP;

    f32x4 acc = f32x4{};
    auto load_group = [&](int64_t t0, u32x4 (&rb)[BT_U], u32x4 (&ra)[BT_U]) {
#pragma unroll
        for (int u = 0; u < BT_U; ++u) {
            const int64_t t = t0 + u;
            const int64_t k = t * KSTEP + 8 * lg;
            if (t < steps) {
                rb[u] = load_bt8<GUARD>(Bt, ldbt, n_row, k, N, K);
                ra[u] = load_a8<true>(A, lda, li, k, M, K);
            } else {
                rb[u] = u32x4{0u, 0u, 0u, 0u};
                ra[u] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    auto compute_group = [&](const u32x4 (&rb)[BT_U], const u32x4 (&ra)[BT_U]) {
#pragma unroll
        for (int u = 0; u < BT_U; ++u)
            acc = E::mfma16(__builtin_bit_cast(f16x8, rb[u]), __builtin_bit_cast(f16x8, ra[u]), acc);
    };

    // Phase kp takes the step groups kp, kp + 2, kp + 4, ... (BT_U steps each).
    const int64_t stride = (int64_t)BT_PHASES * BT_U;
    u32x4 rb0[BT_U], rb1[BT_U], ra0[BT_U], ra1[BT_U];
    int64_t t0 = (int64_t)kp * BT_U;
    if (t0 < steps) load_group(t0, rb0, ra0);
    for (; t0 < steps; t0 += 2 * stride) {
        if (t0 + stride < steps) load_group(t0 + stride, rb1, ra1);
        compute_group(rb0, ra0);
        if (t0 + stride >= steps) break;
        if (t0 + 2 * stride < steps) load_group(t0 + 2 * stride, rb0, ra0);
        compute_group(rb1, ra1);
    }

    // acc holds C^T: lane l, register r is the partial sum of C[m][n] with
    // m = l%16 and n = n_base + 4(l/16) + r.
#pragma unroll
    for (int r = 0; r < 4; ++r) red[kp][li][BT_COLS * cg + 4 * lg + r] = acc[r];
    __syncthreads();
    for (uint32_t o = tid; o < (uint32_t)(MAX_M * BT_NB); o += 64 * BT_WAVES) {
        const uint32_t m = o / BT_NB, nl = o % BT_NB;
        const int64_t n = n_wg + nl;
        if ((int64_t)m < M && n < N) C[(int64_t)m * ldc + n] = epi_value<E>(red[0][m][nl] + red[1][m][nl], n, N, ep);
    }
}

// Bt version with direct-to-LDS copies, for K a multiple of 256: loading MFMA
// operands straight from global memory (above) reads every Bt row in 64-byte
// pieces and re-reads A for every column group.  Measured at 8 x 16384 x 8192
// with Bt cold (four rotating copies), back to back: a workgroup of 4 waves
// sharing each 256-deep chunk of Bt and A through a ring of 4 (2) slots, with
// a barrier per chunk, 55.3 (52.7) us; 128-deep chunks 65-68 us; the variant
// below, with a 2-slot ring per wave and no barrier, 52.2 us; with Bt warm
// (one copy, mostly in the last-level cache) 47.8-49.5 against 49.6-50.3 us.
// At 16 x 4096 x 4096 the two are equal (10.9 and 10.7 us).  Rings of 3 or 4
// slots, 2 waves per workgroup, or only 8 rows of A per slot for M <= 8 were
// no faster (52.8-61 us cold).
// Bt streaming variant (no barrier): the workgroup's W waves each own 16 Bt
// rows (16 columns of C) and stream them through a ring of R slots of their
// own, R - 1 256-deep chunks ahead (512 bytes of each row per chunk), as the
// row-major streaming kernel does for B; each slot also takes the chunk of
// the first MA rows of A (rows >= M copy row M - 1; lanes of rows >= MA read
// row MA - 1: their outputs are never stored).  A wave reads back only what
// it copied itself, so there is no barrier; every copy is a direct-to-LDS
// one, whose completion the hand-placed waits count.
constexpr int BTS_KC = 256;
constexpr int BTS_ROWB = BTS_KC * 2;  // 512 bytes of a row per chunk

template <bool GUARD, typename E = ElemF16, int W = 4, int MA = 16, int R = 2>
__global__ __launch_bounds__(64 * W, 1) void gemm_relu_smallm_bt_stream_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ Bt, uint16_t* __restrict__ C, int64_t M, int64_t N,
    int64_t K, int64_t lda, int64_t ldbt, int64_t ldc, EpiArgs ep) {
    static_assert(MA == 2 || MA == 4 || MA == 8 || MA == 16, "rows of A per slot");
    static_assert(R >= 2 && R <= 4, "ring entries per wave");
    constexpr int BT_BYTES = 16 * BTS_ROWB;                // 8 KiB: the wave's 16 Bt rows
    constexpr int WSLOT = BT_BYTES + MA * BTS_ROWB;
    constexpr int CP_A = MA / 2;
    constexpr int OPS = 8 + CP_A;                          // copies per chunk
    __shared__ __attribute__((aligned(1024))) uint8_t lds[W * R * WSLOT];

    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t n_w = (int64_t)blockIdx.x * (16 * W) + 16 * wave;  // this wave's first column

    // Copy i of a chunk: rows 2i, 2i+1 (of the wave's 16 Bt rows, or of the
    // MA rows of A); lane -> row 2i + lane/32, LDS piece lane%32, which
    // holds global piece (lane%32) ^ (row % 16) of the row's 32.
    // (a wave wholly past N copies row N - 1 for all its rows, from a base
    // moved to that row; none of them is stored)
    const bool past = GUARD && n_w >= N;
    const int64_t n_first = past ? N - 1 : n_w;
    uint32_t off_bt[8], off_a[CP_A];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t row = 2u * i + (lane >> 5);
        const uint32_t piece = (lane & 31u) ^ (row & 15u);
        int64_t n = n_w + row;
        if (GUARD && n >= N) n = N - 1;
        off_bt[i] = past ? piece * 16u : (uint32_t)((n - n_w) * ldbt * 2 + piece * 16);
    }
#pragma unroll
    for (int i = 0; i < CP_A; ++i) {
        const uint32_t row = 2u * i + (lane >> 5);
        const uint32_t piece = (lane & 31u) ^ (row & 15u);
        const int64_t m = (int64_t)row < M ? (int64_t)row : M - 1;
        off_a[i] = (uint32_t)(m * lda * 2 + piece * 16);
    }
    const uint8_t* base_bt = reinterpret_cast<const uint8_t*>(Bt + n_first * ldbt);
    const uint8_t* base_a = reinterpret_cast<const uint8_t*>(A);
    const uint32_t ring = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds + wave * R * WSLOT;

    auto issue = [&](int64_t kc) {
        const uint32_t dst = ring + (uint32_t)(kc % R) * WSLOT;
        const int64_t kb = kc * BTS_ROWB;
#pragma unroll
        for (int i = 0; i < 8; ++i) tile2::dma16(base_bt + kb, off_bt[i], dst + i * 1024u);
#pragma unroll
        for (int i = 0; i < CP_A; ++i) tile2::dma16(base_a + kb, off_a[i], dst + BT_BYTES + i * 1024u);
    };

    // Operands of step s: Bt row l%16 and A row min(l%16, MA - 1), piece
    // 4 s + l/16 of the chunk.
    const uint32_t li = lane & 15u, lg = lane >> 4;
    const uint32_t ar = li < (uint32_t)MA ? li : (uint32_t)MA - 1u;
    f32x4 acc0 = f32x4{}, acc1 = f32x4{};
    const int64_t chunks = K / BTS_KC;
    for (int64_t c = 0; c < R - 1 && c < chunks; ++c) issue(c);
    for (int64_t kc = 0; kc < chunks; ++kc) {
        if (kc + R - 1 < chunks) {
            issue(kc + R - 1);  // into the slot chunk kc - 1 used, whose reads its MFMAs consumed
            tile2::wait_vmcnt<(R - 1) * OPS>();
        } else {
            tile2::wait_vmcnt<0>();
        }
        const uint8_t* slot = lds + wave * R * WSLOT + (kc % R) * WSLOT;
#pragma unroll
        for (int st = 0; st < BTS_KC / KSTEP; ++st) {
            const uint32_t piece = 4u * st + lg;
            const f16x8 b = *reinterpret_cast<const f16x8*>(slot + li * BTS_ROWB + ((piece ^ li) << 4));
            const f16x8 a = *reinterpret_cast<const f16x8*>(slot + BT_BYTES + ar * BTS_ROWB + ((piece ^ ar) << 4));
            if (st & 1) acc1 = E::mfma16(b, a, acc1);
            else acc0 = E::mfma16(b, a, acc0);
        }
    }

    // acc holds C^T: lane l, register r is C[m][n] with m = l%16 and
    // n = n_w + 4(l/16) + r.
    const int64_t m = li;
    if (m < M) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t n = n_w + 4 * lg + r;
            if (!GUARD || n < N) C[m * ldc + n] = epi_value<E>(acc0[r] + acc1[r], n, N, ep);
        }
    }
}

}  // namespace smallm
}  // namespace gr
