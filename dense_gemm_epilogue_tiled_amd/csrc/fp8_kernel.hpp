// fp8 (OCP e4m3) GEMM with the fused epilogue: C = act(scale * A * Bt^T + bias),
// A M x K and Bt N x K, both k-contiguous bytes, fp32 accumulation, fp16 or
// bfloat16 output.  gfx950's v_mfma_f32_32x32x64_f8f6f4 multiplies a 32 x 64
// block of e4m3 values by a 64 x 32 one per instruction, twice the rate of the
// fp16 instruction.
//
// Operand layout.  Each lane supplies 32 bytes (8 VGPRs) per operand: the 32
// rows of a block are the lanes mod 32, and the two lane halves split the 64
// k of the step.  Without scales, which k a given byte position stands for
// inside the instruction does not matter: A and B use the same positions
// for the same k, so filling both operands by one rule -- lane half h gets
// the two 16-byte chunks h and 2 + h (chunk 2s + h, s = 0, 1) of its row's
// 64-byte k strip -- pairs every A[m][k] with B[k][n] exactly once.  (With
// MX scales it does matter; see below.)  The output block follows the usual
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
// MX=true (OCP MX fp8: one E8M0 scale per 32 consecutive k of every row of
// A and Bt): here the k order inside the instruction matters.  The
// assignment above is the instruction's own (register quad s of lane half h
// holds k 32s + 16h .. 32s + 16h + 15 of the step), and the scale byte of
// lane (h, row) multiplies that row's 32-k block h, i.e. quad h of both lane
// halves; so the operands are fetched exactly as without scales, and lane
// half h supplies the scale of block 2kt + h of its row (measured: per-row
// and per-block scales both match the oracle only with this pairing).  The
// scales travel through LDS beside the ring: 4 bytes of each row (the blocks
// of two strips) per copy, with the copies of every even strip.
// MX=4 (OCP MX fp4: E2M1 elements, two per byte, one E8M0 scale per 32 k):
// the same kernel byte for byte -- a 64-byte strip row now holds 128 k --
// with two scaled fp4 instructions per strip and block pair (32 x 32 x 64,
// one 16-byte quad per lane: quad s of the strip, k 64s + 32h .. + 31 in
// lane half h, whose scale is that of block 4kt + 2s + h); the scales of a
// strip (4 blocks per row) travel with every strip's copies.
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

// The same block product with E8M0 scales: lane l scales the 32 bytes of
// its B operand by 2^(sb - 127) and those of its A operand by 2^(sa - 127)
// (the low byte of each scale word; see MX below for which k that is).
__device__ __forceinline__ f32x16 mfma_mx(const u32x4& b0, const u32x4& b1, const u32x4& a0, const u32x4& a1,
                                          f32x16 c, uint32_t sb, uint32_t sa) {
    const i32x8 bo = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
    const i32x8 ao = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bo, ao, c, 0, 0, 0, (int)sb, 0, (int)sa);
}

// One 32 x 32 x 64 product of OCP fp4 E2M1 operands (format code 4): one
// 16-byte quad (32 elements) per lane and operand, with E8M0 scales.
__device__ __forceinline__ f32x16 mfma_mx4(const u32x4& b, const u32x4& a, f32x16 c, uint32_t sb, uint32_t sa) {
    const i32x8 bo = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
    const i32x8 ao = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bo, ao, c, 4, 4, 0, (int)sb, 0, (int)sa);
}

// Copy of 4 bytes per lane from global memory into LDS (lane l writes LDS
// bytes [m0 + 4l, m0 + 4l + 4)); waits as for tile2::dma16.
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t lds_addr) {
    asm volatile(
        "s_nop 0\n\t"
        "global_load_lds_dword %0, %1"
        :
        : "v"(voff), "s"(base), "{m0}"(lds_addr)
        : "memory");
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
    // MX scales: slot q % SC_SLOTS holds 4 bytes (the E8M0 scales of strips
    // 2q and 2q + 1) of every A row, then of every Bt row, after the ring.
    static constexpr int SC_SLOTS = 4;
    static constexpr int SC_SLOT_BYTES = (BM + BN) * 4;
    static constexpr int SC_BASE = LDS_BYTES;
    static constexpr int LDS_BYTES_MX = LDS_BYTES + SC_SLOTS * SC_SLOT_BYTES;  // 136 or 68 KiB
    static constexpr int SC_COPIES = (BM + BN) / 256;  // 64-row scale copies per wave per even strip
    static_assert(BM % 64 == 0 && (SC_COPIES * THREADS / 64) * 64 == BM + BN, "scale copies cover every row");
};

__device__ __forceinline__ u32x4 read16(const GR_LDS uint8_t* p) { return *(const GR_LDS u32x4*)p; }

// E: output element type with the general epilogue (Epi<ElemF16> or
// Epi<ElemBF16>); ep.scale carries scale_a * scale_b.
// SPLIT=true (split-K, with a workspace): workgroup g covers tile g % tiles
// over the K range of split g / tiles (k_per_split bytes, a multiple of 64;
// no split is empty) and writes its unscaled fp32 sums to part[split][m][n];
// a second pass adds the splits in order and applies the epilogue.
// MX = 8 (MX fp8) or 4 (MX fp4; K, lda and ldb then count bytes, two
// elements each): SA (M x K/32, pitch ldsa) and SB (N x K/32, pitch ldsb)
// hold the E8M0 scales; 128 elements per two strips (fp8) or per strip
// (fp4), scale rows 4-byte aligned.  MX = 0: no scales.
template <int BMT, bool EDGE, typename E, bool SPLIT = false, int MX = 0>
__global__ __launch_bounds__(THREADS, Tile<BMT>::MIN_WAVES) void gemm_fp8_tile_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ Bt, uint16_t* __restrict__ C, int64_t M, int64_t N,
    int64_t K, int64_t lda, int64_t ldb, int64_t ldc, uint32_t tiles_m, uint32_t tiles_n, uint32_t group_m,
    int vec_c, float* __restrict__ part, int64_t k_per_split, const uint8_t* __restrict__ SA, int64_t ldsa,
    const uint8_t* __restrict__ SB, int64_t ldsb, EpiArgs ep) {
    static_assert(E::kGeneral, "the fp8 kernels use the general epilogue");
    static_assert(MX == 0 || MX == 8 || MX == 4, "scale formats: none, MX fp8, MX fp4");
    static_assert(!(MX && SPLIT), "the MX path has no split-K variant");
    using T = Tile<BMT>;
    constexpr int FM = T::FM, FN = T::FN, COPIES = T::COPIES;
    constexpr int SC_COPIES = MX ? T::SC_COPIES : 0;
    constexpr bool FP4 = MX == 4;
    constexpr uint32_t SC_EVERY = FP4 ? 1u : 2u;  // strips per 4-byte scale copy
    using tile2::a_off;
    using tile2::barrier;
    using tile2::dma16;
    using tile2::pin;
    using tile2::wait_vmcnt;

    __shared__ __attribute__((aligned(1024))) uint8_t lds[MX ? T::LDS_BYTES_MX : T::LDS_BYTES];

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
    // MX scale copy c of this wave: scale rows R = 64 (SC_COPIES w + c) +
    // lane of the slot (A rows 0 .. BM-1, then Bt rows); a copy never mixes
    // the two (64-row groups), so its base address is wave-uniform.
    const uint8_t* base_s[SC_COPIES > 0 ? SC_COPIES : 1];
    uint32_t off_s[SC_COPIES > 0 ? SC_COPIES : 1];
    if constexpr (MX) {
#pragma unroll
        for (int c = 0; c < SC_COPIES; ++c) {
            const uint32_t g0 = 64u * ((uint32_t)SC_COPIES * wave + (uint32_t)c);  // first row of the group
            const bool is_a = g0 < (uint32_t)T::BM;
            uint32_t r = (is_a ? g0 : g0 - (uint32_t)T::BM) + lane;
            if constexpr (EDGE) {
                if (is_a) r = m0 + r < M ? r : (uint32_t)(M - 1 - m0);
                else r = n0 + r < N ? r : (uint32_t)(N - 1 - n0);
            }
            base_s[c] = is_a ? SA + m0 * ldsa : SB + n0 * ldsb;
            off_s[c] = (uint32_t)(r * (is_a ? ldsa : ldsb));
        }
    }
    // Scale copies of strip kt (kt % SC_EVERY == 0): the blocks of strips
    // kt .. kt + SC_EVERY - 1.
    auto dma_scale = [&](uint32_t kt, int c) {
        if constexpr (MX != 0) {
            const uint32_t q = kt / SC_EVERY;
            dma4(base_s[c] + 4 * (int64_t)q, off_s[c],
                 lds_base + T::SC_BASE + (q % T::SC_SLOTS) * T::SC_SLOT_BYTES +
                     256u * ((uint32_t)SC_COPIES * wave + (uint32_t)c));
        }
    };
    auto issue = [&](uint32_t slot, uint32_t kt) {
#pragma unroll
        for (int c = 0; c < 2 * COPIES; ++c) dma_one(slot, kt, c);
        if (MX && kt % SC_EVERY == 0u) {
#pragma unroll
            for (int c = 0; c < SC_COPIES; ++c) dma_scale(kt, c);
        }
    };

    // ---- fragment addresses: row wm*WAVE_T + 32i + lane%32 (A) or
    // wn*WAVE_T + 32j + lane%32 (Bt), chunk 2s + lane/32; block i or j is
    // 2 KiB on.
    const GR_LDS uint8_t* lds_p = (const GR_LDS uint8_t*)lds;
    const uint32_t ar = wm * T::WAVE_T + (lane & 31u);
    const uint32_t br = wn * T::WAVE_T + (lane & 31u);
    const GR_LDS uint8_t* a_ptr[2];
    const GR_LDS uint8_t* b_ptr[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const uint32_t ch = 2u * (uint32_t)s + (lane >> 5);
        a_ptr[s] = lds_p + a_off(ar, ch);
        b_ptr[s] = lds_p + T::A_BYTES + a_off(br, ch);
    }
    // MX: scale byte of strip kt for A row ar + 32i (Bt row br + 32j) at
    // slot (kt/SC_EVERY) % SC_SLOTS, row * 4 + b + lane/32 with b = 2 (kt %
    // 2) (fp8) or 2s for the fp4 instruction s.
    const uint32_t sc_a = T::SC_BASE + ar * 4u + (lane >> 5);
    const uint32_t sc_b = T::SC_BASE + ((uint32_t)T::BM + br) * 4u + (lane >> 5);

    constexpr int SCS = FP4 ? 2 : 1;  // scale bytes per row block and strip
    struct Frags {
        u32x4 a[2][FM];
        u32x4 b[2][FN];
        uint32_t sa[SCS][FM];
        uint32_t sb[SCS][FN];
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    // The 2 (FM + FN) fragment reads of one strip, in the order the next
    // step's MFMAs (block row i, then column j) first need them: A0, B0 ..,
    // A1 .., each as its two chunks.
    // MX adds SCS (FM + FN) one-byte scale reads (strip kt) after them.
    constexpr int FRAG_READS = 2 * (FM + FN);
    constexpr int READS = FRAG_READS + (MX ? SCS * (FM + FN) : 0);
    auto read_one = [&](Frags& f, uint32_t slot, uint32_t kt, int r) {
        if (r < FRAG_READS) {
            const int q = r >> 1, s = r & 1;
            const uint32_t so = slot * T::STAGE_BYTES;
            if (q == 0) f.a[s][0] = read16(a_ptr[s] + so);
            else if (q <= FN) f.b[s][q - 1] = read16(b_ptr[s] + so + 2048u * (q - 1));
            else f.a[s][q - FN] = read16(a_ptr[s] + so + 2048u * (q - FN));
        } else if constexpr (MX != 0) {
            const int x0 = r - FRAG_READS, sc = x0 / (FM + FN), x = x0 % (FM + FN);
            const uint32_t bsel = FP4 ? 2u * (uint32_t)sc : 2u * (kt & 1u);
            const uint32_t so = ((kt / SC_EVERY) % T::SC_SLOTS) * T::SC_SLOT_BYTES + bsel;
            if (x < FM) f.sa[sc][x] = *(const GR_LDS uint8_t*)(lds_p + sc_a + so + 128u * x);
            else f.sb[sc][x - FM] = *(const GR_LDS uint8_t*)(lds_p + sc_b + so + 128u * (x - FM));
        }
    };
    // fp4: instruction t covers quad t / (FM FN) of the strip.
    constexpr int MFMAS = (FP4 ? 2 : 1) * FM * FN;
    auto mfma_one = [&](const Frags& f, int t) {
        const int q = t / (FM * FN), u = t % (FM * FN);
        const int i = u / FN, j = u % FN;
        if constexpr (FP4)
            acc[i][j] = mfma_mx4(f.b[q][j], f.a[q][i], acc[i][j], f.sb[q][j], f.sa[q][i]);
        else if constexpr (MX == 8)
            acc[i][j] = mfma_mx(f.b[0][j], f.b[1][j], f.a[0][i], f.a[1][i], acc[i][j], f.sb[0][j], f.sa[0][i]);
        else
            acc[i][j] = mfma(f.b[0][j], f.b[1][j], f.a[0][i], f.a[1][i], acc[i][j]);
    };

    const uint32_t KT = (uint32_t)(k_len / BK);  // >= 1, whole strips only

    // Prologue: strips 0, 1, 2 in flight; strip 0 landed and read.
    // (MX fp8: the copies of strips 0 and 2 carry scales; MX fp4: all.)
    constexpr int N1 = 2 * COPIES + (FP4 ? SC_COPIES : 0);  // copies of strip 1
    constexpr int N2 = 2 * COPIES + SC_COPIES;              // copies of strip 2
    issue(0, 0);
    if (KT > 1) issue(1, 1);
    if (KT > 2) issue(2, 2);
    if (KT > 2) wait_vmcnt<N1 + N2>();
    else if (KT > 1) wait_vmcnt<N1>();
    else wait_vmcnt<0>();
    barrier();

    Frags f0, f1;
#pragma unroll
    for (int r = 0; r < READS; ++r) read_one(f0, 0, 0, r);

    // Steady step on strip kt (slot SLOT = kt % 4), fragments in `cur`: PRE
    // MFMAs; wait for this wave's copies of strip kt+1; barrier (all copies of
    // kt+1 landed, every wave done with the slot of kt-1); then the other
    // MFMAs with the READS reads of strip kt+1 and the 2*COPIES copies of
    // strip kt+3 (every third operation) spread evenly behind them.
    // MX fp8: the batch of an even strip adds SC_COPIES scale copies; strip
    // kt+2 (the batch allowed to stay in flight) is even when SLOT is, strip
    // kt+3 (the batch issued here) when SLOT is odd.  MX fp4: every batch.
    constexpr int PRE = 2;
    auto step = [&](auto slot_c, uint32_t kt, Frags& cur, Frags& nxt) {
        constexpr uint32_t SLOT = decltype(slot_c)::value;
        constexpr int IN_FLIGHT = 2 * COPIES + (FP4 || SLOT % 2 == 0 ? SC_COPIES : 0);
        constexpr int CPS = 2 * COPIES + (FP4 || SLOT % 2 == 1 ? SC_COPIES : 0);
        constexpr int OPS = READS + CPS;
        constexpr int PER = (OPS + (MFMAS - PRE) - 1) / (MFMAS - PRE);
        auto copy_one = [&](int cp) {
            if (cp < 2 * COPIES) dma_one((SLOT + 3) % STAGES, kt + 3, cp);
            else dma_scale(kt + 3, cp - 2 * COPIES);
        };
#pragma unroll
        for (int t = 0; t < PRE; ++t) mfma_one(cur, t);
        pin();
        wait_vmcnt<IN_FLIGHT>();
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
                    if (k % 3 == 1 && cp < CPS) {
                        copy_one(cp);
                        ++cp;
                    } else if (rd < READS) {
                        read_one(nxt, (SLOT + 1) % STAGES, kt + 1, rd);
                        ++rd;
                    } else {
                        copy_one(cp);
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
            if (kt + 2 < KT) {
                if (MX && (kt + 2) % SC_EVERY == 0u) wait_vmcnt<2 * COPIES + SC_COPIES>();
                else wait_vmcnt<2 * COPIES>();
            } else {
                wait_vmcnt<0>();
            }
            barrier();
        }
        pin();
        if (kt + 3 < KT) issue((kt + 3) % STAGES, kt + 3);
        pin();
        if (more) {
#pragma unroll
            for (int r = 0; r < READS; ++r) read_one(nxt, (kt + 1) % STAGES, kt + 1, r);
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

// E8M0 scale of the 32-element block holding element k of row `row`: 127 (a
// factor of 1) outside [0, rows) x [0, K), so that the zeros loaded there
// stay zero.
__device__ __forceinline__ uint32_t load_scale(const uint8_t* __restrict__ S, int64_t ld, int64_t row, int64_t rows,
                                               int64_t k, int64_t K) {
    return (row < rows && k < K) ? (uint32_t)S[row * ld + k / 32] : 127u;
}

// MX = 8 or 4: E8M0 scales SA (M x K/32, pitch ldsa) and SB (N x K/32, pitch
// ldsb), K (elements) a multiple of 32; for MX fp4 the K, lda and ldb passed
// here count bytes (two elements each).
template <typename E, int MX = 0>
__global__ __launch_bounds__(256) void gemm_fp8_guarded_kernel(const uint8_t* __restrict__ A,
                                                              const uint8_t* __restrict__ Bt,
                                                              uint16_t* __restrict__ C, int64_t M, int64_t N,
                                                              int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                                                              uint32_t tiles_n, int vec_c,
                                                              const uint8_t* __restrict__ SA, int64_t ldsa,
                                                              const uint8_t* __restrict__ SB, int64_t ldsb,
                                                              EpiArgs ep) {
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
    // two kernels feed the matrix cores identical operands.  MX fp8: lane
    // half h supplies the scale of block k0/32 + h of its row; MX fp4: chunk
    // s of lane half h holds elements 2 k0 + 64s + 32h .. + 31, one block.
    for (int64_t k0 = 0; k0 < K; k0 += BK) {
        u32x4 a[2][2], b[2][2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int64_t kc = k0 + 32 * s + 16 * h;
#pragma unroll
            for (int i = 0; i < 2; ++i) a[i][s] = load16(A, lda, m0 + 32 * i + r, M, kc, K);
#pragma unroll
            for (int j = 0; j < 2; ++j) b[j][s] = load16(Bt, ldb, n0 + 32 * j + r, N, kc, K);
        }
        if constexpr (MX == 8) {
            const int64_t kb = k0 + 32 * h;
            uint32_t sa[2], sb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) sa[i] = load_scale(SA, ldsa, m0 + 32 * i + r, M, kb, K);
#pragma unroll
            for (int j = 0; j < 2; ++j) sb[j] = load_scale(SB, ldsb, n0 + 32 * j + r, N, kb, K);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = mfma_mx(b[j][0], b[j][1], a[i][0], a[i][1], acc[i][j], sb[j], sa[i]);
        } else if constexpr (MX == 4) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int64_t ke = 2 * k0 + 64 * s + 32 * h;  // first element of this lane's block
                uint32_t sa[2], sb[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) sa[i] = load_scale(SA, ldsa, m0 + 32 * i + r, M, ke, 2 * K);
#pragma unroll
                for (int j = 0; j < 2; ++j) sb[j] = load_scale(SB, ldsb, n0 + 32 * j + r, N, ke, 2 * K);
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) acc[i][j] = mfma_mx4(b[j][s], a[i][s], acc[i][j], sb[j], sa[i]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = mfma(b[j][0], b[j][1], a[i][0], a[i][1], acc[i][j]);
        }
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
