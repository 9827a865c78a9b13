// C ABI of the fused fp16 GEMM + ReLU library for MI355X (gfx950).
//
// Host side: argument validation, a pure planner (which kernel, tile and grid)
// and the launch on the caller's stream.  The operation and its contract are
// documented in include/gemm_relu.h.  No allocation, no synchronisation and
// no per-call state: the only state is a once-per-device check that the
// device is a gfx950.  Scratch memory, where a path uses it, is the caller's
// workspace.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/gemm_relu.h"
#include "fp8_kernel.hpp"
#include "pack_kernel.hpp"
#include "probe_kernel.hpp"
#include "smallm_kernel.hpp"
#include "tile2_kernel.hpp"
#include "tile128_kernel.hpp"
#include "tile3_kernel.hpp"
#include "tile3t_kernel.hpp"
#include "tile_kernel.hpp"

// Scratch of gemm_relu_f16_noalloc: a static device array, one copy per GPU
// the library runs on.  Host code never uses this name as an address (on the
// host it is only a stand-in for the symbol); the device address of each
// GPU's copy comes from hipGetSymbolAddress, looked up once per device with
// that device current (scratch_on_current_device below).
static __device__ __align__(256) uint8_t scratch[GR_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kVersion = 200;  // 0.2.0: gr_plan_t.plain_order
constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxSpanBytes = int64_t(1) << 62;
constexpr int kGroupM = 4;          // tile rows per workgroup-order group
constexpr int kSmallMThreshold = 16;  // rows of A handled by the small-M split and Bt kernels
constexpr int kSmallMMaxRows = 64;    // rows the single-pass small-M kernel handles (4 blocks of 16)
constexpr int64_t kPackMinMacs = int64_t(1) << 30;  // smallest M*N*K the planner packs for
constexpr int64_t kWorkspaceAlign = 256;            // required alignment of a workspace (bytes)
#ifndef GR_SMALLM_WAVES
#define GR_SMALLM_WAVES 8
#endif
#ifndef GR_SMALLM_UNROLL
#define GR_SMALLM_UNROLL 2
#endif
constexpr int kSmallMWaves = GR_SMALLM_WAVES;    // waves per small-M workgroup
constexpr int kSmallMUnroll = GR_SMALLM_UNROLL;  // 32-deep K steps per load group

// Number of bytes spanned by a rows x cols matrix with pitch ld (0 if empty);
// -1 when it does not fit the library's limits.
int64_t span_bytes(int64_t rows, int64_t cols, int64_t ld) {
    if (rows == 0 || cols == 0) return 0;
    // (rows - 1) * ld + cols elements, checked against 2^62 bytes.
    const int64_t limit = kMaxSpanBytes / 2;
    if (rows - 1 > 0 && ld > (limit - cols) / (rows - 1)) return -1;
    return ((rows - 1) * ld + cols) * 2;
}

bool overlaps(uintptr_t a, int64_t alen, uintptr_t b, int64_t blen) {
    if (alen <= 0 || blen <= 0) return false;
    return a < b + (uintptr_t)blen && b < a + (uintptr_t)alen;
}

// Widest fp16 vector (8, 2 or 1 elements) every row start of a pitched matrix
// is aligned to.
int vec_width(uintptr_t p, int64_t ld) {
    if (p % 16 == 0 && ld % 8 == 0) return 8;
    if (p % 4 == 0 && ld % 2 == 0) return 2;
    return 1;
}

// Width of the stores into C (16-bit elements): 8, wherever C's rows start.
// The memory system of this part splits a misaligned access itself (the
// direct-to-LDS copies read from any 2-byte address on the same footing),
// and one 16-byte store per 8 elements beats eight 2-byte ones: at 4099 x
// 3071 x 2050 with a row pitch of 3071, 2-byte stores cost 13.7 us more.
// Partial row segments at the edges of C take at most two stores
// (epi::store_run).
int vec_width_c(uintptr_t, int64_t) { return 8; }

// Argument checks.  The workspace (ws, ws_bytes) is optional: a size of 0
// means none; a negative size or a misaligned workspace is GR_ERR_INVALID_ARG,
// NULL with a positive size GR_ERR_NULL_PTR, overlap with A, B or C
// GR_ERR_ALIAS.
int validate(int64_t M, int64_t N, int64_t K, uintptr_t A, int64_t lda, uintptr_t B, int64_t ldb,
             uintptr_t C, int64_t ldc, uintptr_t ws = 0, int64_t ws_bytes = 0) {
    if (M < 0 || N < 0 || K < 0) return GR_ERR_INVALID_DIM;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return GR_ERR_TOO_LARGE;
    const int64_t kmin = K > 1 ? K : 1, nmin = N > 1 ? N : 1;
    if (lda < kmin || ldb < nmin || ldc < nmin) return GR_ERR_INVALID_LD;
    const bool a_used = M > 0 && K > 0 && N > 0;
    const bool b_used = K > 0 && N > 0 && M > 0;
    const bool c_used = M > 0 && N > 0;
    if ((a_used && !A) || (b_used && !B) || (c_used && !C)) return GR_ERR_NULL_PTR;
    const int64_t sa = a_used ? span_bytes(M, K, lda) : 0;
    const int64_t sb = b_used ? span_bytes(K, N, ldb) : 0;
    const int64_t sc = c_used ? span_bytes(M, N, ldc) : 0;
    if (sa < 0 || sb < 0 || sc < 0) return GR_ERR_TOO_LARGE;
    if (overlaps(C, sc, A, sa) || overlaps(C, sc, B, sb)) return GR_ERR_ALIAS;
    if (ws_bytes < 0) return GR_ERR_INVALID_ARG;
    if (ws_bytes > 0) {
        if (!ws) return GR_ERR_NULL_PTR;
        if (ws % kWorkspaceAlign != 0) return GR_ERR_INVALID_ARG;
        if (overlaps(ws, ws_bytes, A, sa) || overlaps(ws, ws_bytes, B, sb) || overlaps(ws, ws_bytes, C, sc))
            return GR_ERR_ALIAS;
    }
    return GR_OK;
}

bool smallm_ok(int64_t M, int64_t N, int64_t K, uintptr_t A, int64_t lda, uintptr_t B, int64_t ldb) {
    (void)N;
    (void)K;
    return M >= 1 && M <= kSmallMThreshold && A % 16 == 0 && lda % 8 == 0 && B % 8 == 0 && ldb % 4 == 0;
}

// The single-pass small-M kernel with 2 or 4 blocks of 16 rows of A.
bool smallm_rows_ok(int64_t M, int64_t N, int64_t K, uintptr_t A, int64_t lda, uintptr_t B, int64_t ldb) {
    (void)N;
    (void)K;
    return M >= 1 && M <= kSmallMMaxRows && A % 16 == 0 && lda % 8 == 0 && B % 8 == 0 && ldb % 4 == 0;
}

// The streaming small-M kernel (gemm_relu_smallm_stream_kernel): M <= 16, K
// a positive multiple of 32 (whole 32-row slots), 16-byte rows of A, B of
// any alignment and a pitch within 32-bit copy offsets, N of at least one
// column block of nb.  Without a split it runs with 64-column blocks; the
// split uses 128-column blocks (256-byte row pieces, the faster read
// pattern, measured 6.5 TB/s for the first pass at 8 x 16384 x 8192).
constexpr int kStreamNB = 64, kStreamW = 4, kStreamR = 2;  // single pass: 64-column blocks, 4 waves x 2 slots
constexpr int kStreamSplitNB = 128, kStreamSplitW = 2, kStreamSplitR = 2;  // split: 128 columns, 2 waves x 2 slots
constexpr int kStreamTaW = 8;  // A given transposed (gathered into registers): 8 waves x 1 slot
// The copy offsets are 32-bit: 32 rows of B and at most 64 rows of A per
// workgroup keep them below 2^32 for pitches up to 2^25 elements.
constexpr int64_t kStreamMaxLd = int64_t(1) << 25;
bool smallm_stream_ok(int64_t M, int64_t N, int64_t K, uintptr_t A, int64_t lda, int64_t ldb, int64_t nb,
                      int64_t max_rows = kSmallMThreshold) {
    return M >= 1 && M <= max_rows && K > 0 && K % 32 == 0 && A % 16 == 0 && lda % 8 == 0 && N >= nb &&
           lda <= kStreamMaxLd && ldb <= kStreamMaxLd;
}

// Split-K layout of the small-M path: S splits of k_per_split (a multiple of
// 32) over ceil(N / NB) column blocks, about 256 workgroups in all, and the
// fp32 partial sums S x M x N in the workspace.  The streaming kernel
// (stream = true, NB = 128) splits whenever its column blocks leave CUs
// idle, with at least four 32-row slots per split; otherwise the
// register-staged split kernel (NB = 256, 16-byte rows of B) where the
// single pass has fewer than 256 strips of 64 columns.
struct SmallMSplit {
    int64_t splits = 0, k_per_split = 0, n_blocks = 0, bytes = 0;
    bool stream = false;
};
constexpr int64_t kSmallMMaxSplits = 64;

// The register-staged split pays only where the single-pass kernel (one
// workgroup per 64-column strip) leaves CUs idle: measured at N = 16384 (256
// strips) its first pass is 4% faster, and its second pass costs more.
bool smallm_split_pays(int64_t N) { return (N + gr::smallm::NB - 1) / gr::smallm::NB < 256; }

bool smallm_split_layout(int64_t M, int64_t N, int64_t K, uintptr_t A, int64_t lda, uintptr_t B, int64_t ldb,
                         SmallMSplit* sp) {
    using namespace gr::smallm;
    if (K < 1 || N < 1) return false;
    SmallMSplit q;
    int64_t nb, min_steps;
    if (smallm_stream_ok(M, N, K, A, lda, ldb, kStreamSplitNB)) {
        q.stream = true;
        nb = kStreamSplitNB;
        min_steps = kStreamSplitW * kStreamSplitR;  // a full ring per wave
    } else if (smallm_ok(M, N, K, A, lda, B, ldb) && B % 16 == 0 && ldb % 8 == 0) {
        nb = SPLIT_NB;
        min_steps = 2;
    } else {
        return false;
    }
    q.n_blocks = (N + nb - 1) / nb;
    int64_t S = 256 / q.n_blocks;
    S = S < 1 ? 1 : (S > kSmallMMaxSplits ? kSmallMMaxSplits : S);
    const int64_t ksteps = (K + KSTEP - 1) / KSTEP;
    if (S > ksteps / min_steps) S = ksteps / min_steps > 0 ? ksteps / min_steps : 1;
    q.k_per_split = (ksteps + S - 1) / S * KSTEP;
    q.splits = (K + q.k_per_split - 1) / q.k_per_split;  // no empty split
    q.bytes = (q.splits * M * N * 4 + kWorkspaceAlign - 1) / kWorkspaceAlign * kWorkspaceAlign;
    *sp = q;
    return true;
}

// Whether the planner takes the split (with a big enough workspace).
bool smallm_split_wanted(int64_t N, const SmallMSplit& sp) {
    return sp.splits >= 2 && (sp.stream || smallm_split_pays(N));
}

// Conditions of the pipelined direct-to-LDS kernels: 16-byte aligned rows of
// A and B (every copy is a whole 16-byte chunk), K a positive multiple of the
// 32-deep strip and pitches small enough for 32-bit per-lane copy offsets.
// Any M, N and C layout (the 256 x 256 kernels, used only for M >= 256, move
// a partial last tile row up to end at row M; the 128 x 128 kernel clamps
// rows past M).
bool tile_fast_ok(int64_t M, int64_t N, int64_t K, uintptr_t A, int64_t lda, uintptr_t B, int64_t ldb) {
    using namespace gr::tile2;
    return M >= 1 && N >= 1 && K % BK == 0 && K > 0 && vec_width(A, lda) == 8 && vec_width(B, ldb) == 8 &&
           lda <= MAX_LDA && ldb <= MAX_LDB;
}

// The persistent tile loop: whole 256 x 256 tiles, K % 64 == 0 (the 64-deep
// A strips), 16-byte stores into C (its 32-row epilogue writes 16-byte
// segments).
constexpr int64_t kPersistentWorkgroups = 256;  // one per CU
bool tile_persistent_ok(int64_t M, int64_t N, int64_t K, uintptr_t A, int64_t lda, uintptr_t B, int64_t ldb,
                        uintptr_t C, int64_t ldc) {
    using namespace gr::tile3;
    return tile_fast_ok(M, N, K, A, lda, B, ldb) && M % BM == 0 && N % BN == 0 && K % BKA == 0 &&
           vec_width_c(C, ldc) == 8;
}

// The pipelined 256 x 256 kernel in place on misaligned rows and a K that
// is no multiple of 64 (tile3's UA variant): M and N of at least one tile
// (the last tile row and column move to end at M and N), K > 128 (the tail
// of 1..64 plus at least two 64-deep strips) and pitches within its 32-bit
// copy offsets.  The planner takes it when there are also more than 128
// tiles (as for the aligned 256 x 256 kernel), and with fewer where neither
// the packed copy (workspace) nor the streaming kernel applies; the forced
// hook only needs the kernel's own conditions.
bool tile_unaligned_ok(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb);

// 256 x 256 tiles unless they would fill less than half of one wave of
// workgroups over the 256 CUs (or M < 256): then 128 x 128 tiles, which give
// four times as many workgroups.
constexpr int64_t kSmallTileMaxLargeTiles = 128;
bool use_large_tiles(int64_t M, int64_t N) {
    using namespace gr::tile2;
    if (M < BM) return false;
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    return tiles > kSmallTileMaxLargeTiles;
}

// Blocks of 64 rows x 64 columns on the streaming kernel (TILE_STREAM): in
// each workgroup the waves (4, or 8 up to 256 blocks: tile_stream_waves)
// take the 32-row slots of K in turn through rings of their own, with no
// barrier in the loop, and add their partial sums in LDS at the end.
// Against 128 x 128 tiles this gives four times as many workgroups and a
// quarter of the K steps per wave.  A 4-wave block holds 64 KiB of LDS, so
// two are resident per CU and 512 fill one round of the 256 CUs.  Where it is planned (blocks = ceil(M / 64) x ceil(N / 64); us, back
// to back):
//  * aligned rows, against the 128 x 128 tile kernel: blocks <= 256 from
//    K = 256 (1024^3 7.4 against 12.3, 1024^2 x 256 5.4 against 5.6; at
//    K = 128 5.1 against 4.5) and <= 512 from K = 512 (1024 x 1536 x 512
//    7.4 against 8.0, 1024 x 2048 x 1024 10.4 against 12.4, x 8192 59.5
//    against 73.7; 1024 x 1536 x 256 6.4 against 5.8).  Beyond one round the
//    tiles win (1536^2 x 1024, 576 blocks: 14.9 against 12.6).  With a
//    workspace the split-K tile path comes first where it splits: it is
//    faster still at long K (1024^2 x 8192 29.4, 1024 x 2048 x 8192 48.3).
//  * rows of A or B not 16-byte aligned: the alternatives are the in-place
//    unaligned 256 x 256 kernel, the packed path (workspace) and the
//    guarded kernel.  Streaming wins up to one round (A misaligned, 1024^3:
//    7.9 against 31.5 unaligned, 16.2 packed, 75.5 guarded; 1024 x 2048 x
//    4096: 39.7 against 83.8, 45.6, 417) and, with no workspace, up to two
//    rounds (2048^2 x 4096: 74.1 against 84.1 unaligned; with a workspace
//    the packed path, 49.4).
// Needs K % 32 == 0 (whole slots) and N >= 64; its direct-to-LDS copies read
// any 2-byte aligned address (as the unaligned tile kernel's do), so rows of
// A and B of any alignment.
constexpr int64_t kTileStreamRows = 64;  // 4 blocks of 16 rows per workgroup
constexpr int64_t kTileStreamRound = 512;  // resident blocks: 2 per CU x 256 CUs
// Up to 256 blocks (one per CU) 8 waves take the slots of a block instead of
// 4 (128 KiB of LDS: twice the copies in flight per CU).  Measured, back to
// back: 1024^3 6.93 against 7.32 us, 512 x 1024 x 2048 8.44 against 9.74,
// 1024^2 x 256 5.05 against 5.39; with 512 blocks they would take two rounds
// (1024 x 2048 x 1024: 12.41 against 10.15).
constexpr int kTileStreamWOne = 8;
int tile_stream_waves(int64_t blocks) { return blocks <= 256 ? kTileStreamWOne : kStreamW; }
// Workgroup order of the row-blocked grid.  All blocks of a launch that fits
// one round are resident together, so what counts is how many distinct
// column blocks of B (and row blocks of A) each XCD's L2 holds.  In plain
// row-major order (workgroup j nb + cb runs block (j, cb) on XCD (j nb + cb)
// mod 8) XCD x gets, over the row blocks j, the column blocks cb with cb = x
// - j nb (mod 8): 8 / gcd(nb, 8) of the 8 residues, so an eighth of B when
// nb % 8 == 0, a quarter when nb % 8 == 4, half when nb % 4 == 2 and all of
// B when nb is odd.  Unless nb % 4 == 0 the XCD renumbering with groups of 4
// row blocks is faster (1088 x 1856 x 8192, nb = 29: 95.5 us against 66.3;
// 1024 x 1984 x 4096, nb = 31: 50.0 against 33.8; nb = 18, 22, 30: 10-20%
// faster at K = 8192); with nb % 4 == 0 plain order is as fast or faster
// (1152 x 1792 x 8192: 63.0 against 70.5; 960 x 2048 x 8192: 57.1 against
// 67.5).
constexpr int32_t kTileStreamGroupM = 4;
bool tile_stream_plain_order(int64_t N) { return ((N + kStreamNB - 1) / kStreamNB) % 4 == 0; }
bool tile_stream_ok(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb) {
    return M >= 1 && K > 0 && K % 32 == 0 && N >= kStreamNB && lda <= kStreamMaxLd && ldb <= kStreamMaxLd;
}
int64_t tile_stream_blocks(int64_t M, int64_t N) {
    return ((M + kTileStreamRows - 1) / kTileStreamRows) * ((N + kStreamNB - 1) / kStreamNB);
}
// Aligned rows: where the streaming path beats the 128 x 128 tile kernel.
bool tile_stream_beats_tiles(int64_t blocks, int64_t K) {
    return (blocks <= 256 && K >= 256) || (blocks <= kTileStreamRound && K >= 512);
}
// With a workspace the split-K tile path usually beats the streaming path
// (1024^2 x 8192: 30.2 against 32.5 us; 512 x 1024 x 8192, 128 blocks: 22.0
// against 30.5), but where the streaming path fills every CU with one 8-wave
// block (129-256 blocks) up to K = 4096 it is the faster one (1024^2 x 4096:
// 18.9 against 20.6; 128 x 8192 x 4096: 18.9 against 23.2).  There the
// planner streams and asks for no workspace.
bool tile_stream_before_split(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb) {
    const int64_t blocks = tile_stream_blocks(M, N);
    return M > kSmallMMaxRows && tile_stream_ok(M, N, K, lda, ldb) && blocks > 128 && blocks <= 256 && K <= 4096 &&
           tile_stream_beats_tiles(blocks, K);
}

// Up to 64 rows of A without a split: one row of 64 x 64 blocks on the
// streaming kernel (8 waves per block up to 256 blocks: twice the copies in
// flight of the small-M kernel's 4) where its blocks leave most CUs idle and
// B is large enough for that to count.  Measured back to back (us, small-M
// kernel / streaming): 64 x 4096 x 4096 30.5 / 19.1, 16 x 4096 x 4096 19.8 /
// 14.5, 8 x 2048 x 4096 16.4 / 12.7, 8 x 8192 x 1024 6.53 / 6.06, 64 x 1024
// x 256 5.00 / 4.90; but 8 x 1024 x 2048 5.85 / 7.55, 16 x 8192 x 512 4.34 /
// 4.97, and with 256 blocks and B cold 8 x 16384 x 8192 46.4 / 51.9.
bool tile_stream_small_m_pays(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb) {
    if (!tile_stream_ok(M, N, K, lda, ldb)) return false;
    const int64_t blocks = tile_stream_blocks(M, N);
    if (blocks > 128) return false;
    if (M > 32) return true;
    const double kn = (double)K * (double)N;
    return N >= 1024 && kn >= 8388608.0 && (blocks <= 64 || kn <= 33554432.0);
}

bool tile_unaligned_ok(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb) {
    using namespace gr::tile3;
    return M >= BM && N >= BN && K > 2 * BKA && lda <= MAX_LDA && ldb <= MAX_LDB;
}

// Split-K of the 128 x 128 tile path (workspace): when the small tiles do not
// fill the chip and K is long, each tile's K range is split S ways (S x tiles
// <= 256, one workgroup per CU; at least 8 strips per split, S <= 16); fp32
// partial sums S x M x N go to the workspace and a second pass adds them in
// order and applies ReLU.  Filling both workgroup slots of every CU (S x
// tiles <= 512) measured 10-25% slower: the extra partial sums cost more than
// the second slot gains (fp16 1024 x 1024 x 4096: 27.1 -> 23.4 us, 128 x 8192
// x 4096: 30.3 -> 26.1 us; fp8 128 x 8192 x 8192: 30.4 -> 23.7 us).  The
// planner splits only when that saves each workgroup at least 64 strips
// (measured, fp16 and fp8 alike: 64 saved strips win -- fp16 256 x 8192 x
// 4096 40.1 -> 34.4 us, fp8 256 x 8192 x 8192 39.0 -> 32.3 us; 32 saved
// strips tie; fp8 1024 x 1024 x 4096 with 48 saved loses, 15.6 -> 19.3 us).
constexpr int64_t kTileSplitMinSavedStrips = 64;
struct TileSplit {
    int64_t splits = 0, k_per_split = 0, bytes = 0;
};
constexpr int64_t kTileMaxSplits = 16;
constexpr int64_t kTileMinSplitK = 256;

// bk: K per strip of the kernel (32 fp16 elements; 64 for the fp8 kernel,
// whose strips take the same matrix-core time); min_k: shortest split.
bool tile_split_layout(int64_t M, int64_t N, int64_t K, bool allow_one, TileSplit* ts,
                       int64_t bk = gr::tile128::BK, int64_t min_k = kTileMinSplitK) {
    using namespace gr::tile128;
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    int64_t S = 256 / tiles;
    if (S > K / min_k) S = K / min_k;
    if (S > kTileMaxSplits) S = kTileMaxSplits;
    if (S < 1) S = 1;
    const int64_t strips = K / bk;
    // Splitting pays only while the unsplit grid fills at most half of the
    // CUs' workgroup slots: with 224-256 tiles a split into 2 measured 15-20%
    // slower (8192 x 28672 x 64..256, 256 x 16384 x 8192).
    if (!allow_one && tiles > kSmallTileMaxLargeTiles) return false;
    if (!allow_one && (S < 2 || strips * (S - 1) < kTileSplitMinSavedStrips * S)) return false;
    TileSplit q;
    q.k_per_split = (strips + S - 1) / S * bk;
    q.splits = (K + q.k_per_split - 1) / q.k_per_split;  // no empty split
    q.bytes = (q.splits * M * N * 4 + kWorkspaceAlign - 1) / kWorkspaceAlign * kWorkspaceAlign;
    *ts = q;
    return true;
}

// Whole tiles of size bm x bn: the edge-free variant of those kernels.
bool tile_whole(int64_t M, int64_t N, int64_t bm, int64_t bn) { return M % bm == 0 && N % bn == 0; }

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// The packed variant of the pipelined path: which operands are copied into
// the workspace, and the problem the tile kernel then sees.  K is padded to a
// multiple of 64 (zeros) unless it already is a multiple of 32; an operand is
// copied when its rows are not 16-byte aligned or when K is padded.
struct Pack {
    bool a = false, b = false;  // operand copied into the workspace
    int64_t kp = 0;             // K of the packed problem
    int64_t lda_p = 0, ldb_p = 0;
    int64_t off_b = 0;          // byte offset of the copy of B in the workspace
    int64_t bytes = 0;          // workspace bytes used
};

bool pack_layout(int64_t M, int64_t N, int64_t K, uintptr_t A, int64_t lda, uintptr_t B, int64_t ldb, Pack* pk) {
    using namespace gr::tile2;
    if (M < 1 || N < 1 || K < 1) return false;
    Pack q;
    q.kp = K % BK == 0 ? K : round_up(K, 2 * BK);
    q.a = vec_width(A, lda) != 8 || lda > MAX_LDA || q.kp != K;
    q.b = vec_width(B, ldb) != 8 || ldb > MAX_LDB || q.kp != K;
    if (!q.a && !q.b) return false;  // the pipelined path runs in place
    q.lda_p = q.a ? q.kp : lda;
    q.ldb_p = q.b ? round_up(N, 8) : ldb;
    if (q.lda_p > MAX_LDA || q.ldb_p > MAX_LDB) return false;
    const int64_t a_bytes = q.a ? round_up(M * q.kp * 2, kWorkspaceAlign) : 0;
    const int64_t b_bytes = q.b ? q.kp * q.ldb_p * 2 : 0;
    q.off_b = a_bytes;
    q.bytes = a_bytes + b_bytes;
    *pk = q;
    return true;
}

void fill_plan(int path, int64_t M, int64_t N, int64_t K, uintptr_t A, int64_t lda, uintptr_t B, int64_t ldb, uintptr_t C,
               int64_t ldc, const Pack& pk, const SmallMSplit& sp, const TileSplit& ts, gr_plan_t* p) {
    std::memset(p, 0, sizeof(*p));
    p->path = path;
    if (path == GR_PATH_TILE_UNALIGNED || path == GR_PATH_TILE_PERSISTENT) {
        using namespace gr::tile3;
        p->block_m = BM;
        p->block_n = BN;
        p->block_k = BK;
        p->stages = B_SLOTS;
        p->threads = THREADS;
        p->grid = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
        if (path == GR_PATH_TILE_PERSISTENT && p->grid > kPersistentWorkgroups) p->grid = kPersistentWorkgroups;
        p->vec_a = vec_width(A, lda);
        p->vec_b = vec_width(B, ldb);
        p->vec_c = vec_width_c(C, ldc);
        p->group_m = kGroupM;
        p->split_k = 1;
    } else if (path == GR_PATH_TILE || path == GR_PATH_TILE_PACKED || path == GR_PATH_TILE_SPLIT) {
        const bool large = path != GR_PATH_TILE_SPLIT && use_large_tiles(M, N);
        const int64_t bm = large ? gr::tile2::BM : gr::tile128::BM;
        const int64_t bn = large ? gr::tile2::BN : gr::tile128::BN;
        p->block_m = (int32_t)bm;
        p->block_n = (int32_t)bn;
        p->block_k = gr::tile2::BK;
        p->stages = large ? gr::tile2::STAGES : gr::tile128::STAGES;
        p->threads = gr::tile2::THREADS;
        p->grid = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
        p->vec_a = 8;
        p->vec_b = 8;
        p->vec_c = vec_width_c(C, ldc);
        p->group_m = kGroupM;
        p->split_k = 1;
        if (path == GR_PATH_TILE_PACKED) {
            p->packed = (pk.a ? 1 : 0) | (pk.b ? 2 : 0);
            p->workspace = pk.bytes;
        } else if (path == GR_PATH_TILE_SPLIT) {
            p->grid *= ts.splits;
            p->split_k = (int32_t)ts.splits;
            p->workspace = ts.bytes;
        }
    } else if (path == GR_PATH_TILE_EDGE) {
        using namespace gr::tile;
        p->block_m = BM;
        p->block_n = BN;
        p->block_k = BK;
        p->stages = 2;
        p->threads = THREADS;
        p->grid = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
        p->vec_a = vec_width(A, lda);
        p->vec_b = vec_width(B, ldb);
        p->vec_c = vec_width_c(C, ldc);
        p->group_m = kGroupM;
    } else if (path == GR_PATH_SMALL_M_SPLIT) {
        using namespace gr::smallm;
        p->block_m = MAX_M;
        p->block_n = sp.stream ? kStreamSplitNB : SPLIT_NB;
        p->block_k = KSTEP;
        p->stages = sp.stream ? 1 : SPLIT_U;
        p->threads = sp.stream ? 64 * kStreamSplitW : SPLIT_THREADS;
        p->grid = sp.n_blocks * sp.splits;
        p->vec_a = 8;
        p->vec_b = sp.stream ? vec_width(B, ldb) : 8;
        p->vec_c = 1;
        p->group_m = 1;
        p->workspace = sp.bytes;
        p->split_k = (int32_t)sp.splits;
    } else if (path == GR_PATH_TILE_STREAM) {
        p->block_m = (int32_t)kTileStreamRows;
        p->block_n = kStreamNB;
        p->block_k = gr::smallm::KSTEP;
        p->stages = kStreamR;
        p->grid = ((N + kStreamNB - 1) / kStreamNB) * ((M + kTileStreamRows - 1) / kTileStreamRows);
        p->threads = 64 * tile_stream_waves(p->grid);
        p->vec_a = 8;
        p->vec_b = 8;  // 16-byte copies from any 2-byte address
        p->vec_c = 1;
        p->plain_order = tile_stream_plain_order(N);
        p->group_m = p->plain_order ? 1 : kTileStreamGroupM;  // plain: row-major
        p->split_k = 1;
    } else if (path == GR_PATH_SMALL_M) {
        using namespace gr::smallm;
        // the streaming kernel where it applies (vec_b 8: 16-byte copies of B
        // from any address), else the register-staged one (vec_b 4)
        const bool stream = smallm_stream_ok(M, N, K, A, lda, ldb, kStreamNB, kSmallMMaxRows);
        p->block_m = M <= MAX_M ? MAX_M : (M <= 2 * MAX_M ? 2 * MAX_M : 4 * MAX_M);  // rows per workgroup
        p->block_n = stream ? kStreamNB : NB;
        p->block_k = KSTEP;
        p->stages = stream ? 1 : kSmallMUnroll;
        p->threads = 64 * (stream ? kStreamW : kSmallMWaves);
        p->grid = (N + p->block_n - 1) / p->block_n;
        p->vec_a = 8;
        p->vec_b = stream ? 8 : 4;
        p->vec_c = 1;
        p->group_m = 1;
        p->split_k = 1;
    }
}

int choose_path(int64_t M, int64_t N, int64_t K, uintptr_t A, int64_t lda, uintptr_t B, int64_t ldb,
                uintptr_t C, int64_t ldc, int64_t ws_bytes, Pack* pk, SmallMSplit* sp, TileSplit* ts) {
    (void)C;
    (void)ldc;
    if (M == 0 || N == 0) return GR_PATH_NONE;
    if (K > 0 && (smallm_ok(M, N, K, A, lda, B, ldb) || smallm_stream_ok(M, N, K, A, lda, ldb, kStreamNB))) {
        if (ws_bytes > 0 && smallm_split_layout(M, N, K, A, lda, B, ldb, sp) && smallm_split_wanted(N, *sp) &&
            sp->bytes <= ws_bytes)
            return GR_PATH_SMALL_M_SPLIT;
        return tile_stream_small_m_pays(M, N, K, lda, ldb) ? GR_PATH_TILE_STREAM : GR_PATH_SMALL_M;
    }
    const bool fast = tile_fast_ok(M, N, K, A, lda, B, ldb);
    if (fast && ws_bytes > 0 && !use_large_tiles(M, N) && !tile_stream_before_split(M, N, K, lda, ldb) &&
        tile_split_layout(M, N, K, false, ts) && ts->bytes <= ws_bytes)
        return GR_PATH_TILE_SPLIT;
    if (K > 0 &&
        (smallm_rows_ok(M, N, K, A, lda, B, ldb) || smallm_stream_ok(M, N, K, A, lda, ldb, kStreamNB, kSmallMMaxRows)) &&
        (N + gr::smallm::NB - 1) / gr::smallm::NB <= 256)
        return tile_stream_small_m_pays(M, N, K, lda, ldb) ? GR_PATH_TILE_STREAM : GR_PATH_SMALL_M;
    // Up to 64 rows reach here when the small-M kernels cannot take A's rows
    // (not 16-byte aligned): the streaming kernel takes them in place (8 x
    // 4096 x 4096 with A's rows odd: 14.3 us against 182 for the guarded
    // kernel; 64 x 16384 x 4096 29.0 against 215).
    const bool stream = (M > kSmallMMaxRows || !fast) && tile_stream_ok(M, N, K, lda, ldb);
    const int64_t blocks = stream ? tile_stream_blocks(M, N) : 0;
    if (stream && (fast ? tile_stream_beats_tiles(blocks, K) : blocks <= kTileStreamRound))
        return GR_PATH_TILE_STREAM;
    if (fast) return GR_PATH_TILE;
    if (tile_unaligned_ok(M, N, K, lda, ldb) && use_large_tiles(M, N)) return GR_PATH_TILE_UNALIGNED;
    if (ws_bytes > 0 && pack_layout(M, N, K, A, lda, B, ldb, pk) && pk->bytes <= ws_bytes &&
        (double)M * (double)N * (double)K >= (double)kPackMinMacs)
        return GR_PATH_TILE_PACKED;
    if (stream && blocks <= 2 * kTileStreamRound) return GR_PATH_TILE_STREAM;
    // Misaligned rows or a ragged K without a workspace: the in-place
    // unaligned kernel wherever it applies (1024 x 2048 x 4096 with A's rows
    // misaligned: 83.6 us against 417 for the guarded kernel; 512 x 1024 x
    // 256 with B's: 18.3 against 21.5).
    if (tile_unaligned_ok(M, N, K, lda, ldb)) return GR_PATH_TILE_UNALIGNED;
    return GR_PATH_TILE_EDGE;
}


// ---- device check (once per device) ------------------------------------------

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GR_ERR_NO_DEVICE;
    if (dev >= kMaxDevices) return GR_ERR_UNSUPPORTED_DEVICE;
    int state = g_device_state[dev].load(std::memory_order_acquire);
    if (state == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GR_ERR_NO_DEVICE;
        state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_device_state[dev].store(state, std::memory_order_release);
    }
    return state == 1 ? GR_OK : GR_ERR_UNSUPPORTED_DEVICE;
}

// Device address of the current device's copy of `scratch`, looked up once
// per device (thread-safe) and kept for later calls.
std::atomic<uintptr_t> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

int scratch_on_current_device(uint8_t** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GR_ERR_NO_DEVICE;
    if (dev >= kMaxDevices) return GR_ERR_UNSUPPORTED_DEVICE;
    uintptr_t p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == 0) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch_ptr[dev].load(std::memory_order_acquire);
        if (p == 0) {
            void* q = nullptr;
            if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return GR_ERR_LAUNCH;
            p = reinterpret_cast<uintptr_t>(q);
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = reinterpret_cast<uint8_t*>(p);
    return GR_OK;
}

// ---- launches ----------------------------------------------------------------

template <typename... Args>
int launch(void (*kernel)(Args...), int64_t grid, int threads, hipStream_t stream, Args... args) {
    void* argv[] = {static_cast<void*>(&args)...};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3((uint32_t)grid), dim3(threads), argv,
                                   0, stream);
    return e == hipSuccess ? GR_OK : GR_ERR_LAUNCH;
}

// The order word the tile kernels take (tile_of_workgroup): the group of tile
// rows, bit 31 set for the plain order (tile order follows the workgroup id).
uint32_t order_word(const gr_plan_t& p) {
    return (uint32_t)p.group_m | (p.plain_order ? gr::kNoXcdRemap : 0u);
}

// Second pass of every split path: sum the fp32 partial sums in order and
// apply the epilogue (4 outputs per thread when rows hold a multiple of 4).
template <typename E>
int launch_reduce(const float* part, uint16_t* C, int64_t M, int64_t N, int64_t ldc, int64_t splits, int vec_c,
                  const gr::EpiArgs& ep, hipStream_t stream) {
    const bool vec4 = N % 4 == 0;
    const int64_t items = vec4 ? M * N / 4 : M * N;
    int64_t blocks = (items + 255) / 256;
    if (blocks > 2048) blocks = 2048;
    const int s = (int)splits;
    if (vec4)
        return launch(gr::smallm::gemm_relu_smallm_reduce_kernel<E, true>, blocks, 256, stream, part, C, M, N, ldc, s,
                      vec_c, ep);
    return launch(gr::smallm::gemm_relu_smallm_reduce_kernel<E, false>, blocks, 256, stream, part, C, M, N, ldc, s,
                  vec_c, ep);
}

template <bool GUARD, int VA, int VB, typename E>
int launch_tile(const gr_plan_t& p, int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                const uint16_t* B, int64_t ldb, uint16_t* C, int64_t ldc, const gr::EpiArgs& ep, hipStream_t stream) {
    using namespace gr::tile;
    const uint32_t tiles_m = (uint32_t)((M + BM - 1) / BM);
    const uint32_t tiles_n = (uint32_t)((N + BN - 1) / BN);
    return launch(gemm_relu_tile_kernel<GUARD, VA, VB, false, E>, p.grid, THREADS, stream, A, B, C, M, N, K, lda,
                  ldb, ldc, tiles_m, tiles_n, order_word(p), (int)p.vec_c, ep);
}

template <bool GUARD, int VA, typename E>
int launch_tile_vb(const gr_plan_t& p, int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                   const uint16_t* B, int64_t ldb, uint16_t* C, int64_t ldc, const gr::EpiArgs& ep,
                   hipStream_t stream) {
    switch (p.vec_b) {
        case 8: return launch_tile<GUARD, VA, 8, E>(p, M, N, K, A, lda, B, ldb, C, ldc, ep, stream);
        case 2: return launch_tile<GUARD, VA, 2, E>(p, M, N, K, A, lda, B, ldb, C, ldc, ep, stream);
        default: return launch_tile<GUARD, VA, 1, E>(p, M, N, K, A, lda, B, ldb, C, ldc, ep, stream);
    }
}

// Copy the operands the layout names into the workspace (one launch).
int launch_pack(const Pack& pk, int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                const uint16_t* B, int64_t ldb, uint8_t* ws, hipStream_t stream) {
    using gr::pack::Job;
    const Job none{nullptr, nullptr, 0, 8, 0, 0, 0};
    const Job ja = pk.a ? Job{A, reinterpret_cast<uint16_t*>(ws), lda, pk.lda_p, M, K, M} : none;
    const Job jb = pk.b ? Job{B, reinterpret_cast<uint16_t*>(ws + pk.off_b), ldb, pk.ldb_p, K, N, pk.kp} : none;
    // UNROLL 16-byte groups per thread, at most 8192 workgroups per job
    // (then a grid-stride loop).
    auto blocks = [](const Job& j) -> int64_t {
        constexpr int64_t per_block = (int64_t)gr::pack::THREADS * gr::pack::UNROLL;
        const int64_t groups = j.rows_d * (j.ldd / 8);
        const int64_t b = (groups + per_block - 1) / per_block;
        return b < 8192 ? b : 8192;
    };
    const int64_t ba = blocks(ja), bb = blocks(jb);
    if (ba + bb == 0) return GR_OK;
    return launch(gr::pack::pack_kernel, ba + bb, gr::pack::THREADS, stream, ja, jb, (uint32_t)ba);
}

// E: element type of A, B and C and the epilogue (the workspace paths exist
// for the fp16 ReLU only); ep: bias and activation of the general epilogue.
template <typename E>
int run(const gr_plan_t& p, int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* B,
        int64_t ldb, uint16_t* C, int64_t ldc, const Pack& pk, const SmallMSplit& sp, const TileSplit& ts,
        uint8_t* ws, const gr::EpiArgs& ep, hipStream_t stream) {
    switch (p.path) {
        case GR_PATH_NONE: return GR_OK;
        case GR_PATH_SMALL_M_SPLIT: {
            using namespace gr::smallm;
            float* part = reinterpret_cast<float*>(ws);
            if (sp.stream) {
                const int st = launch(
                    gemm_relu_smallm_stream_kernel<kStreamSplitNB, kStreamSplitW, kStreamSplitR, stream::PARTIAL, E>,
                    p.grid, p.threads, stream, A, B, C, part, M, N, K, lda, ldb, ldc, sp.k_per_split,
                    (uint32_t)sp.n_blocks, 0u, ep);
                if (st != GR_OK) return st;
                return launch_reduce<E>(part, C, M, N, ldc, sp.splits, p.vec_c, ep, stream);
            }
            const bool whole = N % SPLIT_NB == 0 && K % KSTEP == 0;
            const uint32_t nb = (uint32_t)sp.n_blocks;
            int st = whole ? launch(gemm_relu_smallm_split_kernel<false, E>, p.grid, SPLIT_THREADS, stream, A, B,
                                    part, M, N, K, lda, ldb, sp.k_per_split, nb)
                           : launch(gemm_relu_smallm_split_kernel<true, E>, p.grid, SPLIT_THREADS, stream, A, B, part,
                                    M, N, K, lda, ldb, sp.k_per_split, nb);
            if (st != GR_OK) return st;
            return launch_reduce<E>(part, C, M, N, ldc, sp.splits, p.vec_c, ep, stream);
        }
        case GR_PATH_TILE_SPLIT: {
            using namespace gr::tile128;
            float* part = reinterpret_cast<float*>(ws);
            const bool whole = tile_whole(M, N, BM, BN);
            const uint32_t tiles_m = (uint32_t)((M + BM - 1) / BM);
            const uint32_t tiles_n = (uint32_t)((N + BN - 1) / BN);
            const uint32_t gm = order_word(p);
            const int vc = p.vec_c;
            const int64_t kps = ts.k_per_split;
            int st = whole ? launch(gemm_relu_tile128_kernel<false, true, false, E>, p.grid, THREADS, stream, A, B,
                                    C, M, N, K, lda, ldb, ldc, tiles_m, tiles_n, gm, vc, part, kps, ep)
                           : launch(gemm_relu_tile128_kernel<true, true, false, E>, p.grid, THREADS, stream, A, B, C,
                                    M, N, K, lda, ldb, ldc, tiles_m, tiles_n, gm, vc, part, kps, ep);
            if (st != GR_OK) return st;
            return launch_reduce<E>(part, C, M, N, ldc, ts.splits, p.vec_c, ep, stream);
        }
        case GR_PATH_TILE_PACKED: {
            const int st = launch_pack(pk, M, N, K, A, lda, B, ldb, ws, stream);
            if (st != GR_OK) return st;
            gr_plan_t q = p;
            q.path = GR_PATH_TILE;
            const uint16_t* Ap = pk.a ? reinterpret_cast<const uint16_t*>(ws) : A;
            const uint16_t* Bp = pk.b ? reinterpret_cast<const uint16_t*>(ws + pk.off_b) : B;
            return run<E>(q, M, N, pk.kp, Ap, pk.lda_p, Bp, pk.ldb_p, C, ldc, pk, sp, ts, ws, ep, stream);
        }
        case GR_PATH_TILE: {
            const int64_t bm = p.block_m, bn = p.block_n;
            const bool whole = tile_whole(M, N, bm, bn);
            const uint32_t tiles_m = (uint32_t)((M + bm - 1) / bm);
            const uint32_t tiles_n = (uint32_t)((N + bn - 1) / bn);
            const uint32_t gm = order_word(p);
            const int vc = p.vec_c;
            if (bm == gr::tile128::BM) {
                using namespace gr::tile128;
                float* no_part = nullptr;
                const int64_t no_split = 0;
                if (whole)
                    return launch(gemm_relu_tile128_kernel<false, false, false, E>, p.grid, THREADS, stream, A, B, C,
                                  M, N, K, lda, ldb, ldc, tiles_m, tiles_n, gm, vc, no_part, no_split, ep);
                return launch(gemm_relu_tile128_kernel<true, false, false, E>, p.grid, THREADS, stream, A, B, C, M,
                              N, K, lda, ldb, ldc, tiles_m, tiles_n, gm, vc, no_part, no_split, ep);
            }
            if (K % gr::tile3::BKA == 0) {
                using namespace gr::tile3;
                if (whole)
                    return launch(gemm_relu_tile3_kernel<false, E>, p.grid, THREADS, stream, A, B, C, M, N, K,
                                  lda, ldb, ldc, tiles_m, tiles_n, gm, vc, ep);
                return launch(gemm_relu_tile3_kernel<true, E>, p.grid, THREADS, stream, A, B, C, M, N, K, lda,
                              ldb, ldc, tiles_m, tiles_n, gm, vc, ep);
            }
            using namespace gr::tile2;
            if (whole)
                return launch(gemm_relu_tile2_kernel<false, false, E>, p.grid, THREADS, stream, A, B, C, M, N, K, lda,
                              ldb, ldc, tiles_m, tiles_n, gm, vc, ep);
            return launch(gemm_relu_tile2_kernel<true, false, E>, p.grid, THREADS, stream, A, B, C, M, N, K, lda, ldb,
                          ldc, tiles_m, tiles_n, gm, vc, ep);
        }
        case GR_PATH_TILE_PERSISTENT: {
            using namespace gr::tile3;
            const uint32_t tiles_m = (uint32_t)(M / BM), tiles_n = (uint32_t)(N / BN);
            if constexpr (E::kGeneral) {
                // the bias + activation epilogue stages fp32 blocks through
                // all of LDS: the same tiles, one workgroup each
                return launch(gemm_relu_tile3_kernel<false, E>, (int64_t)tiles_m * tiles_n, THREADS, stream, A, B, C,
                              M, N, K, lda, ldb, ldc, tiles_m, tiles_n, order_word(p), (int)p.vec_c, ep);
            } else {
                return launch(gemm_relu_tile3_kernel<false, E, false, true>, p.grid, THREADS, stream, A, B, C, M, N,
                              K, lda, ldb, ldc, tiles_m, tiles_n, order_word(p), (int)p.vec_c, ep);
            }
        }
        case GR_PATH_TILE_UNALIGNED: {
            using namespace gr::tile3;
            const uint32_t tiles_m = (uint32_t)((M + BM - 1) / BM);
            const uint32_t tiles_n = (uint32_t)((N + BN - 1) / BN);
            return launch(gemm_relu_tile3_kernel<true, E, true>, p.grid, THREADS, stream, A, B, C, M, N, K, lda, ldb,
                          ldc, tiles_m, tiles_n, order_word(p), (int)p.vec_c, ep);
        }
        case GR_PATH_TILE_EDGE:
            switch (p.vec_a) {
                case 8: return launch_tile_vb<true, 8, E>(p, M, N, K, A, lda, B, ldb, C, ldc, ep, stream);
                case 2: return launch_tile_vb<true, 2, E>(p, M, N, K, A, lda, B, ldb, C, ldc, ep, stream);
                default: return launch_tile_vb<true, 1, E>(p, M, N, K, A, lda, B, ldb, C, ldc, ep, stream);
            }
        case GR_PATH_TILE_STREAM: {
            using namespace gr::smallm;
            const uint32_t nb = (uint32_t)((N + kStreamNB - 1) / kStreamNB);
            static_assert(kTileStreamRows == 4 * MAX_M, "4 blocks of 16 rows per workgroup");
            if (p.threads == 64 * kTileStreamWOne)
                return launch(
                    gemm_relu_smallm_stream_kernel<kStreamNB, kTileStreamWOne, kStreamR, stream::WHOLE, E, false, 4, true>,
                    p.grid, p.threads, stream, A, B, C, static_cast<float*>(nullptr), M, N, K, lda, ldb, ldc, K, nb,
                    order_word(p), ep);
            return launch(gemm_relu_smallm_stream_kernel<kStreamNB, kStreamW, kStreamR, stream::WHOLE, E, false, 4, true>,
                          p.grid, p.threads, stream, A, B, C, static_cast<float*>(nullptr), M, N, K, lda, ldb, ldc, K,
                          nb, order_word(p), ep);
        }
        case GR_PATH_SMALL_M: {
            using namespace gr::smallm;
            if (p.vec_b == 8) {
                // the streaming kernel with 1, 2 or 4 blocks of 16 rows of A
                float* no_part = nullptr;
                if (M <= MAX_M)
                    return launch(gemm_relu_smallm_stream_kernel<kStreamNB, kStreamW, kStreamR, stream::WHOLE, E>,
                                  p.grid, p.threads, stream, A, B, C, no_part, M, N, K, lda, ldb, ldc, K,
                                  (uint32_t)p.grid, 0u, ep);
                if (M <= 2 * MAX_M)
                    return launch(
                        gemm_relu_smallm_stream_kernel<kStreamNB, kStreamW, kStreamR, stream::WHOLE, E, false, 2>,
                        p.grid, p.threads, stream, A, B, C, no_part, M, N, K, lda, ldb, ldc, K, (uint32_t)p.grid, 0u, ep);
                return launch(gemm_relu_smallm_stream_kernel<kStreamNB, kStreamW, kStreamR, stream::WHOLE, E, false, 4>,
                              p.grid, p.threads, stream, A, B, C, no_part, M, N, K, lda, ldb, ldc, K,
                              (uint32_t)p.grid, 0u, ep);
            }
            const bool whole = N % NB == 0 && K % KSTEP == 0;
            constexpr int W = kSmallMWaves, U = kSmallMUnroll;
            if (M <= MAX_M) {
                if (whole)
                    return launch(gemm_relu_smallm_kernel<W, U, false, E, 1>, p.grid, p.threads, stream, A, B, C, M,
                                  N, K, lda, ldb, ldc, ep);
                return launch(gemm_relu_smallm_kernel<W, U, true, E, 1>, p.grid, p.threads, stream, A, B, C, M, N, K,
                              lda, ldb, ldc, ep);
            }
            if (M <= 2 * MAX_M) {
                if (whole)
                    return launch(gemm_relu_smallm_kernel<W, U, false, E, 2>, p.grid, p.threads, stream, A, B, C, M,
                                  N, K, lda, ldb, ldc, ep);
                return launch(gemm_relu_smallm_kernel<W, U, true, E, 2>, p.grid, p.threads, stream, A, B, C, M, N, K,
                              lda, ldb, ldc, ep);
            }
            // four row blocks: one load group per register set keeps the
            // kernel within its 256 registers per lane
            if (whole)
                return launch(gemm_relu_smallm_kernel<W, 1, false, E, 4>, p.grid, p.threads, stream, A, B, C, M, N, K,
                              lda, ldb, ldc, ep);
            return launch(gemm_relu_smallm_kernel<W, 1, true, E, 4>, p.grid, p.threads, stream, A, B, C, M, N, K, lda,
                          ldb, ldc, ep);
        }
        default: return GR_ERR_INVALID_PATH;
    }
}

// Validate, choose (or check a forced) path, fill the plan.  No HIP call.
// ws_known: the workspace pointer is real and is checked (a plan made from
// a size alone skips the pointer checks).
int plan_call(int64_t M, int64_t N, int64_t K, uintptr_t a, int64_t lda, uintptr_t b, int64_t ldb, uintptr_t c,
              int64_t ldc, uintptr_t ws, int64_t ws_bytes, bool ws_known, int forced, Pack* pk, SmallMSplit* sp,
              TileSplit* ts, gr_plan_t* p) {
    if (ws_bytes < 0) return GR_ERR_INVALID_ARG;
    int st = ws_known ? validate(M, N, K, a, lda, b, ldb, c, ldc, ws, ws_bytes)
                      : validate(M, N, K, a, lda, b, ldb, c, ldc);
    if (st != GR_OK) return st;
    int path = choose_path(M, N, K, a, lda, b, ldb, c, ldc, ws_bytes, pk, sp, ts);
    if (forced >= 0 && path != GR_PATH_NONE) {
        if (forced == GR_PATH_TILE) {
            if (!tile_fast_ok(M, N, K, a, lda, b, ldb)) return GR_ERR_INVALID_PATH;
        } else if (forced == GR_PATH_TILE_UNALIGNED) {
            if (!tile_unaligned_ok(M, N, K, lda, ldb)) return GR_ERR_INVALID_PATH;
        } else if (forced == GR_PATH_TILE_PERSISTENT) {
            if (!tile_persistent_ok(M, N, K, a, lda, b, ldb, c, ldc)) return GR_ERR_INVALID_PATH;
        } else if (forced == GR_PATH_SMALL_M) {
            if (K == 0 || !(smallm_rows_ok(M, N, K, a, lda, b, ldb) ||
                            smallm_stream_ok(M, N, K, a, lda, ldb, kStreamNB, kSmallMMaxRows)))
                return GR_ERR_INVALID_PATH;
        } else if (forced == GR_PATH_TILE_PACKED) {
            if (!pack_layout(M, N, K, a, lda, b, ldb, pk) || pk->bytes > ws_bytes) return GR_ERR_INVALID_PATH;
        } else if (forced == GR_PATH_TILE_SPLIT) {
            if (!tile_fast_ok(M, N, K, a, lda, b, ldb) || !tile_split_layout(M, N, K, true, ts) ||
                ts->bytes > ws_bytes)
                return GR_ERR_INVALID_PATH;
        } else if (forced == GR_PATH_SMALL_M_SPLIT) {
            if (!smallm_split_layout(M, N, K, a, lda, b, ldb, sp) || sp->bytes > ws_bytes) return GR_ERR_INVALID_PATH;
        } else if (forced == GR_PATH_TILE_STREAM) {
            if (!tile_stream_ok(M, N, K, lda, ldb)) return GR_ERR_INVALID_PATH;
        } else if (forced != GR_PATH_TILE_EDGE) {
            return GR_ERR_INVALID_PATH;
        }
        path = forced;
    }
    fill_plan(path, M, N, K, a, lda, b, ldb, c, ldc, *pk, *sp, *ts, p);
    return GR_OK;
}

static_assert(GR_ACT_NONE == gr::kActNone && GR_ACT_RELU == gr::kActRelu && GR_ACT_GELU == gr::kActGelu &&
                  GR_ACT_GELU_TANH == gr::kActGeluTanh && GR_ACT_SILU == gr::kActSilu &&
                  GR_ACT_SIGMOID == gr::kActSigmoid && GR_ACT_TANH == gr::kActTanh && gr::kActCount == 7,
              "activation codes of the C ABI and the kernels agree");

// Epilogue arguments of the fused-ReLU calls (their kernels ignore them).
const gr::EpiArgs kReluOnly{nullptr, gr::kActRelu, 1.0f};

// order: -1 keeps the planner's workgroup order; otherwise bits 0-30 are the
// group of tile rows (>= 1) and bit 31 turns the XCD renumbering off (the
// test hook gemm_relu_f16_forced_order).
int entry(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
          uint16_t* C, int64_t ldc, void* ws, int64_t ws_bytes, void* stream, int forced, int64_t order = -1) {
    Pack pk;
    SmallMSplit sp;
    TileSplit ts;
    gr_plan_t p;
    int st = plan_call(M, N, K, (uintptr_t)A, lda, (uintptr_t)B, ldb, (uintptr_t)C, ldc, (uintptr_t)ws, ws_bytes,
                       true, forced, &pk, &sp, &ts, &p);
    if (st != GR_OK) return st;
    if (order >= 0) {
        p.group_m = (int32_t)((uint32_t)order & ~gr::kNoXcdRemap);
        p.plain_order = ((uint32_t)order & gr::kNoXcdRemap) != 0;
    }
    if (p.path == GR_PATH_NONE) return GR_OK;
    st = check_device();
    if (st != GR_OK) return st;
    return run<gr::ElemF16>(p, M, N, K, A, lda, B, ldb, C, ldc, pk, sp, ts, static_cast<uint8_t*>(ws), kReluOnly,
                            static_cast<hipStream_t>(stream));
}

// bfloat16 operands and output; the same paths as fp16 (a workspace, when
// given, enables the packed and split paths).
int entry_bf16(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
               uint16_t* C, int64_t ldc, void* ws, int64_t ws_bytes, void* stream, int forced) {
    Pack pk;
    SmallMSplit sp;
    TileSplit ts;
    gr_plan_t p;
    int st = plan_call(M, N, K, (uintptr_t)A, lda, (uintptr_t)B, ldb, (uintptr_t)C, ldc, (uintptr_t)ws, ws_bytes,
                       true, forced, &pk, &sp, &ts, &p);
    if (st != GR_OK) return st;
    if (p.path == GR_PATH_NONE) return GR_OK;
    st = check_device();
    if (st != GR_OK) return st;
    return run<gr::ElemBF16>(p, M, N, K, A, lda, B, ldb, C, ldc, pk, sp, ts, static_cast<uint8_t*>(ws), kReluOnly,
                             static_cast<hipStream_t>(stream));
}

// Bias + activation epilogue (Base: element type), on the planner's paths.
// The bias (N values, or none) must not overlap C or the workspace.
template <typename Base>
int entry_epi(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
              const uint16_t* bias, int act, uint16_t* C, int64_t ldc, void* ws, int64_t ws_bytes, void* stream,
              int forced) {
    if (act < 0 || act >= gr::kActCount) return GR_ERR_INVALID_ARG;
    Pack pk;
    SmallMSplit sp;
    TileSplit ts;
    gr_plan_t p;
    int st = plan_call(M, N, K, (uintptr_t)A, lda, (uintptr_t)B, ldb, (uintptr_t)C, ldc, (uintptr_t)ws, ws_bytes,
                       true, forced, &pk, &sp, &ts, &p);
    if (st != GR_OK) return st;
    if (bias != nullptr && M > 0 && N > 0 &&
        (overlaps((uintptr_t)C, span_bytes(M, N, ldc), (uintptr_t)bias, 2 * N) ||
         overlaps((uintptr_t)ws, ws_bytes, (uintptr_t)bias, 2 * N)))
        return GR_ERR_ALIAS;
    if (p.path == GR_PATH_NONE) return GR_OK;
    st = check_device();
    if (st != GR_OK) return st;
    return run<gr::Epi<Base>>(p, M, N, K, A, lda, B, ldb, C, ldc, pk, sp, ts, static_cast<uint8_t*>(ws),
                              gr::EpiArgs{bias, act, 1.0f}, static_cast<hipStream_t>(stream));
}

bool known_path(int path) {
    return path == GR_PATH_TILE || path == GR_PATH_TILE_EDGE || path == GR_PATH_SMALL_M ||
           path == GR_PATH_TILE_PACKED || path == GR_PATH_SMALL_M_SPLIT || path == GR_PATH_TILE_SPLIT ||
           path == GR_PATH_TILE_UNALIGNED || path == GR_PATH_TILE_PERSISTENT || path == GR_PATH_TILE_STREAM;
}

bool needs_workspace(int path) {
    return path == GR_PATH_TILE_PACKED || path == GR_PATH_SMALL_M_SPLIT || path == GR_PATH_TILE_SPLIT;
}

// ---- B given transposed (Bt, N x K) -------------------------------------------

// Argument checks for the transposed-B calls: Bt is N x K with pitch ldbt >=
// max(1, K); otherwise as validate().
int validate_bt(int64_t M, int64_t N, int64_t K, uintptr_t A, int64_t lda, uintptr_t Bt, int64_t ldbt,
                uintptr_t C, int64_t ldc) {
    if (M < 0 || N < 0 || K < 0) return GR_ERR_INVALID_DIM;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return GR_ERR_TOO_LARGE;
    const int64_t kmin = K > 1 ? K : 1, nmin = N > 1 ? N : 1;
    if (lda < kmin || ldbt < kmin || ldc < nmin) return GR_ERR_INVALID_LD;
    const bool used = M > 0 && N > 0 && K > 0;
    const bool c_used = M > 0 && N > 0;
    if ((used && (!A || !Bt)) || (c_used && !C)) return GR_ERR_NULL_PTR;
    const int64_t sa = used ? span_bytes(M, K, lda) : 0;
    const int64_t sb = used ? span_bytes(N, K, ldbt) : 0;
    const int64_t sc = c_used ? span_bytes(M, N, ldc) : 0;
    if (sa < 0 || sb < 0 || sc < 0) return GR_ERR_TOO_LARGE;
    if (overlaps(C, sc, A, sa) || overlaps(C, sc, Bt, sb)) return GR_ERR_ALIAS;
    return GR_OK;
}

// Largest pitch for which the streaming small-M Bt kernel's per-lane copy
// offsets (16 rows of Bt or A from a wave's base) fit in 32 bits, with room.
constexpr int64_t kBtLdsMaxPitch = (int64_t(1) << 32) / (64 * 2) - 512;

// Small-M kernel for Bt: 16-byte rows of A and of Bt.
bool smallm_bt_ok(int64_t M, int64_t K, uintptr_t A, int64_t lda, uintptr_t Bt, int64_t ldbt) {
    return M >= 1 && M <= kSmallMThreshold && K > 0 && A % 16 == 0 && lda % 8 == 0 && Bt % 16 == 0 &&
           ldbt % 8 == 0;
}

// Pipelined kernels for Bt: 16-byte rows of A and Bt, K % 32 == 0; Bt is
// staged like A, so its pitch has A's limit.
bool tile_bt_ok(int64_t M, int64_t N, int64_t K, uintptr_t A, int64_t lda, uintptr_t Bt, int64_t ldbt) {
    using namespace gr::tile2;
    return M >= 1 && N >= 1 && K > 0 && K % BK == 0 && vec_width(A, lda) == 8 && vec_width(Bt, ldbt) == 8 &&
           lda <= MAX_LDA && ldbt <= MAX_LDA;
}

// The row-blocked streaming kernel with B given transposed (its BT mode):
// blocks of 16 rows of Bt are copied and read like those of A, with the same
// conditions (any alignment, pitch within the 32-bit copy offsets).  M > 16:
// fewer rows take the transposed-B small-M kernels.
bool tile_stream_bt_ok(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldbt) {
    return M > kSmallMThreshold && tile_stream_ok(M, N, K, lda, ldbt);
}
// Where it beats the transposed-B tile kernels.  Its copies of Bt move 64
// bytes of each row per slot (row-major B: 128), so with two blocks per CU it
// needs a longer K than the row-major streaming path (us, back to back):
// 1024^2 x 256 5.3 against 5.6 for the tiles, 32 x 4096 x 4096 17.1 against
// 35.6; with 384-512 blocks from K = 1024 (1024 x 2048 x 1024 11.2 against
// 12.4, x 2048 21.1 against 20.8, x 4096 33.5 against 37.8).
bool tile_stream_bt_beats_tiles(int64_t blocks, int64_t K) {
    return (blocks <= 256 && K >= 256) || (blocks <= kTileStreamRound && K >= 1024);
}

int choose_path_bt(int64_t M, int64_t N, int64_t K, uintptr_t A, int64_t lda, uintptr_t Bt, int64_t ldbt) {
    if (M == 0 || N == 0) return GR_PATH_NONE;
    if (smallm_bt_ok(M, K, A, lda, Bt, ldbt)) return GR_PATH_SMALL_M;
    // Rows of A or Bt not 16-byte aligned: the alternative is the guarded
    // kernel, which streaming beats at any size (1024^3 8.2 against 72.9 us,
    // 4096^2 x 1024, 4096 blocks: 72.9 against 108.7).
    if (tile_stream_bt_ok(M, N, K, lda, ldbt) &&
        (!tile_bt_ok(M, N, K, A, lda, Bt, ldbt) || tile_stream_bt_beats_tiles(tile_stream_blocks(M, N), K)))
        return GR_PATH_TILE_STREAM;
    if (tile_bt_ok(M, N, K, A, lda, Bt, ldbt)) return GR_PATH_TILE;
    return GR_PATH_TILE_EDGE;
}

void fill_plan_bt(int path, int64_t M, int64_t N, uintptr_t A, int64_t lda, uintptr_t Bt, int64_t ldbt, uintptr_t C,
                  int64_t ldc, gr_plan_t* p) {
    Pack pk;
    SmallMSplit sp;
    TileSplit ts;
    // K only matters to the row-major small-M plan, which this one replaces
    fill_plan(path == GR_PATH_SMALL_M ? GR_PATH_NONE : path, M, N, 0, A, lda, Bt, ldbt, C, ldc, pk, sp, ts, p);
    p->path = path;
    if (path == GR_PATH_TILE) {
        p->block_k = gr::tile2::BK;
        p->stages = gr::tile2::STAGES;
    } else if (path == GR_PATH_TILE_EDGE) {
        p->vec_b = vec_width(Bt, ldbt);
    } else if (path == GR_PATH_SMALL_M) {
        using namespace gr::smallm;
        p->block_m = MAX_M;
        p->block_n = BT_NB;
        p->block_k = KSTEP;
        p->stages = BT_U;
        p->threads = 64 * BT_WAVES;
        p->grid = (N + BT_NB - 1) / BT_NB;
        p->vec_a = 8;
        p->vec_b = 8;
        p->vec_c = 1;
        p->group_m = 1;
        p->split_k = 1;
    }
}

template <int VA, int VB, typename E>
int launch_tile_bt(const gr_plan_t& p, int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                   const uint16_t* Bt, int64_t ldbt, uint16_t* C, int64_t ldc, const gr::EpiArgs& ep,
                   hipStream_t stream) {
    using namespace gr::tile;
    const uint32_t tiles_m = (uint32_t)((M + BM - 1) / BM);
    const uint32_t tiles_n = (uint32_t)((N + BN - 1) / BN);
    return launch(gemm_relu_tile_kernel<true, VA, VB, true, E>, p.grid, THREADS, stream, A, Bt, C, M, N, K, lda, ldbt,
                  ldc, tiles_m, tiles_n, order_word(p), (int)p.vec_c, ep);
}

// E: ElemF16 (the fused ReLU; ep is ignored) or Epi<ElemF16 / ElemBF16>.
template <typename E>
int run_bt(const gr_plan_t& p, int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* Bt,
           int64_t ldbt, uint16_t* C, int64_t ldc, const gr::EpiArgs& ep, hipStream_t stream) {
    switch (p.path) {
        case GR_PATH_NONE: return GR_OK;
        case GR_PATH_SMALL_M: {
            using namespace gr::smallm;
            if (K % BTS_KC == 0 && ldbt <= kBtLdsMaxPitch && lda <= kBtLdsMaxPitch) {
                // K in whole 256-deep chunks: the streaming variant, 4 waves
                // of 16 columns each
                constexpr int W = 4;
                const int64_t grid = (N + 16 * W - 1) / (16 * W);
                const bool whole = N % (16 * W) == 0;
                if (whole)
                    return launch(gemm_relu_smallm_bt_stream_kernel<false, E, W, 16>, grid, 64 * W, stream, A, Bt, C,
                                  M, N, K, lda, ldbt, ldc, ep);
                return launch(gemm_relu_smallm_bt_stream_kernel<true, E, W, 16>, grid, 64 * W, stream, A, Bt, C, M,
                              N, K, lda, ldbt, ldc, ep);
            }
            const bool whole = N % BT_NB == 0 && K % KSTEP == 0;
            if (whole)
                return launch(gemm_relu_smallm_bt_kernel<false, E>, p.grid, p.threads, stream, A, Bt, C, M, N, K, lda,
                              ldbt, ldc, ep);
            return launch(gemm_relu_smallm_bt_kernel<true, E>, p.grid, p.threads, stream, A, Bt, C, M, N, K, lda,
                          ldbt, ldc, ep);
        }
        case GR_PATH_TILE: {
            const int64_t bm = p.block_m, bn = p.block_n;
            const bool whole = tile_whole(M, N, bm, bn);
            const uint32_t tiles_m = (uint32_t)((M + bm - 1) / bm);
            const uint32_t tiles_n = (uint32_t)((N + bn - 1) / bn);
            const uint32_t gm = order_word(p);
            const int vc = p.vec_c;
            if (bm == gr::tile128::BM) {
                using namespace gr::tile128;
                float* no_part = nullptr;
                const int64_t no_split = 0;
                if (whole)
                    return launch(gemm_relu_tile128_kernel<false, false, true, E>, p.grid, THREADS, stream, A, Bt, C,
                                  M, N, K, lda, ldbt, ldc, tiles_m, tiles_n, gm, vc, no_part, no_split, ep);
                return launch(gemm_relu_tile128_kernel<true, false, true, E>, p.grid, THREADS, stream, A, Bt, C, M, N,
                              K, lda, ldbt, ldc, tiles_m, tiles_n, gm, vc, no_part, no_split, ep);
            }
            if (K % gr::tile3t::BKS == 0) {
                using namespace gr::tile3t;
                if (whole)
                    return launch(gemm_relu_tile3t_kernel<false, E>, p.grid, THREADS, stream, A, Bt, C, M, N, K, lda,
                                  ldbt, ldc, tiles_m, tiles_n, gm, vc, ep);
                return launch(gemm_relu_tile3t_kernel<true, E>, p.grid, THREADS, stream, A, Bt, C, M, N, K, lda, ldbt,
                              ldc, tiles_m, tiles_n, gm, vc, ep);
            }
            using namespace gr::tile2;
            if (whole)
                return launch(gemm_relu_tile2_kernel<false, true, E>, p.grid, THREADS, stream, A, Bt, C, M, N, K, lda,
                              ldbt, ldc, tiles_m, tiles_n, gm, vc, ep);
            return launch(gemm_relu_tile2_kernel<true, true, E>, p.grid, THREADS, stream, A, Bt, C, M, N, K, lda,
                          ldbt, ldc, tiles_m, tiles_n, gm, vc, ep);
        }
        case GR_PATH_TILE_STREAM: {
            using namespace gr::smallm;
            const uint32_t nb = (uint32_t)((N + kStreamNB - 1) / kStreamNB);
            if (p.threads == 64 * kTileStreamWOne)
                return launch(gemm_relu_smallm_stream_kernel<kStreamNB, kTileStreamWOne, kStreamR, stream::WHOLE, E, false,
                                                             4, true, true>,
                              p.grid, p.threads, stream, A, Bt, C, static_cast<float*>(nullptr), M, N, K, lda, ldbt, ldc,
                              K, nb, order_word(p), ep);
            return launch(
                gemm_relu_smallm_stream_kernel<kStreamNB, kStreamW, kStreamR, stream::WHOLE, E, false, 4, true, true>,
                p.grid, p.threads, stream, A, Bt, C, static_cast<float*>(nullptr), M, N, K, lda, ldbt, ldc, K, nb,
                order_word(p), ep);
        }
        case GR_PATH_TILE_EDGE: {
            const int va = p.vec_a, vb = p.vec_b;
            if (va == 8 && vb == 8) return launch_tile_bt<8, 8, E>(p, M, N, K, A, lda, Bt, ldbt, C, ldc, ep, stream);
            if (va == 8 && vb == 2) return launch_tile_bt<8, 2, E>(p, M, N, K, A, lda, Bt, ldbt, C, ldc, ep, stream);
            if (va == 8) return launch_tile_bt<8, 1, E>(p, M, N, K, A, lda, Bt, ldbt, C, ldc, ep, stream);
            if (va == 2 && vb == 8) return launch_tile_bt<2, 8, E>(p, M, N, K, A, lda, Bt, ldbt, C, ldc, ep, stream);
            if (va == 2 && vb == 2) return launch_tile_bt<2, 2, E>(p, M, N, K, A, lda, Bt, ldbt, C, ldc, ep, stream);
            if (va == 2) return launch_tile_bt<2, 1, E>(p, M, N, K, A, lda, Bt, ldbt, C, ldc, ep, stream);
            if (vb == 8) return launch_tile_bt<1, 8, E>(p, M, N, K, A, lda, Bt, ldbt, C, ldc, ep, stream);
            if (vb == 2) return launch_tile_bt<1, 2, E>(p, M, N, K, A, lda, Bt, ldbt, C, ldc, ep, stream);
            return launch_tile_bt<1, 1, E>(p, M, N, K, A, lda, Bt, ldbt, C, ldc, ep, stream);
        }
        default: return GR_ERR_INVALID_PATH;
    }
}

int plan_call_bt(int64_t M, int64_t N, int64_t K, uintptr_t a, int64_t lda, uintptr_t bt, int64_t ldbt, uintptr_t c,
                 int64_t ldc, int forced, gr_plan_t* p) {
    int st = validate_bt(M, N, K, a, lda, bt, ldbt, c, ldc);
    if (st != GR_OK) return st;
    int path = choose_path_bt(M, N, K, a, lda, bt, ldbt);
    if (forced >= 0 && path != GR_PATH_NONE) {
        if (forced == GR_PATH_TILE) {
            if (!tile_bt_ok(M, N, K, a, lda, bt, ldbt)) return GR_ERR_INVALID_PATH;
        } else if (forced == GR_PATH_SMALL_M) {
            if (!smallm_bt_ok(M, K, a, lda, bt, ldbt)) return GR_ERR_INVALID_PATH;
        } else if (forced == GR_PATH_TILE_STREAM) {
            if (!tile_stream_bt_ok(M, N, K, lda, ldbt)) return GR_ERR_INVALID_PATH;
        } else if (forced != GR_PATH_TILE_EDGE) {
            return GR_ERR_INVALID_PATH;
        }
        path = forced;
    }
    fill_plan_bt(path, M, N, a, lda, bt, ldbt, c, ldc, p);
    return GR_OK;
}

int entry_bt(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* Bt, int64_t ldbt,
             uint16_t* C, int64_t ldc, void* stream, int forced) {
    gr_plan_t p;
    int st = plan_call_bt(M, N, K, (uintptr_t)A, lda, (uintptr_t)Bt, ldbt, (uintptr_t)C, ldc, forced, &p);
    if (st != GR_OK) return st;
    if (p.path == GR_PATH_NONE) return GR_OK;
    st = check_device();
    if (st != GR_OK) return st;
    return run_bt<gr::ElemF16>(p, M, N, K, A, lda, Bt, ldbt, C, ldc, kReluOnly, static_cast<hipStream_t>(stream));
}

// C = act(A Bt^T + bias) in fp16 or bfloat16 (fmt): the transposed-B paths
// with the general epilogue.
template <typename Base>
int entry_bt_epi(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* Bt, int64_t ldbt,
                 const uint16_t* bias, int act, uint16_t* C, int64_t ldc, void* stream, int forced) {
    if (act < 0 || act >= gr::kActCount) return GR_ERR_INVALID_ARG;
    gr_plan_t p;
    int st = plan_call_bt(M, N, K, (uintptr_t)A, lda, (uintptr_t)Bt, ldbt, (uintptr_t)C, ldc, forced, &p);
    if (st != GR_OK) return st;
    if (bias != nullptr && M > 0 && N > 0 && overlaps((uintptr_t)C, span_bytes(M, N, ldc), (uintptr_t)bias, 2 * N))
        return GR_ERR_ALIAS;
    if (p.path == GR_PATH_NONE) return GR_OK;
    st = check_device();
    if (st != GR_OK) return st;
    return run_bt<gr::Epi<Base>>(p, M, N, K, A, lda, Bt, ldbt, C, ldc, gr::EpiArgs{bias, act, 1.0f},
                                 static_cast<hipStream_t>(stream));
}

// ---- A given transposed (At, K x M) --------------------------------------------

// Argument checks for the transposed-A call: At is K x M with pitch ldat >=
// max(1, M); otherwise as validate().
int validate_ta(int64_t M, int64_t N, int64_t K, uintptr_t At, int64_t ldat, uintptr_t B, int64_t ldb,
                uintptr_t C, int64_t ldc) {
    if (M < 0 || N < 0 || K < 0) return GR_ERR_INVALID_DIM;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return GR_ERR_TOO_LARGE;
    const int64_t mmin = M > 1 ? M : 1, nmin = N > 1 ? N : 1;
    if (ldat < mmin || ldb < nmin || ldc < nmin) return GR_ERR_INVALID_LD;
    const bool used = M > 0 && N > 0 && K > 0;
    const bool c_used = M > 0 && N > 0;
    if ((used && (!At || !B)) || (c_used && !C)) return GR_ERR_NULL_PTR;
    const int64_t sa = used ? span_bytes(K, M, ldat) : 0;
    const int64_t sb = used ? span_bytes(K, N, ldb) : 0;
    const int64_t sc = c_used ? span_bytes(M, N, ldc) : 0;
    if (sa < 0 || sb < 0 || sc < 0) return GR_ERR_TOO_LARGE;
    if (overlaps(C, sc, At, sa) || overlaps(C, sc, B, sb)) return GR_ERR_ALIAS;
    return GR_OK;
}

// The streaming small-M kernel with At: M <= 16, K % 32 == 0, N of at least
// one 64-column block, B of any alignment, pitches within 32-bit offsets.
bool smallm_ta_ok(int64_t M, int64_t N, int64_t K, int64_t ldb) {
    return M >= 1 && M <= kSmallMThreshold && K > 0 && K % 32 == 0 && N >= kStreamNB && ldb <= gr::tile2::MAX_LDB;
}

// The 32-deep pipelined kernel with At staged like B: 16-byte rows of At and
// B, K a positive multiple of 32, M >= 256 (the last tile row moves up to end
// at M, so no copy reads a column of At past M), pitches within its 32-bit
// copy offsets (32 rows of At or B per strip).
bool tile_ta_ok(int64_t M, int64_t N, int64_t K, uintptr_t At, int64_t ldat, uintptr_t B, int64_t ldb) {
    using namespace gr::tile2;
    return M >= BM && N >= 1 && K > 0 && K % BK == 0 && vec_width(At, ldat) == 8 && vec_width(B, ldb) == 8 &&
           ldat <= MAX_LDB && ldb <= MAX_LDB;
}

int choose_path_ta(int64_t M, int64_t N, int64_t K, uintptr_t At, int64_t ldat, uintptr_t B, int64_t ldb) {
    if (M == 0 || N == 0) return GR_PATH_NONE;
    if (smallm_ta_ok(M, N, K, ldb)) return GR_PATH_SMALL_M;
    if (tile_ta_ok(M, N, K, At, ldat, B, ldb)) return GR_PATH_TILE;
    return GR_PATH_TILE_EDGE;
}

void fill_plan_ta(int path, int64_t M, int64_t N, int64_t K, uintptr_t At, int64_t ldat, uintptr_t B, int64_t ldb,
                  uintptr_t C, int64_t ldc, gr_plan_t* p) {
    Pack pk;
    SmallMSplit sp;
    TileSplit ts;
    std::memset(p, 0, sizeof(*p));
    if (path == GR_PATH_TILE) {
        using namespace gr::tile2;
        p->block_m = BM;
        p->block_n = BN;
        p->block_k = BK;
        p->stages = STAGES;
        p->threads = THREADS;
        p->grid = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
        p->vec_a = 8;
        p->vec_b = 8;
        p->vec_c = vec_width_c(C, ldc);
        p->group_m = kGroupM;
        p->split_k = 1;
    } else if (path == GR_PATH_SMALL_M) {
        using namespace gr::smallm;
        p->block_m = MAX_M;
        p->block_n = kStreamNB;
        p->block_k = KSTEP;
        p->stages = 1;
        p->threads = 64 * kStreamTaW;
        p->grid = (N + kStreamNB - 1) / kStreamNB;
        p->vec_a = 1;
        p->vec_b = 8;
        p->vec_c = 1;
        p->group_m = 1;
        p->split_k = 1;
    } else if (path == GR_PATH_TILE_EDGE) {
        fill_plan(path, M, N, K, At, ldat, B, ldb, C, ldc, pk, sp, ts, p);
    }
    p->path = path;
}

template <int VA, int VB>
int launch_tile_ta(const gr_plan_t& p, int64_t M, int64_t N, int64_t K, const uint16_t* At, int64_t ldat,
                   const uint16_t* B, int64_t ldb, uint16_t* C, int64_t ldc, hipStream_t stream) {
    using namespace gr::tile;
    const uint32_t tiles_m = (uint32_t)((M + BM - 1) / BM);
    const uint32_t tiles_n = (uint32_t)((N + BN - 1) / BN);
    return launch(gemm_relu_tile_kernel<true, VA, VB, false, gr::ElemF16, true>, p.grid, THREADS, stream, At, B, C,
                  M, N, K, ldat, ldb, ldc, tiles_m, tiles_n, order_word(p), (int)p.vec_c, kReluOnly);
}

int run_ta(const gr_plan_t& p, int64_t M, int64_t N, int64_t K, const uint16_t* At, int64_t ldat, const uint16_t* B,
           int64_t ldb, uint16_t* C, int64_t ldc, hipStream_t stream) {
    using E = gr::ElemF16;
    switch (p.path) {
        case GR_PATH_NONE: return GR_OK;
        case GR_PATH_SMALL_M: {
            float* no_part = nullptr;
            return launch(gr::smallm::gemm_relu_smallm_stream_kernel<kStreamNB, kStreamTaW, 1,
                                                                     gr::smallm::stream::WHOLE, E, true>,
                          p.grid, p.threads, stream, At, B, C, no_part, M, N, K, ldat, ldb, ldc, K, (uint32_t)p.grid,
                          0u, kReluOnly);
        }
        case GR_PATH_TILE: {
            using namespace gr::tile2;
            const bool whole = tile_whole(M, N, BM, BN);
            const uint32_t tiles_m = (uint32_t)((M + BM - 1) / BM);
            const uint32_t tiles_n = (uint32_t)((N + BN - 1) / BN);
            const uint32_t gm = order_word(p);
            const int vc = p.vec_c;
            if (whole)
                return launch(gemm_relu_tile2_kernel<false, false, E, true>, p.grid, THREADS, stream, At, B, C, M, N,
                              K, ldat, ldb, ldc, tiles_m, tiles_n, gm, vc, kReluOnly);
            return launch(gemm_relu_tile2_kernel<true, false, E, true>, p.grid, THREADS, stream, At, B, C, M, N, K,
                          ldat, ldb, ldc, tiles_m, tiles_n, gm, vc, kReluOnly);
        }
        case GR_PATH_TILE_EDGE: {
            const int va = p.vec_a, vb = p.vec_b;
            if (va == 8 && vb == 8) return launch_tile_ta<8, 8>(p, M, N, K, At, ldat, B, ldb, C, ldc, stream);
            if (va == 8 && vb == 2) return launch_tile_ta<8, 2>(p, M, N, K, At, ldat, B, ldb, C, ldc, stream);
            if (va == 8) return launch_tile_ta<8, 1>(p, M, N, K, At, ldat, B, ldb, C, ldc, stream);
            if (va == 2 && vb == 8) return launch_tile_ta<2, 8>(p, M, N, K, At, ldat, B, ldb, C, ldc, stream);
            if (va == 2 && vb == 2) return launch_tile_ta<2, 2>(p, M, N, K, At, ldat, B, ldb, C, ldc, stream);
            if (va == 2) return launch_tile_ta<2, 1>(p, M, N, K, At, ldat, B, ldb, C, ldc, stream);
            if (vb == 8) return launch_tile_ta<1, 8>(p, M, N, K, At, ldat, B, ldb, C, ldc, stream);
            if (vb == 2) return launch_tile_ta<1, 2>(p, M, N, K, At, ldat, B, ldb, C, ldc, stream);
            return launch_tile_ta<1, 1>(p, M, N, K, At, ldat, B, ldb, C, ldc, stream);
        }
        default: return GR_ERR_INVALID_PATH;
    }
}

int plan_call_ta(int64_t M, int64_t N, int64_t K, uintptr_t at, int64_t ldat, uintptr_t b, int64_t ldb, uintptr_t c,
                 int64_t ldc, int forced, gr_plan_t* p) {
    int st = validate_ta(M, N, K, at, ldat, b, ldb, c, ldc);
    if (st != GR_OK) return st;
    int path = choose_path_ta(M, N, K, at, ldat, b, ldb);
    if (forced >= 0 && path != GR_PATH_NONE) {
        if (forced == GR_PATH_TILE) {
            if (!tile_ta_ok(M, N, K, at, ldat, b, ldb)) return GR_ERR_INVALID_PATH;
        } else if (forced == GR_PATH_SMALL_M) {
            if (!smallm_ta_ok(M, N, K, ldb)) return GR_ERR_INVALID_PATH;
        } else if (forced != GR_PATH_TILE_EDGE) {
            return GR_ERR_INVALID_PATH;
        }
        path = forced;
    }
    fill_plan_ta(path, M, N, K, at, ldat, b, ldb, c, ldc, p);
    return GR_OK;
}

int entry_ta(int64_t M, int64_t N, int64_t K, const uint16_t* At, int64_t ldat, const uint16_t* B, int64_t ldb,
             uint16_t* C, int64_t ldc, void* stream, int forced) {
    gr_plan_t p;
    int st = plan_call_ta(M, N, K, (uintptr_t)At, ldat, (uintptr_t)B, ldb, (uintptr_t)C, ldc, forced, &p);
    if (st != GR_OK) return st;
    if (p.path == GR_PATH_NONE) return GR_OK;
    st = check_device();
    if (st != GR_OK) return st;
    return run_ta(p, M, N, K, At, ldat, B, ldb, C, ldc, static_cast<hipStream_t>(stream));
}

// ---- fp8 (e4m3) operands, B given transposed -----------------------------------

// Bytes spanned by a rows x cols matrix of 1-byte elements with pitch ld.
int64_t span_bytes8(int64_t rows, int64_t cols, int64_t ld) {
    if (rows == 0 || cols == 0) return 0;
    const int64_t limit = kMaxSpanBytes;
    if (rows - 1 > 0 && ld > (limit - cols) / (rows - 1)) return -1;
    return (rows - 1) * ld + cols;
}

// Argument checks of the fp8 calls; the workspace (ws, ws_bytes) as in
// validate(), and it must not overlap the bias either.
int validate_fp8(int64_t M, int64_t N, int64_t K, uintptr_t A, int64_t lda, uintptr_t Bt, int64_t ldbt,
                 uintptr_t bias, int act, uintptr_t C, int64_t ldc, int out_fmt, uintptr_t ws = 0,
                 int64_t ws_bytes = 0) {
    if (M < 0 || N < 0 || K < 0) return GR_ERR_INVALID_DIM;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return GR_ERR_TOO_LARGE;
    const int64_t kmin = K > 1 ? K : 1, nmin = N > 1 ? N : 1;
    if (lda < kmin || ldbt < kmin || ldc < nmin) return GR_ERR_INVALID_LD;
    if (act < 0 || act >= gr::kActCount || (out_fmt != GR_FMT_F16 && out_fmt != GR_FMT_BF16))
        return GR_ERR_INVALID_ARG;
    const bool used = M > 0 && N > 0 && K > 0;
    const bool c_used = M > 0 && N > 0;
    if ((used && (!A || !Bt)) || (c_used && !C)) return GR_ERR_NULL_PTR;
    const int64_t sa = used ? span_bytes8(M, K, lda) : 0;
    const int64_t sb = used ? span_bytes8(N, K, ldbt) : 0;
    const int64_t sc = c_used ? span_bytes(M, N, ldc) : 0;
    if (sa < 0 || sb < 0 || sc < 0) return GR_ERR_TOO_LARGE;
    if (overlaps(C, sc, A, sa) || overlaps(C, sc, Bt, sb)) return GR_ERR_ALIAS;
    if (bias && c_used && overlaps(C, sc, bias, 2 * N)) return GR_ERR_ALIAS;
    if (ws_bytes < 0) return GR_ERR_INVALID_ARG;
    if (ws_bytes > 0) {
        if (!ws) return GR_ERR_NULL_PTR;
        if (ws % kWorkspaceAlign != 0) return GR_ERR_INVALID_ARG;
        if (overlaps(ws, ws_bytes, A, sa) || overlaps(ws, ws_bytes, Bt, sb) || overlaps(ws, ws_bytes, C, sc) ||
            (bias && c_used && overlaps(ws, ws_bytes, bias, 2 * N)))
            return GR_ERR_ALIAS;
    }
    return GR_OK;
}

// The pipelined fp8 kernel: K a positive multiple of 64, 16-byte aligned rows
// of A and Bt, pitches within the 32-bit copy offsets.
bool fp8_tile_ok(int64_t M, int64_t N, int64_t K, uintptr_t A, int64_t lda, uintptr_t Bt, int64_t ldbt) {
    using namespace gr::fp8;
    return M >= 1 && N >= 1 && K > 0 && K % BK == 0 && A % 16 == 0 && lda % 16 == 0 && Bt % 16 == 0 &&
           ldbt % 16 == 0 && lda <= MAX_LD && ldbt <= MAX_LD;
}

// The fp8 small-M stream: M <= 16, K a positive multiple of the 512-deep
// chunk, 16-byte aligned rows.
bool fp8_smallm_ok(int64_t M, int64_t N, int64_t K, uintptr_t A, int64_t lda, uintptr_t Bt, int64_t ldbt) {
    using namespace gr::fp8;
    return M >= 1 && M <= SM_MAX_M && N >= 1 && K > 0 && K % SM_KC == 0 && A % 16 == 0 && lda % 16 == 0 &&
           Bt % 16 == 0 && ldbt % 16 == 0 && lda <= SM_MAX_LD && ldbt <= SM_MAX_LD;
}

// 256 x 256 fp8 tiles unless they would fill less than half of one wave of
// workgroups (or M < 256): then 128 x 128 tiles, two workgroups per CU.
bool fp8_large_tiles(int64_t M, int64_t N) {
    if (M < 256) return false;
    return ((M + 255) / 256) * ((N + 255) / 256) > kSmallTileMaxLargeTiles;
}

// Split-K of the 128 x 128 fp8 tiles (workspace): the rule of the fp16 tile
// split, in 64-byte strips, each split at least 8 strips long.
constexpr int64_t kFp8MinSplitK = 512;
bool fp8_split_layout(int64_t M, int64_t N, int64_t K, bool forced, TileSplit* ts) {
    if (!forced && fp8_large_tiles(M, N)) return false;
    return tile_split_layout(M, N, K, forced, ts, gr::fp8::BK, kFp8MinSplitK);
}

void fill_plan_fp8(int path, int64_t M, int64_t N, uintptr_t C, int64_t ldc, const TileSplit& ts,
                   gr_plan_t* p) {
    std::memset(p, 0, sizeof(*p));
    p->path = path;
    p->block_k = gr::fp8::BK;
    p->threads = gr::fp8::THREADS;
    p->vec_c = vec_width_c(C, ldc);
    p->split_k = 1;
    if (path == GR_PATH_TILE) {
        using namespace gr::fp8;
        const int64_t bm = fp8_large_tiles(M, N) ? 256 : 128;
        p->block_m = (int32_t)bm;
        p->block_n = (int32_t)bm;
        p->stages = STAGES;
        p->grid = ((M + bm - 1) / bm) * ((N + bm - 1) / bm);
        p->vec_a = 16;
        p->vec_b = 16;
        p->group_m = kGroupM;
    } else if (path == GR_PATH_TILE_SPLIT) {
        using namespace gr::fp8;
        p->block_m = 128;
        p->block_n = 128;
        p->stages = STAGES;
        p->grid = ((M + 127) / 128) * ((N + 127) / 128) * ts.splits;
        p->vec_a = 16;
        p->vec_b = 16;
        p->group_m = kGroupM;
        p->split_k = (int32_t)ts.splits;
        p->workspace = ts.bytes;
    } else if (path == GR_PATH_SMALL_M) {
        using namespace gr::fp8;
        p->block_m = SM_MAX_M;
        p->block_n = SM_NB;
        p->block_k = SM_KC;
        p->stages = SM_SLOTS;
        p->grid = (N + SM_NB - 1) / SM_NB;
        p->vec_a = 16;
        p->vec_b = 16;
        p->group_m = 1;
    } else if (path == GR_PATH_TILE_EDGE) {
        using namespace gr::fp8;
        p->block_m = G_BM;
        p->block_n = G_BN;
        p->stages = 1;
        p->grid = ((M + G_BM - 1) / G_BM) * ((N + G_BN - 1) / G_BN);
        p->vec_a = 1;
        p->vec_b = 1;
        p->group_m = 1;
    }
}

// Validate, choose (or check a forced) path, fill the plan; no HIP call.
// ws_known: the workspace pointer is real and is checked (a plan made from a
// size alone skips the pointer checks).
int plan_call_fp8(int64_t M, int64_t N, int64_t K, uintptr_t A, int64_t lda, uintptr_t Bt, int64_t ldbt,
                  uintptr_t bias, int act, uintptr_t C, int64_t ldc, int out_fmt, uintptr_t ws, int64_t ws_bytes,
                  bool ws_known, int forced, TileSplit* ts, gr_plan_t* p) {
    if (ws_bytes < 0) return GR_ERR_INVALID_ARG;
    int st = ws_known ? validate_fp8(M, N, K, A, lda, Bt, ldbt, bias, act, C, ldc, out_fmt, ws, ws_bytes)
                      : validate_fp8(M, N, K, A, lda, Bt, ldbt, bias, act, C, ldc, out_fmt);
    if (st != GR_OK) return st;
    const bool tile_ok = fp8_tile_ok(M, N, K, A, lda, Bt, ldbt);
    const bool smallm_ok = fp8_smallm_ok(M, N, K, A, lda, Bt, ldbt);
    int path;
    if (M == 0 || N == 0) path = GR_PATH_NONE;
    else if (smallm_ok) path = GR_PATH_SMALL_M;
    else if (tile_ok && ws_bytes > 0 && fp8_split_layout(M, N, K, false, ts) && ts->bytes <= ws_bytes)
        path = GR_PATH_TILE_SPLIT;
    else path = tile_ok ? GR_PATH_TILE : GR_PATH_TILE_EDGE;
    if (forced >= 0 && path != GR_PATH_NONE) {
        if (forced == GR_PATH_TILE_SPLIT) {
            if (!tile_ok || !fp8_split_layout(M, N, K, true, ts) || ts->bytes > ws_bytes) return GR_ERR_INVALID_PATH;
        } else if ((forced == GR_PATH_TILE && !tile_ok) || (forced == GR_PATH_SMALL_M && !smallm_ok) ||
                   (forced != GR_PATH_TILE && forced != GR_PATH_TILE_EDGE && forced != GR_PATH_SMALL_M)) {
            return GR_ERR_INVALID_PATH;
        }
        path = forced;
    }
    fill_plan_fp8(path, M, N, C, ldc, *ts, p);
    return GR_OK;
}

template <typename E>
int run_fp8(const gr_plan_t& p, int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, const uint8_t* Bt,
            int64_t ldbt, uint16_t* C, int64_t ldc, const TileSplit& ts, uint8_t* ws, const gr::EpiArgs& ep,
            hipStream_t stream) {
    using namespace gr::fp8;
    float* const no_part = nullptr;  // the unsplit kernels take no workspace
    const int64_t no_kps = 0;
    const uint8_t* const no_s = nullptr;  // nor MX scales
    const int64_t no_ld = 0;
    if (p.path == GR_PATH_TILE_SPLIT) {
        float* part = reinterpret_cast<float*>(ws);
        const uint32_t tiles_m = (uint32_t)((M + 127) / 128);
        const uint32_t tiles_n = (uint32_t)((N + 127) / 128);
        const uint32_t gm = order_word(p);
        const int vc = (int)p.vec_c;
        const int64_t kps = ts.k_per_split;
        const bool whole = M % 128 == 0 && N % 128 == 0;
        int st = whole ? launch(gemm_fp8_tile_kernel<128, false, E, true>, p.grid, THREADS, stream, A, Bt, C, M, N, K,
                                lda, ldbt, ldc, tiles_m, tiles_n, gm, vc, part, kps, no_s, no_ld, no_s, no_ld, ep)
                       : launch(gemm_fp8_tile_kernel<128, true, E, true>, p.grid, THREADS, stream, A, Bt, C, M, N, K,
                                lda, ldbt, ldc, tiles_m, tiles_n, gm, vc, part, kps, no_s, no_ld, no_s, no_ld, ep);
        if (st != GR_OK) return st;
        return launch_reduce<E>(part, C, M, N, ldc, ts.splits, p.vec_c, ep, stream);
    }
    if (p.path == GR_PATH_TILE) {
        const int64_t bm = p.block_m;
        const uint32_t tiles_m = (uint32_t)((M + bm - 1) / bm);
        const uint32_t tiles_n = (uint32_t)((N + bm - 1) / bm);
        const bool whole = M % bm == 0 && N % bm == 0;
        const uint32_t gm = order_word(p);
        const int vc = (int)p.vec_c;
        if (bm == 256) {
            if (whole)
                return launch(gemm_fp8_tile_kernel<256, false, E>, p.grid, THREADS, stream, A, Bt, C, M, N, K, lda,
                              ldbt, ldc, tiles_m, tiles_n, gm, vc, no_part, no_kps, no_s, no_ld, no_s, no_ld, ep);
            return launch(gemm_fp8_tile_kernel<256, true, E>, p.grid, THREADS, stream, A, Bt, C, M, N, K, lda, ldbt,
                          ldc, tiles_m, tiles_n, gm, vc, no_part, no_kps, no_s, no_ld, no_s, no_ld, ep);
        }
        if (whole)
            return launch(gemm_fp8_tile_kernel<128, false, E>, p.grid, THREADS, stream, A, Bt, C, M, N, K, lda, ldbt,
                          ldc, tiles_m, tiles_n, gm, vc, no_part, no_kps, no_s, no_ld, no_s, no_ld, ep);
        return launch(gemm_fp8_tile_kernel<128, true, E>, p.grid, THREADS, stream, A, Bt, C, M, N, K, lda, ldbt, ldc,
                      tiles_m, tiles_n, gm, vc, no_part, no_kps, no_s, no_ld, no_s, no_ld, ep);
    }
    if (p.path == GR_PATH_SMALL_M) {
        if (N % SM_NB == 0)
            return launch(gemm_fp8_smallm_kernel<false, E>, p.grid, 256, stream, A, Bt, C, M, N, K, lda, ldbt, ldc,
                          ep);
        return launch(gemm_fp8_smallm_kernel<true, E>, p.grid, 256, stream, A, Bt, C, M, N, K, lda, ldbt, ldc, ep);
    }
    if (p.path == GR_PATH_TILE_EDGE) {
        const uint32_t tiles_n = (uint32_t)((N + G_BN - 1) / G_BN);
        return launch(gemm_fp8_guarded_kernel<E>, p.grid, 256, stream, A, Bt, C, M, N, K, lda, ldbt, ldc, tiles_n,
                      (int)p.vec_c, no_s, no_ld, no_s, no_ld, ep);
    }
    return p.path == GR_PATH_NONE ? GR_OK : GR_ERR_INVALID_PATH;
}

int entry_fp8(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, const uint8_t* Bt, int64_t ldbt,
              float scale_a, float scale_b, const uint16_t* bias, int act, uint16_t* C, int64_t ldc, int out_fmt,
              void* ws, int64_t ws_bytes, void* stream, int forced) {
    gr_plan_t p;
    TileSplit ts;
    int st = plan_call_fp8(M, N, K, (uintptr_t)A, lda, (uintptr_t)Bt, ldbt, (uintptr_t)bias, act, (uintptr_t)C, ldc,
                           out_fmt, (uintptr_t)ws, ws_bytes, true, forced, &ts, &p);
    if (st != GR_OK) return st;
    if (p.path == GR_PATH_NONE) return GR_OK;
    st = check_device();
    if (st != GR_OK) return st;
    // One scale for the product: the two per-tensor scales multiplied in fp32.
    const gr::EpiArgs ep{bias, act, scale_a * scale_b};
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* w = static_cast<uint8_t*>(ws);
    if (out_fmt == GR_FMT_BF16)
        return run_fp8<gr::Epi<gr::ElemBF16>>(p, M, N, K, A, lda, Bt, ldbt, C, ldc, ts, w, ep, s);
    return run_fp8<gr::Epi<gr::ElemF16>>(p, M, N, K, A, lda, Bt, ldbt, C, ldc, ts, w, ep, s);
}

// ---- MX fp8 and fp4: E4M3 / E2M1 operands with one E8M0 scale per 32 k -----------

// mxf: 8 (MX fp8, one byte per element) or 4 (MX fp4, two elements per
// byte).  Bytes of K elements of one row.
int64_t mx_row_bytes(int64_t K, int mxf) { return mxf == 4 ? K / 2 : K; }

// Argument checks of the MX calls: K a multiple of the 32-element block
// (GR_ERR_INVALID_DIM), then those of the fp8 calls on the operand bytes,
// scale pitches of at least K/32 bytes, scale arrays present and clear of C.
int validate_mx(int64_t M, int64_t N, int64_t K, uintptr_t A, int64_t lda, uintptr_t SA, int64_t ldsa, uintptr_t Bt,
                int64_t ldbt, uintptr_t SB, int64_t ldsb, uintptr_t bias, int act, uintptr_t C, int64_t ldc,
                int out_fmt, int mxf) {
    if (M < 0 || N < 0 || K < 0) return GR_ERR_INVALID_DIM;
    if (K % 32 != 0) return GR_ERR_INVALID_DIM;
    int st = validate_fp8(M, N, mx_row_bytes(K, mxf), A, lda, Bt, ldbt, bias, act, C, ldc, out_fmt);
    if (st != GR_OK) return st;
    const int64_t kb = K / 32, kbmin = kb > 1 ? kb : 1;
    if (ldsa < kbmin || ldsb < kbmin) return GR_ERR_INVALID_LD;
    const bool used = M > 0 && N > 0 && K > 0;
    if (used && (!SA || !SB)) return GR_ERR_NULL_PTR;
    const int64_t ssa = used ? span_bytes8(M, kb, ldsa) : 0;
    const int64_t ssb = used ? span_bytes8(N, kb, ldsb) : 0;
    if (ssa < 0 || ssb < 0) return GR_ERR_TOO_LARGE;
    const int64_t sc = (M > 0 && N > 0) ? span_bytes(M, N, ldc) : 0;
    if (overlaps(C, sc, SA, ssa) || overlaps(C, sc, SB, ssb)) return GR_ERR_ALIAS;
    return GR_OK;
}

// The pipelined kernel with MX scales: its fp8 conditions on the operand
// bytes, K a multiple of 128 elements (every scale copy moves 4 bytes of a
// row: two strips of MX fp8, one of MX fp4) and 4-byte aligned scale rows.
bool mx_tile_ok(int64_t M, int64_t N, int64_t K, uintptr_t A, int64_t lda, uintptr_t SA, int64_t ldsa, uintptr_t Bt,
                int64_t ldbt, uintptr_t SB, int64_t ldsb, int mxf) {
    using namespace gr::fp8;
    return fp8_tile_ok(M, N, mx_row_bytes(K, mxf), A, lda, Bt, ldbt) && K % 128 == 0 && SA % 4 == 0 &&
           ldsa % 4 == 0 && SB % 4 == 0 && ldsb % 4 == 0 && ldsa <= MAX_LD && ldsb <= MAX_LD;
}

int plan_call_mx(int64_t M, int64_t N, int64_t K, uintptr_t A, int64_t lda, uintptr_t SA, int64_t ldsa,
                 uintptr_t Bt, int64_t ldbt, uintptr_t SB, int64_t ldsb, uintptr_t bias, int act, uintptr_t C,
                 int64_t ldc, int out_fmt, int mxf, int forced, gr_plan_t* p) {
    int st = validate_mx(M, N, K, A, lda, SA, ldsa, Bt, ldbt, SB, ldsb, bias, act, C, ldc, out_fmt, mxf);
    if (st != GR_OK) return st;
    const bool tile_ok = mx_tile_ok(M, N, K, A, lda, SA, ldsa, Bt, ldbt, SB, ldsb, mxf);
    int path = (M == 0 || N == 0) ? GR_PATH_NONE : (tile_ok ? GR_PATH_TILE : GR_PATH_TILE_EDGE);
    if (forced >= 0 && path != GR_PATH_NONE) {
        if ((forced == GR_PATH_TILE && !tile_ok) || (forced != GR_PATH_TILE && forced != GR_PATH_TILE_EDGE))
            return GR_ERR_INVALID_PATH;
        path = forced;
    }
    fill_plan_fp8(path, M, N, C, ldc, TileSplit{}, p);
    return GR_OK;
}

// Kb: bytes of K per row (the kernels count bytes).
template <typename E, int MXF>
int run_mx(const gr_plan_t& p, int64_t M, int64_t N, int64_t Kb, const uint8_t* A, int64_t lda, const uint8_t* SA,
           int64_t ldsa, const uint8_t* Bt, int64_t ldbt, const uint8_t* SB, int64_t ldsb, uint16_t* C, int64_t ldc,
           const gr::EpiArgs& ep, hipStream_t stream) {
    using namespace gr::fp8;
    float* const no_part = nullptr;
    const int64_t no_kps = 0;
    if (p.path == GR_PATH_TILE) {
        const int64_t bm = p.block_m;
        const uint32_t tiles_m = (uint32_t)((M + bm - 1) / bm);
        const uint32_t tiles_n = (uint32_t)((N + bm - 1) / bm);
        const bool whole = M % bm == 0 && N % bm == 0;
        const uint32_t gm = order_word(p);
        const int vc = (int)p.vec_c;
        if (bm == 256) {
            if (whole)
                return launch(gemm_fp8_tile_kernel<256, false, E, false, MXF>, p.grid, THREADS, stream, A, Bt, C, M, N,
                              Kb, lda, ldbt, ldc, tiles_m, tiles_n, gm, vc, no_part, no_kps, SA, ldsa, SB, ldsb, ep);
            return launch(gemm_fp8_tile_kernel<256, true, E, false, MXF>, p.grid, THREADS, stream, A, Bt, C, M, N, Kb,
                          lda, ldbt, ldc, tiles_m, tiles_n, gm, vc, no_part, no_kps, SA, ldsa, SB, ldsb, ep);
        }
        if (whole)
            return launch(gemm_fp8_tile_kernel<128, false, E, false, MXF>, p.grid, THREADS, stream, A, Bt, C, M, N, Kb,
                          lda, ldbt, ldc, tiles_m, tiles_n, gm, vc, no_part, no_kps, SA, ldsa, SB, ldsb, ep);
        return launch(gemm_fp8_tile_kernel<128, true, E, false, MXF>, p.grid, THREADS, stream, A, Bt, C, M, N, Kb, lda,
                      ldbt, ldc, tiles_m, tiles_n, gm, vc, no_part, no_kps, SA, ldsa, SB, ldsb, ep);
    }
    if (p.path == GR_PATH_TILE_EDGE) {
        const uint32_t tiles_n = (uint32_t)((N + G_BN - 1) / G_BN);
        return launch(gemm_fp8_guarded_kernel<E, MXF>, p.grid, 256, stream, A, Bt, C, M, N, Kb, lda, ldbt, ldc, tiles_n,
                      (int)p.vec_c, SA, ldsa, SB, ldsb, ep);
    }
    return p.path == GR_PATH_NONE ? GR_OK : GR_ERR_INVALID_PATH;
}

int entry_mx(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, const uint8_t* SA, int64_t ldsa,
             const uint8_t* Bt, int64_t ldbt, const uint8_t* SB, int64_t ldsb, const uint16_t* bias, int act,
             uint16_t* C, int64_t ldc, int out_fmt, int mxf, void* stream, int forced) {
    gr_plan_t p;
    int st = plan_call_mx(M, N, K, (uintptr_t)A, lda, (uintptr_t)SA, ldsa, (uintptr_t)Bt, ldbt, (uintptr_t)SB, ldsb,
                          (uintptr_t)bias, act, (uintptr_t)C, ldc, out_fmt, mxf, forced, &p);
    if (st != GR_OK) return st;
    if (p.path == GR_PATH_NONE) return GR_OK;
    st = check_device();
    if (st != GR_OK) return st;
    const gr::EpiArgs ep{bias, act, 1.0f};
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t Kb = mx_row_bytes(K, mxf);
    if (mxf == 4) {
        if (out_fmt == GR_FMT_BF16)
            return run_mx<gr::Epi<gr::ElemBF16>, 4>(p, M, N, Kb, A, lda, SA, ldsa, Bt, ldbt, SB, ldsb, C, ldc, ep, s);
        return run_mx<gr::Epi<gr::ElemF16>, 4>(p, M, N, Kb, A, lda, SA, ldsa, Bt, ldbt, SB, ldsb, C, ldc, ep, s);
    }
    if (out_fmt == GR_FMT_BF16)
        return run_mx<gr::Epi<gr::ElemBF16>, 8>(p, M, N, Kb, A, lda, SA, ldsa, Bt, ldbt, SB, ldsb, C, ldc, ep, s);
    return run_mx<gr::Epi<gr::ElemF16>, 8>(p, M, N, Kb, A, lda, SA, ldsa, Bt, ldbt, SB, ldsb, C, ldc, ep, s);
}

}  // namespace

extern "C" {

int gemm_relu_bf16(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                   uint16_t* C, int64_t ldc, void* stream) {
    return entry_bf16(M, N, K, A, lda, B, ldb, C, ldc, nullptr, 0, stream, -1);
}

int gemm_relu_bf16_forced(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* B,
                          int64_t ldb, uint16_t* C, int64_t ldc, void* stream, int path) {
    if (!known_path(path) || needs_workspace(path)) return GR_ERR_INVALID_PATH;
    return entry_bf16(M, N, K, A, lda, B, ldb, C, ldc, nullptr, 0, stream, path);
}

int gemm_relu_bf16_ws(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                      uint16_t* C, int64_t ldc, void* workspace, int64_t workspace_bytes, void* stream) {
    return entry_bf16(M, N, K, A, lda, B, ldb, C, ldc, workspace, workspace_bytes, stream, -1);
}

int gemm_relu_bf16_forced_ws(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* B,
                             int64_t ldb, uint16_t* C, int64_t ldc, void* workspace, int64_t workspace_bytes,
                             void* stream, int path) {
    if (!known_path(path)) return GR_ERR_INVALID_PATH;
    return entry_bf16(M, N, K, A, lda, B, ldb, C, ldc, workspace, workspace_bytes, stream, path);
}

int gemm_bias_act_f16(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* B,
                      int64_t ldb, const uint16_t* bias, int act, uint16_t* C, int64_t ldc, void* stream) {
    return entry_epi<gr::ElemF16>(M, N, K, A, lda, B, ldb, bias, act, C, ldc, nullptr, 0, stream, -1);
}

int gemm_bias_act_f16_forced(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* B,
                             int64_t ldb, const uint16_t* bias, int act, uint16_t* C, int64_t ldc, void* stream,
                             int path) {
    if (!known_path(path) || needs_workspace(path)) return GR_ERR_INVALID_PATH;
    return entry_epi<gr::ElemF16>(M, N, K, A, lda, B, ldb, bias, act, C, ldc, nullptr, 0, stream, path);
}

int gemm_bias_act_bf16(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* B,
                       int64_t ldb, const uint16_t* bias, int act, uint16_t* C, int64_t ldc, void* stream) {
    return entry_epi<gr::ElemBF16>(M, N, K, A, lda, B, ldb, bias, act, C, ldc, nullptr, 0, stream, -1);
}

int gemm_bias_act_bf16_forced(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* B,
                              int64_t ldb, const uint16_t* bias, int act, uint16_t* C, int64_t ldc, void* stream,
                              int path) {
    if (!known_path(path) || needs_workspace(path)) return GR_ERR_INVALID_PATH;
    return entry_epi<gr::ElemBF16>(M, N, K, A, lda, B, ldb, bias, act, C, ldc, nullptr, 0, stream, path);
}

int gemm_bias_act_ws(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                     const uint16_t* bias, int act, uint16_t* C, int64_t ldc, int fmt, void* workspace,
                     int64_t workspace_bytes, void* stream, int path) {
    if (path != -1 && !known_path(path)) return GR_ERR_INVALID_PATH;
    if (fmt == GR_FMT_BF16)
        return entry_epi<gr::ElemBF16>(M, N, K, A, lda, B, ldb, bias, act, C, ldc, workspace, workspace_bytes, stream,
                                       path);
    if (fmt != GR_FMT_F16) return GR_ERR_INVALID_ARG;
    return entry_epi<gr::ElemF16>(M, N, K, A, lda, B, ldb, bias, act, C, ldc, workspace, workspace_bytes, stream,
                                  path);
}

int gemm_relu_f16_bt(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* Bt,
                     int64_t ldbt, uint16_t* C, int64_t ldc, void* stream) {
    return entry_bt(M, N, K, A, lda, Bt, ldbt, C, ldc, stream, -1);
}

int gemm_relu_f16_bt_forced(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* Bt,
                            int64_t ldbt, uint16_t* C, int64_t ldc, void* stream, int path) {
    if (path != GR_PATH_TILE && path != GR_PATH_TILE_EDGE && path != GR_PATH_SMALL_M && path != GR_PATH_TILE_STREAM)
        return GR_ERR_INVALID_PATH;
    return entry_bt(M, N, K, A, lda, Bt, ldbt, C, ldc, stream, path);
}

int gemm_relu_f16_bt_plan(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* Bt,
                          int64_t ldbt, const uint16_t* C, int64_t ldc, gr_plan_t* out) {
    if (!out) return GR_ERR_INVALID_ARG;
    return plan_call_bt(M, N, K, (uintptr_t)A, lda, (uintptr_t)Bt, ldbt, (uintptr_t)C, ldc, -1, out);
}


int gemm_relu_f16(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                  uint16_t* C, int64_t ldc, void* stream) {
    return entry(M, N, K, A, lda, B, ldb, C, ldc, nullptr, 0, stream, -1);
}

int gemm_relu_f16_forced(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* B,
                         int64_t ldb, uint16_t* C, int64_t ldc, void* stream, int path) {
    if (!known_path(path) || needs_workspace(path)) return GR_ERR_INVALID_PATH;
    return entry(M, N, K, A, lda, B, ldb, C, ldc, nullptr, 0, stream, path);
}

int gemm_relu_f16_plan(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* B,
                       int64_t ldb, const uint16_t* C, int64_t ldc, gr_plan_t* out) {
    return gemm_relu_f16_plan_ws(M, N, K, A, lda, B, ldb, C, ldc, 0, out);
}

int gemm_relu_f16_workspace_size(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                                 const uint16_t* B, int64_t ldb, const uint16_t* C, int64_t ldc, int64_t* bytes) {
    if (!bytes) return GR_ERR_INVALID_ARG;
    const uintptr_t a = (uintptr_t)A, b = (uintptr_t)B, c = (uintptr_t)C;
    int st = validate(M, N, K, a, lda, b, ldb, c, ldc);
    if (st != GR_OK) return st;
    *bytes = 0;
    if (M == 0 || N == 0) return GR_OK;
    Pack pk;
    SmallMSplit sp;
    TileSplit ts;
    if (K > 0 && (smallm_ok(M, N, K, a, lda, b, ldb) || smallm_stream_ok(M, N, K, a, lda, ldb, kStreamNB))) {
        if (smallm_split_layout(M, N, K, a, lda, b, ldb, &sp) && smallm_split_wanted(N, sp)) *bytes = sp.bytes;
    } else if (tile_fast_ok(M, N, K, a, lda, b, ldb)) {
        if (!use_large_tiles(M, N) && !tile_stream_before_split(M, N, K, lda, ldb) &&
            tile_split_layout(M, N, K, false, &ts))
            *bytes = ts.bytes;
    } else if (tile_unaligned_ok(M, N, K, lda, ldb) && use_large_tiles(M, N)) {
        // the pipelined kernel runs in place on these rows: no workspace
    } else if (tile_stream_ok(M, N, K, lda, ldb) && tile_stream_blocks(M, N) <= kTileStreamRound) {
        // one round of the streaming kernel, planned ahead of the packed copy
    } else if (pack_layout(M, N, K, a, lda, b, ldb, &pk)) {
        *bytes = pk.bytes;
    }
    return GR_OK;
}

int gemm_relu_f16_ws(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* B,
                     int64_t ldb, uint16_t* C, int64_t ldc, void* workspace, int64_t workspace_bytes, void* stream) {
    return entry(M, N, K, A, lda, B, ldb, C, ldc, workspace, workspace_bytes, stream, -1);
}

int gemm_relu_f16_forced_ws(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* B,
                            int64_t ldb, uint16_t* C, int64_t ldc, void* workspace, int64_t workspace_bytes,
                            void* stream, int path) {
    if (!known_path(path)) return GR_ERR_INVALID_PATH;
    return entry(M, N, K, A, lda, B, ldb, C, ldc, workspace, workspace_bytes, stream, path);
}

int gemm_relu_f16_plan_ws(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* B,
                          int64_t ldb, const uint16_t* C, int64_t ldc, int64_t workspace_bytes, gr_plan_t* out) {
    if (!out) return GR_ERR_INVALID_ARG;
    Pack pk;
    SmallMSplit sp;
    TileSplit ts;
    return plan_call(M, N, K, (uintptr_t)A, lda, (uintptr_t)B, ldb, (uintptr_t)C, ldc, 0, workspace_bytes, false,
                     -1, &pk, &sp, &ts, out);
}

int gemm_bias_act_bt(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* Bt,
                     int64_t ldbt, const uint16_t* bias, int act, uint16_t* C, int64_t ldc, int fmt, void* stream,
                     int path) {
    if (path != -1 && path != GR_PATH_TILE && path != GR_PATH_TILE_EDGE && path != GR_PATH_SMALL_M &&
        path != GR_PATH_TILE_STREAM)
        return GR_ERR_INVALID_PATH;
    if (fmt == GR_FMT_BF16)
        return entry_bt_epi<gr::ElemBF16>(M, N, K, A, lda, Bt, ldbt, bias, act, C, ldc, stream, path);
    if (fmt != GR_FMT_F16) return GR_ERR_INVALID_ARG;
    return entry_bt_epi<gr::ElemF16>(M, N, K, A, lda, Bt, ldbt, bias, act, C, ldc, stream, path);
}

int gemm_fp8_bt(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, const uint8_t* Bt, int64_t ldbt,
                float scale_a, float scale_b, const uint16_t* bias, int act, uint16_t* C, int64_t ldc, int out_fmt,
                void* stream) {
    return entry_fp8(M, N, K, A, lda, Bt, ldbt, scale_a, scale_b, bias, act, C, ldc, out_fmt, nullptr, 0, stream,
                     -1);
}

int gemm_fp8_bt_forced(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, const uint8_t* Bt,
                       int64_t ldbt, float scale_a, float scale_b, const uint16_t* bias, int act, uint16_t* C,
                       int64_t ldc, int out_fmt, void* stream, int path) {
    if (path != GR_PATH_TILE && path != GR_PATH_TILE_EDGE && path != GR_PATH_SMALL_M) return GR_ERR_INVALID_PATH;
    return entry_fp8(M, N, K, A, lda, Bt, ldbt, scale_a, scale_b, bias, act, C, ldc, out_fmt, nullptr, 0, stream,
                     path);
}

int gemm_fp8_bt_ws(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, const uint8_t* Bt, int64_t ldbt,
                   float scale_a, float scale_b, const uint16_t* bias, int act, uint16_t* C, int64_t ldc,
                   int out_fmt, void* workspace, int64_t workspace_bytes, void* stream, int path) {
    if (path != -1 && path != GR_PATH_TILE && path != GR_PATH_TILE_EDGE && path != GR_PATH_SMALL_M &&
        path != GR_PATH_TILE_SPLIT)
        return GR_ERR_INVALID_PATH;
    return entry_fp8(M, N, K, A, lda, Bt, ldbt, scale_a, scale_b, bias, act, C, ldc, out_fmt, workspace,
                     workspace_bytes, stream, path);
}

int gemm_fp8_bt_workspace_size(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, const uint8_t* Bt,
                               int64_t ldbt, const uint16_t* C, int64_t ldc, int64_t* bytes) {
    if (!bytes) return GR_ERR_INVALID_ARG;
    *bytes = 0;
    int st = validate_fp8(M, N, K, (uintptr_t)A, lda, (uintptr_t)Bt, ldbt, 0, GR_ACT_RELU, (uintptr_t)C, ldc,
                          GR_FMT_F16);
    if (st != GR_OK) return st;
    TileSplit ts;
    if (M > 0 && N > 0 && !fp8_smallm_ok(M, N, K, (uintptr_t)A, lda, (uintptr_t)Bt, ldbt) &&
        fp8_tile_ok(M, N, K, (uintptr_t)A, lda, (uintptr_t)Bt, ldbt) && fp8_split_layout(M, N, K, false, &ts))
        *bytes = ts.bytes;
    return GR_OK;
}

int gemm_fp8_bt_plan_ws(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, const uint8_t* Bt,
                        int64_t ldbt, const uint16_t* bias, int act, const uint16_t* C, int64_t ldc, int out_fmt,
                        int64_t workspace_bytes, gr_plan_t* out) {
    if (!out) return GR_ERR_INVALID_ARG;
    TileSplit ts;
    return plan_call_fp8(M, N, K, (uintptr_t)A, lda, (uintptr_t)Bt, ldbt, (uintptr_t)bias, act, (uintptr_t)C, ldc,
                         out_fmt, 0, workspace_bytes, false, -1, &ts, out);
}

int gemm_fp8_bt_plan(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, const uint8_t* Bt,
                     int64_t ldbt, const uint16_t* bias, int act, const uint16_t* C, int64_t ldc, int out_fmt,
                     gr_plan_t* out) {
    if (!out) return GR_ERR_INVALID_ARG;
    TileSplit ts;
    return plan_call_fp8(M, N, K, (uintptr_t)A, lda, (uintptr_t)Bt, ldbt, (uintptr_t)bias, act, (uintptr_t)C, ldc,
                         out_fmt, 0, 0, false, -1, &ts, out);
}

int gemm_mxfp8_bt(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, const uint8_t* scale_a,
                  int64_t ld_sa, const uint8_t* Bt, int64_t ldbt, const uint8_t* scale_b, int64_t ld_sb,
                  const uint16_t* bias, int act, uint16_t* C, int64_t ldc, int out_fmt, void* stream) {
    return entry_mx(M, N, K, A, lda, scale_a, ld_sa, Bt, ldbt, scale_b, ld_sb, bias, act, C, ldc, out_fmt, 8, stream,
                    -1);
}

int gemm_mxfp8_bt_forced(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, const uint8_t* scale_a,
                         int64_t ld_sa, const uint8_t* Bt, int64_t ldbt, const uint8_t* scale_b, int64_t ld_sb,
                         const uint16_t* bias, int act, uint16_t* C, int64_t ldc, int out_fmt, void* stream,
                         int path) {
    if (path != GR_PATH_TILE && path != GR_PATH_TILE_EDGE) return GR_ERR_INVALID_PATH;
    return entry_mx(M, N, K, A, lda, scale_a, ld_sa, Bt, ldbt, scale_b, ld_sb, bias, act, C, ldc, out_fmt, 8, stream,
                    path);
}

int gemm_mxfp8_bt_plan(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, const uint8_t* scale_a,
                       int64_t ld_sa, const uint8_t* Bt, int64_t ldbt, const uint8_t* scale_b, int64_t ld_sb,
                       const uint16_t* bias, int act, const uint16_t* C, int64_t ldc, int out_fmt, gr_plan_t* out) {
    if (!out) return GR_ERR_INVALID_ARG;
    return plan_call_mx(M, N, K, (uintptr_t)A, lda, (uintptr_t)scale_a, ld_sa, (uintptr_t)Bt, ldbt,
                        (uintptr_t)scale_b, ld_sb, (uintptr_t)bias, act, (uintptr_t)C, ldc, out_fmt, 8, -1, out);
}

int gemm_mxfp4_bt(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, const uint8_t* scale_a,
                  int64_t ld_sa, const uint8_t* Bt, int64_t ldbt, const uint8_t* scale_b, int64_t ld_sb,
                  const uint16_t* bias, int act, uint16_t* C, int64_t ldc, int out_fmt, void* stream) {
    return entry_mx(M, N, K, A, lda, scale_a, ld_sa, Bt, ldbt, scale_b, ld_sb, bias, act, C, ldc, out_fmt, 4, stream,
                    -1);
}

int gemm_mxfp4_bt_forced(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, const uint8_t* scale_a,
                         int64_t ld_sa, const uint8_t* Bt, int64_t ldbt, const uint8_t* scale_b, int64_t ld_sb,
                         const uint16_t* bias, int act, uint16_t* C, int64_t ldc, int out_fmt, void* stream,
                         int path) {
    if (path != GR_PATH_TILE && path != GR_PATH_TILE_EDGE) return GR_ERR_INVALID_PATH;
    return entry_mx(M, N, K, A, lda, scale_a, ld_sa, Bt, ldbt, scale_b, ld_sb, bias, act, C, ldc, out_fmt, 4, stream,
                    path);
}

int gemm_mxfp4_bt_plan(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, const uint8_t* scale_a,
                       int64_t ld_sa, const uint8_t* Bt, int64_t ldbt, const uint8_t* scale_b, int64_t ld_sb,
                       const uint16_t* bias, int act, const uint16_t* C, int64_t ldc, int out_fmt, gr_plan_t* out) {
    if (!out) return GR_ERR_INVALID_ARG;
    return plan_call_mx(M, N, K, (uintptr_t)A, lda, (uintptr_t)scale_a, ld_sa, (uintptr_t)Bt, ldbt,
                        (uintptr_t)scale_b, ld_sb, (uintptr_t)bias, act, (uintptr_t)C, ldc, out_fmt, 4, -1, out);
}

int gemm_relu_f16_ta(int64_t M, int64_t N, int64_t K, const uint16_t* At, int64_t ldat, const uint16_t* B,
                     int64_t ldb, uint16_t* C, int64_t ldc, void* stream) {
    return entry_ta(M, N, K, At, ldat, B, ldb, C, ldc, stream, -1);
}

int gemm_relu_f16_ta_forced(int64_t M, int64_t N, int64_t K, const uint16_t* At, int64_t ldat, const uint16_t* B,
                            int64_t ldb, uint16_t* C, int64_t ldc, void* stream, int path) {
    if (path != GR_PATH_TILE && path != GR_PATH_TILE_EDGE && path != GR_PATH_SMALL_M) return GR_ERR_INVALID_PATH;
    return entry_ta(M, N, K, At, ldat, B, ldb, C, ldc, stream, path);
}

int gemm_relu_f16_ta_plan(int64_t M, int64_t N, int64_t K, const uint16_t* At, int64_t ldat, const uint16_t* B,
                          int64_t ldb, const uint16_t* C, int64_t ldc, gr_plan_t* out) {
    if (!out) return GR_ERR_INVALID_ARG;
    return plan_call_ta(M, N, K, (uintptr_t)At, ldat, (uintptr_t)B, ldb, (uintptr_t)C, ldc, -1, out);
}

int gemm_relu_f16_forced_order(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* B,
                               int64_t ldb, uint16_t* C, int64_t ldc, void* stream, int path, int group_m,
                               int xcd_remap) {
    if (!known_path(path) || needs_workspace(path)) return GR_ERR_INVALID_PATH;
    if (group_m < 1 || (xcd_remap != 0 && xcd_remap != 1)) return GR_ERR_INVALID_ARG;
    const int64_t order = (int64_t)(uint32_t)group_m | (xcd_remap ? 0 : (int64_t)gr::kNoXcdRemap);
    return entry(M, N, K, A, lda, B, ldb, C, ldc, nullptr, 0, stream, path, order);
}

int gemm_relu_f16_noalloc(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* B,
                          int64_t ldb, uint16_t* C, int64_t ldc, void* stream) {
    int64_t need = 0;
    int st = gemm_relu_f16_workspace_size(M, N, K, A, lda, B, ldb, C, ldc, &need);
    if (st != GR_OK) return st;
    if (need > GR_NOALLOC_SCRATCH_BYTES) return GR_ERR_SCRATCH;
    if (need == 0) return entry(M, N, K, A, lda, B, ldb, C, ldc, nullptr, 0, stream, -1);
    st = check_device();
    if (st != GR_OK) return st;
    uint8_t* ws = nullptr;
    st = scratch_on_current_device(&ws);
    if (st != GR_OK) return st;
    return entry(M, N, K, A, lda, B, ldb, C, ldc, ws, need, stream, -1);
}

int gemm_relu_stream_read(const void* src, int64_t bytes, int pattern, uint64_t* sink, void* stream) {
    using namespace gr::probe;
    if (bytes <= 0 || bytes % GRANULE != 0) return GR_ERR_INVALID_ARG;
    if (pattern != CONTIGUOUS && pattern != ROW_PIECES) return GR_ERR_INVALID_ARG;
    if (!src || !sink) return GR_ERR_NULL_PTR;
    if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(sink) % 8 != 0)
        return GR_ERR_INVALID_ARG;
    if (overlaps(reinterpret_cast<uintptr_t>(src), bytes, reinterpret_cast<uintptr_t>(sink), 8 * WGS))
        return GR_ERR_ALIAS;
    int st = check_device();
    if (st != GR_OK) return st;
    const gr::u32x4* s = reinterpret_cast<const gr::u32x4*>(src);
    if (pattern == ROW_PIECES)
        return launch(stream_read_kernel<ROW_PIECES>, WGS, THREADS, static_cast<hipStream_t>(stream), s, bytes, sink);
    return launch(stream_read_kernel<CONTIGUOUS>, WGS, THREADS, static_cast<hipStream_t>(stream), s, bytes, sink);
}

const char* gemm_relu_status_string(int status) {
    switch (status) {
        case GR_OK: return "GR_OK";
        case GR_ERR_INVALID_DIM: return "GR_ERR_INVALID_DIM";
        case GR_ERR_INVALID_LD: return "GR_ERR_INVALID_LD";
        case GR_ERR_NULL_PTR: return "GR_ERR_NULL_PTR";
        case GR_ERR_ALIAS: return "GR_ERR_ALIAS";
        case GR_ERR_TOO_LARGE: return "GR_ERR_TOO_LARGE";
        case GR_ERR_NO_DEVICE: return "GR_ERR_NO_DEVICE";
        case GR_ERR_UNSUPPORTED_DEVICE: return "GR_ERR_UNSUPPORTED_DEVICE";
        case GR_ERR_LAUNCH: return "GR_ERR_LAUNCH";
        case GR_ERR_INVALID_PATH: return "GR_ERR_INVALID_PATH";
        case GR_ERR_INVALID_ARG: return "GR_ERR_INVALID_ARG";
        case GR_ERR_SCRATCH: return "GR_ERR_SCRATCH";
        default: return "GR_ERR_UNKNOWN";
    }
}

int gemm_relu_version(void) { return kVersion; }

}  // extern "C"
