/*
 * gemm_relu.h -- C ABI of the MI355X (gfx950) fused fp16 GEMM + ReLU library
 * (with bfloat16, transposed-B, bias + activation, fp8 and block-scaled MX
 * fp8 / fp4 variants further down).
 *
 * The one operation:  C := ReLU(A * B)
 *   A  M x K, B  K x N, C  M x N, all IEEE binary16, row-major with a row
 *   pitch (element (i, k) of A at A[i*lda + k], likewise B and C).
 *   Products accumulate in fp32 from a cleared accumulator; ReLU acts on the
 *   fp32 sum; the result is rounded to fp16 (nearest, ties to even) only when
 *   it is written.  This is the tiled GEMM with a fused elementwise epilogue
 *   of the TileLang tutorial, chapter "GEMM walkthrough and parameter
 *   derivation" (fp16 operands, fp32 fragment cleared before the K loop), of
 *   the blog "TileLang programming basics", section 2 (the FP16 GEMM + ReLU
 *   listing: max(C_local, 0) on the fp32 fragment, cast on write-back), and of
 *   "Writing high-performance kernels in TileLang", section "Writing a GEMM"
 *   (the caller passes C, which is only written).
 *
 * Conventions shared by every entry point:
 *   - Pointers A, B, C are DEVICE pointers (HIP) to fp16 bit patterns, owned
 *     by the caller.  The library allocates nothing on the call path, keeps no
 *     per-call state and never frees caller memory; the only scratch memory
 *     it uses is a workspace the caller passes (the *_ws calls).
 *   - C is never read (there is no beta); elements of C outside the M x N
 *     window (columns N..ldc-1, rows >= M) are never written.  Padding columns
 *     of A (K..lda-1) and B (N..ldb-1) never affect the result.  Reads stay
 *     inside the 16-byte aligned blocks that hold elements of A and B: the
 *     pipelined kernel copies whole 16-byte chunks, so it may read the padding
 *     of B's rows and up to 14 bytes after B's last element.
 *   - Any M, N, K >= 0 work with the same library: tile shapes are fixed when
 *     the library is built; edges that do not fill a tile are guarded.
 *     M == 0 or N == 0: nothing is launched, GR_OK.  K == 0: C = +0.
 *     (One compiled kernel serving every shape, with the sizes read from the
 *     arguments of each call and guards on the ragged edges: TileLang
 *     tutorial, chapter "动态形状与变长序列" (dynamic shapes and variable
 *     length), section "T.dynamic 的机制".  Zero K iterations leave the
 *     cleared accumulator: chapter "GEMM 走读与参数推导", T.clear.)
 *   - Pitches: lda >= max(1, K), ldb >= max(1, N), ldc >= max(1, N).  Any
 *     element alignment is accepted; 16-byte aligned rows take faster code.
 *   - The byte range C spans must not overlap the ranges of A or B.
 *   - stream: a hipStream_t passed as void* (NULL = the null stream).  The
 *     call only enqueues work and returns; a fault inside a kernel surfaces at
 *     the caller's next synchronisation.  There is no implicit device sync.
 *   - Errors: every entry point returns GR_OK (0) or a negative GR_ERR_* code
 *     and never throws across the ABI.  Argument checks run before any HIP
 *     call, so they work without a GPU.  gemm_relu_status_string() names a
 *     code.  A call never degrades silently: a problem it cannot run is
 *     refused with a code before anything is launched, the way the pages'
 *     tool chain rejects what it cannot lower (TileLang tutorial: chapter
 *     "自动调优", an unknown config key is an error; chapter "归约、扫描与
 *     原子", a mismatched output shape raises ValueError; chapter "动态形状
 *     与变长序列", a size with no source raises TypeError; chapter "后端与
 *     codegen", a missing lowering is a compile error, never silently wrong
 *     code; chapter "CUDA 硬件故障手册", launch-time errors are fatal).
 *   - Thread safety: calls are reentrant; per-device properties are cached
 *     once with thread-safe initialisation.
 */
#ifndef GEMM_RELU_H_
#define GEMM_RELU_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ----------------------------------------------------------
 * Each code names one way a call is refused before launch (GR_ERR_LAUNCH:
 * the runtime rejected the launch).  Failing loudly, with the cause named,
 * follows the pages' error behaviour listed under "Errors" above (TileLang
 * tutorial, chapters "自动调优", "归约、扫描与原子", "动态形状与变长序列",
 * "后端与 codegen" and "CUDA 硬件故障手册").
 */
#define GR_OK                        0
#define GR_ERR_INVALID_DIM          -1 /* M, N or K negative (MX calls: K % 32 != 0)     */
#define GR_ERR_INVALID_LD           -2 /* lda < max(1,K), ldb < max(1,N) or ldc < max(1,N) */
#define GR_ERR_NULL_PTR             -3 /* NULL pointer for a non-empty operand            */
#define GR_ERR_ALIAS                -4 /* C's byte range overlaps A's or B's              */
#define GR_ERR_TOO_LARGE            -5 /* a dimension >= 2^31 or an operand span >= 2^62 B */
#define GR_ERR_NO_DEVICE            -6 /* no HIP device visible                            */
#define GR_ERR_UNSUPPORTED_DEVICE   -7 /* current device is not gfx950                     */
#define GR_ERR_LAUNCH               -8 /* the kernel launch was rejected by the runtime    */
#define GR_ERR_INVALID_PATH         -9 /* forced path unknown or not applicable            */
#define GR_ERR_INVALID_ARG         -10 /* a NULL output struct or other bad argument        */
#define GR_ERR_SCRATCH             -11 /* gemm_relu_f16_noalloc: the problem needs more      */
                                       /* scratch than the library's static buffer holds   */

/* ---- element formats (fmt / out_fmt arguments) ----------------------------- */
#define GR_FMT_F16         0 /* IEEE binary16                                        */
#define GR_FMT_BF16        1 /* bfloat16                                             */

/* ---- execution paths chosen by the planner --------------------------------- */
#define GR_PATH_NONE       0 /* empty output: nothing to launch                            */
#define GR_PATH_TILE       1 /* pipelined MFMA tile kernel, direct-to-LDS copies: 16-B rows  */
                             /* of A and B, K % 32 == 0; any M, N and C layout; 256x256    */
                             /* tiles, or 128x128 when M < 256 or fewer than 129 large ones */
#define GR_PATH_TILE_EDGE  2 /* MFMA tile kernel with edge guards and narrow loads          */
#define GR_PATH_SMALL_M    3 /* bandwidth kernel for GEMV-like shapes (few rows of A)       */
#define GR_PATH_TILE_PACKED 4 /* copy A and/or B into the caller's workspace (aligned rows, */
                              /* K zero-padded), then the pipelined kernel; needs workspace */
#define GR_PATH_SMALL_M_SPLIT 5 /* small-M split over K: fp32 partial sums in the caller's   */
                                /* workspace, then a pass that sums them and applies ReLU  */
#define GR_PATH_TILE_SPLIT    6 /* 128x128-tile kernel split over K (few tiles, long K):     */
                                /* fp32 partial sums in the workspace, then the same pass  */
#define GR_PATH_TILE_UNALIGNED 7 /* the pipelined 256x256 kernel in place on rows that are  */
                                 /* not 16-byte aligned and/or K % 64 != 0: direct-to-LDS */
                                 /* copies from any 2-byte address, the K tail (1..64)    */
                                 /* copied as one strip and masked; M, N >= 256, K > 128; */
                                 /* the planner's choice for such rows with more than 128 */
                                 /* tiles, and with fewer when no workspace lets it pack  */
                                 /* and the streaming kernel does not apply; no workspace */
#define GR_PATH_TILE_PERSISTENT 8 /* the pipelined 256x256 kernel as a persistent tile loop: */
                                  /* at most one workgroup per CU, each storing a finished */
                                  /* tile while the next tile's first copies are in flight */
                                  /* (TileLang tutorial, "Persistent kernel"); whole tiles, */
                                  /* K % 64 == 0, 16-byte rows of A and B                  */
#define GR_PATH_TILE_STREAM 9 /* blocks of 64 rows x 64 columns on the streaming kernel:  */
                              /* the block's 4 waves (8 up to 256 blocks) split K (rings */
                              /* of direct-to-LDS copies of their own, no barrier in the */
                              /* loop) and add their partial sums in order at the end;   */
                              /* K % 32 == 0, N >= 64, rows of A and B of any alignment; */
                              /* blocks placed for L2 reuse per XCD                     */
                              /* (plain_order).  The planner's choice for few blocks     */
                              /* (ceil(M/64) x ceil(N/64), 512 fill one round): with     */
                              /* aligned rows up to 256 of them from K = 256 and 512     */
                              /* from K = 512; with rows of A or B misaligned up to      */
                              /* 512, and 1024 when no workspace lets the operands be    */
                              /* packed (few tiles: the split-K                          */
                              /* remedy of the TileLang tutorial's "性能取证", within one */
                              /* workgroup); no workspace.  Up to 64 rows without a     */
                              /* split: one row of blocks where the small-M kernel's    */
                              /* few blocks would leave CUs idle (at most 128 blocks;   */
                              /* more than 32 rows, or K x N >= 2^23 with N >= 1024),   */
                              /* and whenever A's rows are not 16-byte aligned          */

/* What the planner decided for one problem.  Filled by gemm_relu_f16_plan. */
typedef struct gr_plan_t {
    int32_t path;        /* GR_PATH_*                                                  */
    int32_t block_m;     /* rows of C per workgroup                                   */
    int32_t block_n;     /* columns of C per workgroup                                */
    int32_t block_k;     /* K step per pipeline stage                                 */
    int32_t stages;      /* LDS buffers in the K pipeline                             */
    int32_t threads;     /* threads per workgroup                                     */
    int64_t grid;        /* workgroups launched (1-D grid)                            */
    int32_t vec_a;       /* fp16 elements per global load of A (8, 4, 2 or 1)         */
    int32_t vec_b;       /* fp16 elements per global load of B                        */
    int32_t vec_c;       /* fp16 elements per global store of C (8 at any alignment; 1
                            on the small-M paths, which store elements)               */
    int32_t group_m;     /* tile rows per workgroup-order group (L2 reuse)           */
    int32_t packed;      /* GR_PATH_TILE_PACKED: bit 0 = A copied, bit 1 = B copied     */
    int64_t workspace;   /* bytes of the caller's workspace the path uses (else 0)     */
    int32_t split_k;     /* K splits (the *_SPLIT paths); 1 for the tile and small-M  */
                         /* paths                                                       */
    int32_t plain_order; /* workgroup order of the tiled grids: 0 = each XCD takes a   */
                         /* contiguous range of tiles, walked in groups of group_m     */
                         /* tile rows; 1 = tile order follows the workgroup id         */
                         /* (GR_PATH_TILE_STREAM when its number of 64-column blocks   */
                         /* is a multiple of 4)                                        */
} gr_plan_t;

/*
 * gemm_relu_f16 -- C := ReLU(A * B), fp16 in, fp32 accumulate, fp16 out.
 *   M, N, K   problem size (>= 0)
 *   A, lda    device pointer to M x K fp16, row pitch lda elements
 *   B, ldb    device pointer to K x N fp16, row pitch ldb elements
 *   C, ldc    device pointer to M x N fp16 output, row pitch ldc elements
 *   stream    hipStream_t as void* (NULL = null stream)
 * Returns GR_OK or a GR_ERR_* code (see above); on error nothing is launched.
 * The path (tile, edge-guarded tile, small-M) is chosen by the same planner
 * gemm_relu_f16_plan exposes; all paths produce the same result up to fp32
 * summation order.
 */
int gemm_relu_f16(int64_t M, int64_t N, int64_t K,
                  const uint16_t* A, int64_t lda,
                  const uint16_t* B, int64_t ldb,
                  uint16_t* C, int64_t ldc,
                  void* stream);

/*
 * gemm_relu_f16_plan -- pure planner: validates the arguments exactly as
 * gemm_relu_f16 does and reports the path, tile and grid it would launch.
 * It is the library's "look at what the kernel became" hook: the pages
 * inspect the generated kernel (tile sizes, stages, shared-memory buffers)
 * before any performance discussion ("TileLang programming basics", section
 * "六、写完之后的三个动作", step 2, get_kernel_source; TileLang tutorial,
 * chapter "安装与第一个 kernel").  Tests and the benchmark use it to name the
 * tile edges they check and the path they time.
 * Makes no HIP call and touches no memory behind the pointers: it only uses
 * their values (for alignment and overlap checks), so it runs without a GPU.
 *   out   host pointer to a gr_plan_t to fill (must not be NULL)
 * Returns GR_OK or the GR_ERR_* code gemm_relu_f16 would return for the same
 * arguments (device errors excepted).
 */
int gemm_relu_f16_plan(int64_t M, int64_t N, int64_t K,
                       const uint16_t* A, int64_t lda,
                       const uint16_t* B, int64_t ldb,
                       const uint16_t* C, int64_t ldc,
                       gr_plan_t* out);

/*
 * gemm_relu_f16_forced -- as gemm_relu_f16, but runs the given path instead of
 * the planner's choice, for tests that cross-check the paths on one input.
 * The pages check every candidate kernel configuration against one
 * reference on the same inputs ("TileLang programming basics", section
 * "六、写完之后的三个动作", step 1: the autotuner validates each config the
 * same way); this hook lets the tests do that for every path.
 *   path  GR_PATH_TILE, GR_PATH_TILE_UNALIGNED, GR_PATH_TILE_EDGE or
 *         GR_PATH_SMALL_M.
 * GR_PATH_TILE is accepted only when the planner's conditions for it hold
 * (16-byte aligned rows of A and B, K a positive multiple of 32, pitches of
 * at most 2^22 elements for A and 2^25 for B); GR_PATH_TILE_UNALIGNED when M
 * >= 256, N >= 256, K > 128, there are more than 128 tiles of 256 x 256 and
 * the pitches are within the same limits (any alignment; the planner also
 * asks for more than 128 tiles of 256 x 256, the forced hook does not);
 * GR_PATH_SMALL_M
 * only when the small-M kernel's alignment conditions hold (see
 * gemm_relu_f16_plan).  Otherwise GR_ERR_INVALID_PATH and nothing is
 * launched.  GR_PATH_TILE_EDGE accepts any valid problem.
 */
int gemm_relu_f16_forced(int64_t M, int64_t N, int64_t K,
                         const uint16_t* A, int64_t lda,
                         const uint16_t* B, int64_t ldb,
                         uint16_t* C, int64_t ldc,
                         void* stream, int path);

/*
 * gemm_relu_f16_forced_order -- gemm_relu_f16_forced with the workgroup order
 * of the tile kernels chosen by the caller: `group_m` tile rows per group of
 * the grid-level swizzle (>= 1; the planner uses 4) and `xcd_remap` 1 (each
 * XCD takes a contiguous range of tiles: the planner's choice, plain_order =
 * 0) or 0 (tile order follows the workgroup id: plain_order = 1, which the
 * planner takes for GR_PATH_TILE_STREAM when its number of 64-column blocks
 * is a multiple of 4).  The order decides only when each tile
 * runs, never what it computes, so every setting must give the same bits:
 * the test hook that checks exactly that.  The pages give the grid swizzle
 * (panel size, ordering) as a free scheduling choice for L2 reuse (TileLang
 * tutorial, chapter "布局与存储体冲突", T.use_swizzle; "Writing
 * high-performance kernels in TileLang", section "編寫一個 GEMM").
 * GR_ERR_INVALID_ARG for group_m < 1 or xcd_remap not 0 or 1; paths as
 * gemm_relu_f16_forced.
 */
int gemm_relu_f16_forced_order(int64_t M, int64_t N, int64_t K,
                               const uint16_t* A, int64_t lda,
                               const uint16_t* B, int64_t ldb,
                               uint16_t* C, int64_t ldc,
                               void* stream, int path, int group_m, int xcd_remap);

/*
 * ---- calls with a caller-provided workspace ---------------------------------
 * Two paths use scratch device memory when the caller provides it:
 *   - GR_PATH_TILE_PACKED.  The pipelined kernel reads A and B in whole
 *     16-byte chunks and walks K in whole 32-deep strips.  When an operand's
 *     rows are not 16-byte aligned, or K is not a multiple of 32, the calls
 *     above take GR_PATH_TILE_UNALIGNED where its conditions hold and fall
 *     back to the guarded register-staged kernel otherwise.  With a
 *     workspace, for the problems GR_PATH_TILE_UNALIGNED does not take, the
 *     library instead copies the offending operand(s) into it
 *     -- rows 16-byte aligned, K padded with zeros to a multiple of 64 (the
 *     padded steps add exact zeros, the same rule as the edge guards) -- and
 *     runs the pipelined kernel on the copies: two launches on the stream,
 *     one extra read and write of the copied operands.  Bit-exact against
 *     the other tile paths (same MFMA steps, same k order).
 *   - GR_PATH_SMALL_M_SPLIT.  For M <= 16 where the single pass would leave
 *     CUs idle, the K range is split so that each workgroup streams 128
 *     columns of B (256 columns on the register-staged kernel, for K % 32
 *     != 0) over a part of K; the fp32 partial sums (splits x M x N) go to
 *     the workspace and a second launch adds them in split order, applies
 *     ReLU and rounds.  Same result as GR_PATH_SMALL_M up to fp32 summation
 *     order.
 *   - GR_PATH_TILE_SPLIT.  For pipelined-path problems with too few 128x128
 *     tiles to fill the chip and a long K, each tile's K range is split; the
 *     fp32 partial sums go to the workspace and the same second launch sums
 *     them in order and applies ReLU.  Same result as GR_PATH_TILE up to fp32
 *     summation order.
 *
 * Where this comes from: the packed copy applies, ahead of time, the pages'
 * edge rule that out-of-range elements of both operands read as zero
 * (TileLang tutorial, chapter "动态形状与变长序列"); the split paths are the
 * split-K of "TileLang programming basics", section 5.1 "Split-K" and of the
 * tutorial's chapter "归约、扫描与原子" (partial sums over K slices), made
 * deterministic by adding the partials in a fixed order, and with ReLU
 * applied once to the complete sum.  The caller owns the scratch memory as
 * it owns C (destination passing: "Writing high-performance kernels in
 * TileLang", section "編寫一個 GEMM").
 *
 * Workspace rules: a DEVICE pointer, 256-byte aligned, owned by the caller,
 * not overlapping A, B or C; its contents on entry are ignored and on return
 * are unspecified.  The work is stream-ordered: the caller may reuse or free
 * the workspace once the call's work on `stream` is done, and two calls in
 * flight at once (on different streams) need two workspaces.
 */

/*
 * gemm_relu_f16_workspace_size -- bytes of workspace that let this problem
 * take GR_PATH_TILE_PACKED, GR_PATH_SMALL_M_SPLIT or GR_PATH_TILE_SPLIT; 0
 * when the problem never uses a workspace (it fills the chip on the pipelined
 * or small-M kernel as it is, has a K too short to split, or is empty).
 * Validates like gemm_relu_f16; no HIP call.
 *   bytes  host pointer receiving the size (must not be NULL)
 */
int gemm_relu_f16_workspace_size(int64_t M, int64_t N, int64_t K,
                                 const uint16_t* A, int64_t lda,
                                 const uint16_t* B, int64_t ldb,
                                 const uint16_t* C, int64_t ldc,
                                 int64_t* bytes);

/*
 * gemm_relu_f16_ws -- gemm_relu_f16 with a workspace.
 *   workspace, workspace_bytes  the caller's scratch (NULL, 0 = none)
 * Takes GR_PATH_TILE_PACKED, GR_PATH_SMALL_M_SPLIT or GR_PATH_TILE_SPLIT
 * when the workspace holds at least the size gemm_relu_f16_workspace_size
 * reports (the packed path only when the problem is large enough for the
 * copies to pay, M*N*K >= 2^30); otherwise does exactly what gemm_relu_f16
 * does.  Extra errors: GR_ERR_INVALID_ARG for a negative size
 * or a workspace not 256-byte aligned, GR_ERR_NULL_PTR for NULL with a
 * positive size, GR_ERR_ALIAS when the workspace overlaps A, B or C.
 */
int gemm_relu_f16_ws(int64_t M, int64_t N, int64_t K,
                     const uint16_t* A, int64_t lda,
                     const uint16_t* B, int64_t ldb,
                     uint16_t* C, int64_t ldc,
                     void* workspace, int64_t workspace_bytes,
                     void* stream);

/*
 * gemm_relu_f16_forced_ws -- gemm_relu_f16_forced with a workspace, which
 * also accepts GR_PATH_TILE_PACKED, GR_PATH_SMALL_M_SPLIT and
 * GR_PATH_TILE_SPLIT when the problem qualifies and the workspace holds the
 * bytes that path needs, whatever the size of the problem (a split path may
 * then use a single split).  Test hook.
 */
int gemm_relu_f16_forced_ws(int64_t M, int64_t N, int64_t K,
                            const uint16_t* A, int64_t lda,
                            const uint16_t* B, int64_t ldb,
                            uint16_t* C, int64_t ldc,
                            void* workspace, int64_t workspace_bytes,
                            void* stream, int path);

/*
 * gemm_relu_f16_plan_ws -- the planner's decision for gemm_relu_f16_ws with a
 * workspace of `workspace_bytes` bytes (its address is not checked).  Pure,
 * like gemm_relu_f16_plan.
 */
int gemm_relu_f16_plan_ws(int64_t M, int64_t N, int64_t K,
                          const uint16_t* A, int64_t lda,
                          const uint16_t* B, int64_t ldb,
                          const uint16_t* C, int64_t ldc,
                          int64_t workspace_bytes, gr_plan_t* out);

/*
 * ---- B given transposed -----------------------------------------------------
 * The same operation with B stored as its transpose Bt (N x K row-major,
 * element (n, k) at Bt[n*ldbt + k], pitch ldbt >= max(1, K)): C := ReLU(A *
 * Bt^T).  This is the layout of a weight matrix in the GEMV pattern of "Tilelang
 * Cuda Patterns", section 4 (B as N x K, each output a dot product of two
 * contiguous rows) and of the B_T option of the tutorial's GEMM.  Every
 * convention above holds, with Bt in the place of B; the paths are:
 *   GR_PATH_SMALL_M   M <= 16, 16-byte rows of A and Bt: each wave streams 16
 *                     rows of Bt, whose 16-byte pieces are MFMA operands as
 *                     they stand;
 *   GR_PATH_TILE_STREAM  M > 16, K % 32 == 0, N >= 64, rows of A and Bt
 *                     of any alignment: the row-blocked streaming kernel (64 x
 *                     64 blocks, K split between a block's 4 or 8 waves) with
 *                     blocks of 16 rows of Bt copied and read like those of
 *                     A; the planner takes it for up to 256 blocks from K =
 *                     256 and up to 512 from K = 1024, and at any size when
 *                     rows of A or Bt are not 16-byte aligned;
 *   GR_PATH_TILE      16-byte rows of A and Bt, K % 32 == 0, pitches of at
 *                     most 2^22 elements: the pipelined kernel with Bt staged
 *                     like A;
 *   GR_PATH_TILE_EDGE everything else (guarded register-staged kernel).
 * There is no workspace variant.
 */
int gemm_relu_f16_bt(int64_t M, int64_t N, int64_t K,
                     const uint16_t* A, int64_t lda,
                     const uint16_t* Bt, int64_t ldbt,
                     uint16_t* C, int64_t ldc,
                     void* stream);

/* Pure planner for gemm_relu_f16_bt (no GPU needed); see gemm_relu_f16_plan. */
int gemm_relu_f16_bt_plan(int64_t M, int64_t N, int64_t K,
                          const uint16_t* A, int64_t lda,
                          const uint16_t* Bt, int64_t ldbt,
                          const uint16_t* C, int64_t ldc,
                          gr_plan_t* out);

/* gemm_relu_f16_bt on a given path (GR_PATH_TILE, GR_PATH_TILE_EDGE,
   GR_PATH_SMALL_M or GR_PATH_TILE_STREAM; GR_ERR_INVALID_PATH when the path's
   conditions do not hold).  Test hook. */
int gemm_relu_f16_bt_forced(int64_t M, int64_t N, int64_t K,
                            const uint16_t* A, int64_t lda,
                            const uint16_t* Bt, int64_t ldbt,
                            uint16_t* C, int64_t ldc,
                            void* stream, int path);

/*
 * ---- A given transposed -----------------------------------------------------
 * The same operation with A stored as its transpose At (K x M row-major,
 * element (k, m) at At[k*ldat + m], pitch ldat >= max(1, M)): C := ReLU(At^T
 * * B).  This is the transpose_A option of the pages' tile GEMM (T.gemm takes
 * transpose_A and transpose_B: "Writing high-performance kernels in
 * TileLang", section "編寫一個 GEMM"; the tutorial's dynamic-shape GEMM takes
 * trans_A and trans_B, chapter "动态形状与变长序列").  Every convention above
 * holds, with At in the place of A; the paths are:
 *   GR_PATH_SMALL_M   M <= 16, K % 32 == 0, N >= 64: the streaming small-M
 *                     kernel (B of any alignment), each lane gathering its k
 *                     run of one column of At;
 *   GR_PATH_TILE      M >= 256, 16-byte rows of At and B, K % 32 == 0,
 *                     pitches of at most 2^25 elements: the 32-deep pipelined
 *                     kernel with At strips staged and read like B's;
 *   GR_PATH_TILE_EDGE everything else (the guarded kernel, At transposed in
 *                     registers).
 * There is no workspace variant; fp16 with the fused ReLU only.
 */
int gemm_relu_f16_ta(int64_t M, int64_t N, int64_t K,
                     const uint16_t* At, int64_t ldat,
                     const uint16_t* B, int64_t ldb,
                     uint16_t* C, int64_t ldc,
                     void* stream);

/* Pure planner for gemm_relu_f16_ta (no GPU needed); see gemm_relu_f16_plan. */
int gemm_relu_f16_ta_plan(int64_t M, int64_t N, int64_t K,
                          const uint16_t* At, int64_t ldat,
                          const uint16_t* B, int64_t ldb,
                          const uint16_t* C, int64_t ldc,
                          gr_plan_t* out);

/* gemm_relu_f16_ta on a given path (GR_PATH_TILE, GR_PATH_TILE_EDGE or
   GR_PATH_SMALL_M; GR_ERR_INVALID_PATH otherwise or when the path's
   conditions do not hold).  Test hook. */
int gemm_relu_f16_ta_forced(int64_t M, int64_t N, int64_t K,
                            const uint16_t* At, int64_t ldat,
                            const uint16_t* B, int64_t ldb,
                            uint16_t* C, int64_t ldc,
                            void* stream, int path);

/*
 * ---- bfloat16 operands and result ---------------------------------------------
 * The same operation with A, B and C in bfloat16 (1 sign, 8 exponent, 7
 * fraction bits: the upper half of a binary32): products accumulate in fp32,
 * ReLU acts on the fp32 sum, and the result is rounded to bfloat16 (nearest,
 * ties to even) when it is written.  The TileLang tutorial, section "张量核与
 * CUDA core", names fp16 and bf16 as the inputs a GEMM feeds to the matrix
 * engines; the epilogue is the one defined above.  Every convention above
 * holds (layouts, pitches, edges, errors, streams); the paths are those of
 * gemm_relu_f16 without a workspace, chosen by the same rules:
 *   GR_PATH_SMALL_M        M <= 64, the small-M kernels;
 *   GR_PATH_TILE_STREAM    64 x 64 blocks on the streaming kernel (few
 *                          blocks, also one row of them for M <= 64; rows
 *                          of any alignment, K % 32 == 0);
 *   GR_PATH_TILE           16-byte rows of A and B, K % 32 == 0 (256x256 or
 *                          128x128 tiles);
 *   GR_PATH_TILE_UNALIGNED misaligned rows or K % 64 != 0, in place;
 *   GR_PATH_TILE_EDGE      everything else (guarded register-staged kernel).
 * gemm_relu_f16_plan describes the plan these calls follow (the path does not
 * depend on the element format).  gemm_relu_bf16_ws takes a caller workspace
 * exactly like gemm_relu_f16_ws (same sizes: gemm_relu_f16_workspace_size)
 * and then also uses the packed and split paths.
 */
int gemm_relu_bf16(int64_t M, int64_t N, int64_t K,
                   const uint16_t* A, int64_t lda,
                   const uint16_t* B, int64_t ldb,
                   uint16_t* C, int64_t ldc,
                   void* stream);

/* gemm_relu_bf16 on a given path (any path that needs no workspace;
   GR_ERR_INVALID_PATH for the others, or when the path's conditions do not
   hold).  Test hook. */
int gemm_relu_bf16_forced(int64_t M, int64_t N, int64_t K,
                          const uint16_t* A, int64_t lda,
                          const uint16_t* B, int64_t ldb,
                          uint16_t* C, int64_t ldc,
                          void* stream, int path);

/* gemm_relu_bf16 with a caller workspace (see gemm_relu_f16_ws). */
int gemm_relu_bf16_ws(int64_t M, int64_t N, int64_t K,
                      const uint16_t* A, int64_t lda,
                      const uint16_t* B, int64_t ldb,
                      uint16_t* C, int64_t ldc,
                      void* workspace, int64_t workspace_bytes,
                      void* stream);

/* gemm_relu_bf16_ws on a given path (any GR_PATH_*; see
   gemm_relu_f16_forced_ws).  Test hook. */
int gemm_relu_bf16_forced_ws(int64_t M, int64_t N, int64_t K,
                             const uint16_t* A, int64_t lda,
                             const uint16_t* B, int64_t ldb,
                             uint16_t* C, int64_t ldc,
                             void* workspace, int64_t workspace_bytes,
                             void* stream, int path);

/*
 * ---- bias and other activations -------------------------------------------------
 * C := act(A * B + bias), the same tiled GEMM with a wider epilogue: bias is
 * a row vector of N values broadcast down the columns (bias[n] is added to
 * every element of column n; NULL for none), and act is one of the GR_ACT_*
 * codes below, applied to the fp32 sum.  The result is rounded once to the
 * output type (nearest, ties to even).  The elementwise pattern of "Tilelang
 * Cuda Patterns", section 1, lists relu, sigmoid, tanh and gelu among the
 * activations and a broadcast among the operations; the tutorial's GEMM
 * chapters fuse such elementwise work into the write-back of the fp32
 * fragment.  The activations, on x = acc + bias[n] in fp32:
 *   GR_ACT_NONE       x (a plain GEMM; negative values are kept)
 *   GR_ACT_RELU       x > 0 ? x : +0 (with bias NULL: bit for bit gemm_relu_*)
 *   GR_ACT_GELU       x * Phi(x) = x/2 * (1 + erf(x / sqrt(2)))
 *   GR_ACT_GELU_TANH  x/2 * (1 + tanh(sqrt(2/pi) * (x + 0.044715 x^3)))
 *   GR_ACT_SILU       x / (1 + exp(-x))
 *   GR_ACT_SIGMOID    1 / (1 + exp(-x))
 *   GR_ACT_TANH       tanh(x)
 * The transcendental functions are the device library's fp32 ones (a few
 * ulp of fp32, far below the output's rounding).  A, B, bias and C share the
 * element type: fp16 for gemm_bias_act_f16, bfloat16 for gemm_bias_act_bf16.
 * Every convention of gemm_relu_f16 holds; in addition GR_ERR_INVALID_ARG
 * for an unknown act and GR_ERR_ALIAS when the bias overlaps C.  K == 0
 * gives C = act(bias) (act(0) without a bias).  Paths: GR_PATH_SMALL_M,
 * GR_PATH_TILE, GR_PATH_TILE_EDGE, chosen as gemm_relu_f16_plan says;
 * gemm_bias_act_ws below adds the workspace paths.
 */
#define GR_ACT_NONE        0
#define GR_ACT_RELU        1
#define GR_ACT_GELU        2
#define GR_ACT_GELU_TANH   3
#define GR_ACT_SILU        4
#define GR_ACT_SIGMOID     5
#define GR_ACT_TANH        6

int gemm_bias_act_f16(int64_t M, int64_t N, int64_t K,
                      const uint16_t* A, int64_t lda,
                      const uint16_t* B, int64_t ldb,
                      const uint16_t* bias, int act,
                      uint16_t* C, int64_t ldc,
                      void* stream);

int gemm_bias_act_bf16(int64_t M, int64_t N, int64_t K,
                       const uint16_t* A, int64_t lda,
                       const uint16_t* B, int64_t ldb,
                       const uint16_t* bias, int act,
                       uint16_t* C, int64_t ldc,
                       void* stream);

/* The two calls above on a given path (any path that needs no workspace;
   GR_PATH_TILE_PERSISTENT runs the same tiles one workgroup each, since the
   bias + activation epilogue stages fp32 blocks through all of LDS;
   GR_ERR_INVALID_PATH for the others or when the path's conditions do not
   hold).  Test hooks. */
int gemm_bias_act_f16_forced(int64_t M, int64_t N, int64_t K,
                             const uint16_t* A, int64_t lda,
                             const uint16_t* B, int64_t ldb,
                             const uint16_t* bias, int act,
                             uint16_t* C, int64_t ldc,
                             void* stream, int path);

int gemm_bias_act_bf16_forced(int64_t M, int64_t N, int64_t K,
                              const uint16_t* A, int64_t lda,
                              const uint16_t* B, int64_t ldb,
                              const uint16_t* bias, int act,
                              uint16_t* C, int64_t ldc,
                              void* stream, int path);

/* gemm_bias_act_f16 / _bf16 with a caller workspace (see gemm_relu_f16_ws;
   the sizes of gemm_relu_f16_workspace_size apply): fmt is GR_FMT_F16 or GR_FMT_BF16 (the
   format of A, B, bias and C), path -1 lets the planner choose (then the
   packed and split paths run bias and activation in their final pass), any
   GR_PATH_* forces one.  The bias must not overlap C or the workspace. */
int gemm_bias_act_ws(int64_t M, int64_t N, int64_t K,
                     const uint16_t* A, int64_t lda,
                     const uint16_t* B, int64_t ldb,
                     const uint16_t* bias, int act,
                     uint16_t* C, int64_t ldc, int fmt,
                     void* workspace, int64_t workspace_bytes,
                     void* stream, int path);

/*
 * gemm_bias_act_bt -- C := act(A * Bt^T + bias) with B given transposed (Bt,
 * N x K row-major, pitch ldbt; the layout of a linear layer's weight), in
 * fp16 or bfloat16 (fmt: GR_FMT_F16 / GR_FMT_BF16, the format of A, Bt, bias
 * and C): the epilogue of gemm_bias_act_f16 on the paths of gemm_relu_f16_bt
 * (GR_PATH_SMALL_M, GR_PATH_TILE_STREAM, GR_PATH_TILE, GR_PATH_TILE_EDGE,
 * chosen as gemm_relu_f16_bt_plan says).  path -1 lets the planner choose;
 * one of those four forces it (test hook; GR_ERR_INVALID_PATH when its
 * conditions do not hold).  Errors as gemm_bias_act_f16, plus GR_ERR_INVALID_ARG for an unknown
 * fmt.
 */
int gemm_bias_act_bt(int64_t M, int64_t N, int64_t K,
                     const uint16_t* A, int64_t lda,
                     const uint16_t* Bt, int64_t ldbt,
                     const uint16_t* bias, int act,
                     uint16_t* C, int64_t ldc, int fmt,
                     void* stream, int path);

/*
 * ---- fp8 operands ---------------------------------------------------------------
 * C := act(scale_a * scale_b * (A * Bt^T) + bias) with A (M x K) and Bt
 * (N x K) in OCP fp8 E4M3 (1 sign, 4 exponent bits with bias 7, 3 fraction
 * bits; no infinities; S.1111.111 is NaN; largest finite 448), one byte per
 * element, both row-major with row pitches lda, ldbt >= max(1, K) in bytes
 * (elements).  B is given transposed, the layout of a weight matrix and of
 * the usual fp8 GEMM; products accumulate in fp32; scale_a and scale_b are
 * per-tensor dequantisation scales (host floats), multiplied together in fp32
 * and applied to the fp32 sum; then the optional bias (N values in the output
 * format) and the activation (GR_ACT_*), and one rounding to the output
 * format out_fmt (GR_FMT_F16 or GR_FMT_BF16, nearest even).  The pages list
 * an fp8 GEMM with per-block scales among the TileLang examples (blog
 * "TileLang programming basics", section "推荐顺序", step 6) and fp8 as the
 * tensor-core format after tf32 and int8 (TileLang tutorial, section
 * "张量核与 CUDA core"); per-tensor scales are the plainest form of those
 * scales.  Paths: GR_PATH_SMALL_M (M <= 16, K a multiple of 512, A, Bt and
 * their pitches 16-byte aligned: a stream over Bt), GR_PATH_TILE (K a
 * multiple of 64, the same alignment, any M and N; 256 x 256 tiles, or
 * 128 x 128 when those would leave compute units idle) and GR_PATH_TILE_EDGE
 * (everything else, including K == 0, which gives act(bias)).  C is fp16 or bfloat16 bits with
 * pitch ldc; the conventions of gemm_relu_f16 hold otherwise (C never read,
 * outside the M x N window never written, GR_ERR_ALIAS when C overlaps A,
 * Bt or the bias, GR_ERR_INVALID_ARG for an unknown act or out_fmt).
 */
int gemm_fp8_bt(int64_t M, int64_t N, int64_t K,
                const uint8_t* A, int64_t lda,
                const uint8_t* Bt, int64_t ldbt,
                float scale_a, float scale_b,
                const uint16_t* bias, int act,
                uint16_t* C, int64_t ldc, int out_fmt,
                void* stream);

/* gemm_fp8_bt on a given path (GR_PATH_TILE, GR_PATH_TILE_EDGE or
   GR_PATH_SMALL_M; GR_ERR_INVALID_PATH otherwise or when the path's
   conditions do not hold).  Test hook. */
int gemm_fp8_bt_forced(int64_t M, int64_t N, int64_t K,
                       const uint8_t* A, int64_t lda,
                       const uint8_t* Bt, int64_t ldbt,
                       float scale_a, float scale_b,
                       const uint16_t* bias, int act,
                       uint16_t* C, int64_t ldc, int out_fmt,
                       void* stream, int path);

/* Pure planner for gemm_fp8_bt (no GPU needed): vec_a and vec_b are in
   bytes (16 on the pipelined path). */
int gemm_fp8_bt_plan(int64_t M, int64_t N, int64_t K,
                     const uint8_t* A, int64_t lda,
                     const uint8_t* Bt, int64_t ldbt,
                     const uint16_t* bias, int act,
                     const uint16_t* C, int64_t ldc, int out_fmt,
                     gr_plan_t* out);

/*
 * gemm_fp8_bt with a caller workspace.  When the 128 x 128 tiles of the
 * pipelined kernel would leave most CUs idle (at most 128 tiles) and K is
 * long, K is split S ways (GR_PATH_TILE_SPLIT): each split's fp32 sums of
 * A * Bt^T go to the workspace (S x M x N floats), and a second kernel adds
 * the splits in order, then applies scale_a * scale_b, the bias, the
 * activation and the rounding once, as the unsplit path does.  This is the
 * split-K the pages give for a small M x N with a long K (blog "TileLang
 * programming basics", section 5.1 "Split-K"), with ordered fp32 partial
 * sums in place of atomic adds.  Workspace rules as for
 * gemm_relu_f16_ws (256-byte aligned; NULL, 0 = none; GR_ERR_ALIAS when it
 * overlaps A, Bt, C or the bias).  path -1 lets the planner choose;
 * GR_PATH_TILE, GR_PATH_TILE_EDGE, GR_PATH_SMALL_M or GR_PATH_TILE_SPLIT
 * force one (GR_ERR_INVALID_PATH when its conditions do not hold or the
 * workspace is too small).
 */
int gemm_fp8_bt_ws(int64_t M, int64_t N, int64_t K,
                   const uint8_t* A, int64_t lda,
                   const uint8_t* Bt, int64_t ldbt,
                   float scale_a, float scale_b,
                   const uint16_t* bias, int act,
                   uint16_t* C, int64_t ldc, int out_fmt,
                   void* workspace, int64_t workspace_bytes,
                   void* stream, int path);

/* Bytes of workspace with which gemm_fp8_bt_ws splits K for this problem
   (0: it never does).  Validates like gemm_fp8_bt; no HIP call.  bytes is a
   host pointer (not NULL). */
int gemm_fp8_bt_workspace_size(int64_t M, int64_t N, int64_t K,
                               const uint8_t* A, int64_t lda,
                               const uint8_t* Bt, int64_t ldbt,
                               const uint16_t* C, int64_t ldc,
                               int64_t* bytes);

/* The planner's decision for gemm_fp8_bt_ws with a workspace of
   workspace_bytes bytes (its address is not checked).  Pure. */
int gemm_fp8_bt_plan_ws(int64_t M, int64_t N, int64_t K,
                        const uint8_t* A, int64_t lda,
                        const uint8_t* Bt, int64_t ldbt,
                        const uint16_t* bias, int act,
                        const uint16_t* C, int64_t ldc, int out_fmt,
                        int64_t workspace_bytes, gr_plan_t* out);

/*
 * ---- MX fp8 (block-scaled) operands ---------------------------------------------
 * C := act(A~ * Bt~^T + bias) where A~[m][k] = A[m][k] * 2^(SA[m][k/32] - 127)
 * and Bt~[n][k] = Bt[n][k] * 2^(SB[n][k/32] - 127): A (M x K) and Bt (N x K)
 * hold OCP fp8 E4M3 bytes as for gemm_fp8_bt, and every run of 32 consecutive
 * k of a row shares one OCP MX E8M0 scale byte (value 2^(x - 127), 0 <= x <=
 * 254; x = 255 is NaN).  scale_a is M x K/32 bytes (row pitch ld_sa >=
 * max(1, K/32)), scale_b is N x K/32 bytes (pitch ld_sb).  Products
 * accumulate in fp32 (the matrix cores apply the scales, one per lane and
 * 32-k block); then bias, activation and one rounding to out_fmt as for
 * gemm_fp8_bt.  The pages name block-scaled GEMMs -- quantised operands with
 * per-block scales -- among the TileLang examples (blog "TileLang programming
 * basics", section "推荐顺序", step 6, and the block-scaled MMA row of the
 * table in section 5.4); OCP MX is the block format gfx950 scales in
 * hardware.
 *   K must be a multiple of 32 (GR_ERR_INVALID_DIM otherwise).
 *   Paths: GR_PATH_TILE (the pipelined fp8 kernel; K % 128 == 0, 16-byte
 *   aligned rows of A and Bt, 4-byte aligned scale rows: scale pointers and
 *   pitches multiples of 4) or GR_PATH_TILE_EDGE (guarded, any alignment).
 *   Other conventions as gemm_fp8_bt; the scale arrays must not overlap C
 *   (GR_ERR_ALIAS).  No workspace variant.
 */
int gemm_mxfp8_bt(int64_t M, int64_t N, int64_t K,
                  const uint8_t* A, int64_t lda,
                  const uint8_t* scale_a, int64_t ld_sa,
                  const uint8_t* Bt, int64_t ldbt,
                  const uint8_t* scale_b, int64_t ld_sb,
                  const uint16_t* bias, int act,
                  uint16_t* C, int64_t ldc, int out_fmt,
                  void* stream);

/* gemm_mxfp8_bt on a given path (GR_PATH_TILE or GR_PATH_TILE_EDGE;
   GR_ERR_INVALID_PATH otherwise or when the path's conditions do not hold).
   Test hook. */
int gemm_mxfp8_bt_forced(int64_t M, int64_t N, int64_t K,
                         const uint8_t* A, int64_t lda,
                         const uint8_t* scale_a, int64_t ld_sa,
                         const uint8_t* Bt, int64_t ldbt,
                         const uint8_t* scale_b, int64_t ld_sb,
                         const uint16_t* bias, int act,
                         uint16_t* C, int64_t ldc, int out_fmt,
                         void* stream, int path);

/* Pure planner for gemm_mxfp8_bt (no GPU needed). */
int gemm_mxfp8_bt_plan(int64_t M, int64_t N, int64_t K,
                       const uint8_t* A, int64_t lda,
                       const uint8_t* scale_a, int64_t ld_sa,
                       const uint8_t* Bt, int64_t ldbt,
                       const uint8_t* scale_b, int64_t ld_sb,
                       const uint16_t* bias, int act,
                       const uint16_t* C, int64_t ldc, int out_fmt,
                       gr_plan_t* out);

/*
 * ---- MX fp4 (block-scaled) operands ---------------------------------------------
 * gemm_mxfp8_bt with OCP fp4 E2M1 elements (1 sign bit, 2 exponent bits with
 * bias 1, 1 fraction bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) packed two
 * per byte, element k of a row in the low nibble of byte k/2 when k is even
 * and in the high nibble when it is odd.  K counts elements (a multiple of
 * 32); lda and ldbt count bytes (>= K/2); the scales are as for MX fp8 (one
 * E8M0 byte per 32 elements).  The pages name NVFP4 block-scaled MMA (fp4
 * elements with per-block scales; blog "TileLang programming basics", table
 * of section 5.4); MX fp4 is the fp4 block format gfx950 scales in hardware.
 * Paths: GR_PATH_TILE (K % 128 == 0, 16-byte aligned rows, 4-byte aligned
 * scale rows) or GR_PATH_TILE_EDGE.  Other conventions as gemm_mxfp8_bt.
 */
int gemm_mxfp4_bt(int64_t M, int64_t N, int64_t K,
                  const uint8_t* A, int64_t lda,
                  const uint8_t* scale_a, int64_t ld_sa,
                  const uint8_t* Bt, int64_t ldbt,
                  const uint8_t* scale_b, int64_t ld_sb,
                  const uint16_t* bias, int act,
                  uint16_t* C, int64_t ldc, int out_fmt,
                  void* stream);

/* gemm_mxfp4_bt on a given path (GR_PATH_TILE or GR_PATH_TILE_EDGE).
   Test hook. */
int gemm_mxfp4_bt_forced(int64_t M, int64_t N, int64_t K,
                         const uint8_t* A, int64_t lda,
                         const uint8_t* scale_a, int64_t ld_sa,
                         const uint8_t* Bt, int64_t ldbt,
                         const uint8_t* scale_b, int64_t ld_sb,
                         const uint16_t* bias, int act,
                         uint16_t* C, int64_t ldc, int out_fmt,
                         void* stream, int path);

/* Pure planner for gemm_mxfp4_bt (no GPU needed). */
int gemm_mxfp4_bt_plan(int64_t M, int64_t N, int64_t K,
                       const uint8_t* A, int64_t lda,
                       const uint8_t* scale_a, int64_t ld_sa,
                       const uint8_t* Bt, int64_t ldbt,
                       const uint8_t* scale_b, int64_t ld_sb,
                       const uint16_t* bias, int act,
                       const uint16_t* C, int64_t ldc, int out_fmt,
                       gr_plan_t* out);

/*
 * gemm_relu_f16_noalloc -- gemm_relu_f16_ws without a caller workspace and
 * without any allocation: for callers that cannot allocate device memory
 * (code being captured into a HIP graph, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, result and paths as gemm_relu_f16_ws
 * with a workspace of the size gemm_relu_f16_workspace_size reports; the
 * workspace is a static device array of the library, GR_NOALLOC_SCRATCH_BYTES
 * bytes, one per GPU, held from the library's first use of that GPU until
 * the process ends.  Problems whose workspace would exceed it are refused
 * with GR_ERR_SCRATCH before anything is launched (pure check, no HIP call);
 * problems that need no workspace run the in-place paths and do not touch
 * it.  Calls no hipMalloc, hipFree or allocating library routine.
 * Every call on one GPU shares that GPU's array: two calls that overlap in
 * time on one GPU (on different streams, or from different threads) race
 * and give undefined results; calls ordered on one stream are safe.  The
 * paths that use it overwrite what they read within the call (nothing in it
 * has to start at zero).
 */
#define GR_NOALLOC_SCRATCH_BYTES (32ll << 20)
int gemm_relu_f16_noalloc(int64_t M, int64_t N, int64_t K,
                          const uint16_t* A, int64_t lda,
                          const uint16_t* B, int64_t ldb,
                          uint16_t* C, int64_t ldc,
                          void* stream);

/*
 * gemm_relu_stream_read -- a measurement aid, not part of the operation:
 * reads `bytes` bytes of the device buffer `src` once with 256 workgroups of
 * 512 threads and nontemporal 16-byte loads, and writes the 64-bit XOR of
 * each workgroup's words to `sink` (device, 256 x 8 bytes), so that timing
 * it gives the HBM read ceiling a bandwidth-bound path is judged against
 * (the roofline's memory leg; TileLang tutorial, chapter "性能取证",
 * sections "三层归因" and "Roofline 计算器").  pattern 0
 * (GR_READ_CONTIGUOUS): workgroup g reads the g-th contiguous 1/256 of the
 * buffer; pattern 1 (GR_READ_ROW_PIECES): the buffer as rows of 32 KiB,
 * workgroup g reads 256-byte piece g % 128 of each row of half g / 128 of
 * the rows.  bytes: a positive multiple of 8 MiB; src 16-byte and sink
 * 8-byte aligned and disjoint.  Errors: GR_ERR_INVALID_ARG, GR_ERR_NULL_PTR,
 * GR_ERR_ALIAS, device errors.  Enqueues on `stream`.
 */
#define GR_READ_CONTIGUOUS 0
#define GR_READ_ROW_PIECES 1
int gemm_relu_stream_read(const void* src, int64_t bytes, int pattern, uint64_t* sink, void* stream);

/* Static, NUL-terminated name of a status code ("GR_OK", "GR_ERR_ALIAS", ...),
 * so that a refused call can be reported with its cause (the fail-loudly
 * behaviour cited at the status codes above).  Unknown codes give
 * "GR_ERR_UNKNOWN". */
const char* gemm_relu_status_string(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH.  Not an operation of
 * the pages: it identifies the build in test and benchmark reports. */
int gemm_relu_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_RELU_H_ */
