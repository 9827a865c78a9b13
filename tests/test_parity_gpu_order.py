"""The workgroup order (grid-level swizzle and XCD renumbering) decides only
when each tile runs, never what it computes: every order gives the same bits.
Likewise a permutation of the rows of A permutes the rows of C bit for bit
(each output row's k order does not depend on where its tile lands).

The pages treat the grid swizzle as a free scheduling choice for L2 reuse
(TileLang tutorial, chapter "布局与存储体冲突", T.use_swizzle with any panel
size); these tests pin that the library's choice is equally free.
"""
import numpy as np
import pytest

import dense_gemm_epilogue_tiled_amd as gr
import oracle
import synth
from gpu_util import assert_parity, call, from_dev, full_dev, log, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("oracle_lib")]

SENTINEL = 0x7E5A
ORDERS = [(1, 1), (2, 0), (3, 1), (7, 0), (16, 1), (64, 0), (1000, 1)]

# M, N, K, pitch pad of A and B, path: every tile kernel the order reaches
SHAPES = [
    (2304, 4096, 128, 0, 0, gr.GR_PATH_TILE),             # 256 x 256, K % 64 == 0, 144 tiles
    (2304, 4096, 96, 0, 0, gr.GR_PATH_TILE),              # 256 x 256, 32-deep strips (K % 64 == 32)
    (1000, 1000, 256, 0, 0, gr.GR_PATH_TILE),             # 128 x 128 tiles (few large ones), ragged
    (2304, 4099, 300, 3, 5, gr.GR_PATH_TILE_UNALIGNED),   # misaligned rows, ragged K and N
    (700, 600, 130, 1, 1, gr.GR_PATH_TILE_EDGE),          # guarded kernel
]


def _call_order(M, N, K, dA, lda, dB, ldb, path, group_m, remap):
    import torch as t
    dC = full_dev((M * N,), SENTINEL)
    st = gr.gemm_relu_f16_forced_order(M, N, K, dA.data_ptr(), lda, dB.data_ptr(), ldb, dC.data_ptr(), N,
                                       t.cuda.current_stream().cuda_stream, path, group_m, remap)
    t.cuda.synchronize()
    assert st == gr.GR_OK, gr.gemm_relu_status_string(st)
    return from_dev(dC)


@pytest.mark.parametrize("M,N,K,pa,pb,path", SHAPES)
def test_workgroup_order_changes_no_bit(M, N, K, pa, pb, path):
    lda, ldb = K + pa, N + pb
    A, B = synth.random_operands(M, N, K, seed=M + N + K, lda=lda, ldb=ldb)
    dA, dB = to_dev(A), to_dev(B)
    base = _call_order(M, N, K, dA, lda, dB, ldb, path, 4, 1)  # the planner's order
    ii, jj = synth.sample_indices(M, N, 2048, 3)
    ref = oracle.gemm_relu_elems(A, B, ii, jj, M=M, N=N, K=K, lda=lda, ldb=ldb)
    assert_parity(base.reshape(M, N)[ii, jj], ref, "order base")
    for gm, remap in ORDERS:
        log("order %dx%dx%d path=%d group_m=%d remap=%d" % (M, N, K, path, gm, remap))
        assert np.array_equal(base, _call_order(M, N, K, dA, lda, dB, ldb, path, gm, remap)), (gm, remap)


def test_order_hook_rejects_bad_arguments():
    import torch as t
    args = (512, 512, 64, 0x100000, 64, 0x200000000000, 512, 0x400000000000, 512, None)
    assert gr.gemm_relu_f16_forced_order(*args, gr.GR_PATH_TILE, 0, 1) == gr.GR_ERR_INVALID_ARG
    assert gr.gemm_relu_f16_forced_order(*args, gr.GR_PATH_TILE, 4, 2) == gr.GR_ERR_INVALID_ARG
    assert gr.gemm_relu_f16_forced_order(*args, gr.GR_PATH_TILE_PACKED, 4, 1) == gr.GR_ERR_INVALID_PATH
    del t


@pytest.mark.parametrize("M,N,K,path", [(2304, 4096, 256, gr.GR_PATH_TILE), (1000, 1000, 256, gr.GR_PATH_TILE),
                                        (2304, 4096, 300, gr.GR_PATH_TILE_UNALIGNED),
                                        (8, 4096, 2048, gr.GR_PATH_SMALL_M)])
def test_row_permutation_of_A_permutes_C_bitwise(M, N, K, path):
    A, B = synth.random_operands(M, N, K, seed=2 * M + K, b_scale=K ** -0.5)
    perm = np.random.default_rng(M + N).permutation(M)
    dB = to_dev(B)
    dC1 = full_dev((M * N,), SENTINEL)
    dC2 = full_dev((M * N,), SENTINEL)
    assert call(M, N, K, to_dev(A), K, dB, N, dC1, N, path=path) == gr.GR_OK
    assert call(M, N, K, to_dev(np.ascontiguousarray(A[perm])), K, dB, N, dC2, N, path=path) == gr.GR_OK
    C1 = from_dev(dC1).reshape(M, N)
    C2 = from_dev(dC2).reshape(M, N)
    assert np.array_equal(C1[perm], C2)
