"""GPU parity of the transposed-A call (gemm_relu_f16_ta: A given as At, K x
M row-major) against the CPU oracle on A = At^T.

The transpose_A option of the pages' tile GEMM ("Writing high-performance
kernels in TileLang", section "編寫一個 GEMM"; TileLang tutorial, chapter
"动态形状与变长序列", trans_A).  Bar: |gpu - oracle| <= 1e-2 + 1e-2 |oracle|
per element, no NaN or Inf, C's padding untouched.
"""
import numpy as np
import pytest

import dense_gemm_epilogue_tiled_amd as gr
import oracle
import synth
from gpu_util import assert_parity, call, from_dev, full_dev, log, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("oracle_lib")]

SENTINEL = 0x7E5A


def transposed(A, M, K, ldat, pad=0x7BFF):
    """At (K x ldat) holding A^T, padding columns set to 65504."""
    At = np.full((K, ldat), pad, dtype=np.uint16)
    At[:, :M] = A[:M, :K].T
    return At


def run_ta(At, B, M, N, K, ldat, ldb, ldc, path=None, offs=(0, 0, 0)):
    import torch as t
    Atp = np.concatenate([np.zeros(offs[0], np.uint16), At.ravel()])
    Bp = np.concatenate([np.zeros(offs[1], np.uint16), B.ravel()])
    dA, dB = to_dev(Atp), to_dev(Bp)
    dC = full_dev((offs[2] + (M + 2) * ldc,), SENTINEL)
    s = t.cuda.current_stream().cuda_stream
    a, b, c = dA.data_ptr() + 2 * offs[0], dB.data_ptr() + 2 * offs[1], dC.data_ptr() + 2 * offs[2]
    if path is None:
        st = gr.gemm_relu_f16_ta(M, N, K, a, ldat, b, ldb, c, ldc, s)
    else:
        st = gr.gemm_relu_f16_ta_forced(M, N, K, a, ldat, b, ldb, c, ldc, s, path)
    t.cuda.synchronize()
    assert st == gr.GR_OK, gr.gemm_relu_status_string(st)
    Cflat = from_dev(dC)
    C = Cflat[offs[2]:offs[2] + M * ldc].reshape(M, ldc)
    assert np.all(Cflat[:offs[2]] == SENTINEL)
    assert np.all(C[:, N:] == SENTINEL), "a padding column of C was written"
    assert np.all(Cflat[offs[2] + M * ldc:] == SENTINEL), "a row past M was written"
    return C[:, :N]


# M, N, K, ldat, ldb, ldc, path, element offsets of At, B, C
CASES = [
    (512, 768, 256, 512, 768, 768, gr.GR_PATH_TILE, (0, 0, 0)),       # whole tiles
    (300, 520, 96, 304, 520, 521, gr.GR_PATH_TILE, (0, 0, 0)),        # last tile row moved up, partial N
    (2304, 4096, 128, 2304, 4096, 4096, gr.GR_PATH_TILE, (0, 0, 0)),  # 144 tiles
    (8, 4096, 4096, 8, 4096, 4096, gr.GR_PATH_SMALL_M, (0, 0, 0)),    # GEMV-like
    (3, 1000, 1024, 5, 1003, 1001, gr.GR_PATH_SMALL_M, (1, 3, 1)),    # odd pitches, misaligned B
    (16, 640, 96, 17, 640, 640, gr.GR_PATH_SMALL_M, (0, 0, 0)),
    (257, 300, 130, 259, 301, 300, gr.GR_PATH_TILE_EDGE, (1, 1, 0)),  # ragged K, odd pitches
    (100, 200, 70, 100, 200, 200, gr.GR_PATH_TILE_EDGE, (0, 0, 0)),   # M < 256
    (8, 60, 50, 9, 60, 61, gr.GR_PATH_TILE_EDGE, (0, 0, 0)),          # tiny
]


@pytest.mark.parametrize("M,N,K,ldat,ldb,ldc,path,offs", CASES)
def test_transposed_a_parity(M, N, K, ldat, ldb, ldc, path, offs):
    A, B = synth.random_operands(M, N, K, seed=M + 3 * N + 5 * K, ldb=ldb, b_scale=K ** -0.5)
    At = transposed(A, M, K, ldat)
    st, plan = gr.gemm_relu_f16_ta_plan(M, N, K, 0x100000 + 2 * offs[0], ldat, 0x200000000000 + 2 * offs[1], ldb,
                                        0x400000000000 + 2 * offs[2], ldc)
    log("ta %dx%dx%d ldat=%d plan=%s forced=%d" % (M, N, K, ldat, plan["path_name"], path))
    assert st == gr.GR_OK and plan["path"] == path
    ref = oracle.gemm_relu_full(A, B, M=M, N=N, K=K, ldb=ldb)
    C = run_ta(At, B, M, N, K, ldat, ldb, ldc, offs=offs)
    assert_parity(C, ref, "ta %dx%dx%d" % (M, N, K))
    # the guarded kernel takes every problem
    C2 = run_ta(At, B, M, N, K, ldat, ldb, ldc, path=gr.GR_PATH_TILE_EDGE, offs=offs)
    assert_parity(C2, ref, "ta guarded %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K", [(2304, 4096, 96), (2560, 4096, 160)])
def test_transposed_a_pipelined_matches_plain_layout_bitwise(M, N, K):
    """K % 64 == 32 and more than 128 tiles: the plain call runs the same
    32-deep 256 x 256 kernel with A staged row by row, so the two layouts give
    the same bits."""
    A, B = synth.random_operands(M, N, K, seed=11 * M + K)
    At = transposed(A, M, K, M)
    Cta = run_ta(At, B, M, N, K, M, N, N, path=gr.GR_PATH_TILE)
    dC = full_dev((M * N,), SENTINEL)
    assert call(M, N, K, to_dev(A), K, to_dev(B), N, dC, N, path=gr.GR_PATH_TILE) == gr.GR_OK
    assert np.array_equal(Cta, from_dev(dC).reshape(M, N))
