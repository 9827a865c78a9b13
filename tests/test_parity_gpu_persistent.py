"""GPU parity of the persistent tile loop (GR_PATH_TILE_PERSISTENT): at most
one workgroup per CU walks the tiles g, g + grid, g + 2 grid, ... and stores
each finished tile 32 rows at a time while the next tile's first copies are
in flight (TileLang tutorial, "Persistent kernel").

Each tile adds its k terms in the same order as the one-workgroup-per-tile
kernel (GR_PATH_TILE), so the two must agree bit for bit; both are checked
against the CPU oracle (|gpu - oracle| <= 1e-2 + 1e-2 |oracle|), with C's
padding and the rows after C never written.
"""
import numpy as np
import pytest

import dense_gemm_epilogue_tiled_amd as gr
import oracle
import synth
from gpu_util import as_f64, assert_parity, call, from_dev, full_dev, log, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("oracle_lib")]

SENTINEL = 0x7E5A

# M, N, K, pitch pads of A, B and C (multiples of 8).  Tile counts: below one
# wave of CUs, exactly one, one and a fraction, two; K from one 64-deep strip
# (no steady step) through every prologue variant to a long steady loop.
CASES = [
    (256, 256, 64, 0, 0, 0),        # one tile, K = 64: two 32-deep steps, one A strip
    (512, 768, 128, 8, 0, 8),       # 6 tiles, K = 128, padded pitches
    (2304, 4096, 192, 0, 8, 0),     # 144 tiles, K = 192 (three A strips)
    (4096, 4096, 256, 0, 0, 0),     # 256 tiles: one per workgroup
    (4608, 4096, 320, 0, 0, 16),    # 288 tiles: 32 workgroups take a second tile
    (4096, 8192, 512, 8, 8, 8),     # 512 tiles: two each
    (8192, 8192, 64, 0, 0, 0),      # 1024 tiles of one strip each: four per workgroup
]


def _run(M, N, K, dA, lda, dB, ldb, ldc, path, extra_rows=2):
    dC = full_dev(((M + extra_rows) * ldc,), SENTINEL)
    assert call(M, N, K, dA, lda, dB, ldb, dC, ldc, path=path) == gr.GR_OK
    Cf = from_dev(dC)
    return Cf


@pytest.mark.parametrize("M,N,K,pa,pb,pc", CASES)
def test_persistent_matches_tile_kernel_and_oracle(M, N, K, pa, pb, pc):
    lda, ldb, ldc = K + pa, N + pb, N + pc
    A, B = synth.random_operands(M, N, K, seed=11 * M + N + K, lda=lda, ldb=ldb)
    dA, dB = to_dev(A), to_dev(B)
    st, p = gr.gemm_relu_f16_plan(M, N, K, 0x100000, lda, 0x200000000000, ldb, 0x400000000000, ldc)
    log("persistent %dx%dx%d lda=%d ldb=%d ldc=%d" % (M, N, K, lda, ldb, ldc))
    Cp = _run(M, N, K, dA, lda, dB, ldb, ldc, gr.GR_PATH_TILE_PERSISTENT)
    Ct = _run(M, N, K, dA, lda, dB, ldb, ldc, gr.GR_PATH_TILE)
    assert np.array_equal(Cp, Ct), "persistent and one-tile-per-workgroup results differ"
    C = Cp[:M * ldc].reshape(M, ldc)
    assert np.all(C[:, N:] == SENTINEL), "a padding column of C was written"
    assert np.all(Cp[M * ldc:] == SENTINEL), "a row past M was written"
    if M * N * K <= 2 ** 28:
        ref = oracle.gemm_relu_full(A, B, M=M, N=N, K=K, lda=lda, ldb=ldb)
        assert_parity(C[:, :N], ref, "persistent full")
    else:
        ii, jj = synth.sample_indices(M, N, 4096, M + K)
        ref = oracle.gemm_relu_elems(A, B, ii, jj, M=M, N=N, K=K, lda=lda, ldb=ldb)
        assert_parity(C[ii, jj], ref, "persistent sampled")
        # the first and last row of every tile row band a workgroup's later
        # tiles write
        rows = sorted({0, 255, 256, M - 256, M - 1})
        assert_parity(C[rows, :N], oracle.gemm_relu_rows(A, B, rows, M=M, N=N, K=K, lda=lda, ldb=ldb),
                      "persistent rows")


def test_persistent_bf16_matches_tile_kernel():
    import torch as t
    M, N, K = 4608, 4096, 256
    A, B = synth.random_operands(M, N, K, seed=5, fmt="bf16")
    dA, dB = to_dev(A), to_dev(B)
    s = t.cuda.current_stream().cuda_stream
    outs = []
    for path in (gr.GR_PATH_TILE_PERSISTENT, gr.GR_PATH_TILE):
        dC = full_dev((M * N,), SENTINEL)
        assert gr.gemm_relu_bf16_forced(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, dC.data_ptr(), N, s,
                                        path) == gr.GR_OK
        t.cuda.synchronize()
        outs.append(from_dev(dC))
    assert np.array_equal(outs[0], outs[1])
    ii, jj = synth.sample_indices(M, N, 4096, 9)
    got = as_f64(outs[0].reshape(M, N)[ii, jj], "bf16")
    ref = as_f64(oracle.gemm_relu_elems(A, B, ii, jj, fmt="bf16"), "bf16")
    assert np.all(np.abs(got - ref) <= 1e-2 + 1e-2 * np.abs(ref))


def test_persistent_with_bias_and_activation_falls_back_to_one_tile_per_workgroup():
    """The bias + activation epilogue has no 32-row form: forced onto the
    persistent path it runs the same tiles one workgroup each."""
    import torch as t
    M, N, K = 2304, 4096, 128
    A, B = synth.random_operands(M, N, K, seed=8)
    bias = synth.random_operands(1, N, 1, seed=9)[1].reshape(N)
    dA, dB, db = to_dev(A), to_dev(B), to_dev(bias)
    s = t.cuda.current_stream().cuda_stream
    outs = []
    for path in (gr.GR_PATH_TILE_PERSISTENT, gr.GR_PATH_TILE):
        dC = full_dev((M * N,), SENTINEL)
        assert gr.gemm_bias_act_f16_forced(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, db.data_ptr(),
                                           gr.ACT_CODES["gelu"], dC.data_ptr(), N, s, path) == gr.GR_OK
        t.cuda.synchronize()
        outs.append(from_dev(dC))
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("group_m,remap", [(1, 1), (3, 0), (16, 1), (1000, 0)])
def test_persistent_order_changes_no_bit(group_m, remap):
    import torch as t
    M, N, K = 4608, 4096, 128
    A, B = synth.random_operands(M, N, K, seed=21)
    dA, dB = to_dev(A), to_dev(B)
    base = _run(M, N, K, dA, K, dB, N, N, gr.GR_PATH_TILE_PERSISTENT, extra_rows=0)
    dC = full_dev((M * N,), SENTINEL)
    st = gr.gemm_relu_f16_forced_order(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, dC.data_ptr(), N,
                                       t.cuda.current_stream().cuda_stream, gr.GR_PATH_TILE_PERSISTENT, group_m,
                                       remap)
    t.cuda.synchronize()
    assert st == gr.GR_OK
    assert np.array_equal(base, from_dev(dC))


def test_mlp_workload_on_the_persistent_path():
    """The MLP projection (8192 x 28672 x 8192, 3584 tiles, 14 per workgroup):
    bitwise equal to the one-tile-per-workgroup kernel, sampled oracle check."""
    w = synth.WORKLOADS["mlp8192x28672x8192"]
    M, N, K = w.M, w.N, w.K
    A, B = synth.operands(w)
    dA, dB = to_dev(A), to_dev(B)
    log("persistent mlp")
    Cp = _run(M, N, K, dA, K, dB, N, N, gr.GR_PATH_TILE_PERSISTENT, extra_rows=0)
    Ct = _run(M, N, K, dA, K, dB, N, N, gr.GR_PATH_TILE, extra_rows=0)
    assert np.array_equal(Cp, Ct)
    ii, jj = synth.sample_indices(M, N, 4096, w.seed)
    assert_parity(Cp.reshape(M, N)[ii, jj], oracle.gemm_relu_elems(A, B, ii, jj), "mlp persistent sampled")
