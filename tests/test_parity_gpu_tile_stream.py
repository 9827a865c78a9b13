"""GPU parity of the row-blocked streaming path (GR_PATH_TILE_STREAM) against
the CPU oracle.

Blocks of 64 rows x 64 columns of C, one per workgroup; the workgroup's
waves (4, or 8 up to 256 blocks) take the 32-row slots of K in turn through
rings of direct-to-LDS copies of their own and add their fp32 partial sums
in wave order at the end, so ReLU sees the complete sum (the split-K of the
TileLang tutorial's chapter "性能取证", kept inside one workgroup).  The
planner takes it for few blocks with K long enough (e.g. the 1024^3
workload) and, for misaligned rows, up to one or two rounds of blocks; the
workgroup order (plain row-major, or XCD renumbering with groups of 4 row
blocks) never changes a bit.
Bar: |gpu - oracle| <= 1e-2 + 1e-2 |oracle| per element, no NaN or Inf,
C's padding and rows past M untouched.
"""
import numpy as np
import pytest

import dense_gemm_epilogue_tiled_amd as gr
import oracle
import synth
from gpu_util import as_f64, assert_parity, call, from_dev, full_dev, log, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("oracle_lib")]

SENTINEL = 0x7E5A

# M, N, K, lda, ldb, ldc, element offsets of A, B, C (A's rows 16-byte
# aligned: lda and A's offset multiples of 8)
CASES = [
    (65, 64, 32, 32, 64, 64, (0, 0, 0)),            # 2 row blocks (the second 1 row), 1 slot: 7 idle waves
    (130, 65, 64, 64, 65, 70, (0, 1, 3)),           # last column block moved left to column 1, B odd pitch
    (1000, 1000, 1024, 1032, 1003, 1005, (8, 3, 1)),  # ragged M and N, B and C misaligned
    (200, 300, 96, 104, 301, 300, (0, 5, 0)),        # 3 slots, 8 waves (5 idle)
    (64, 128, 4096, 4096, 128, 128, (0, 0, 0)),      # one row block, long K
    (513, 200, 160, 168, 200, 203, (16, 0, 2)),      # 5 slots, a 1-row last block
]


def _run(M, N, K, lda, ldb, ldc, offs, path, seed):
    A, B = synth.random_operands(M, N, K, seed=seed, lda=lda, ldb=ldb)
    Ap = np.concatenate([np.zeros(offs[0], np.uint16), A.ravel()])
    Bp = np.concatenate([np.full(offs[1], 0x7BFF, np.uint16), B.ravel()])
    extra = 2
    dC = full_dev((offs[2] + (M + extra) * ldc,), SENTINEL)
    log("tile_stream %dx%dx%d lda=%d ldb=%d ldc=%d offs=%s path=%s" % (M, N, K, lda, ldb, ldc, offs, path))
    st = call(M, N, K, to_dev(Ap), lda, to_dev(Bp), ldb, dC, ldc, path=path, offsets=offs)
    assert st == gr.GR_OK, gr.gemm_relu_status_string(st)
    Cflat = from_dev(dC)
    C = Cflat[offs[2]:offs[2] + M * ldc].reshape(M, ldc)
    assert np.all(Cflat[:offs[2]] == SENTINEL), "an element before C was written"
    assert np.all(C[:, N:] == SENTINEL), "a padding column of C was written"
    assert np.all(Cflat[offs[2] + M * ldc:] == SENTINEL), "a row past M was written"
    return A, B, C[:, :N]


MISALIGNED_A_CASES = [
    (65, 64, 32, 33, 64, 64, (1, 0, 0)),             # one slot, A's base and pitch odd
    (130, 200, 96, 97, 201, 203, (1, 3, 5)),          # A, B and C misaligned, ragged edges
    (1000, 1000, 1024, 1025, 1000, 1000, (3, 0, 0)),  # long K, A's rows 2-byte aligned only
    (300, 520, 512, 516, 520, 520, (2, 0, 0)),        # A's rows 8-byte aligned
]


@pytest.mark.parametrize("M,N,K,lda,ldb,ldc,offs", MISALIGNED_A_CASES)
def test_tile_stream_parity_misaligned_a(M, N, K, lda, ldb, ldc, offs):
    """The streaming kernel copies A's rows from any 2-byte aligned address:
    full oracle check with A's and B's padding poisoned with 65504."""
    A, B = synth.random_operands(M, N, K, seed=M * 13 + N + K, lda=lda, ldb=ldb)
    A = A.copy()
    A.reshape(M, lda)[:, K:] = 0x7BFF
    Ap = np.concatenate([np.full(offs[0], 0x7BFF, np.uint16), A.ravel()])
    Bp = np.concatenate([np.full(offs[1], 0x7BFF, np.uint16), B.ravel()])
    dC = full_dev((offs[2] + (M + 2) * ldc,), SENTINEL)
    log("tile_stream misaligned A %dx%dx%d lda=%d ldb=%d ldc=%d offs=%s" % (M, N, K, lda, ldb, ldc, offs))
    st = call(M, N, K, to_dev(Ap), lda, to_dev(Bp), ldb, dC, ldc, path=gr.GR_PATH_TILE_STREAM, offsets=offs)
    assert st == gr.GR_OK, gr.gemm_relu_status_string(st)
    Cflat = from_dev(dC)
    C = Cflat[offs[2]:offs[2] + M * ldc].reshape(M, ldc)
    assert np.all(Cflat[:offs[2]] == SENTINEL), "an element before C was written"
    assert np.all(C[:, N:] == SENTINEL), "a padding column of C was written"
    assert np.all(Cflat[offs[2] + M * ldc:] == SENTINEL), "a row past M was written"
    ref = oracle.gemm_relu_full(A, B, M=M, N=N, K=K, lda=lda, ldb=ldb)
    log("parity %s" % (assert_parity(C[:, :N], ref, "tile_stream misaligned A %dx%dx%d" % (M, N, K)),))


@pytest.mark.parametrize("M,N,K,lda,ldb,ldc,offs", CASES)
def test_tile_stream_parity(M, N, K, lda, ldb, ldc, offs):
    """Forced row-blocked streaming path on padded, misaligned operands: full
    oracle check, padding of B poisoned with 65504."""
    A, B, C = _run(M, N, K, lda, ldb, ldc, offs, gr.GR_PATH_TILE_STREAM, seed=M * 31 + N + K)
    ref = oracle.gemm_relu_full(A, B, M=M, N=N, K=K, lda=lda, ldb=ldb)
    log("parity %s" % (assert_parity(C, ref, "tile_stream %dx%dx%d" % (M, N, K)),))


def test_square1024_workload_takes_tile_stream_and_matches_oracle():
    """The 1024^3 workload through the plain call: the planner picks the
    row-blocked streaming path (256 workgroups where 128 x 128 tiles give
    64); full oracle check; two calls agree bit for bit."""
    w = synth.WORKLOADS["square1024"]
    M, N, K = w.M, w.N, w.K
    st, p = gr.gemm_relu_f16_plan(M, N, K, 0x100000, K, 0x200000000000, N, 0x400000000000, N)
    assert st == gr.GR_OK and p["path"] == gr.GR_PATH_TILE_STREAM and p["grid"] == 256
    A, B = synth.operands(w)
    dA, dB = to_dev(A), to_dev(B)
    dC1 = full_dev((M * N,), SENTINEL)
    dC2 = full_dev((M * N,), SENTINEL)
    assert call(M, N, K, dA, K, dB, N, dC1, N) == gr.GR_OK
    assert call(M, N, K, dA, K, dB, N, dC2, N) == gr.GR_OK
    C = from_dev(dC1).reshape(M, N)
    assert np.array_equal(C, from_dev(dC2).reshape(M, N)), "two runs differ"
    log("parity %s" % (assert_parity(C, oracle.gemm_relu_full(A, B), "square1024"),))


def test_tile_stream_and_tile_kernel_agree():
    """The same problem on the row-blocked streaming path and on the 128 x 128
    tile kernel: both within the bar of the oracle, and within a few fp16
    ulps of each other (they add the k terms in different orders)."""
    M, N, K = 384, 640, 1024
    A, B = synth.random_operands(M, N, K, seed=123)
    dA, dB = to_dev(A), to_dev(B)
    out = {}
    for path in (gr.GR_PATH_TILE_STREAM, gr.GR_PATH_TILE):
        dC = full_dev((M * N,), SENTINEL)
        assert call(M, N, K, dA, K, dB, N, dC, N, path=path) == gr.GR_OK
        out[path] = from_dev(dC).reshape(M, N)
    ref = oracle.gemm_relu_full(A, B)
    for path, C in out.items():
        assert_parity(C, ref, "path %d" % path)
    c1 = out[gr.GR_PATH_TILE_STREAM].view(np.float16).astype(np.float64)
    c2 = out[gr.GR_PATH_TILE].view(np.float16).astype(np.float64)
    assert np.all(np.abs(c1 - c2) <= 1e-2 + 1e-2 * np.abs(c2))


@pytest.mark.parametrize("M,N,K,ldb", [(1088, 1856, 2048, 1856), (1024, 2048, 512, 2049), (700, 1100, 128, 1101),
                                     (2048, 2048, 256, 2049)])
def test_planned_tile_stream_matches_oracle(M, N, K, ldb):
    """The plain call where the planner picks the streaming path: 29 column
    blocks (XCD renumbering, 493 workgroups), B's rows misaligned over one
    full round (512 blocks, plain order), a short K with misaligned B and 18
    column blocks (XCD renumbering), and misaligned B over two rounds (1024
    blocks, no workspace); sampled oracle check, and every workgroup order
    gives the same bits."""
    import torch as t
    A, B = synth.random_operands(M, N, K, seed=M + K, ldb=ldb)
    st, p = gr.gemm_relu_f16_plan(M, N, K, 0x100000, K, 0x200000000000, ldb, 0x400000000000, N)
    assert st == gr.GR_OK and p["path"] == gr.GR_PATH_TILE_STREAM, p
    dA, dB = to_dev(A), to_dev(B)
    dC = full_dev((M * N,), SENTINEL)
    log("planned tile_stream %dx%dx%d ldb=%d order=%d/%d" % (M, N, K, ldb, p["group_m"], p["plain_order"]))
    assert call(M, N, K, dA, K, dB, ldb, dC, N) == gr.GR_OK
    C = from_dev(dC).reshape(M, N)
    ii, jj = synth.sample_indices(M, N, 4096, M)
    ref = oracle.gemm_relu_elems(A, B, ii, jj, M=M, N=N, K=K, lda=K, ldb=ldb)
    log("parity %s" % (assert_parity(C[ii, jj], ref, "planned tile_stream %dx%dx%d" % (M, N, K)),))
    for gm, remap in ((1, 0), (4, 1), (3, 1), (64, 0)):
        dC2 = full_dev((M * N,), SENTINEL)
        assert gr.gemm_relu_f16_forced_order(M, N, K, dA.data_ptr(), K, dB.data_ptr(), ldb, dC2.data_ptr(), N,
                                             t.cuda.current_stream().cuda_stream, gr.GR_PATH_TILE_STREAM, gm,
                                             remap) == gr.GR_OK
        t.cuda.synchronize()
        assert np.array_equal(C, from_dev(dC2).reshape(M, N)), (gm, remap)


BT_CASES = [
    # M, N, K, lda, ldbt, ldc, element offsets of A, Bt, C
    (17, 64, 32, 32, 32, 64, (0, 0, 0)),             # one row block of 17 rows, one slot
    (130, 65, 64, 64, 72, 70, (0, 8, 3)),            # last column block moved left, Bt padded
    (1000, 1000, 1024, 1032, 1024, 1005, (8, 0, 1)),  # ragged M and N, C misaligned
    (300, 300, 96, 104, 104, 300, (0, 16, 0)),        # 3 slots
    (64, 128, 4096, 4096, 4096, 128, (0, 0, 0)),      # one row block, long K
    (130, 65, 64, 65, 67, 70, (1, 1, 0)),             # rows of A and Bt 2-byte aligned only
    (300, 300, 96, 97, 99, 300, (3, 5, 0)),           # odd pitches and offsets
]


@pytest.mark.parametrize("M,N,K,lda,ldbt,ldc,offs", BT_CASES)
def test_tile_stream_transposed_b_parity(M, N, K, lda, ldbt, ldc, offs):
    """The streaming kernel with B given as N x K (16-row blocks of Bt copied
    and read like those of A): full oracle check on padded operands (Bt's
    padding poisoned with 65504), C's padding and rows past M untouched, and
    the same bits as the row-major layout on the same kernel (the same MFMA
    sequence on the same fragment values)."""
    import torch as t
    A, B = synth.random_operands(M, N, K, seed=7 * M + N + K, lda=lda)
    Bt = np.full((N, ldbt), 0x7BFF, np.uint16)
    Bt[:, :K] = B[:K, :N].T
    Ap = np.concatenate([np.zeros(offs[0], np.uint16), A.ravel()])
    Btp = np.concatenate([np.full(offs[1], 0x7BFF, np.uint16), Bt.ravel()])
    dC = full_dev((offs[2] + (M + 2) * ldc,), SENTINEL)
    dA, dBt = to_dev(Ap), to_dev(Btp)
    s = t.cuda.current_stream().cuda_stream
    log("tile_stream bt %dx%dx%d lda=%d ldbt=%d ldc=%d offs=%s" % (M, N, K, lda, ldbt, ldc, offs))
    st = gr.gemm_relu_f16_bt_forced(M, N, K, dA.data_ptr() + 2 * offs[0], lda, dBt.data_ptr() + 2 * offs[1], ldbt,
                                    dC.data_ptr() + 2 * offs[2], ldc, s, gr.GR_PATH_TILE_STREAM)
    t.cuda.synchronize()
    assert st == gr.GR_OK, gr.gemm_relu_status_string(st)
    Cflat = from_dev(dC)
    C = Cflat[offs[2]:offs[2] + M * ldc].reshape(M, ldc)
    assert np.all(Cflat[:offs[2]] == SENTINEL), "an element before C was written"
    assert np.all(C[:, N:] == SENTINEL), "a padding column of C was written"
    assert np.all(Cflat[offs[2] + M * ldc:] == SENTINEL), "a row past M was written"
    ref = oracle.gemm_relu_full(A, B, M=M, N=N, K=K, lda=lda, ldb=N)
    log("parity %s" % (assert_parity(C[:, :N], ref, "tile_stream bt %dx%dx%d" % (M, N, K)),))
    dC2 = full_dev((M * N,), SENTINEL)
    assert call(M, N, K, to_dev(A), lda, to_dev(np.ascontiguousarray(B[:K, :N])), N, dC2, N,
                path=gr.GR_PATH_TILE_STREAM) == gr.GR_OK
    assert np.array_equal(C[:, :N], from_dev(dC2).reshape(M, N)), "transposed and row-major B differ"


def test_all_ones_exact_on_tile_stream():
    """All-ones operands give exactly K in every element (every partial sum
    is an integer below 2^24, whatever the order of the waves' sums)."""
    for M, N, K in ((130, 200, 32), (300, 520, 1024), (64, 64, 2080)):
        A = np.full((M, K), 0x3C00, np.uint16)
        B = np.full((K, N), 0x3C00, np.uint16)
        dC = full_dev((M * N,), SENTINEL)
        assert call(M, N, K, to_dev(A), K, to_dev(B), N, dC, N, path=gr.GR_PATH_TILE_STREAM) == gr.GR_OK
        assert np.all(from_dev(dC) == np.float16(K).view(np.uint16)), (M, N, K)


@pytest.mark.parametrize("fmt,act", [("f16", "relu"), ("bf16", "relu"), ("f16", "gelu"), ("bf16", "silu"),
                                     ("f16", "none")])
def test_tile_stream_with_bias_and_activation(fmt, act):
    """The bias + activation epilogue and bfloat16 on the row-blocked
    streaming path, against the oracle's double-precision epilogue."""
    import torch as t
    M, N, K = 300, 1000, 512
    A, B = synth.random_operands(M, N, K, seed=97, b_scale=K ** -0.5, fmt=fmt)
    bias = synth.random_operands(1, N, 1, seed=98, fmt=fmt)[1].reshape(N)
    dA, dB, db = to_dev(A), to_dev(B), to_dev(bias)
    dC = full_dev(((M + 2) * N,), SENTINEL)
    s = t.cuda.current_stream().cuda_stream
    fn = gr.gemm_bias_act_f16_forced if fmt == "f16" else gr.gemm_bias_act_bf16_forced
    st = fn(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, db.data_ptr(), gr.ACT_CODES[act], dC.data_ptr(), N, s,
            gr.GR_PATH_TILE_STREAM)
    t.cuda.synchronize()
    assert st == gr.GR_OK
    Cflat = from_dev(dC)
    assert np.all(Cflat[M * N:] == SENTINEL), "a row past M was written"
    got = as_f64(Cflat[:M * N].reshape(M, N), fmt)
    ref = as_f64(oracle.gemm_relu_full(A, B, fmt=fmt, bias=bias, act=act), fmt)
    assert np.all(np.isfinite(got))
    err = np.abs(got - ref)
    assert np.all(err <= 1e-2 + 1e-2 * np.abs(ref)), (fmt, act, float(err.max()))


def test_bf16_plain_call_takes_tile_stream():
    """gemm_relu_bf16 on a 1024^3 problem plans the same path and matches the
    oracle's bfloat16 result on sampled elements."""
    import torch as t
    M = N = K = 1024
    A, B = synth.random_operands(M, N, K, seed=99, fmt="bf16")
    dA, dB = to_dev(A), to_dev(B)
    dC = full_dev((M * N,), SENTINEL)
    st = gr.gemm_relu_bf16(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, dC.data_ptr(), N,
                           t.cuda.current_stream().cuda_stream)
    t.cuda.synchronize()
    assert st == gr.GR_OK
    ii, jj = synth.sample_indices(M, N, 4096, 99)
    got = as_f64(from_dev(dC).reshape(M, N)[ii, jj], "bf16")
    ref = as_f64(oracle.gemm_relu_elems(A, B, ii, jj, fmt="bf16"), "bf16")
    err = np.abs(got - ref)
    assert np.all(err <= 1e-2 + 1e-2 * np.abs(ref)), float(err.max())


SMALL_M_ROWS_CASES = [
    # M, N, K, lda, ldb, ldc, offs: up to 64 rows planned onto one row of streaming blocks
    (8, 1024, 8192, 8192, 1024, 1024, (0, 0, 0)),    # K x N = 2^23: 16 blocks of 8 waves, 32 slots each
    (64, 1024, 1024, 1024, 1024, 1024, (0, 0, 0)),   # more than 32 rows
    (40, 1100, 512, 512, 1100, 1103, (0, 2, 1)),     # ragged N, B and C misaligned
    (5, 200, 96, 97, 200, 200, (1, 0, 0)),           # A's rows odd: the small-M kernels cannot take them
    (33, 2048, 1024, 1030, 2056, 2048, (3, 8, 0)),   # A's rows 4-byte aligned, padded B
]


@pytest.mark.parametrize("M,N,K,lda,ldb,ldc,offs", SMALL_M_ROWS_CASES)
def test_planned_small_m_rows_on_tile_stream(M, N, K, lda, ldb, ldc, offs):
    """The plain call plans the streaming kernel for these few-row shapes
    (rows past M read row M - 1 and are never stored): full oracle check,
    canaries around C."""
    base = (0x100000 + 2 * offs[0], 0x200000000000 + 2 * offs[1], 0x400000000000 + 2 * offs[2])
    st, p = gr.gemm_relu_f16_plan(M, N, K, base[0], lda, base[1], ldb, base[2], ldc)
    assert st == gr.GR_OK and p["path"] == gr.GR_PATH_TILE_STREAM, p
    A, B, C = _run(M, N, K, lda, ldb, ldc, offs, None, seed=M * 13 + N + K)
    ref = oracle.gemm_relu_full(A, B, M=M, N=N, K=K, lda=lda, ldb=ldb)
    log("parity %s" % (assert_parity(C, ref, "planned few-row tile_stream %dx%dx%d" % (M, N, K)),))


def test_bf16_plain_call_few_rows_takes_tile_stream():
    """gemm_relu_bf16 with 24 rows and few columns (K x N = 2^23) plans one row
    of streaming blocks, as for fp16, and matches the oracle's bfloat16
    result on sampled elements; rows past M stay untouched."""
    import torch as t
    M, N, K = 24, 2048, 4096
    st, p = gr.gemm_relu_f16_plan(M, N, K, 0x100000, K, 0x200000000000, N, 0x400000000000, N)
    assert st == gr.GR_OK and p["path"] == gr.GR_PATH_TILE_STREAM, p
    A, B = synth.random_operands(M, N, K, seed=24, fmt="bf16")
    dA, dB = to_dev(A), to_dev(B)
    dC = full_dev(((M + 1) * N,), SENTINEL)
    log("bf16 few-row tile_stream %dx%dx%d" % (M, N, K))
    st = gr.gemm_relu_bf16(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, dC.data_ptr(), N,
                           t.cuda.current_stream().cuda_stream)
    t.cuda.synchronize()
    assert st == gr.GR_OK
    Cf = from_dev(dC)
    assert np.all(Cf[M * N:] == SENTINEL), "a row past M was written"
    ii, jj = synth.sample_indices(M, N, 4096, 24)
    got = as_f64(Cf[:M * N].reshape(M, N)[ii, jj], "bf16")
    ref = as_f64(oracle.gemm_relu_elems(A, B, ii, jj, fmt="bf16"), "bf16")
    err = np.abs(got - ref)
    assert np.all(err <= 1e-2 + 1e-2 * np.abs(ref)), float(err.max())
