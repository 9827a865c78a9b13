"""GPU parity of the pipelined 256 x 256 kernel on misaligned rows and ragged K
(GR_PATH_TILE_UNALIGNED) against the CPU oracle.

The path copies operand rows into LDS from any 2-byte aligned address,
multiplies the last (K - 1) % 64 + 1 steps of k first, from a strip copied
from k = K - 64 whose elements before the tail are zeroed in both operands (the
pages' rule that out-of-range elements of both operands read as zero,
TileLang tutorial, chapter "动态形状与变长序列"), and moves the last tile row
and column to end at M and N.  Bar as everywhere: |gpu - oracle| <= 1e-2 +
1e-2 |oracle| per element, no NaN or Inf, padding of C and rows past M never
written.
"""
import numpy as np
import pytest

import dense_gemm_epilogue_tiled_amd as gr
import oracle
import synth
from gpu_util import assert_parity, call, from_dev, full_dev, log, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("oracle_lib")]

SENTINEL = 0x7E5A

# M, N, K, lda, ldb, ldc, element offsets of A, B, C.  K covers every tail
# class: 1 (K % 64 == 1), 2, 31, 32, 33, 63, 64 (K % 64 == 0: a whole 64-deep
# tail), with 2..4 pipeline strips after it.
CASES = [
    (256, 256, 129, 129, 256, 256, (0, 0, 0)),      # one tile, tail 1
    (300, 270, 130, 131, 271, 270, (1, 0, 0)),      # ragged M and N, tail 2, odd pitches
    (513, 300, 223, 223, 301, 303, (0, 1, 3)),      # tail 31
    (384, 768, 224, 230, 770, 768, (3, 5, 7)),      # tail 32
    (511, 257, 161, 163, 257, 260, (0, 0, 1)),      # tail 33
    (260, 520, 319, 320, 522, 520, (5, 3, 0)),      # tail 63
    (520, 260, 192, 192, 262, 261, (0, 7, 0)),      # tail 64 (K % 64 == 0, rows misaligned)
    (1024, 1024, 4100, 4100, 1024, 1024, (0, 0, 0)),  # aligned rows, K % 64 == 4, long K
    # 16-byte rows of C (16-byte stores) while the last tile column, moved
    # left to end at N, starts at an odd column (267, 515): its stores are
    # 2-byte aligned and must still leave columns N.. of C alone
    (300, 523, 130, 130, 528, 528, (0, 0, 0)),      # tail 2
    (513, 771, 200, 200, 776, 776, (0, 0, 8)),      # tail 8, C offset by 16 bytes
]


@pytest.mark.parametrize("M,N,K,lda,ldb,ldc,offs", CASES)
def test_unaligned_path_parity(M, N, K, lda, ldb, ldc, offs):
    """Forced unaligned path on misaligned, padded operands: full oracle check,
    padding poisoned with 65504 (the largest finite fp16) so that a read of
    it would show, C's padding, the rows after C and the elements before C's
    start keep the sentinel."""
    A, B = synth.random_operands(M, N, K, seed=3 * M + 5 * N + K, lda=lda, ldb=ldb)
    Ap = np.concatenate([np.full(offs[0], 0x7BFF, np.uint16), A.ravel()])
    Bp = np.concatenate([np.full(offs[1], 0x7BFF, np.uint16), B.ravel()])
    extra = 2
    dC = full_dev((offs[2] + (M + extra) * ldc,), SENTINEL)
    log("unaligned %dx%dx%d lda=%d ldb=%d ldc=%d offsets=%s" % (M, N, K, lda, ldb, ldc, offs))
    st = call(M, N, K, to_dev(Ap), lda, to_dev(Bp), ldb, dC, ldc, path=gr.GR_PATH_TILE_UNALIGNED, offsets=offs)
    assert st == gr.GR_OK, gr.gemm_relu_status_string(st)
    Cflat = from_dev(dC)
    C = Cflat[offs[2]:offs[2] + M * ldc].reshape(M, ldc)
    ref = oracle.gemm_relu_full(A, B, M=M, N=N, K=K, lda=lda, ldb=ldb)
    rep = assert_parity(C[:, :N], ref, "unaligned %dx%dx%d" % (M, N, K))
    log("parity %s" % (rep,))
    assert np.all(Cflat[:offs[2]] == SENTINEL), "an element before C was written"
    assert np.all(C[:, N:] == SENTINEL), "a padding column of C was written"
    assert np.all(Cflat[offs[2] + M * ldc:] == SENTINEL), "a row past M was written"


def test_unaligned_path_matches_guarded_kernel_closely():
    """The same problem through the unaligned pipelined kernel and the guarded
    kernel: both within the bar of the oracle, and within a few fp16 ulps of
    each other (they add the k terms in different orders)."""
    M, N, K = 768, 1280, 1000
    A, B = synth.random_operands(M, N, K, seed=77)
    dA, dB = to_dev(A), to_dev(B)
    dC1 = full_dev((M * N,), SENTINEL)
    dC2 = full_dev((M * N,), SENTINEL)
    assert call(M, N, K, dA, K, dB, N, dC1, N, path=gr.GR_PATH_TILE_UNALIGNED) == gr.GR_OK
    assert call(M, N, K, dA, K, dB, N, dC2, N, path=gr.GR_PATH_TILE_EDGE) == gr.GR_OK
    c1 = from_dev(dC1).view(np.float16).astype(np.float64)
    c2 = from_dev(dC2).view(np.float16).astype(np.float64)
    assert np.all(np.abs(c1 - c2) <= 1e-2 + 1e-2 * np.abs(c2))
    ii, jj = synth.sample_indices(M, N, 4096, 77)
    assert_parity(from_dev(dC1).reshape(M, N)[ii, jj], oracle.gemm_relu_elems(A, B, ii, jj), "unaligned sample")


def test_all_ones_exact_on_the_unaligned_path():
    """All-ones operands give exactly K in every element, whatever the tail
    (every partial sum is an integer below 2^24)."""
    for K in (129, 160, 191, 192, 2050):
        M, N = 300, 520
        A = np.full((M, K), 0x3C00, np.uint16)
        B = np.full((K, N + 1), 0x3C00, np.uint16)
        dC = full_dev((M * N,), SENTINEL)
        st = call(M, N, K, to_dev(A), K, to_dev(B), N + 1, dC, N, path=gr.GR_PATH_TILE_UNALIGNED)
        assert st == gr.GR_OK
        expect = np.float16(K).view(np.uint16)
        assert np.all(from_dev(dC) == expect), K


def test_ragged_workload_runs_in_place_with_or_without_workspace():
    """The ragged workload (4099 x 3071 x 2050, pitches 4100 B and 6142 B)
    takes the unaligned path whether or not a workspace is offered, so the two
    calls agree bit for bit; sampled oracle check plus every row and column of
    the partial last tiles."""
    import torch as t
    w = synth.WORKLOADS["ragged4099x3071x2050"]
    M, N, K = w.M, w.N, w.K
    st, p = gr.gemm_relu_f16_plan(M, N, K, 0x100000, K, 0x200000000000, N, 0x400000000000, N)
    assert st == gr.GR_OK and p["path"] == gr.GR_PATH_TILE_UNALIGNED
    A, B = synth.operands(w)
    dA, dB = to_dev(A), to_dev(B)
    dC1 = full_dev((M * N,), SENTINEL)
    dC2 = full_dev((M * N,), SENTINEL)
    assert call(M, N, K, dA, K, dB, N, dC1, N) == gr.GR_OK
    ws = t.empty(1 << 20, dtype=t.uint8, device="cuda")
    st = gr.gemm_relu_f16_ws(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, dC2.data_ptr(), N, ws.data_ptr(),
                             1 << 20, t.cuda.current_stream().cuda_stream)
    t.cuda.synchronize()
    assert st == gr.GR_OK
    C = from_dev(dC1).reshape(M, N)
    assert np.array_equal(C, from_dev(dC2).reshape(M, N))
    ii, jj = synth.sample_indices(M, N, 4096, w.seed)
    assert_parity(C[ii, jj], oracle.gemm_relu_elems(A, B, ii, jj), "ragged sampled")
    # the last tile row starts at 3843 and owns rows 4096.., the last tile
    # column starts at 2815 and owns columns 2816..
    rows = [0, 255, 256, 3839, 3840, 3843, 4095, 4096, 4098]
    cols = [0, 255, 256, 2559, 2560, 2815, 2816, 3070]
    assert_parity(C[rows, :], oracle.gemm_relu_rows(A, B, rows), "ragged rows")
    assert_parity(C[:, cols].T, oracle.gemm_relu_cols(A, B, cols), "ragged cols")


@pytest.mark.parametrize("M,N,K,lda,ldb,offs", [
    (512, 512, 500, 500, 512, (1, 0, 0)),     # A's base pointer misaligned, ragged K
    (300, 300, 300, 300, 300, (0, 0, 0)),     # 600-byte rows: 8-byte aligned only
    (1000, 700, 1000, 1001, 700, (0, 0, 0)),  # ragged K, odd pitch of A
    (256, 2000, 130, 130, 2003, (0, 3, 0)),   # one tile row, tail 2, B misaligned
])
def test_plain_call_takes_the_unaligned_kernel_on_misaligned_mid_size_problems(M, N, K, lda, ldb, offs):
    """Without a workspace, a ragged K (which the streaming kernel cannot
    take) with M, N >= 256 and K > 128 runs on the unaligned kernel in place,
    whatever the rows' alignment (the guarded kernel was 2-5x slower there):
    full oracle check."""
    A, B = synth.random_operands(M, N, K, seed=M + 2 * N + K, lda=lda, ldb=ldb)
    Ap = np.concatenate([np.full(offs[0], 0x7BFF, np.uint16), A.ravel()])
    Bp = np.concatenate([np.full(offs[1], 0x7BFF, np.uint16), B.ravel()])
    st, p = gr.gemm_relu_f16_plan(M, N, K, 0x100000 + 2 * offs[0], lda, 0x200000000000 + 2 * offs[1], ldb,
                                  0x400000000000, N)
    assert st == gr.GR_OK and p["path"] == gr.GR_PATH_TILE_UNALIGNED, p
    dC = full_dev(((M + 2) * N,), SENTINEL)
    log("planned unaligned %dx%dx%d lda=%d ldb=%d offsets=%s" % (M, N, K, lda, ldb, offs))
    assert call(M, N, K, to_dev(Ap), lda, to_dev(Bp), ldb, dC, N, offsets=offs) == gr.GR_OK
    Cflat = from_dev(dC)
    assert np.all(Cflat[M * N:] == SENTINEL), "a row past M was written"
    assert_parity(Cflat[:M * N].reshape(M, N), oracle.gemm_relu_full(A, B, M=M, N=N, K=K, lda=lda, ldb=ldb),
                  "planned unaligned %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("r", range(1, 8))
@pytest.mark.parametrize("path", [gr.GR_PATH_TILE_UNALIGNED, gr.GR_PATH_TILE])
def test_partial_row_segments_of_every_length(r, path):
    """N = 512 + r: the last 8-column segment of each row of C holds r columns
    (and, on the unaligned path, the last tile column moved left to end at N
    starts r columns into a segment, so its first segment holds 8 - r of
    them).  Each partial segment is written with at most two overlapping
    stores; the full result must match the oracle and C's padding columns
    must keep the sentinel."""
    M, N = 300, 512 + r
    K, lda = (130, 130) if path == gr.GR_PATH_TILE_UNALIGNED else (128, 128)
    ldb = ldc = N + (-N) % 8  # 16-byte rows of B and C
    A, B = synth.random_operands(M, N, K, seed=17 * r + K, lda=lda, ldb=ldb)
    dC = full_dev(((M + 1) * ldc,), SENTINEL)
    log("partial segments %dx%dx%d path=%d" % (M, N, K, path))
    st = call(M, N, K, to_dev(A), lda, to_dev(B), ldb, dC, ldc, path=path)
    assert st == gr.GR_OK, gr.gemm_relu_status_string(st)
    Cflat = from_dev(dC)
    C = Cflat[:M * ldc].reshape(M, ldc)
    assert_parity(C[:, :N], oracle.gemm_relu_full(A, B, M=M, N=N, K=K, lda=lda, ldb=ldb), "segments r=%d" % r)
    assert np.all(C[:, N:] == SENTINEL), "a padding column of C was written"
    assert np.all(Cflat[M * ldc:] == SENTINEL), "a row past M was written"
