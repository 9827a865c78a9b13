"""GPU parity of the streaming small-M kernel (B copied straight into LDS, any
alignment of B) against the CPU oracle: single pass (GR_PATH_SMALL_M) and the
split-K first pass plus ordered sum (GR_PATH_SMALL_M_SPLIT).

The path is the GEMV-like pattern of "Tilelang Cuda Patterns", section 4
(stream the large operand once, fp32 accumulation, one cast at the end) with
the split-K of "TileLang programming basics", section 5.1, made deterministic
and with ReLU after the complete sum.  Bar: |gpu - oracle| <= 1e-2 + 1e-2
|oracle| per element, no NaN or Inf, C's padding and rows past M untouched.
"""
import numpy as np
import pytest

import dense_gemm_epilogue_tiled_amd as gr
import oracle
import synth
from gpu_util import as_f64, assert_parity, call, call_ws, from_dev, full_dev, log, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("oracle_lib")]

SENTINEL = 0x7E5A
WS_POISON = 0x7E5A

# M, N, K, lda, ldb, ldc, element offsets of A, B, C (A's rows stay 16-byte
# aligned: offsets of A are multiples of 8)
CASES = [
    (8, 16384, 8192, 8192, 16384, 16384, (0, 0, 0)),  # the small-M workload's shape
    (1, 64, 32, 32, 64, 64, (0, 0, 0)),               # one row, one block, one slot
    (3, 1000, 1024, 1024, 1003, 1001, (0, 1, 1)),     # ragged N (last block moved left), B odd pitch
    (16, 777, 4096, 4104, 777, 780, (8, 3, 5)),       # 16 rows, B and C misaligned
    (5, 130, 96, 96, 131, 130, (0, 7, 0)),            # N just above one block, three slots
    (8, 4096, 8192, 8192, 4100, 4096, (0, 2, 0)),     # B rows 8-byte aligned only
]


def _run(M, N, K, lda, ldb, ldc, offs, path, ws_bytes=0):
    import torch as t
    A, B = synth.random_operands(M, N, K, seed=M * 977 + N + K, lda=lda, ldb=ldb, b_scale=K ** -0.5)
    Ap = np.concatenate([np.zeros(offs[0], np.uint16), A.ravel()])
    Bp = np.concatenate([np.full(offs[1], 0x7BFF, np.uint16), B.ravel()])
    extra = 2
    dC = full_dev((offs[2] + (M + extra) * ldc,), SENTINEL)
    log("stream %dx%dx%d lda=%d ldb=%d ldc=%d offs=%s path=%d ws=%d" % (M, N, K, lda, ldb, ldc, offs, path,
                                                                     ws_bytes))
    if ws_bytes:
        ws = full_dev(((ws_bytes + 4096) // 2,), WS_POISON).view(t.uint8)
        st = call_ws(M, N, K, to_dev(Ap), lda, to_dev(Bp), ldb, dC, ldc, ws, ws_bytes, path=path, offsets=offs)
        w = ws.view(t.int16).cpu().numpy().view(np.uint16)
        assert np.all(w[ws_bytes // 2:] == WS_POISON), "workspace written past the size asked for"
    else:
        st = call(M, N, K, to_dev(Ap), lda, to_dev(Bp), ldb, dC, ldc, path=path, offsets=offs)
    assert st == gr.GR_OK, gr.gemm_relu_status_string(st)
    Cflat = from_dev(dC)
    C = Cflat[offs[2]:offs[2] + M * ldc].reshape(M, ldc)
    assert np.all(Cflat[:offs[2]] == SENTINEL), "an element before C was written"
    assert np.all(C[:, N:] == SENTINEL), "a padding column of C was written"
    assert np.all(Cflat[offs[2] + M * ldc:] == SENTINEL), "a row past M was written"
    return A, B, C[:, :N]


@pytest.mark.parametrize("M,N,K,lda,ldb,ldc,offs", CASES)
def test_stream_single_pass_parity(M, N, K, lda, ldb, ldc, offs):
    st, p = gr.gemm_relu_f16_plan(M, N, K, 0x100000 + 2 * offs[0], lda, 0x200000000000 + 2 * offs[1], ldb,
                                  0x400000000000 + 2 * offs[2], ldc)
    # planned: the streaming small-M kernel, or (few column blocks, K x N
    # large) one row of row-blocked streaming blocks; forced here: the former
    assert p["path"] == gr.GR_PATH_TILE_STREAM or (p["path"] == gr.GR_PATH_SMALL_M and p["vec_b"] == 8 and
                                                   p["block_n"] == 64), p
    A, B, C = _run(M, N, K, lda, ldb, ldc, offs, gr.GR_PATH_SMALL_M)
    assert_parity(C, oracle.gemm_relu_full(A, B, M=M, N=N, K=K, lda=lda, ldb=ldb), "stream %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K,lda,ldb,ldc,offs", [c for c in CASES if c[1] >= 128])
def test_stream_split_parity(M, N, K, lda, ldb, ldc, offs):
    """Forced split (the planner's split count, or one split where it would
    not split); a dirty workspace gives the same bits on a second call."""
    args = (M, N, K, 0x100000 + 2 * offs[0], lda, 0x200000000000 + 2 * offs[1], ldb,
            0x400000000000 + 2 * offs[2], ldc)
    st, size = gr.gemm_relu_f16_workspace_size(*args)
    if size == 0:
        size = 4 * M * N + 256
    st, p = gr.gemm_relu_f16_plan_ws(*args, size)
    log("split plan %s" % (p,))
    A, B, C = _run(M, N, K, lda, ldb, ldc, offs, gr.GR_PATH_SMALL_M_SPLIT, size)
    ref = oracle.gemm_relu_full(A, B, M=M, N=N, K=K, lda=lda, ldb=ldb)
    assert_parity(C, ref, "stream split %dx%dx%d" % (M, N, K))
    _, _, C2 = _run(M, N, K, lda, ldb, ldc, offs, gr.GR_PATH_SMALL_M_SPLIT, size)
    assert np.array_equal(C, C2)


def test_small_m_workload_with_workspace():
    """The small-M workload as the benchmark runs it with a workspace: two
    splits of 128-column blocks, full oracle check, and within the bar of the
    single pass."""
    import torch as t
    w = synth.WORKLOADS["smallm8x16384x8192"]
    M, N, K = w.M, w.N, w.K
    st, size = gr.gemm_relu_f16_workspace_size(M, N, K, 0x100000, K, 0x200000000000, N, 0x400000000000, N)
    st, p = gr.gemm_relu_f16_plan_ws(M, N, K, 0x100000, K, 0x200000000000, N, 0x400000000000, N, size)
    assert p["path"] == gr.GR_PATH_SMALL_M_SPLIT and p["split_k"] == 2 and p["grid"] == 256
    A, B = synth.operands(w)
    dA, dB = to_dev(A), to_dev(B)
    ws = t.empty(size, dtype=t.uint8, device="cuda")
    dC = full_dev((M * N,), SENTINEL)
    assert call_ws(M, N, K, dA, K, dB, N, dC, N, ws, size) == gr.GR_OK
    C = from_dev(dC).reshape(M, N)
    ref = oracle.gemm_relu_full(A, B)
    assert_parity(C, ref, "small-M workload, split")
    dC2 = full_dev((M * N,), SENTINEL)
    assert call(M, N, K, dA, K, dB, N, dC2, N) == gr.GR_OK
    assert_parity(C, from_dev(dC2).reshape(M, N), "split vs single pass")


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("act", ["relu", "gelu", "silu", "none"])
def test_stream_kernel_with_bias_and_activation(fmt, act):
    """The bias + activation epilogue and bfloat16 on the streaming kernel
    (single pass), against the oracle's double-precision epilogue."""
    import torch as t
    M, N, K = 8, 1088, 2048
    A, B = synth.random_operands(M, N, K, seed=91, b_scale=K ** -0.5, fmt=fmt)
    bias = synth.random_operands(1, N, 1, seed=92, fmt=fmt)[1].reshape(N)
    dA, dB, db = to_dev(A), to_dev(B), to_dev(bias)
    dC = full_dev((M * N,), SENTINEL)
    s = t.cuda.current_stream().cuda_stream
    fn = gr.gemm_bias_act_f16_forced if fmt == "f16" else gr.gemm_bias_act_bf16_forced
    st = fn(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, db.data_ptr(), gr.ACT_CODES[act], dC.data_ptr(), N, s,
            gr.GR_PATH_SMALL_M)
    t.cuda.synchronize()
    assert st == gr.GR_OK
    got = as_f64(from_dev(dC).reshape(M, N), fmt)
    ref = as_f64(oracle.gemm_relu_full(A, B, fmt=fmt, bias=bias, act=act), fmt)
    assert np.all(np.isfinite(got))
    err = np.abs(got - ref)
    assert np.all(err <= 1e-2 + 1e-2 * np.abs(ref)), (fmt, act, float(err.max()))


@pytest.mark.parametrize("M", [24, 64])
@pytest.mark.parametrize("fmt,act", [("f16", "gelu"), ("bf16", "silu"), ("bf16", "relu")])
def test_stream_kernel_row_blocks_with_bias_and_activation(M, fmt, act):
    """The streaming kernel with 2 and 4 blocks of 16 rows of A (M = 24, 64)
    under the bias + activation epilogue and bfloat16, against the oracle's
    double-precision epilogue; rows past M of the last block are never
    stored."""
    import torch as t
    N, K = 1088, 2048
    A, B = synth.random_operands(M, N, K, seed=M + 93, b_scale=K ** -0.5, fmt=fmt)
    bias = synth.random_operands(1, N, 1, seed=94, fmt=fmt)[1].reshape(N)
    dA, dB, db = to_dev(A), to_dev(B), to_dev(bias)
    dC = full_dev(((M + 2) * N,), SENTINEL)
    s = t.cuda.current_stream().cuda_stream
    fn = gr.gemm_bias_act_f16_forced if fmt == "f16" else gr.gemm_bias_act_bf16_forced
    st = fn(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, db.data_ptr(), gr.ACT_CODES[act], dC.data_ptr(), N, s,
            gr.GR_PATH_SMALL_M)
    t.cuda.synchronize()
    assert st == gr.GR_OK
    Cf = from_dev(dC)
    assert np.all(Cf[M * N:] == SENTINEL), "a row past M was written"
    got = as_f64(Cf[:M * N].reshape(M, N), fmt)
    ref = as_f64(oracle.gemm_relu_full(A, B, fmt=fmt, bias=bias, act=act), fmt)
    assert np.all(np.isfinite(got))
    err = np.abs(got - ref)
    assert np.all(err <= 1e-2 + 1e-2 * np.abs(ref)), (M, fmt, act, float(err.max()))
