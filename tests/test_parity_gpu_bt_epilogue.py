"""GPU parity of gemm_bias_act_bt -- C = act(A Bt^T + bias) with B given
transposed (N x K, a linear layer's weight), fp16 and bfloat16 -- against the
oracle (which takes B = Bt^T), on every kernel family of the transposed-B
planner: the small-M stream straight from memory and through LDS, the
pipelined 256 x 256 kernels (64- and 32-deep A strips), the 128 x 128 kernel
and the guarded kernel.  Same bar as every other path (|gpu - oracle| <=
1e-2 + 1e-2 |oracle|, "Writing high-performance kernels in TileLang",
section "Writing a GEMM"); ReLU without a bias in fp16 equals
gemm_relu_f16_bt bit for bit.
"""
import numpy as np
import pytest

import dense_gemm_epilogue_tiled_amd as gr
import oracle
import synth
from gpu_util import assert_parity, from_dev, full_dev, log, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("oracle_lib")]

SENTINEL = 0x7FC1
FMTS = {"f16": gr.GR_FMT_F16, "bf16": gr.GR_FMT_BF16}

CASES = [
    # M, N, K, lda, ldbt, ldc, expected (path, block_m), what
    (8, 4096, 1024, 1024, 1024, 4096, (gr.GR_PATH_SMALL_M, None), "small-M through LDS (K % 256 = 0)"),
    (13, 1000, 1000, 1000, 1000, 1001, (gr.GR_PATH_SMALL_M, None), "small-M from memory, partial"),
    (2600, 3000, 128, 128, 136, 3001, (gr.GR_PATH_TILE, 256), "256 tiles, 64-deep A strips, partial"),
    (4096, 3072, 96, 96, 96, 3072, (gr.GR_PATH_TILE, 256), "256 tiles, 32-deep strips"),
    (300, 270, 224, 232, 224, 273, (gr.GR_PATH_TILE, 128), "128 tiles, partial"),
    (300, 270, 100, 101, 103, 273, (gr.GR_PATH_TILE_EDGE, None), "guarded, odd pitches"),
    (300, 1000, 1024, 1032, 1032, 1001, (gr.GR_PATH_TILE_STREAM, 64), "row-blocked streaming, Bt copied like A"),
]


def plan(M, N, K, lda, ldbt, ldc):
    st, p = gr.gemm_relu_f16_bt_plan(M, N, K, 0x100000, lda, 0x200000000000, ldbt, 0x400000000000, ldc)
    assert st == gr.GR_OK
    return p


def operands(M, N, K, seed, lda, ldbt, fmt):
    """A (M x lda) and Bt (N x ldbt), N(0,1) with Bt scaled by 2/sqrt(K), plus
    a bias and B = Bt^T for the oracle."""
    A, B = synth.random_operands(M, N, K, seed=seed, lda=lda, b_scale=2.0 * max(K, 1) ** -0.5, fmt=fmt)
    Bt = np.full((N, ldbt), B.flat[0] if B.size else 0, dtype=np.uint16)
    Bt[:, :K] = B[:K, :N].T
    if ldbt > K:
        Bt[:, K:] = 0x7BFF if fmt == "f16" else 0x7F7F  # large finite padding
    _, b2 = synth.random_operands(1, N, 1, seed=seed + 1, fmt=fmt)
    return A, np.ascontiguousarray(Bt), np.ascontiguousarray(B[:K, :N]), np.ascontiguousarray(b2[0])


def run(A, Bt, bias, M, N, K, lda, ldbt, ldc, act, fmt, path=-1):
    import torch as t
    dA, dB = to_dev(A), to_dev(Bt)
    db = to_dev(bias) if bias is not None else None
    dC = full_dev((M * ldc + 8,), SENTINEL)
    log("bt-epi %s %s M=%d N=%d K=%d lda=%d ldbt=%d ldc=%d bias=%s path=%s" %
        (fmt, act, M, N, K, lda, ldbt, ldc, bias is not None, path))
    st = gr.gemm_bias_act_bt(M, N, K, dA.data_ptr(), lda, dB.data_ptr(), ldbt,
                             db.data_ptr() if db is not None else None, gr.ACT_CODES[act], dC.data_ptr(), ldc,
                             FMTS[fmt], t.cuda.current_stream().cuda_stream, path)
    t.cuda.synchronize()
    assert st == gr.GR_OK, gr.gemm_relu_status_string(st)
    return from_dev(dC)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("act", ["gelu", "silu", "relu"])
@pytest.mark.parametrize("case", CASES, ids=[c[-1] for c in CASES])
def test_bt_epilogue_parity(case, act, fmt):
    M, N, K, lda, ldbt, ldc, expect, what = case
    p = plan(M, N, K, lda, ldbt, ldc)
    assert p["path"] == expect[0] and (expect[1] is None or p["block_m"] == expect[1]), p
    A, Bt, B, bias = operands(M, N, K, M + N + K, lda, ldbt, fmt)
    Cflat = run(A, Bt, bias, M, N, K, lda, ldbt, ldc, act, fmt)
    C = Cflat[:M * ldc].reshape(M, ldc)
    ref = oracle.gemm_relu_full(A, B, M=M, N=N, K=K, lda=lda, ldb=N, fmt=fmt, bias=bias, act=act)
    assert_parity(C[:, :N], ref, "bt-epi %s %s %s" % (what, act, fmt), fmt=fmt)
    assert np.all(C[:, N:] == SENTINEL) and np.all(Cflat[M * ldc:] == SENTINEL)


@pytest.mark.parametrize("act", list(gr.ACT_CODES))
def test_bt_every_activation(act):
    M, N, K = 300, 270, 256
    A, Bt, B, bias = operands(M, N, K, 7, K, K, "bf16")
    C = run(A, Bt, bias, M, N, K, K, K, N, act, "bf16")[:M * N].reshape(M, N)
    assert_parity(C, oracle.gemm_relu_full(A, B, fmt="bf16", bias=bias, act=act), "bt %s" % act, fmt="bf16")


@pytest.mark.parametrize("case", CASES, ids=[c[-1] for c in CASES])
def test_relu_without_bias_is_the_fused_bt_call_bitwise(case):
    import torch as t
    M, N, K, lda, ldbt, ldc = case[:6]
    A, Bt, _, _ = operands(M, N, K, 3, lda, ldbt, "f16")
    C1 = run(A, Bt, None, M, N, K, lda, ldbt, ldc, "relu", "f16")
    dA, dB = to_dev(A), to_dev(Bt)
    dC = full_dev((M * ldc + 8,), SENTINEL)
    st = gr.gemm_relu_f16_bt(M, N, K, dA.data_ptr(), lda, dB.data_ptr(), ldbt, dC.data_ptr(), ldc,
                             t.cuda.current_stream().cuda_stream)
    t.cuda.synchronize()
    assert st == gr.GR_OK
    assert np.array_equal(C1, from_dev(dC))


def test_linear_wrapper():
    t = pytest.importorskip("torch")
    M, N, K = 40, 300, 512
    A, Bt, B, bias = operands(M, N, K, 11, K, K, "bf16")
    x = to_dev(A).view(t.bfloat16).reshape(M, K)
    w = to_dev(Bt).view(t.bfloat16).reshape(N, K)
    b = to_dev(bias).view(t.bfloat16)
    y = gr.linear(x, w, b, "gelu_tanh")
    t.cuda.synchronize()
    ref = oracle.gemm_relu_full(A, B, fmt="bf16", bias=bias, act="gelu_tanh")
    assert_parity(y.view(t.int16).cpu().numpy().view(np.uint16), ref, "linear", fmt="bf16")
