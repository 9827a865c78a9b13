"""GPU parity of gemm_mxfp8_bt (OCP MX fp8: E4M3 operands, one E8M0 scale per
32 consecutive k of each row, B given transposed) with the CPU oracle.

Same bar as every other path (|gpu - oracle| <= 1e-2 + 1e-2 |oracle|,
"Writing high-performance kernels in TileLang", section "Writing a GEMM"),
plus bit-for-bit agreement of the pipelined and guarded kernels, which feed
the matrix cores the same operands and scales in the same order.  Inputs are
N(0,1) values times 2^u (u from -2..2, drawn per 32-k block) quantised the
OCP MX way (shared exponent floor(log2 max|x|) - 8 per block, elements
rounded to E4M3), so the scales change from block to block while the
dequantised operands stay as well conditioned as the per-tensor fp8 inputs;
the padding of every operand and scale array holds 448 or the NaN scale
code, so a read outside the matrices shows in the result.
"""
import numpy as np
import pytest

import dense_gemm_epilogue_tiled_amd as gr
import oracle
import synth
from gpu_util import assert_parity, from_dev, full_dev, log

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("oracle_lib")]

SENTINEL = 0x7FC1  # NaN in fp16 and bfloat16
FMTS = {"f16": gr.GR_FMT_F16, "bf16": gr.GR_FMT_BF16}


def dev8(x, offset=0):
    import torch as t
    flat = np.concatenate([np.zeros(offset, np.uint8), np.ascontiguousarray(x).ravel(), np.zeros(16, np.uint8)])
    return t.from_numpy(flat).to("cuda")


def dev16(x):
    import torch as t
    return t.from_numpy(np.ascontiguousarray(x).view(np.int16)).to("cuda")


def bias_for(N, fmt, seed):
    import torch as t
    g = t.Generator().manual_seed(seed)
    x = t.randn(N, generator=g)
    return x.to(t.bfloat16 if fmt == "bf16" else t.float16).view(t.int16).numpy().view(np.uint16)


def run(A, SA, Bt, SB, M, N, K, lda, ldsa, ldbt, ldsb, ldc, bias=None, act="relu", fmt="f16", path=None,
        s_offsets=(0, 0)):
    import torch as t
    dA, dB = dev8(A), dev8(Bt)
    dSA, dSB = dev8(SA, s_offsets[0]), dev8(SB, s_offsets[1])
    db = dev16(bias) if bias is not None else None
    dC = full_dev(((M + 1) * ldc + 8,), SENTINEL)
    log("mxfp8 M=%d N=%d K=%d lda=%d ldsa=%d ldbt=%d ldsb=%d ldc=%d act=%s fmt=%s path=%s soff=%s" %
        (M, N, K, lda, ldsa, ldbt, ldsb, ldc, act, fmt, path, s_offsets))
    args = (M, N, K, dA.data_ptr(), lda, dSA.data_ptr() + s_offsets[0], ldsa, dB.data_ptr(), ldbt,
            dSB.data_ptr() + s_offsets[1], ldsb, db.data_ptr() if db is not None else None, gr.ACT_CODES[act],
            dC.data_ptr(), ldc, FMTS[fmt], t.cuda.current_stream().cuda_stream)
    st = gr.gemm_mxfp8_bt(*args) if path is None else gr.gemm_mxfp8_bt_forced(*args, path)
    t.cuda.synchronize()
    assert st == gr.GR_OK, gr.gemm_relu_status_string(st)
    return from_dev(dC)


def plan(M, N, K, lda, ldsa, ldbt, ldsb, ldc, s_off=0):
    st, p = gr.gemm_mxfp8_bt_plan(M, N, K, 0x100000, lda, 0x300000 + s_off, ldsa, 0x200000000000, ldbt, 0x300000,
                                  ldsb, None, 1, 0x400000000000, ldc)
    assert st == gr.GR_OK
    return p


CASES = [
    # M, N, K, lda, ldsa, ldbt, ldsb, ldc, expected (path, tile), what
    (512, 512, 256, 256, 8, 256, 8, 512, (gr.GR_PATH_TILE, 128), "128 tiles, whole"),
    (300, 270, 384, 400, 12, 384, 16, 273, (gr.GR_PATH_TILE, 128), "128 tiles, partial, padded"),
    (17, 600, 128, 128, 4, 128, 4, 601, (gr.GR_PATH_TILE, 128), "M = 17, one strip pair"),
    (2600, 3000, 128, 128, 4, 144, 8, 3001, (gr.GR_PATH_TILE, 256), "256 tiles, partial"),
    (3072, 3072, 256, 256, 8, 256, 8, 3072, (gr.GR_PATH_TILE, 256), "256 tiles, whole"),
    (300, 270, 96, 96, 3, 96, 3, 273, (gr.GR_PATH_TILE_EDGE, 128), "guarded, K % 64 = 32"),
    (129, 200, 640, 640, 21, 640, 20, 200, (gr.GR_PATH_TILE_EDGE, 128), "guarded, odd scale pitch"),
    (70, 90, 160, 161, 5, 170, 5, 90, (gr.GR_PATH_TILE_EDGE, 128), "guarded, misaligned rows"),
]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=[c[-1] for c in CASES])
def test_mxfp8_parity(case, fmt):
    M, N, K, lda, ldsa, ldbt, ldsb, ldc, expect, what = case
    p = plan(M, N, K, lda, ldsa, ldbt, ldsb, ldc)
    assert (p["path"], p["block_m"]) == expect, p
    A, SA, Bt, SB = synth.mx_operands(M, N, K, seed=M + N + K, lda=lda, ldbt=ldbt, ldsa=ldsa, ldsb=ldsb)
    bias = bias_for(N, fmt, 3)
    Cflat = run(A, SA, Bt, SB, M, N, K, lda, ldsa, ldbt, ldsb, ldc, bias, "gelu", fmt)
    C = Cflat[:M * ldc].reshape(M, ldc)
    ref = oracle.gemm_mxfp8_bt_full(A, SA, Bt, SB, fmt, bias, "gelu", M=M, N=N, K=K, lda=lda, ldsa=ldsa, ldbt=ldbt,
                                    ldsb=ldsb)
    assert_parity(C[:, :N], ref, "mxfp8 %s %s" % (what, fmt), fmt=fmt)
    assert np.all(C[:, N:] == SENTINEL) and np.all(Cflat[M * ldc:] == SENTINEL)


@pytest.mark.parametrize("act", list(gr.ACT_CODES))
@pytest.mark.parametrize("path", [gr.GR_PATH_TILE, gr.GR_PATH_TILE_EDGE], ids=["tile", "guarded"])
def test_mxfp8_every_activation(act, path):
    M, N, K = 300, 270, 512
    A, SA, Bt, SB = synth.mx_operands(M, N, K, seed=21)
    bias = bias_for(N, "f16", 4) if act != "relu" else None
    C = run(A, SA, Bt, SB, M, N, K, K, K // 32, K, K // 32, N, bias, act, path=path)[:M * N].reshape(M, N)
    assert_parity(C, oracle.gemm_mxfp8_bt_full(A, SA, Bt, SB, bias=bias, act=act), "mxfp8 %s" % act)


@pytest.mark.parametrize("M,N,K", [(512, 512, 256), (300, 270, 1024), (2304, 1100, 384), (40, 2048, 512),
                                   (2600, 3000, 128)])
def test_mxfp8_tile_and_guarded_bitwise(M, N, K):
    A, SA, Bt, SB = synth.mx_operands(M, N, K, seed=31)
    kb = K // 32
    C1 = run(A, SA, Bt, SB, M, N, K, K, kb, K, kb, N, None, "silu", path=gr.GR_PATH_TILE)
    C2 = run(A, SA, Bt, SB, M, N, K, K, kb, K, kb, N, None, "silu", path=gr.GR_PATH_TILE_EDGE)
    assert np.array_equal(C1, C2)


def test_mxfp8_square_4096_sampled():
    """4096^3 on the pipelined kernel (256 tiles of 256^2): 4096 sampled
    elements plus the edge rows and columns of the first and last tiles."""
    M = N = K = 4096
    A, SA, Bt, SB = synth.mx_operands(M, N, K, seed=41)
    kb = K // 32
    C = run(A, SA, Bt, SB, M, N, K, K, kb, K, kb, N)[:M * N].reshape(M, N)
    ii, jj = synth.sample_indices(M, N, 4096, 41)
    assert_parity(C[ii, jj], oracle.gemm_mxfp8_bt_elems(A, SA, Bt, SB, ii, jj), "mxfp8 4096^3 sampled")
    for r in (0, 255, 256, 4095):
        jj = np.arange(N)
        assert_parity(C[r, :], oracle.gemm_mxfp8_bt_elems(A, SA, Bt, SB, np.full(N, r), jj), "row %d" % r)
        assert_parity(C[:, r], oracle.gemm_mxfp8_bt_elems(A, SA, Bt, SB, jj, np.full(M, r)), "col %d" % r)


def test_mxfp8_unit_scales_match_per_tensor_path():
    """All scale codes 127: the per-tensor fp8 call with unit scales computes
    the same products (within the tolerance: the two kernels give the
    matrix cores the k of a step in a different order)."""
    import torch as t
    M, N, K = 300, 500, 1024
    A, Bt = synth.fp8_operands(M, N, K, seed=51)
    SA = np.full((M, K // 32), 127, np.uint8)
    SB = np.full((N, K // 32), 127, np.uint8)
    C1 = run(A, SA, Bt, SB, M, N, K, K, K // 32, K, K // 32, N)[:M * N].reshape(M, N)
    dA, dB = dev8(A), dev8(Bt)  # held until the call has run
    dC = full_dev((M * N,), SENTINEL)
    st = gr.gemm_fp8_bt(M, N, K, dA.data_ptr(), K, dB.data_ptr(), K, 1.0, 1.0, None, gr.GR_ACT_RELU,
                        dC.data_ptr(), N, gr.GR_FMT_F16, t.cuda.current_stream().cuda_stream)
    t.cuda.synchronize()
    assert st == gr.GR_OK
    assert_parity(C1, from_dev(dC).reshape(M, N), "mx unit scales vs per-tensor")


def test_mxfp8_scale_pointer_offsets_and_k_zero():
    """Scale arrays at an odd byte offset take the guarded kernel; K = 0 gives
    act(bias)."""
    M, N, K = 260, 300, 256
    A, SA, Bt, SB = synth.mx_operands(M, N, K, seed=61)
    kb = K // 32
    assert plan(M, N, K, K, kb, K, kb, N, s_off=1)["path"] == gr.GR_PATH_TILE_EDGE
    C = run(A, SA, Bt, SB, M, N, K, K, kb, K, kb, N, s_offsets=(1, 3))[:M * N].reshape(M, N)
    assert_parity(C, oracle.gemm_mxfp8_bt_full(A, SA, Bt, SB), "mx scale offsets")
    bias = bias_for(N, "f16", 5)
    z = np.zeros((M, 1), np.uint8)
    C0 = run(z, z, np.zeros((N, 1), np.uint8), np.zeros((N, 1), np.uint8), M, N, 0, 1, 1, 1, 1, N, bias,
             "tanh")[:M * N].reshape(M, N)
    ref = oracle.gemm_fp8_bt_full(z, np.zeros((N, 1), np.uint8), bias=bias, act="tanh", M=M, N=N, K=0, lda=1, ldbt=1)
    assert_parity(C0, ref, "mx K=0")


def test_mxfp8_tensor_wrapper():
    t = pytest.importorskip("torch")
    M, N, K = 300, 200, 512
    A, SA, Bt, SB = synth.mx_operands(M, N, K, seed=71)
    a = dev8(A)[:M * K].view(t.float8_e4m3fn).reshape(M, K)
    bt = dev8(Bt)[:N * K].view(t.float8_e4m3fn).reshape(N, K)
    sa = dev8(SA)[:SA.size].reshape(SA.shape)
    sb = dev8(SB)[:SB.size].reshape(SB.shape)
    bias = dev16(bias_for(N, "bf16", 6)).view(t.bfloat16)
    c = gr.gemm_mxfp8(a, sa, bt, sb, bias=bias, act="gelu_tanh", out_dtype=t.bfloat16)
    t.cuda.synchronize()
    ref = oracle.gemm_mxfp8_bt_full(A, SA, Bt, SB, "bf16", bias_for(N, "bf16", 6), "gelu_tanh")
    assert_parity(c.view(t.int16).cpu().numpy().view(np.uint16), ref, "mx wrapper", fmt="bf16")
