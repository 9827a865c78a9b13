"""GPU parity of gemm_mxfp4_bt (OCP MX fp4: E2M1 elements two per byte, one
E8M0 scale per 32 consecutive k of each row, B given transposed) with the CPU
oracle.

Same bar as every other path (|gpu - oracle| <= 1e-2 + 1e-2 |oracle|,
"Writing high-performance kernels in TileLang", section "Writing a GEMM"),
plus bit-for-bit agreement of the pipelined and guarded kernels.  Inputs are
N(0,1) values times 2^u (u from -2..2 per 32-k block) quantised the OCP MX
way to E2M1 (synth.mxfp4_operands); padding bytes hold 6.0 twice and the
scale padding the NaN code, so a read outside the matrices shows.
"""
import numpy as np
import pytest

import dense_gemm_epilogue_tiled_amd as gr
import oracle
import synth
from gpu_util import assert_parity, from_dev, full_dev, log

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("oracle_lib")]

SENTINEL = 0x7FC1
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


def run(A, SA, Bt, SB, M, N, K, lda, ldsa, ldbt, ldsb, ldc, bias=None, act="relu", fmt="f16", path=None):
    import torch as t
    dA, dB, dSA, dSB = dev8(A), dev8(Bt), dev8(SA), dev8(SB)
    db = dev16(bias) if bias is not None else None
    dC = full_dev(((M + 1) * ldc + 8,), SENTINEL)
    log("mxfp4 M=%d N=%d K=%d lda=%d ldsa=%d ldbt=%d ldsb=%d ldc=%d act=%s fmt=%s path=%s" %
        (M, N, K, lda, ldsa, ldbt, ldsb, ldc, act, fmt, path))
    args = (M, N, K, dA.data_ptr(), lda, dSA.data_ptr(), ldsa, dB.data_ptr(), ldbt, dSB.data_ptr(), ldsb,
            db.data_ptr() if db is not None else None, gr.ACT_CODES[act], dC.data_ptr(), ldc, FMTS[fmt],
            t.cuda.current_stream().cuda_stream)
    st = gr.gemm_mxfp4_bt(*args) if path is None else gr.gemm_mxfp4_bt_forced(*args, path)
    t.cuda.synchronize()
    assert st == gr.GR_OK, gr.gemm_relu_status_string(st)
    return from_dev(dC)


def plan(M, N, K, lda, ldsa, ldbt, ldsb, ldc):
    st, p = gr.gemm_mxfp4_bt_plan(M, N, K, 0x100000, lda, 0x300000, ldsa, 0x200000000000, ldbt, 0x300000, ldsb,
                                  None, 1, 0x400000000000, ldc)
    assert st == gr.GR_OK
    return p


CASES = [
    # M, N, K (elements), lda, ldsa, ldbt, ldsb (bytes), ldc, expected (path, tile), what
    (512, 512, 256, 128, 8, 128, 8, 512, (gr.GR_PATH_TILE, 128), "128 tiles, whole"),
    (300, 270, 384, 208, 12, 192, 16, 273, (gr.GR_PATH_TILE, 128), "128 tiles, partial, padded"),
    (17, 600, 128, 64, 4, 64, 4, 601, (gr.GR_PATH_TILE, 128), "M = 17, one strip"),
    (2600, 3000, 256, 128, 8, 144, 8, 3001, (gr.GR_PATH_TILE, 256), "256 tiles, partial"),
    (3072, 3072, 512, 256, 16, 256, 16, 3072, (gr.GR_PATH_TILE, 256), "256 tiles, whole"),
    (300, 270, 96, 48, 3, 48, 3, 273, (gr.GR_PATH_TILE_EDGE, 128), "guarded, K % 128 = 96"),
    (129, 200, 640, 320, 21, 320, 20, 200, (gr.GR_PATH_TILE_EDGE, 128), "guarded, odd scale pitch"),
    (70, 90, 160, 81, 5, 85, 5, 90, (gr.GR_PATH_TILE_EDGE, 128), "guarded, misaligned rows"),
]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=[c[-1] for c in CASES])
def test_mxfp4_parity(case, fmt):
    M, N, K, lda, ldsa, ldbt, ldsb, ldc, expect, what = case
    p = plan(M, N, K, lda, ldsa, ldbt, ldsb, ldc)
    assert (p["path"], p["block_m"]) == expect, p
    A, SA, Bt, SB = synth.mxfp4_operands(M, N, K, seed=M + N + K, lda=lda, ldbt=ldbt, ldsa=ldsa, ldsb=ldsb)
    bias = bias_for(N, fmt, 3)
    Cflat = run(A, SA, Bt, SB, M, N, K, lda, ldsa, ldbt, ldsb, ldc, bias, "gelu", fmt)
    C = Cflat[:M * ldc].reshape(M, ldc)
    ref = oracle.gemm_mxfp4_bt_full(A, SA, Bt, SB, fmt, bias, "gelu", M=M, N=N, K=K, lda=lda, ldsa=ldsa, ldbt=ldbt,
                                    ldsb=ldsb)
    assert_parity(C[:, :N], ref, "mxfp4 %s %s" % (what, fmt), fmt=fmt)
    assert np.all(C[:, N:] == SENTINEL) and np.all(Cflat[M * ldc:] == SENTINEL)


@pytest.mark.parametrize("act", list(gr.ACT_CODES))
@pytest.mark.parametrize("path", [gr.GR_PATH_TILE, gr.GR_PATH_TILE_EDGE], ids=["tile", "guarded"])
def test_mxfp4_every_activation(act, path):
    M, N, K = 300, 270, 512
    A, SA, Bt, SB = synth.mxfp4_operands(M, N, K, seed=21)
    bias = bias_for(N, "f16", 4) if act != "relu" else None
    C = run(A, SA, Bt, SB, M, N, K, K // 2, K // 32, K // 2, K // 32, N, bias, act, path=path)[:M * N].reshape(M, N)
    assert_parity(C, oracle.gemm_mxfp4_bt_full(A, SA, Bt, SB, bias=bias, act=act), "mxfp4 %s" % act)


@pytest.mark.parametrize("M,N,K", [(512, 512, 256), (300, 270, 1024), (40, 2048, 512), (2600, 3000, 256)])
def test_mxfp4_tile_and_guarded_bitwise(M, N, K):
    A, SA, Bt, SB = synth.mxfp4_operands(M, N, K, seed=31)
    kb = K // 32
    C1 = run(A, SA, Bt, SB, M, N, K, K // 2, kb, K // 2, kb, N, None, "silu", path=gr.GR_PATH_TILE)
    C2 = run(A, SA, Bt, SB, M, N, K, K // 2, kb, K // 2, kb, N, None, "silu", path=gr.GR_PATH_TILE_EDGE)
    assert np.array_equal(C1, C2)


def test_mxfp4_square_4096_sampled():
    M = N = K = 4096
    A, SA, Bt, SB = synth.mxfp4_operands(M, N, K, seed=41)
    kb = K // 32
    C = run(A, SA, Bt, SB, M, N, K, K // 2, kb, K // 2, kb, N)[:M * N].reshape(M, N)
    ii, jj = synth.sample_indices(M, N, 4096, 41)
    assert_parity(C[ii, jj], oracle.gemm_mxfp4_bt_elems(A, SA, Bt, SB, ii, jj), "mxfp4 4096^3 sampled")
    for r in (0, 255, 256, 4095):
        jj = np.arange(N)
        assert_parity(C[r, :], oracle.gemm_mxfp4_bt_elems(A, SA, Bt, SB, np.full(N, r), jj), "row %d" % r)
        assert_parity(C[:, r], oracle.gemm_mxfp4_bt_elems(A, SA, Bt, SB, jj, np.full(M, r)), "col %d" % r)


def test_mxfp4_matches_mxfp8_on_the_same_values():
    """E2M1 values are exact in E4M3: the fp4 call and the fp8 call on the
    re-encoded operands (same scales) agree within the tolerance (the two
    instructions add the k of a step in different orders)."""
    import torch as t
    M, N, K = 300, 500, 1024
    A, SA, Bt, SB = synth.mxfp4_operands(M, N, K, seed=51)
    C4 = run(A, SA, Bt, SB, M, N, K, K // 2, K // 32, K // 2, K // 32, N)[:M * N].reshape(M, N)

    def to_e4m3(P):
        codes = np.empty((P.shape[0], K), np.uint8)
        codes[:, 0::2], codes[:, 1::2] = P[:, :K // 2] & 15, P[:, :K // 2] >> 4
        v = oracle.e2m1_to_f32(codes)
        return t.from_numpy(v).to(t.float8_e4m3fn).view(t.uint8).numpy()
    A8, B8 = to_e4m3(A), to_e4m3(Bt)
    dA, dSA, dB, dSB = dev8(A8), dev8(SA), dev8(B8), dev8(SB)
    dC = full_dev((M * N,), SENTINEL)
    st = gr.gemm_mxfp8_bt(M, N, K, dA.data_ptr(), K, dSA.data_ptr(), K // 32, dB.data_ptr(), K, dSB.data_ptr(),
                          K // 32, None, gr.GR_ACT_RELU, dC.data_ptr(), N, gr.GR_FMT_F16,
                          t.cuda.current_stream().cuda_stream)
    t.cuda.synchronize()
    assert st == gr.GR_OK
    assert_parity(C4, from_dev(dC).reshape(M, N), "mxfp4 vs mxfp8")
