"""GPU parity of gemm_fp8_bt (OCP fp8 E4M3 operands, B given transposed) with
the CPU oracle.

Same bar as every other path (|gpu - oracle| <= 1e-2 + 1e-2 |oracle|,
"Writing high-performance kernels in TileLang", section "Writing a GEMM"),
plus bit-for-bit agreement of the pipelined and guarded kernels, which feed
the matrix cores the same operands in the same order. Inputs are N(0,1)
values rounded to E4M3, with per-tensor scales as a quantised GEMM uses them.
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


def dev8(x):
    import torch as t
    return t.from_numpy(np.ascontiguousarray(x)).to("cuda")


def dev16(x):
    import torch as t
    return t.from_numpy(np.ascontiguousarray(x).view(np.int16)).to("cuda")


def plan(M, N, K, lda, ldbt, ldc, a_off=0, b_off=0):
    st, p = gr.gemm_fp8_bt_plan(M, N, K, 0x100000 + a_off, lda, 0x200000000000 + b_off, ldbt, None, 1,
                                0x400000000000, ldc)
    assert st == gr.GR_OK
    return p


def run(A, Bt, M, N, K, lda, ldbt, ldc, sa=1.0, sb=1.0, bias=None, act="relu", fmt="f16", path=None, c_rows=None,
        offsets=(0, 0)):
    import torch as t
    dA = dev8(np.concatenate([np.zeros(offsets[0], np.uint8), A.ravel(), np.zeros(16, np.uint8)]))
    dB = dev8(np.concatenate([np.zeros(offsets[1], np.uint8), Bt.ravel(), np.zeros(16, np.uint8)]))
    db = dev16(bias) if bias is not None else None
    rows = M if c_rows is None else c_rows
    dC = full_dev((rows * ldc + 8,), SENTINEL)
    log("fp8 M=%d N=%d K=%d lda=%d ldbt=%d ldc=%d act=%s fmt=%s path=%s offsets=%s" %
        (M, N, K, lda, ldbt, ldc, act, fmt, path, offsets))
    args = (M, N, K, dA.data_ptr() + offsets[0], lda, dB.data_ptr() + offsets[1], ldbt, sa, sb,
            db.data_ptr() if db is not None else None, gr.ACT_CODES[act], dC.data_ptr(), ldc, FMTS[fmt],
            t.cuda.current_stream().cuda_stream)
    st = gr.gemm_fp8_bt(*args) if path is None else gr.gemm_fp8_bt_forced(*args, path)
    t.cuda.synchronize()
    assert st == gr.GR_OK, gr.gemm_relu_status_string(st)
    return from_dev(dC)


def bias_for(N, fmt, seed):
    import torch as t
    g = t.Generator().manual_seed(seed)
    x = t.randn(N, generator=g)
    return x.to(t.bfloat16 if fmt == "bf16" else t.float16).view(t.int16).numpy().view(np.uint16)


CASES = [
    # M, N, K, lda, ldbt, ldc, expected path (tile size), what
    (512, 512, 256, 256, 256, 512, (gr.GR_PATH_TILE, 128), "128 tiles, whole"),
    (1024, 768, 512, 528, 512, 768, (gr.GR_PATH_TILE, 128), "128 tiles, padded A"),
    (300, 270, 128, 128, 144, 273, (gr.GR_PATH_TILE, 128), "128 tiles, partial"),
    (17, 600, 256, 256, 256, 601, (gr.GR_PATH_TILE, 128), "M = 17"),
    (2304, 1100, 192, 192, 192, 1100, (gr.GR_PATH_TILE, 128), "128 tiles, 3 strips"),
    (2600, 3000, 128, 128, 144, 3001, (gr.GR_PATH_TILE, 256), "256 tiles, partial"),
    (3072, 3072, 192, 192, 192, 3072, (gr.GR_PATH_TILE, 256), "256 tiles, whole"),
    (8, 4096, 1024, 1024, 1024, 4096, (gr.GR_PATH_SMALL_M, 16), "small-M"),
    (16, 1000, 512, 512, 528, 1001, (gr.GR_PATH_SMALL_M, 16), "small-M, partial column block"),
    (1, 64, 2048, 2048, 2048, 64, (gr.GR_PATH_SMALL_M, 16), "small-M, one row"),
    (12, 300, 640, 640, 640, 300, (gr.GR_PATH_TILE, 128), "M <= 16, K % 512 != 0"),
    (300, 270, 100, 101, 103, 273, gr.GR_PATH_TILE_EDGE, "guarded, odd K and pitches"),
    (5, 130, 1000, 1000, 1000, 130, gr.GR_PATH_TILE_EDGE, "guarded, K % 64 != 0"),
    (700, 500, 320, 330, 320, 500, gr.GR_PATH_TILE_EDGE, "guarded, misaligned A rows"),
]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=[c[-1] for c in CASES])
def test_fp8_parity(case, fmt):
    M, N, K, lda, ldbt, ldc, path, what = case
    p = plan(M, N, K, lda, ldbt, ldc)
    if isinstance(path, tuple):
        assert (p["path"], p["block_m"]) == path, p
    else:
        assert p["path"] == path, p
    A, Bt = synth.fp8_operands(M, N, K, seed=M + N + K, lda=lda, ldbt=ldbt)
    sa, sb = 0.125, 2.0 / np.sqrt(K)
    bias = bias_for(N, fmt, 3)
    Cflat = run(A, Bt, M, N, K, lda, ldbt, ldc, sa, sb, bias, "gelu", fmt, c_rows=M + 1)
    C = Cflat[:M * ldc].reshape(M, ldc)
    ref = oracle.gemm_fp8_bt_full(A, Bt, sa, sb, fmt, bias, "gelu", M=M, N=N, K=K, lda=lda, ldbt=ldbt)
    assert_parity(C[:, :N], ref, "fp8 %s %s" % (what, fmt), fmt=fmt)
    assert np.all(C[:, N:] == SENTINEL) and np.all(Cflat[M * ldc:] == SENTINEL)


@pytest.mark.parametrize("act", list(gr.ACT_CODES))
@pytest.mark.parametrize("path_case", [(300, 270, 128, 128, 128, 270), (300, 270, 100, 100, 100, 270),
                                       (7, 270, 1024, 1024, 1024, 270)],
                         ids=["tile", "guarded", "small-M"])
def test_fp8_every_activation(act, path_case):
    M, N, K, lda, ldbt, ldc = path_case
    A, Bt = synth.fp8_operands(M, N, K, seed=21, lda=lda, ldbt=ldbt)
    sa, sb = 0.25, 0.5
    bias = bias_for(N, "f16", 4) if act != "relu" else None
    C = run(A, Bt, M, N, K, lda, ldbt, ldc, sa, sb, bias, act)[:M * N].reshape(M, N)
    ref = oracle.gemm_fp8_bt_full(A, Bt, sa, sb, "f16", bias, act, lda=lda, ldbt=ldbt)
    assert_parity(C, ref, "fp8 %s" % act)


@pytest.mark.parametrize("M,N,K", [(512, 512, 256), (300, 270, 128), (2304, 1100, 192), (40, 2048, 1024),
                                   (2600, 3000, 128)])
def test_fp8_tile_and_guarded_bitwise(M, N, K):
    A, Bt = synth.fp8_operands(M, N, K, seed=31)
    C1 = run(A, Bt, M, N, K, K, K, N, 0.5, 0.5, None, "silu", path=gr.GR_PATH_TILE)
    C2 = run(A, Bt, M, N, K, K, K, N, 0.5, 0.5, None, "silu", path=gr.GR_PATH_TILE_EDGE)
    assert np.array_equal(C1, C2)


def test_fp8_headline_shape_sampled():
    """4096^3, the pipelined kernel on whole tiles: 4096 sampled elements plus
    the first and last rows and columns of the first and last tiles."""
    M = N = K = 4096
    A, Bt = synth.fp8_operands(M, N, K, seed=41)
    sa, sb = 1.0 / 64, 1.0
    C = run(A, Bt, M, N, K, K, K, N, sa, sb)[:M * N].reshape(M, N)
    ii, jj = synth.sample_indices(M, N, 4096, 41)
    assert_parity(C[ii, jj], oracle.gemm_fp8_bt_elems(A, Bt, ii, jj, sa, sb), "fp8 4096^3 sampled")
    edges = [0, 255, 256, 3839, 3840, 4095]
    for r in edges:
        jj = np.arange(N)
        assert_parity(C[r, :], oracle.gemm_fp8_bt_elems(A, Bt, np.full(N, r), jj, sa, sb), "row %d" % r)
        assert_parity(C[:, r], oracle.gemm_fp8_bt_elems(A, Bt, jj, np.full(M, r), sa, sb), "col %d" % r)


def test_fp8_k_zero_and_unaligned_pointers():
    M, N = 33, 70
    bias = bias_for(N, "f16", 5)
    C = run(np.zeros((M, 1), np.uint8), np.zeros((N, 1), np.uint8), M, N, 0, 1, 1, N, bias=bias, act="tanh")
    ref = oracle.gemm_fp8_bt_full(np.zeros((M, 1), np.uint8), np.zeros((N, 1), np.uint8), bias=bias, act="tanh",
                                  M=M, N=N, K=0, lda=1, ldbt=1)
    assert_parity(C[:M * N].reshape(M, N), ref, "K=0")
    M, N, K = 260, 300, 256
    A, Bt = synth.fp8_operands(M, N, K, seed=51)
    assert plan(M, N, K, K, K, N, a_off=3)["path"] == gr.GR_PATH_TILE_EDGE
    C = run(A, Bt, M, N, K, K, K, N, 0.5, 0.25, offsets=(3, 5))[:M * N].reshape(M, N)
    assert_parity(C, oracle.gemm_fp8_bt_full(A, Bt, 0.5, 0.25), "fp8 unaligned")


def test_fp8_tensor_wrapper():
    t = pytest.importorskip("torch")
    M, N, K = 300, 200, 256
    A, Bt = synth.fp8_operands(M, N, K, seed=61)
    a = dev8(A).view(t.float8_e4m3fn)
    bt = dev8(Bt).view(t.float8_e4m3fn)
    bias = dev16(bias_for(N, "bf16", 6)).view(t.bfloat16)
    c = gr.gemm_fp8(a, bt, 0.5, 0.125, bias=bias, act="gelu_tanh", out_dtype=t.bfloat16)
    t.cuda.synchronize()
    assert c.dtype == t.bfloat16
    ref = oracle.gemm_fp8_bt_full(A, Bt, 0.5, 0.125, "bf16", bias_for(N, "bf16", 6), "gelu_tanh")
    assert_parity(c.view(t.int16).cpu().numpy().view(np.uint16), ref, "fp8 wrapper", fmt="bf16")


@pytest.mark.parametrize("M,N,K", [(8, 16384, 8192), (16, 256, 512)])
def test_fp8_small_m_against_tile(M, N, K):
    """The small-M stream and the 128 x 128 tile kernel on the same input
    (different matrix-core shapes: equal within the tolerance), and the
    small-M result against the oracle."""
    A, Bt = synth.fp8_operands(M, N, K, seed=71)
    sa, sb = 1.0 / 16, 1.0 / 16
    C1 = run(A, Bt, M, N, K, K, K, N, sa, sb, path=gr.GR_PATH_SMALL_M)[:M * N].reshape(M, N)
    C2 = run(A, Bt, M, N, K, K, K, N, sa, sb, path=gr.GR_PATH_TILE)[:M * N].reshape(M, N)
    assert_parity(C1, C2, "small-M vs tile")
    assert_parity(C1, oracle.gemm_fp8_bt_full(A, Bt, sa, sb), "small-M vs oracle")


# ---- split-K with a workspace (gemm_fp8_bt_ws) -------------------------------------

def run_ws(A, Bt, M, N, K, lda, ldbt, ldc, sa, sb, bias, act, fmt, path=-1, ws_bytes=None):
    import torch as t
    dA = dev8(np.concatenate([A.ravel(), np.zeros(16, np.uint8)]))
    dB = dev8(np.concatenate([Bt.ravel(), np.zeros(16, np.uint8)]))
    db = dev16(bias) if bias is not None else None
    dC = full_dev((M * ldc + 8,), SENTINEL)
    if ws_bytes is None:
        st, ws_bytes = gr.gemm_fp8_bt_workspace_size(M, N, K, dA.data_ptr(), lda, dB.data_ptr(), ldbt, dC.data_ptr(),
                                                     ldc)
        assert st == gr.GR_OK
        ws_bytes = max(ws_bytes, 32 << 20)  # forced splits may need more than the planner's choice
    ws = t.full((ws_bytes,), 0x7F, dtype=t.uint8, device="cuda")  # dirty: NaN-ish floats if a partial is not written
    log("fp8 ws M=%d N=%d K=%d lda=%d ldbt=%d ldc=%d act=%s fmt=%s path=%s ws=%d" %
        (M, N, K, lda, ldbt, ldc, act, fmt, path, ws_bytes))
    st = gr.gemm_fp8_bt_ws(M, N, K, dA.data_ptr(), lda, dB.data_ptr(), ldbt, sa, sb,
                           db.data_ptr() if db is not None else None, gr.ACT_CODES[act], dC.data_ptr(), ldc, FMTS[fmt],
                           ws.data_ptr(), ws_bytes, t.cuda.current_stream().cuda_stream, path)
    t.cuda.synchronize()
    assert st == gr.GR_OK, gr.gemm_relu_status_string(st)
    return from_dev(dC)


SPLIT_CASES = [
    # M, N, K, lda, ldbt, ldc, forced path (-1: the planner must pick the split), what
    (300, 270, 8192, 8192, 8192, 273, -1, "3 x 3 partial tiles, 16 splits"),
    (256, 512, 4096, 4096, 4112, 512, gr.GR_PATH_TILE_SPLIT, "whole tiles, padded Bt"),
    (129, 1000, 2048, 2064, 2048, 1001, gr.GR_PATH_TILE_SPLIT, "partial tiles, odd N"),
    (40, 256, 64, 64, 64, 256, gr.GR_PATH_TILE_SPLIT, "one strip: a single split"),
    (17, 130, 1984, 1984, 1984, 130, gr.GR_PATH_TILE_SPLIT, "K not a multiple of the split"),
]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("case", SPLIT_CASES, ids=[c[-1] for c in SPLIT_CASES])
def test_fp8_split_parity(case, fmt):
    M, N, K, lda, ldbt, ldc, path, what = case
    if path == -1:
        st, p = gr.gemm_fp8_bt_plan_ws(M, N, K, 0x100000, lda, 0x200000000000, ldbt, None, 2, 0x400000000000, ldc,
                                       FMTS[fmt], 1 << 30)
        assert p["path"] == gr.GR_PATH_TILE_SPLIT and p["split_k"] > 1, p
    A, Bt = synth.fp8_operands(M, N, K, seed=M + N + K + 7, lda=lda, ldbt=ldbt)
    sa, sb = 0.125, 2.0 / np.sqrt(K)
    bias = bias_for(N, fmt, 9)
    Cflat = run_ws(A, Bt, M, N, K, lda, ldbt, ldc, sa, sb, bias, "gelu", fmt, path)
    C = Cflat[:M * ldc].reshape(M, ldc)
    ref = oracle.gemm_fp8_bt_full(A, Bt, sa, sb, fmt, bias, "gelu", M=M, N=N, K=K, lda=lda, ldbt=ldbt)
    assert_parity(C[:, :N], ref, "fp8 split %s %s" % (what, fmt), fmt=fmt)
    assert np.all(C[:, N:] == SENTINEL) and np.all(Cflat[M * ldc:] == SENTINEL)


@pytest.mark.parametrize("act", list(gr.ACT_CODES))
def test_fp8_split_every_activation(act):
    M, N, K = 200, 300, 4096
    A, Bt = synth.fp8_operands(M, N, K, seed=81)
    sa, sb = 0.25, 1.0 / 16
    bias = bias_for(N, "f16", 8) if act != "relu" else None
    C = run_ws(A, Bt, M, N, K, K, K, N, sa, sb, bias, act, "f16", gr.GR_PATH_TILE_SPLIT)[:M * N].reshape(M, N)
    assert_parity(C, oracle.gemm_fp8_bt_full(A, Bt, sa, sb, "f16", bias, act), "fp8 split %s" % act)


def test_fp8_split_mid_m_sampled():
    """128 x 8192 x 8192 (64 tiles, 4 splits): the planner's split on the
    shape it is for, sampled against the oracle, and against the unsplit
    kernel within the tolerance."""
    M, N, K = 128, 8192, 8192
    A, Bt = synth.fp8_operands(M, N, K, seed=91)
    sa, sb = 1.0 / 16, 1.0 / 16
    st, p = gr.gemm_fp8_bt_plan_ws(M, N, K, 0x100000, K, 0x200000000000, K, None, 1, 0x400000000000, N, 0, 1 << 30)
    assert p["path"] == gr.GR_PATH_TILE_SPLIT
    C = run_ws(A, Bt, M, N, K, K, K, N, sa, sb, None, "relu", "f16")[:M * N].reshape(M, N)
    ii, jj = synth.sample_indices(M, N, 4096, 91)
    assert_parity(C[ii, jj], oracle.gemm_fp8_bt_elems(A, Bt, ii, jj, sa, sb), "fp8 split 128x8192x8192 sampled")
    for r in (0, 127):
        jj = np.arange(N)
        assert_parity(C[r, :], oracle.gemm_fp8_bt_elems(A, Bt, np.full(N, r), jj, sa, sb), "row %d" % r)
    C1 = run(A, Bt, M, N, K, K, K, N, sa, sb)[:M * N].reshape(M, N)
    assert_parity(C, C1, "split vs unsplit")


def test_fp8_split_workspace_reuse_and_wrapper():
    """Two calls in a row on one workspace (the second smaller), then the
    tensor helper with its own workspace."""
    t = pytest.importorskip("torch")
    ws = t.empty(64 << 20, dtype=t.uint8, device="cuda")
    for (M, N, K) in ((256, 1024, 8192), (100, 300, 2048)):
        A, Bt = synth.fp8_operands(M, N, K, seed=M)
        dA, dB = dev8(A), dev8(Bt)
        dC = full_dev((M * N,), SENTINEL)
        st = gr.gemm_fp8_bt_ws(M, N, K, dA.data_ptr(), K, dB.data_ptr(), K, 0.5, 0.25, None, gr.GR_ACT_RELU,
                               dC.data_ptr(), N, gr.GR_FMT_F16, ws.data_ptr(), ws.numel(),
                               t.cuda.current_stream().cuda_stream, gr.GR_PATH_TILE_SPLIT)
        t.cuda.synchronize()
        assert st == gr.GR_OK
        assert_parity(from_dev(dC).reshape(M, N), oracle.gemm_fp8_bt_full(A, Bt, 0.5, 0.25), "reuse %d" % M)
    M, N, K = 300, 270, 8192
    A, Bt = synth.fp8_operands(M, N, K, seed=95)
    c = gr.gemm_fp8(dev8(A).view(t.float8_e4m3fn), dev8(Bt).view(t.float8_e4m3fn), 0.5, 1.0 / 64, act="silu")
    t.cuda.synchronize()
    assert_parity(c.view(t.int16).cpu().numpy().view(np.uint16),
                  oracle.gemm_fp8_bt_full(A, Bt, 0.5, 1.0 / 64, act="silu"), "fp8 wrapper split")
