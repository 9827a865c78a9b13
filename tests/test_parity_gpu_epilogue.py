"""GPU parity of gemm_bias_act_* (C = act(A.B + bias)) against the CPU oracle.

Same bar as the fused-ReLU paths (|gpu - oracle| <= 1e-2 + 1e-2 |oracle|,
"Writing high-performance kernels in TileLang", section "Writing a GEMM"):
the kernels evaluate the activation in fp32 with the device library, the
oracle in double precision, and both round once to the output format. Every
activation runs on every kernel family (pipelined 128 x 128 and 256 x 256
tiles with partial tiles, the guarded kernel, the small-M kernel), in fp16 and
bfloat16, with and without a bias; with ReLU and no bias the result must equal
the fused-ReLU call bit for bit, and the pipelined and guarded kernels agree
bit for bit with each other.
"""
import numpy as np
import pytest

import dense_gemm_epilogue_tiled_amd as gr
import oracle
import synth
from gpu_util import as_f64, assert_parity, from_dev, full_dev, log, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("oracle_lib")]


def planned_agrees(planned, path):
    """The planner's path for a case written for the kernel family `path`:
    that family, or the faster paths it plans for the same rows (the
    streaming kernel for few blocks; the unaligned kernel or the streaming
    kernel for rows the guarded kernel would take)."""
    if path == gr.GR_PATH_TILE:
        return planned in (gr.GR_PATH_TILE, gr.GR_PATH_TILE_STREAM)
    if path == gr.GR_PATH_TILE_EDGE:
        return planned in (gr.GR_PATH_TILE_EDGE, gr.GR_PATH_TILE_UNALIGNED, gr.GR_PATH_TILE_STREAM)
    if path == gr.GR_PATH_SMALL_M:
        return planned in (gr.GR_PATH_SMALL_M, gr.GR_PATH_TILE_STREAM)
    return planned == path


SENTINEL = 0x7FC1  # NaN in fp16 and in bfloat16
ACTS = list(gr.ACT_CODES)

FAMILY_CASES = [
    # M, N, K, lda, ldb, ldc, expected path, kernel family
    (300, 250, 96, 104, 256, 251, gr.GR_PATH_TILE, "tile128 partial"),
    (2400, 4000, 128, 128, 4008, 4001, gr.GR_PATH_TILE, "tile 256 64-deep partial"),
    (2400, 4000, 96, 96, 4000, 4001, gr.GR_PATH_TILE, "tile 256 32-deep partial"),
    (300, 270, 100, 109, 277, 273, gr.GR_PATH_TILE_EDGE, "guarded"),
    (13, 1000, 1000, 1000, 1000, 1001, gr.GR_PATH_SMALL_M, "small-M guarded"),
    (45, 700, 512, 512, 704, 701, gr.GR_PATH_SMALL_M, "small-M four row blocks"),
]

EXTRA_CASES = [
    (512, 768, 256, 256, 768, 768, gr.GR_PATH_TILE, "tile128 whole"),
    (4352, 4100, 128, 128, 4104, 4101, gr.GR_PATH_TILE, "tile 256, 289 tiles"),
    (4096, 2304, 256, 256, 2304, 2304, gr.GR_PATH_TILE, "tile 256 whole"),
    (257, 130, 70, 70, 130, 130, gr.GR_PATH_TILE_EDGE, "guarded 4-byte rows"),
    (8, 4096, 1024, 1024, 4096, 4096, gr.GR_PATH_SMALL_M, "small-M whole"),
]


def plan_path(M, N, K, lda, ldb, ldc):
    st, p = gr.gemm_relu_f16_plan(M, N, K, 0x100000, lda, 0x200000000000, ldb, 0x400000000000, ldc)
    assert st == gr.GR_OK
    return p["path"]


def operands(M, N, K, seed, lda, ldb, fmt):
    A, B = synth.random_operands(M, N, K, seed=seed, lda=lda, ldb=ldb, b_scale=2.0 * max(K, 1) ** -0.5, fmt=fmt)
    _, b2 = synth.random_operands(1, N, 1, seed=seed + 1, fmt=fmt)
    return A, B, np.ascontiguousarray(b2[0])


def run(A, B, bias, M, N, K, lda, ldb, ldc, act, fmt, path=None, c_rows=None, bias_offset=0):
    """Flat C buffer (c_rows x ldc + tail, prefilled with SENTINEL) after the call."""
    import torch as t
    dA = to_dev(A) if A.size else None
    dB = to_dev(B) if B.size else None
    dbias = None
    if bias is not None:
        dbias = to_dev(np.concatenate([np.zeros(bias_offset, np.uint16), bias]))
    rows = M if c_rows is None else c_rows
    dC = full_dev((rows * ldc + 8,), SENTINEL)
    a = dA.data_ptr() if dA is not None else 0
    b = dB.data_ptr() if dB is not None else 0
    bp = dbias.data_ptr() + 2 * bias_offset if dbias is not None else 0
    s = t.cuda.current_stream().cuda_stream
    code = gr.ACT_CODES[act]
    log("epi %s %s M=%d N=%d K=%d lda=%d ldb=%d ldc=%d bias=%s path=%s" %
        (fmt, act, M, N, K, lda, ldb, ldc, bias is not None, path))
    if path is None:
        f = gr.gemm_bias_act_bf16 if fmt == "bf16" else gr.gemm_bias_act_f16
        st = f(M, N, K, a, lda, b, ldb, bp, code, dC.data_ptr(), ldc, s)
    else:
        f = gr.gemm_bias_act_bf16_forced if fmt == "bf16" else gr.gemm_bias_act_f16_forced
        st = f(M, N, K, a, lda, b, ldb, bp, code, dC.data_ptr(), ldc, s, path)
    t.cuda.synchronize()
    assert st == gr.GR_OK, gr.gemm_relu_status_string(st)
    return from_dev(dC)


def check(M, N, K, lda, ldb, ldc, path, act, fmt, with_bias=True, seed=0):
    # the kernel family under test is forced; the planner picks it, or 64 x
    # 64 blocks on the streaming kernel where 128 x 128 tiles would be few
    planned = plan_path(M, N, K, lda, ldb, ldc)
    assert planned_agrees(planned, path), (planned, path)
    A, B, bias = operands(M, N, K, seed + M + N + K, lda, ldb, fmt)
    bias = bias if with_bias else None
    Cflat = run(A, B, bias, M, N, K, lda, ldb, ldc, act, fmt, path=path, c_rows=M + 1)
    C = Cflat[:M * ldc].reshape(M, ldc)
    ref = oracle.gemm_relu_full(A, B, M=M, N=N, K=K, lda=lda, ldb=ldb, fmt=fmt, bias=bias, act=act)
    rep = assert_parity(C[:, :N], ref, "%s %s %dx%dx%d" % (fmt, act, M, N, K), fmt=fmt)
    assert np.all(C[:, N:] == SENTINEL) and np.all(Cflat[M * ldc:] == SENTINEL)
    return C[:, :N], rep


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("case", FAMILY_CASES, ids=[c[-1] for c in FAMILY_CASES])
def test_every_activation_on_every_kernel(case, act, fmt):
    M, N, K, lda, ldb, ldc, path, _ = case
    C, _ = check(M, N, K, lda, ldb, ldc, path, act, fmt)
    if act == "none":
        assert np.any(C & 0x8000)  # negative sums are kept without an activation


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("case", EXTRA_CASES, ids=[c[-1] for c in EXTRA_CASES])
def test_gelu_and_identity_on_whole_tiles(case, fmt):
    M, N, K, lda, ldb, ldc, path, _ = case
    check(M, N, K, lda, ldb, ldc, path, "gelu", fmt)
    check(M, N, K, lda, ldb, ldc, path, "none", fmt, with_bias=False)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("M,N,K", [(512, 768, 256), (2400, 4000, 128), (300, 256, 96), (12, 1000, 512)])
def test_relu_without_bias_is_the_fused_relu_bitwise(M, N, K, fmt):
    A, B, _ = operands(M, N, K, 5, K, N, fmt)
    C1 = run(A, B, None, M, N, K, K, N, N, "relu", fmt)
    import torch as t
    dA, dB = to_dev(A), to_dev(B)
    dC = full_dev((M * N + 8,), SENTINEL)
    f = gr.gemm_relu_bf16 if fmt == "bf16" else gr.gemm_relu_f16
    assert f(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, dC.data_ptr(), N,
             t.cuda.current_stream().cuda_stream) == gr.GR_OK
    t.cuda.synchronize()
    assert np.array_equal(C1, from_dev(dC))


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("act", ["gelu", "silu", "none"])
@pytest.mark.parametrize("M,N,K", [(512, 768, 256), (4096, 2304, 96), (300, 256, 96)])
def test_tile_and_guarded_kernels_bitwise_equal(M, N, K, act, fmt):
    A, B, bias = operands(M, N, K, 6, K, N, fmt)
    C1 = run(A, B, bias, M, N, K, K, N, N, act, fmt, path=gr.GR_PATH_TILE)
    C2 = run(A, B, bias, M, N, K, K, N, N, act, fmt, path=gr.GR_PATH_TILE_EDGE)
    assert np.array_equal(C1, C2)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_k_zero_gives_act_of_bias(fmt):
    M, N = 40, 72
    _, _, bias = operands(1, N, 1, 7, 1, N, fmt)
    for act in ACTS:
        C = run(np.zeros((M, 1), np.uint16), np.zeros((1, N), np.uint16), bias, M, N, 0, 1, N, N, act, fmt)
        ref = oracle.gemm_relu_full(np.zeros((M, 1), np.uint16), np.zeros((1, N), np.uint16), M=M, N=N, K=0, lda=1,
                                    ldb=N, fmt=fmt, bias=bias, act=act)
        assert_parity(C[:M * N].reshape(M, N), ref, "K=0 %s" % act, fmt=fmt)


@pytest.mark.parametrize("offset", [1, 3])
def test_unaligned_bias_pointer(offset):
    M, N, K = 520, 264, 128
    A, B, bias = operands(M, N, K, 8, K, N, "f16")
    C = run(A, B, bias, M, N, K, K, N, N, "silu", "f16", bias_offset=offset)
    ref = oracle.gemm_relu_full(A, B, bias=bias, act="silu")
    assert_parity(C[:M * N].reshape(M, N), ref, "bias offset %d" % offset)


def test_large_magnitudes_saturate():
    """Sums of +-50 and more: sigmoid and tanh reach +-1 and 0 exactly, GELU
    and SiLU give x or 0, the identity keeps the value."""
    M, N, K = 256, 256, 64
    rng = np.random.default_rng(9)
    a = rng.choice([-1.0, 1.0], size=(M, K))
    b = rng.choice([-1.0, 1.0], size=(K, N)) * 2.0
    A = a.astype(np.float16).view(np.uint16)
    B = b.astype(np.float16).view(np.uint16)
    for act in ("sigmoid", "tanh", "gelu", "silu", "none"):
        C = run(A, B, None, M, N, K, K, N, N, act, "f16")[:M * N].reshape(M, N)
        ref = oracle.gemm_relu_full(A, B, act=act)
        assert_parity(C, ref, "saturate %s" % act)
        x = a @ b
        if act in ("sigmoid", "tanh"):
            big = np.abs(x) >= 20
            assert np.array_equal(as_f64(C)[big], as_f64(ref)[big])


def test_tensor_wrapper():
    t = pytest.importorskip("torch")
    M, N, K = 300, 200, 128
    for fmt, dt in (("f16", t.float16), ("bf16", t.bfloat16)):
        A, B, bias = operands(M, N, K, 10, K, N, fmt)
        a = to_dev(A).view(dt).reshape(M, K)
        b = to_dev(B).view(dt).reshape(K, N)
        bb = to_dev(bias).view(dt)
        c = gr.gemm_bias_act(a, b, bb, act="gelu_tanh")
        t.cuda.synchronize()
        assert c.dtype == dt
        assert_parity(c.view(t.int16).cpu().numpy().view(np.uint16),
                      oracle.gemm_relu_full(A, B, fmt=fmt, bias=bias, act="gelu_tanh"), "wrapper " + fmt, fmt=fmt)
    with pytest.raises(ValueError):
        gr.gemm_bias_act(a, b, bb[:10], act="gelu")


# ---- workspace paths: packed operands and the split passes ------------------------

WS_CASES = [
    # M, N, K, lda, ldb, ldc, path
    (700, 500, 322, 322, 501, 500, gr.GR_PATH_TILE_PACKED),   # misaligned pitches, K % 32 != 0
    (8, 4096, 8192, 8192, 4096, 4096, gr.GR_PATH_SMALL_M_SPLIT),
    (13, 1000, 1000, 1000, 1000, 1001, gr.GR_PATH_SMALL_M_SPLIT),
    (300, 520, 4096, 4104, 520, 521, gr.GR_PATH_TILE_SPLIT),
    (128, 128, 1024, 1024, 128, 128, gr.GR_PATH_TILE_SPLIT),
]


def run_ws(A, B, bias, M, N, K, lda, ldb, ldc, act, fmt, path):
    import torch as t
    st, size = gr.gemm_relu_f16_workspace_size(M, N, K, 0x100000, lda, 0x200000000000, ldb, 0x400000000000, ldc)
    assert st == gr.GR_OK
    size = max(size, 4 << 20)  # the forced paths may need more than the planner's own choice
    ws = t.full((size,), 0x5A, dtype=t.uint8, device="cuda")  # dirty: every path must overwrite what it reads
    dA, dB = to_dev(A), to_dev(B)
    db = to_dev(bias) if bias is not None else None
    dC = full_dev((M * ldc + 8,), SENTINEL)
    log("epi ws %s %s M=%d N=%d K=%d path=%s" % (fmt, act, M, N, K, path))
    st = gr.gemm_bias_act_ws(M, N, K, dA.data_ptr(), lda, dB.data_ptr(), ldb,
                             db.data_ptr() if db is not None else None, gr.ACT_CODES[act], dC.data_ptr(), ldc,
                             gr.GR_FMT_BF16 if fmt == "bf16" else gr.GR_FMT_F16, ws.data_ptr(), ws.numel(),
                             t.cuda.current_stream().cuda_stream, path)
    t.cuda.synchronize()
    assert st == gr.GR_OK, gr.gemm_relu_status_string(st)
    return from_dev(dC)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("act", ["relu", "gelu", "none"])
@pytest.mark.parametrize("case", WS_CASES, ids=["packed", "smallm-split", "smallm-split-guarded", "tile-split",
                                                "tile-split-one-tile"])
def test_workspace_paths(case, act, fmt):
    """Bias + activation (and bfloat16) through the packed copy and the two
    split-K passes: the epilogue runs once, on the complete sum."""
    M, N, K, lda, ldb, ldc, path = case
    A, B, bias = operands(M, N, K, 11 + M, lda, ldb, fmt)
    Cflat = run_ws(A, B, bias, M, N, K, lda, ldb, ldc, act, fmt, path)
    C = Cflat[:M * ldc].reshape(M, ldc)
    ref = oracle.gemm_relu_full(A, B, M=M, N=N, K=K, lda=lda, ldb=ldb, fmt=fmt, bias=bias, act=act)
    assert_parity(C[:, :N], ref, "ws %s %s %s" % (fmt, act, path), fmt=fmt)
    assert np.all(C[:, N:] == SENTINEL) and np.all(Cflat[M * ldc:] == SENTINEL)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_planner_picks_workspace_paths(fmt):
    """With a workspace the planner's own choice (path -1) matches the
    forced runs above for the narrow small-M shape."""
    M, N, K = 8, 4096, 8192
    A, B, bias = operands(M, N, K, 3, K, N, fmt)
    st, p = gr.gemm_relu_f16_plan_ws(M, N, K, 0x100000, K, 0x200000000000, N, 0x400000000000, N, 1 << 24)
    assert p["path"] == gr.GR_PATH_SMALL_M_SPLIT
    C = run_ws(A, B, bias, M, N, K, K, N, N, "silu", fmt, -1)[:M * N].reshape(M, N)
    assert_parity(C, oracle.gemm_relu_full(A, B, fmt=fmt, bias=bias, act="silu"), "ws auto", fmt=fmt)


def test_bf16_tensor_wrapper_workspace():
    t = pytest.importorskip("torch")
    M, N, K = 700, 500, 322
    A, B, _ = operands(M, N, K, 17, K, N, "bf16")
    a = to_dev(A).view(t.bfloat16).reshape(M, K)
    b = to_dev(B).view(t.bfloat16).reshape(K, N)
    c = gr.gemm_relu(a, b, path=gr.GR_PATH_TILE_PACKED, workspace=t.empty(1 << 22, dtype=t.uint8, device="cuda"))
    t.cuda.synchronize()
    assert_parity(c.view(t.int16).cpu().numpy().view(np.uint16), oracle.gemm_relu_full(A, B, fmt="bf16"),
                  "bf16 packed wrapper", fmt="bf16")
