"""Seeded random problems for the low-precision entry points -- gemm_fp8_bt
(with and without a workspace), gemm_mxfp8_bt and gemm_mxfp4_bt -- against
the oracle, whatever path the planner picks: random shapes (K a multiple of
32 for the MX calls), pitches, pointer offsets, activations, bias and output
format.  Bar as everywhere (|gpu - oracle| <= 1e-2 + 1e-2 |oracle|,
"Writing high-performance kernels in TileLang", section "Writing a GEMM"),
plus the allowance for the fp8 instructions' own summation (gpu_util
f8_extra: 2^-16 of the absolute sum of the dequantised products, from the
measured 2^-17.6); C's padding and the bytes around it keep their sentinel.
"""
import numpy as np
import pytest

import dense_gemm_epilogue_tiled_amd as gr
import oracle
import synth
from gpu_util import assert_parity, f8_extra, from_dev, full_dev, log

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("oracle_lib")]

SENTINEL = 0x7FC1
FMTS = {"f16": gr.GR_FMT_F16, "bf16": gr.GR_FMT_BF16}
ACTS = list(gr.ACT_CODES)


def dev8(x, offset):
    import torch as t
    flat = np.concatenate([np.zeros(offset, np.uint8), np.ascontiguousarray(x).ravel(), np.zeros(32, np.uint8)])
    return t.from_numpy(flat).to("cuda")


def bias_for(N, fmt, seed):
    import torch as t
    g = t.Generator().manual_seed(seed)
    return t.randn(N, generator=g).to(t.bfloat16 if fmt == "bf16" else t.float16).view(t.int16).numpy() \
        .view(np.uint16)


def _cases(kind, count, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        aligned = i % 3 != 2
        long_k = kind == "fp8" and i % 6 == 4  # few tiles, long K: the split path when a workspace is given
        M = int(rng.choice([rng.integers(1, 17), rng.integers(17, 300), rng.integers(300, 1100)]))
        N = int(rng.integers(1, 900))
        if long_k:
            M, N = int(rng.integers(17, 300)), int(rng.integers(1, 600))
            K = int(64 * rng.integers(100, 160))
        elif kind == "fp8":
            K = int(64 * rng.integers(1, 80)) if aligned else int(rng.integers(1, 2000))
        else:
            K = int(128 * rng.integers(1, 24)) if aligned else int(32 * rng.integers(1, 60))
        row = K // 2 if kind == "mxfp4" else K
        pad = (lambda: 16 * int(rng.integers(0, 2))) if aligned else (lambda: int(rng.integers(0, 9)))
        lda, ldbt = row + pad(), row + pad()
        kb = K // 32
        ldsa = kb + (4 * int(rng.integers(0, 2)) if aligned else int(rng.integers(0, 3)))
        ldsb = kb + (4 * int(rng.integers(0, 2)) if aligned else int(rng.integers(0, 3)))
        ldc = N + int(rng.integers(0, 9))
        offs = [0, 0, 0, 0] if aligned else [int(rng.integers(0, 16)) for _ in range(4)]
        fmt = ["f16", "bf16"][int(rng.integers(0, 2))]
        act = ACTS[int(rng.integers(0, len(ACTS)))]
        with_bias = bool(rng.integers(0, 2))
        use_ws = bool(rng.integers(0, 2)) or long_k
        out.append((i, M, N, K, lda, ldbt, ldsa, ldsb, ldc, offs, fmt, act, with_bias, use_ws))
    return out


def _run(kind, case):
    import torch as t
    i, M, N, K, lda, ldbt, ldsa, ldsb, ldc, offs, fmt, act, with_bias, use_ws = case
    seed = 5000 + 97 * i + (0 if kind == "fp8" else 31 if kind == "mxfp8" else 57)
    SA = SB = None
    if kind == "fp8":
        A, Bt = synth.fp8_operands(M, N, K, seed=seed, lda=lda, ldbt=ldbt, scale_b=2.0 * max(K, 1) ** -0.5)
    elif kind == "mxfp8":
        A, SA, Bt, SB = synth.mx_operands(M, N, K, seed=seed, lda=lda, ldbt=ldbt, ldsa=ldsa, ldsb=ldsb)
    else:
        A, SA, Bt, SB = synth.mxfp4_operands(M, N, K, seed=seed, lda=lda, ldbt=ldbt, ldsa=ldsa, ldsb=ldsb)
    bias = bias_for(N, fmt, seed) if with_bias else None
    dA, dB = dev8(A, offs[0]), dev8(Bt, offs[1])
    a, b = dA.data_ptr() + offs[0], dB.data_ptr() + offs[1]
    db = t.from_numpy(bias.view(np.int16)).to("cuda") if bias is not None else None
    bp = db.data_ptr() if db is not None else None
    dC = full_dev((M * ldc + 16,), SENTINEL)
    s = t.cuda.current_stream().cuda_stream
    code = gr.ACT_CODES[act]
    if kind == "fp8":
        sa, sb = 0.5, 0.75
        st, size = gr.gemm_fp8_bt_workspace_size(M, N, K, a, lda, b, ldbt, dC.data_ptr(), ldc)
        assert st == gr.GR_OK
        ws = t.empty(max(size, 256), dtype=t.uint8, device="cuda") if use_ws and size else None
        wb = size if ws is not None else 0
        st, p = gr.gemm_fp8_bt_plan_ws(M, N, K, a, lda, b, ldbt, bp, code, dC.data_ptr(), ldc, FMTS[fmt], wb)
        log("fuzz-fp8 %d M=%d N=%d K=%d ld=%d,%d,%d offs=%s %s %s bias=%s ws=%d path=%s" %
            (i, M, N, K, lda, ldbt, ldc, offs[:2], fmt, act, with_bias, wb, p["path_name"]))
        st = gr.gemm_fp8_bt_ws(M, N, K, a, lda, b, ldbt, sa, sb, bp, code, dC.data_ptr(), ldc, FMTS[fmt],
                               ws.data_ptr() if ws is not None else None, wb, s)
        ref = (lambda: oracle.gemm_fp8_bt_full(A, Bt, sa, sb, fmt, bias, act, M=M, N=N, K=K, lda=lda, ldbt=ldbt))
    else:
        dSA, dSB = dev8(SA, offs[2]), dev8(SB, offs[3])
        pa, pb = dSA.data_ptr() + offs[2], dSB.data_ptr() + offs[3]
        call = gr.gemm_mxfp8_bt if kind == "mxfp8" else gr.gemm_mxfp4_bt
        plan = gr.gemm_mxfp8_bt_plan if kind == "mxfp8" else gr.gemm_mxfp4_bt_plan
        st, p = plan(M, N, K, a, lda, pa, ldsa, b, ldbt, pb, ldsb, bp, code, dC.data_ptr(), ldc, FMTS[fmt])
        log("fuzz-%s %d M=%d N=%d K=%d ld=%d,%d,%d,%d,%d offs=%s %s %s bias=%s path=%s" %
            (kind, i, M, N, K, lda, ldbt, ldsa, ldsb, ldc, offs, fmt, act, with_bias, p["path_name"]))
        st = call(M, N, K, a, lda, pa, ldsa, b, ldbt, pb, ldsb, bp, code, dC.data_ptr(), ldc, FMTS[fmt], s)
        f = oracle.gemm_mxfp8_bt_full if kind == "mxfp8" else oracle.gemm_mxfp4_bt_full
        ref = (lambda: f(A, SA, Bt, SB, fmt, bias, act, M=M, N=N, K=K, lda=lda, ldsa=ldsa, ldbt=ldbt, ldsb=ldsb))
    t.cuda.synchronize()
    assert st == gr.GR_OK, gr.gemm_relu_status_string(st)
    Cflat = from_dev(dC)
    C = Cflat[:M * ldc].reshape(M, ldc)
    extra = f8_extra(_abs_sums(kind, case, A, SA, Bt, SB))
    assert_parity(C[:, :N], ref(), "fuzz-%s %d" % (kind, i), fmt=fmt, extra=extra)
    assert np.all(C[:, N:] == SENTINEL) and np.all(Cflat[M * ldc:] == SENTINEL)


def _abs_sums(kind, case, A, SA, Bt, SB):
    """sum_k |a_k b_k| of the dequantised operands, M x N (float64)."""
    _, M, N, K = case[:4]
    if kind == "mxfp4":
        def dec(P):
            c = np.empty((P.shape[0], K), np.uint8)
            c[:, 0::2], c[:, 1::2] = P[:, :K // 2] & 15, P[:, :K // 2] >> 4
            return np.abs(oracle.e2m1_to_f32(c).astype(np.float64))
    else:
        def dec(P):
            return np.abs(oracle.e4m3_to_f32(P[:, :K]).astype(np.float64))
    a, b = dec(A), dec(Bt)
    if kind == "fp8":
        return 0.5 * 0.75 * (a @ b.T)
    a = a * np.repeat(oracle.e8m0_to_f64(SA[:, :K // 32]), 32, axis=1)
    b = b * np.repeat(oracle.e8m0_to_f64(SB[:, :K // 32]), 32, axis=1)
    return a @ b.T


@pytest.mark.parametrize("case", _cases("fp8", 18, 71), ids=lambda c: "fp8-%d" % c[0])
def test_fp8_random(case):
    _run("fp8", case)


@pytest.mark.parametrize("case", _cases("mxfp8", 18, 72), ids=lambda c: "mxfp8-%d" % c[0])
def test_mxfp8_random(case):
    _run("mxfp8", case)


@pytest.mark.parametrize("case", _cases("mxfp4", 18, 73), ids=lambda c: "mxfp4-%d" % c[0])
def test_mxfp4_random(case):
    _run("mxfp4", case)
