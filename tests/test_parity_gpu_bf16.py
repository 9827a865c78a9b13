"""GPU parity of the bfloat16 entry points against the CPU oracle.

Same bar as the fp16 paths: |gpu - oracle| <= 1e-2 + 1e-2 |oracle| for every
checked element ("Writing high-performance kernels in TileLang", section
"Writing a GEMM", verifies its GEMM with that tolerance); one bfloat16 ulp is
at most 2^-7 < 1e-2 of the value, so two fp32 sums that round to neighbouring
bfloat16 values still pass, while a wrong operand format, a lost term or a
missing ReLU does not. Closed forms whose rounding is worked out by hand are
checked bit for bit. Every kernel the bfloat16 calls can reach runs here: the
256 x 256 pipelined kernels (64-deep and 32-deep K steps), the 128 x 128 one,
each with whole and partial tiles, the guarded kernel with 16-, 4- and 2-byte
operand loads, and the small-M kernel with and without guards.
"""
import numpy as np
import pytest

import dense_gemm_epilogue_tiled_amd as gr
import oracle
import synth
from gpu_util import as_f64, assert_parity, edge_indices, from_dev, full_dev, log, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("oracle_lib")]

FMT = "bf16"
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


SENTINEL = 0x7FC1  # a NaN in bfloat16: any survivor in the window was never written
ONE = 0x3F80


def call_bf16(M, N, K, dA, lda, dB, ldb, dC, ldc, path=None, offsets=(0, 0, 0)):
    import torch as t
    a = dA.data_ptr() + 2 * offsets[0] if dA is not None else 0
    b = dB.data_ptr() + 2 * offsets[1] if dB is not None else 0
    c = dC.data_ptr() + 2 * offsets[2] if dC is not None else 0
    s = t.cuda.current_stream().cuda_stream
    if path is None:
        st = gr.gemm_relu_bf16(M, N, K, a, lda, b, ldb, c, ldc, s)
    else:
        st = gr.gemm_relu_bf16_forced(M, N, K, a, lda, b, ldb, c, ldc, s, path)
    t.cuda.synchronize()
    return st


def run(A, B, M, N, K, lda=None, ldb=None, ldc=None, path=None, offsets=(0, 0, 0), c_rows=None):
    """Flat C buffer (c_rows x ldc + tail, prefilled with SENTINEL) after the call."""
    lda = max(K, 1) if lda is None else lda
    ldb = max(N, 1) if ldb is None else ldb
    ldc = max(N, 1) if ldc is None else ldc
    dA = to_dev(A) if A.size else None
    dB = to_dev(B) if B.size else None
    rows = M if c_rows is None else c_rows
    dC = full_dev((rows * ldc + offsets[2] + 8,), SENTINEL)
    log("bf16 M=%d N=%d K=%d lda=%d ldb=%d ldc=%d path=%s offsets=%s" % (M, N, K, lda, ldb, ldc, path, offsets))
    st = call_bf16(M, N, K, dA, lda, dB, ldb, dC, ldc, path=path, offsets=offsets)
    assert st == gr.GR_OK, gr.gemm_relu_status_string(st)
    return from_dev(dC)


def window(Cflat, M, N, ldc, off=0):
    return Cflat[off:off + M * ldc].reshape(M, ldc)[:, :N]


def plan_path(M, N, K, lda, ldb, ldc):
    st, p = gr.gemm_relu_f16_plan(M, N, K, 0x100000, lda, 0x200000000000, ldb, 0x400000000000, ldc)
    assert st == gr.GR_OK
    return p


def operands(M, N, K, seed, lda=None, ldb=None, b_scale=None):
    return synth.random_operands(M, N, K, seed=seed, lda=lda, ldb=ldb, b_scale=b_scale, fmt=FMT)


def ref_full(A, B, M, N, K, lda, ldb):
    return oracle.gemm_relu_full(A, B, M=M, N=N, K=K, lda=lda, ldb=ldb, fmt=FMT)


def no_nan_inf(C):
    return not np.any((C & 0x7F80) == 0x7F80)


# ---- the five workloads, with bfloat16 operands ---------------------------------

@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_parity(name):
    w = synth.WORKLOADS[name]
    A, B = synth.operands(w, fmt=FMT)
    M, N, K = w.M, w.N, w.K
    plan = plan_path(M, N, K, K, N, N)
    log("%s bf16 plan=%s" % (name, plan))
    dA, dB = to_dev(A), to_dev(B)
    dC = full_dev((M * N,), SENTINEL)
    assert call_bf16(M, N, K, dA, K, dB, N, dC, N) == gr.GR_OK
    C = from_dev(dC).reshape(M, N)
    del dA, dB, dC
    assert no_nan_inf(C)
    if w.check == "full":
        rep = assert_parity(C, oracle.gemm_relu_full(A, B, fmt=FMT), name, fmt=FMT)
    else:
        bm, bn = max(plan["block_m"], 1), max(plan["block_n"], 1)
        ii, jj = synth.sample_indices(M, N, 4096, w.seed)
        rep = assert_parity(C[ii, jj], oracle.gemm_relu_elems(A, B, ii, jj, fmt=FMT), name + " sampled", fmt=FMT)
        rows = edge_indices(M, bm)
        cols = edge_indices(N, bn)
        assert_parity(C[rows, :], oracle.gemm_relu_rows(A, B, rows, fmt=FMT), name + " rows", fmt=FMT)
        assert_parity(C[:, cols].T, oracle.gemm_relu_cols(A, B, cols, fmt=FMT), name + " cols", fmt=FMT)
    log("%s bf16 parity %s" % (name, rep))
    assert not np.any(C & 0x8000)


# ---- each kernel, whole and partial tiles ------------------------------------------

KERNEL_CASES = [
    # M, N, K, lda, ldb, ldc, expected path, what it exercises
    (512, 768, 256, 256, 768, 768, gr.GR_PATH_TILE, "128x128 whole"),
    (300, 250, 96, 104, 256, 251, gr.GR_PATH_TILE, "128x128 partial, rows clamped"),
    (65, 264, 64, 72, 264, 265, gr.GR_PATH_TILE, "128x128, one row of tiles"),
    (4096, 2304, 256, 256, 2304, 2304, gr.GR_PATH_TILE, "256x256 64-deep whole"),
    (2400, 4000, 128, 128, 4008, 4001, gr.GR_PATH_TILE, "256x256 64-deep partial"),
    (4096, 2304, 160, 160, 2304, 2304, gr.GR_PATH_TILE, "256x256 32-deep whole"),
    (2400, 4000, 96, 96, 4000, 4001, gr.GR_PATH_TILE, "256x256 32-deep partial"),
    (300, 270, 100, 109, 277, 273, gr.GR_PATH_TILE_EDGE, "guarded, odd pitches"),
    (257, 130, 70, 70, 130, 130, gr.GR_PATH_TILE_EDGE, "guarded, 4-byte rows"),
    (520, 260, 200, 200, 264, 261, gr.GR_PATH_TILE_EDGE, "guarded, K % 32 != 0, 16-byte rows"),
    (8, 16384, 8192, 8192, 16384, 16384, gr.GR_PATH_SMALL_M, "small-M whole"),
    (16, 1000, 1000, 1000, 1000, 1000, gr.GR_PATH_SMALL_M, "small-M guarded"),
    (5, 128, 8200, 8200, 128, 129, gr.GR_PATH_SMALL_M, "small-M long K tail"),
    (1, 100, 96, 96, 104, 100, gr.GR_PATH_SMALL_M, "small-M one row"),
    (40, 1000, 512, 512, 1000, 1001, gr.GR_PATH_SMALL_M, "small-M four row blocks"),
    (20, 4096, 300, 304, 4096, 4096, gr.GR_PATH_SMALL_M, "small-M two row blocks, K tail"),
]


@pytest.mark.parametrize("M,N,K,lda,ldb,ldc,path,what", KERNEL_CASES, ids=[c[-1] for c in KERNEL_CASES])
def test_kernel_parity(M, N, K, lda, ldb, ldc, path, what):
    """Full comparison with the oracle, padding of A and B poisoned with the
    largest finite bfloat16, C canaries beside and below the window."""
    planned = plan_path(M, N, K, lda, ldb, ldc)["path"]
    assert planned_agrees(planned, path), (planned, path)
    A, B = operands(M, N, K, seed=M * 7 + N + K, lda=lda, ldb=ldb, b_scale=K ** -0.5)
    extra = 2
    Cflat = run(A, B, M, N, K, lda, ldb, ldc, path=path, c_rows=M + extra)
    C = Cflat[:M * ldc].reshape(M, ldc)
    assert no_nan_inf(C[:, :N])
    assert_parity(C[:, :N], ref_full(A, B, M, N, K, lda, ldb), what, fmt=FMT)
    assert np.all(C[:, N:] == SENTINEL) and np.all(Cflat[M * ldc:] == SENTINEL)


@pytest.mark.parametrize("M,N,K", [(512, 768, 256), (4096, 2304, 256), (4096, 2304, 96), (300, 256, 96)])
def test_tile_and_edge_paths_bitwise_equal(M, N, K):
    """The pipelined and guarded kernels run the same MFMA sequence in the same
    k order, so their bfloat16 results agree bit for bit."""
    A, B = operands(M, N, K, seed=K + 1)
    C1 = run(A, B, M, N, K, path=gr.GR_PATH_TILE)
    C2 = run(A, B, M, N, K, path=gr.GR_PATH_TILE_EDGE)
    assert np.array_equal(C1, C2)


@pytest.mark.parametrize("offs", [(1, 0, 0), (0, 1, 0), (2, 2, 0), (3, 5, 7)])
def test_unaligned_base_pointers(offs):
    """Base pointers off 16-byte alignment select the guarded kernel's 4-byte
    and 2-byte load forms."""
    M, N, K = 200, 136, 96
    A, B = operands(M, N, K, seed=sum(offs) + 3)
    Ap = np.concatenate([np.zeros(offs[0], np.uint16), A.ravel(), np.zeros(8, np.uint16)])
    Bp = np.concatenate([np.zeros(offs[1], np.uint16), B.ravel(), np.zeros(8, np.uint16)])
    Cflat = run(Ap, Bp, M, N, K, K, N, N, offsets=offs)
    C = Cflat[offs[2]:offs[2] + M * N].reshape(M, N)
    assert_parity(C, oracle.gemm_relu_full(A, B, fmt=FMT), "offsets %s" % (offs,), fmt=FMT)
    assert np.all(Cflat[:offs[2]] == SENTINEL) and np.all(Cflat[offs[2] + M * N:] == SENTINEL)


# ---- closed forms, bit for bit ----------------------------------------------------

@pytest.mark.parametrize("M,N,K,expect,path", [
    (512, 512, 8224, 8192.0, gr.GR_PATH_TILE),        # 8192 + 32: tie between 8192 and 8256 -> even 8192
    (4096, 512, 8288, 8320.0, gr.GR_PATH_TILE),       # 8192 + 96: tie between 8256 and 8320 -> even 8320
    (300, 130, 2050, 2048.0, gr.GR_PATH_TILE_EDGE),   # spacing 16 above 2048: rounds down
    (300, 130, 259, 260.0, gr.GR_PATH_TILE_EDGE),     # spacing 2 above 256: tie -> even 260
    (8, 256, 8224, 8192.0, gr.GR_PATH_SMALL_M),
    (5, 104, 2072, 2080.0, gr.GR_PATH_SMALL_M),       # tie between 2064 and 2080 -> even 2080
])
def test_all_ones_rounding(M, N, K, expect, path):
    """Sum of K ones is exactly K in fp32 on every path; the kernel's final
    rounding to bfloat16 must land where the worked cases say."""
    planned = plan_path(M, N, K, K, N, N)["path"]
    assert planned_agrees(planned, path), (planned, path)
    A = np.full((M, K), ONE, dtype=np.uint16)
    B = np.full((K, N), ONE, dtype=np.uint16)
    C = window(run(A, B, M, N, K, path=path), M, N, N)
    assert np.all(as_f64(C, FMT) == expect)


@pytest.mark.parametrize("M,K,path", [(512, 256, gr.GR_PATH_TILE), (300, 100, gr.GR_PATH_TILE_EDGE),
                                      (12, 256, gr.GR_PATH_SMALL_M)])
def test_diagonal_B_exact_rounding(M, K, path):
    """B = diag(d): each result is one exact fp32 product rounded once."""
    A, _ = operands(M, K, K, seed=31)
    rng = np.random.default_rng(32)
    d = oracle.f32_to_bf16((rng.standard_normal(K) * 3).astype(np.float32))
    B = np.zeros((K, K), dtype=np.uint16)
    B[np.arange(K), np.arange(K)] = d
    C = window(run(A, B, M, K, K, path=path), M, K, K)
    assert np.array_equal(C, oracle.gemm_relu_full(A, B, fmt=FMT))


@pytest.mark.parametrize("path", [gr.GR_PATH_TILE, gr.GR_PATH_TILE_EDGE, gr.GR_PATH_SMALL_M])
def test_rank1_powers_of_two_beyond_fp16_range(path):
    """A[i,k] = 2^p_i, B[k,j] = 2^q_j with exponents from -60 to +50: exact,
    and far outside what fp16 could hold, so a stray fp16 step shows."""
    M = 16 if path == gr.GR_PATH_SMALL_M else 256
    N, K = 256, 64
    p = (np.arange(M) % 12) * 5 - 30
    q = (np.arange(N) % 8) * 5 - 30
    A = oracle.f32_to_bf16(np.repeat((2.0 ** p)[:, None], K, axis=1).astype(np.float32))
    B = oracle.f32_to_bf16(np.repeat((2.0 ** q)[None, :], K, axis=0).astype(np.float32))
    C = window(run(A, B, M, N, K, path=path), M, N, N)
    assert np.array_equal(as_f64(C, FMT), K * 2.0 ** (p[:, None] + q[None, :]))


@pytest.mark.parametrize("path", [gr.GR_PATH_TILE, gr.GR_PATH_TILE_EDGE, gr.GR_PATH_SMALL_M])
def test_negative_products_give_plus_zero(path):
    """-1 times 1 summed: the fp32 sum is negative, ReLU gives +0 (0x0000)."""
    M = 8 if path == gr.GR_PATH_SMALL_M else 256
    N, K = 256, 96
    A = np.full((M, K), 0xBF80, dtype=np.uint16)
    B = np.full((K, N), ONE, dtype=np.uint16)
    assert np.all(window(run(A, B, M, N, K, path=path), M, N, N) == 0)


def test_k_zero_writes_zeros():
    M, N = 40, 72
    C = run(np.zeros((M, 1), np.uint16), np.zeros((1, N), np.uint16), M, N, 0, lda=1, ldb=N)
    assert np.all(window(C, M, N, N) == 0)


# ---- seeded random problems --------------------------------------------------------

def _fuzz_cases(count, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        mode = i % 4
        if mode == 0:    # aligned: pipelined kernels
            M = int(rng.integers(1, 900))
            N = int(rng.integers(1, 120)) * 8
            K = int(rng.integers(1, 20)) * 32
        elif mode == 1:  # anything: mostly guarded
            M, N, K = (int(x) for x in rng.integers(1, 700, size=3))
        elif mode == 2:  # small M, 16-byte rows
            M = int(rng.integers(1, 17))
            N = int(rng.integers(1, 250)) * 8
            K = int(rng.integers(1, 400)) * 8
        else:            # larger aligned, 256 tiles
            M = int(rng.integers(1000, 3000))
            N = int(rng.integers(100, 400)) * 8
            K = int(rng.integers(1, 6)) * 64
        out.append((i, M, N, K, int(rng.integers(1 << 30))))
    return out


@pytest.mark.parametrize("case", _fuzz_cases(24, 77), ids=lambda c: "bf16fuzz%d" % c[0])
def test_random_problems_against_oracle(case):
    i, M, N, K, s = case
    A, B = operands(M, N, K, seed=s, b_scale=max(K, 1) ** -0.5)
    plan = plan_path(M, N, K, K, N, N)
    log("bf16 fuzz %d plan %s" % (i, plan))
    C = window(run(A, B, M, N, K), M, N, N)
    assert_parity(C, oracle.gemm_relu_full(A, B, fmt=FMT), "fuzz %d %s" % (i, (M, N, K)), fmt=FMT)


# ---- tensor convenience -------------------------------------------------------------

def test_tensor_wrapper_bfloat16():
    t = pytest.importorskip("torch")
    M, N, K = 300, 200, 128
    A, B = operands(M, N, K, seed=93)
    a = to_dev(A).view(t.bfloat16).reshape(M, K)
    b = to_dev(B).view(t.bfloat16).reshape(K, N)
    c = gr.gemm_relu(a, b)
    t.cuda.synchronize()
    assert c.dtype == t.bfloat16
    assert_parity(c.view(t.int16).cpu().numpy().view(np.uint16), oracle.gemm_relu_full(A, B, fmt=FMT),
                  "bf16 wrapper", fmt=FMT)
    with pytest.raises(TypeError):
        gr.gemm_relu(a, b.to(t.float16))
