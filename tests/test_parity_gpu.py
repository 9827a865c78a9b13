"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar: for every checked element |gpu - oracle| <= 1e-2 + 1e-2 |oracle| (the
tolerance the GEMM+ReLU listings verify with, "Writing high-performance
kernels in TileLang", section "Writing a GEMM"; the blog "TileLang programming
basics", section 6, explains why the reference must accumulate in fp32), no
NaN or Inf, and bit-exact where the closed form is exact.
"""
import numpy as np
import pytest

import dense_gemm_epilogue_tiled_amd as gr
import oracle
import synth
from gpu_util import (as_f64, assert_parity, call, call_ws, edge_indices, from_dev, full_dev, log,
                      to_dev)

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("oracle_lib")]

SENTINEL = 0x7E5A  # a quiet NaN: the kernel never writes NaN, so any survivor was never written


def run_full(A, B, M, N, K, lda=None, ldb=None, ldc=None, path=None, offsets=(0, 0, 0), c_fill=SENTINEL,
             c_rows=None):
    lda = max(K, 1) if lda is None else lda
    ldb = max(N, 1) if ldb is None else ldb
    ldc = max(N, 1) if ldc is None else ldc
    dA = to_dev(A) if A.size else None
    dB = to_dev(B) if B.size else None
    rows = M if c_rows is None else c_rows
    dC = full_dev((rows * ldc + offsets[2] + 8,), c_fill)
    log("M=%d N=%d K=%d lda=%d ldb=%d ldc=%d path=%s offsets=%s" % (M, N, K, lda, ldb, ldc, path, offsets))
    st = call(M, N, K, dA, lda, dB, ldb, dC, ldc, path=path, offsets=offsets)
    assert st == gr.GR_OK, gr.gemm_relu_status_string(st)
    return from_dev(dC)


def window(Cflat, M, N, ldc, off=0):
    return Cflat[off:off + M * ldc].reshape(M, ldc)[:, :N]


# ---- the five workloads, in the launch configuration the benchmark times ----

@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_parity(name):
    w = synth.WORKLOADS[name]
    A, B = synth.operands(w)
    M, N, K = w.M, w.N, w.K
    st, plan = gr.gemm_relu_f16_plan(M, N, K, 0x100000, K, 0x200000000000, N, 0x400000000000, N)
    log("%s plan=%s" % (name, plan))
    dA, dB = to_dev(A), to_dev(B)
    dC = full_dev((M * N,), SENTINEL)
    assert call(M, N, K, dA, K, dB, N, dC, N) == gr.GR_OK
    C = from_dev(dC).reshape(M, N)
    del dA, dB, dC
    # every element written, none NaN/Inf (the sentinel is a NaN)
    assert not np.any((C & 0x7C00) == 0x7C00)
    if w.check == "full":
        ref = oracle.gemm_relu_full(A, B)
        rep = assert_parity(C, ref, name)
    else:
        bm, bn = max(plan["block_m"], 1), max(plan["block_n"], 1)
        ii, jj = synth.sample_indices(M, N, 4096, w.seed)
        rep = assert_parity(C[ii, jj], oracle.gemm_relu_elems(A, B, ii, jj), name + " sampled")
        rows = edge_indices(M, bm)
        cols = edge_indices(N, bn)
        # one seeded interior tile boundary as well
        rng = np.random.default_rng(w.seed)
        tr = int(rng.integers(1, max(2, (M - 1) // bm))) * bm
        tc = int(rng.integers(1, max(2, (N - 1) // bn))) * bn
        rows = sorted(set(rows) | {r for r in (tr - 1, tr) if 0 <= r < M})
        cols = sorted(set(cols) | {c for c in (tc - 1, tc) if 0 <= c < N})
        assert_parity(C[rows, :], oracle.gemm_relu_rows(A, B, rows), name + " rows")
        assert_parity(C[:, cols].T, oracle.gemm_relu_cols(A, B, cols), name + " cols")
    log("%s parity %s" % (name, rep))
    # C >= 0 everywhere, no -0
    assert not np.any(C & 0x8000)


# ---- shapes that do not fill tiles --------------------------------------------

SWEEP = [1, 2, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]


def _sweep_cases(count, seed):
    rng = np.random.default_rng(seed)
    cases = set()
    while len(cases) < count:
        cases.add(tuple(int(x) for x in rng.choice(SWEEP, 3)))
    return sorted(cases)


@pytest.mark.parametrize("M,N,K", _sweep_cases(60, 7))
def test_tiny_shape_sweep(M, N, K):
    A, B = synth.random_operands(M, N, K, seed=M * 7919 + N * 131 + K)
    C = window(run_full(A, B, M, N, K), M, N, N)
    assert_parity(C, oracle.gemm_relu_full(A, B), "sweep %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K", [(300, 520, 200), (257, 257, 257), (513, 255, 130), (1000, 700, 333)])
def test_multi_tile_ragged(M, N, K):
    A, B = synth.random_operands(M, N, K, seed=M + N + K)
    C = window(run_full(A, B, M, N, K), M, N, N)
    assert_parity(C, oracle.gemm_relu_full(A, B), "ragged %dx%dx%d" % (M, N, K))


# ---- guards: poisoned padding, canaries, unaligned rows -----------------------

@pytest.mark.parametrize("M,N,K,pa,pb,pc", [
    (300, 270, 100, 9, 5, 3),      # odd pitches: element loads
    (512, 512, 128, 8, 8, 8),      # aligned pitches larger than the rows
    (260, 300, 70, 2, 2, 4),       # even pitches: 4-byte loads
    (8, 1000, 300, 12, 8, 5),      # small-M path with padding
])
def test_poisoned_padding_and_canary(M, N, K, pa, pb, pc):
    lda, ldb, ldc = K + pa, N + pb, N + pc
    A, B = synth.random_operands(M, N, K, seed=41, lda=lda, ldb=ldb)  # padding = 65504
    extra_rows = 3
    Cflat = run_full(A, B, M, N, K, lda=lda, ldb=ldb, ldc=ldc, c_rows=M + extra_rows)
    C = Cflat[:M * ldc].reshape(M, ldc)
    assert_parity(C[:, :N], oracle.gemm_relu_full(A, B, M=M, N=N, K=K, lda=lda, ldb=ldb), "padded")
    assert np.all(C[:, N:] == SENTINEL), "a padding column of C was written"
    assert np.all(Cflat[M * ldc:] == SENTINEL), "a row past M was written"


@pytest.mark.parametrize("offs", [(1, 0, 0), (0, 1, 0), (0, 0, 1), (3, 5, 7)])
def test_unaligned_base_pointers(offs):
    M, N, K = 320, 288, 96
    A, B = synth.random_operands(M, N, K, seed=43)
    Ap = np.concatenate([np.zeros(offs[0], np.uint16), A.ravel()])
    Bp = np.concatenate([np.zeros(offs[1], np.uint16), B.ravel()])
    Cflat = run_full(Ap, Bp, M, N, K, offsets=offs)
    C = Cflat[offs[2]:offs[2] + M * N].reshape(M, N)
    assert_parity(C, oracle.gemm_relu_full(A, B), "offsets %s" % (offs,))
    assert np.all(Cflat[:offs[2]] == SENTINEL)
    assert np.all(Cflat[offs[2] + M * N:] == SENTINEL)


def test_k_zero_writes_zeros():
    M, N = 300, 260
    Cflat = run_full(np.zeros((M, 0), np.uint16), np.zeros((0, N), np.uint16), M, N, 0, lda=1)
    assert np.all(Cflat[:M * N] == 0)
    assert np.all(Cflat[M * N:] == SENTINEL)


def test_empty_problems_launch_nothing():
    dC = full_dev((64,), SENTINEL)
    assert call(0, 8, 8, None, 8, None, 8, None, 8) == gr.GR_OK
    assert call(8, 0, 8, None, 8, None, 1, dC, 1) == gr.GR_OK
    assert np.all(from_dev(dC) == SENTINEL)


# ---- closed forms on the GPU (exact) ------------------------------------------

@pytest.mark.parametrize("M,N,K", [(1024, 1024, 1024), (300, 270, 2050), (8, 16384, 8192), (512, 256, 4096)])
def test_all_ones_exact(M, N, K):
    A = np.full((M, K), 0x3C00, np.uint16)
    B = np.full((K, N), 0x3C00, np.uint16)
    C = window(run_full(A, B, M, N, K), M, N, N)
    assert np.all(as_f64(C) == K)


def test_minus_one_times_one_exact_zero():
    M, N, K = 260, 300, 96
    C = window(run_full(np.full((M, K), 0xBC00, np.uint16), np.full((K, N), 0x3C00, np.uint16), M, N, K), M, N, N)
    assert np.all(C == 0)


@pytest.mark.parametrize("K", [64, 100, 256])
def test_identity_A_exact(K):
    A = np.eye(K, dtype=np.float16).view(np.uint16)
    _, B = synth.random_operands(K, 280, K, seed=K)
    C = window(run_full(A, B, K, 280, K), K, 280, 280)
    assert np.array_equal(C, np.where(B.view(np.float16) > 0, B, np.uint16(0)))


def test_diagonal_B_exact_rounding():
    M, K = 512, 256
    A, _ = synth.random_operands(M, K, K, seed=51)
    d = (np.random.default_rng(52).standard_normal(K) * 3).astype(np.float16)
    B = np.diag(d.astype(np.float64)).astype(np.float16).view(np.uint16)
    C = window(run_full(A, B, M, K, K), M, K, K)
    prod = A.view(np.float16).astype(np.float64) * d.astype(np.float64)[None, :]
    assert np.array_equal(C, np.maximum(prod, 0.0).astype(np.float16).view(np.uint16))


def test_rank1_powers_of_two_exact():
    M, N, K = 256, 256, 512
    p = (np.arange(M) % 9) - 6  # K * 2^(p+q) spans 2^0 .. 2^14: all exact in fp16
    q = (np.arange(N) % 7) - 3
    A = np.repeat((2.0 ** p)[:, None], K, axis=1).astype(np.float16).view(np.uint16)
    B = np.repeat((2.0 ** q)[None, :], K, axis=0).astype(np.float16).view(np.uint16)
    C = window(run_full(A, B, M, N, K), M, N, N)
    assert np.array_equal(as_f64(C), K * 2.0 ** (p[:, None] + q[None, :]))


# ---- invariants ---------------------------------------------------------------

def test_scaling_by_two_bitwise():
    M, N, K = 512, 512, 512
    A, B = synth.random_operands(M, N, K, seed=61)
    A2 = (A.view(np.float16).astype(np.float32) * 2).astype(np.float16).view(np.uint16)
    C1 = as_f64(window(run_full(A, B, M, N, K), M, N, N))
    C2 = as_f64(window(run_full(A2, B, M, N, K), M, N, N))
    normal = (C1 >= 2.0 ** -14) & (C1 * 2 <= 65504)
    assert np.array_equal(C2[normal], 2 * C1[normal])


@pytest.mark.parametrize("M,N,K,path", [(512, 640, 384, None), (4096, 4096, 256, gr.GR_PATH_TILE_PERSISTENT),
                                          (300, 520, 130, None), (8, 4096, 1024, None)])
def test_relu_of_a_minus_relu_of_minus_a_is_the_product(M, N, K, path):
    """ReLU(x) - ReLU(-x) = x: C(A) - C(-A) matches the float64 product A.B
    within the bar at every element, and at every element one of the two is
    +0 (covers the planner's tile, unaligned and small-M paths and the
    persistent loop)."""
    A, B = synth.random_operands(M, N, K, seed=63 + M)
    An = A ^ np.uint16(0x8000)  # -A, exactly (sign bit)
    C1 = as_f64(window(run_full(A, B, M, N, K, path=path), M, N, N))
    C2 = as_f64(window(run_full(An, B, M, N, K, path=path), M, N, N))
    x = A.view(np.float16).astype(np.float64) @ B.view(np.float16).astype(np.float64)
    assert np.all((C1 == 0) | (C2 == 0))
    assert np.all(np.abs((C1 - C2) - x) <= 1e-2 + 1e-2 * np.abs(x))


def test_deterministic_bitwise():
    M, N, K = 1024, 768, 512
    A, B = synth.random_operands(M, N, K, seed=62)
    C1 = run_full(A, B, M, N, K)
    C2 = run_full(A, B, M, N, K)
    assert np.array_equal(C1, C2)


@pytest.mark.parametrize("M,N,K", [(512, 768, 256), (4096, 2304, 256)])
def test_tile_and_edge_paths_bitwise_equal(M, N, K):
    """The guarded variant runs the same MFMA sequence on whole tiles (small
    tiles at 512 x 768, large ones at 4096 x 2304)."""
    A, B = synth.random_operands(M, N, K, seed=63)
    C1 = run_full(A, B, M, N, K, path=gr.GR_PATH_TILE)
    C2 = run_full(A, B, M, N, K, path=gr.GR_PATH_TILE_EDGE)
    assert np.array_equal(C1, C2)


@pytest.mark.parametrize("M,N", [(512, 256), (2304, 4096)])
@pytest.mark.parametrize("K", [32, 64, 96, 128, 160, 192, 224, 256, 288, 320, 384, 448, 512, 1056, 1088])
def test_tile_pipeline_every_strip_count(M, N, K):
    """Whole tiles through the pipelined kernels (128 x 128 tiles at 512 x 256,
    forced: the planner gives that shape to the streaming kernel from K = 256
    on; 256 x 256
    tiles at 2304 x 4096: the 32- and 64-deep variants), for every K-loop
    length up to the steady state plus odd and even tails, bitwise against
    the guarded kernel (all accumulate the same 16-deep MFMA steps in the
    same order).  The large shape is checked against the oracle on edge rows
    and columns, the small one in full."""
    st, plan = gr.gemm_relu_f16_plan(M, N, K, 0x100000, K, 0x200000000000, N, 0x400000000000, N)
    if M == 512:
        assert plan["path"] == (gr.GR_PATH_TILE_STREAM if K >= 256 else gr.GR_PATH_TILE), plan
    else:
        assert plan["path"] == gr.GR_PATH_TILE and plan["block_m"] == 256, plan
    A, B = synth.random_operands(M, N, K, seed=K)
    C1 = run_full(A, B, M, N, K, path=gr.GR_PATH_TILE)
    C2 = run_full(A, B, M, N, K, path=gr.GR_PATH_TILE_EDGE)
    C = window(C1, M, N, N)
    if M == 512:
        assert_parity(C, oracle.gemm_relu_full(A, B), "tile K=%d" % K)
    else:
        rows = edge_indices(M, plan["block_m"]) + [1000, 1024]
        cols = edge_indices(N, plan["block_n"]) + [2000, 2048]
        assert_parity(C[rows, :], oracle.gemm_relu_rows(A, B, rows), "tile K=%d rows" % K)
        assert_parity(C[:, cols].T, oracle.gemm_relu_cols(A, B, cols), "tile K=%d cols" % K)
    assert np.array_equal(C1, C2)


# ---- the pipelined kernels on partial tiles (16-byte rows, K % 32 == 0) -------

PARTIAL_TILE_CASES = [
    (65, 264, 64, 72, 264, 265),           # 65 rows: rows past M clamped, padded A, odd ldc
    (100, 304, 96, 96, 304, 300 + 4),      # fewer rows than one tile, K % 64 == 32
    (128, 136, 32, 32, 136, 136),          # 128 x 128 tiles: one tile row, one partial tile column
    (257, 264, 64, 64, 264, 264),          # one row past a tile; N a multiple of 8
    (2400, 4000, 96, 96, 4000, 4001),      # 256 x 256 tiles, K % 64 == 32 (32-deep kernel), odd ldc
    (300, 250, 96, 96, 256, 251),          # K % 64 == 32 (32-deep kernel); odd ldc: 2-byte stores
    (511, 1, 128, 136, 8, 1),              # a single column; padded A rows
    (1000, 700, 320, 320, 704, 700),       # 4 x 3 tiles, last tile row shifted by 24 rows
    (4099, 3071, 2048, 2048, 3072, 3071),  # the ragged workload's M and N with 16-byte rows
]


@pytest.mark.parametrize("M,N,K,lda,ldb,ldc", PARTIAL_TILE_CASES)
def test_pipelined_kernel_partial_tiles(M, N, K, lda, ldb, ldc):
    """Shapes whose M and N do not fill tiles run the pipelined kernel (the
    last tile row moved up to end at M, copies past N clamped to the last
    chunk, guarded stores).  Full oracle check, padding of A and B poisoned,
    C's padding columns and the rows after it must keep the sentinel, and
    the result must equal the register-staged guarded kernel's bit for bit
    (same MFMA steps in the same k order)."""
    st, plan = gr.gemm_relu_f16_plan(M, N, K, 0x100000, lda, 0x200000000000, ldb, 0x400000000000, ldc)
    # the planner's choice, or 64 x 64 blocks on the streaming kernel where
    # 128 x 128 tiles would be few: the pipelined kernel is forced here
    assert st == gr.GR_OK and plan["path"] in (gr.GR_PATH_TILE, gr.GR_PATH_TILE_STREAM), plan
    log("partial %dx%dx%d plan %s" % (M, N, K, plan["path_name"]))
    A, B = synth.random_operands(M, N, K, seed=M + 3 * N + 7 * K, lda=lda, ldb=ldb)
    extra_rows = 2
    C1 = run_full(A, B, M, N, K, lda=lda, ldb=ldb, ldc=ldc, c_rows=M + extra_rows, path=gr.GR_PATH_TILE)
    C = C1[:M * ldc].reshape(M, ldc)
    assert_parity(C[:, :N], oracle.gemm_relu_full(A, B, M=M, N=N, K=K, lda=lda, ldb=ldb),
                  "pipelined partial %dx%dx%d" % (M, N, K))
    assert np.all(C[:, N:] == SENTINEL), "a padding column of C was written"
    assert np.all(C1[M * ldc:] == SENTINEL), "a row past M was written"
    C2 = run_full(A, B, M, N, K, lda=lda, ldb=ldb, ldc=ldc, c_rows=M + extra_rows, path=gr.GR_PATH_TILE_EDGE)
    assert np.array_equal(C1, C2)


# ---- the packed path: operands copied into a workspace, then pipelined ------

WS_POISON = 0x7E5A  # the workspace starts as NaN bit patterns: the copy must overwrite what it uses

PACKED_CASES = [
    # M, N, K, lda, ldb, ldc, expected `packed` bits
    (4099, 3071, 2050, 2050, 3071, 3071, 3),  # the ragged workload (forced): both copied, K padded to 2112
    (300, 270, 100, 109, 275, 273, 3),        # odd pitches, padding poisoned
    (256, 8, 33, 33, 8, 8, 3),                # one tile, K padded from 33 to 64
    (512, 640, 1000, 1000, 640, 640, 3),      # aligned rows, K % 32 == 8: both padded
    (1000, 3071, 2048, 2048, 3071, 3071, 2),  # only B misaligned: K unchanged
    (777, 512, 96, 97, 512, 512, 1),          # only A misaligned, K % 64 == 32 (32-deep kernel)
]


@pytest.mark.parametrize("M,N,K,lda,ldb,ldc,bits", PACKED_CASES)
def test_packed_path_parity(M, N, K, lda, ldb, ldc, bits):
    """Forced packed path against the oracle (full), C's padding and the rows
    after it keep the sentinel, bytes of the workspace past the size the
    library asked for are never written, and the result equals the guarded
    kernel's bit for bit (the padded K steps add exact zeros)."""
    import torch as t
    kp = K if K % 32 == 0 else -(-K // 64) * 64
    expect = (-(-(M * kp * 2) // 256) * 256 if bits & 1 else 0) + (kp * (-(-N // 8) * 8) * 2 if bits & 2 else 0)
    st, size = gr.gemm_relu_f16_workspace_size(M, N, K, 0x100000, lda, 0x200000000000, ldb, 0x400000000000, ldc)
    assert st == gr.GR_OK
    if size == 0:
        # the unaligned pipelined kernel or the streaming kernel takes this
        # problem in place, so the planner asks for no workspace; the forced
        # packed path still needs the copies' bytes
        st, p0 = gr.gemm_relu_f16_plan(M, N, K, 0x100000, lda, 0x200000000000, ldb, 0x400000000000, ldc)
        assert p0["path"] in (gr.GR_PATH_TILE_UNALIGNED, gr.GR_PATH_TILE_STREAM)
        size = expect
    st, plan = gr.gemm_relu_f16_plan_ws(M, N, K, 0x100000, lda, 0x200000000000, ldb, 0x400000000000, ldc, size)
    log("packed %dx%dx%d size=%d plan=%s" % (M, N, K, size, plan))
    A, B = synth.random_operands(M, N, K, seed=5 * M + N + K, lda=lda, ldb=ldb)
    dA, dB = to_dev(A), to_dev(B)
    extra_rows = 2
    dC = full_dev(((M + extra_rows) * ldc,), SENTINEL)
    tail = 4096
    ws = full_dev(((size + tail) // 2,), WS_POISON).view(t.uint8)
    assert call_ws(M, N, K, dA, lda, dB, ldb, dC, ldc, ws, size, path=gr.GR_PATH_TILE_PACKED) == gr.GR_OK
    C1 = from_dev(dC)
    C = C1[:M * ldc].reshape(M, ldc)
    assert_parity(C[:, :N], oracle.gemm_relu_full(A, B, M=M, N=N, K=K, lda=lda, ldb=ldb),
                  "packed %dx%dx%d" % (M, N, K))
    assert np.all(C[:, N:] == SENTINEL), "a padding column of C was written"
    assert np.all(C1[M * ldc:] == SENTINEL), "a row past M was written"
    w = ws.view(t.int16).cpu().numpy().view(np.uint16)
    assert np.all(w[size // 2:] == WS_POISON), "workspace written past the size the library asked for"
    dC2 = full_dev(((M + extra_rows) * ldc,), SENTINEL)
    assert call(M, N, K, dA, lda, dB, ldb, dC2, ldc, path=gr.GR_PATH_TILE_EDGE) == gr.GR_OK
    assert np.array_equal(C1, from_dev(dC2))
    # the workspace holds exactly the copies the case expects
    assert size == expect
    if plan["path"] == gr.GR_PATH_TILE_PACKED:
        assert plan["packed"] == bits


@pytest.mark.parametrize("offs", [(1, 0, 0), (0, 3, 0), (3, 5, 7), (7, 7, 1)])
def test_packed_path_unaligned_base_pointers(offs):
    """Operands starting at any element offset: the copy reads each group from
    the aligned 16-byte blocks that hold it and shifts it into place."""
    import torch as t
    M, N, K = 320, 296, 100
    A, B = synth.random_operands(M, N, K, seed=sum(offs) + 50)
    Ap = np.concatenate([np.zeros(offs[0], np.uint16), A.ravel(), np.zeros(8, np.uint16)])
    Bp = np.concatenate([np.zeros(offs[1], np.uint16), B.ravel(), np.zeros(8, np.uint16)])
    args = (M, N, K, 0x100000 + 2 * offs[0], K, 0x200000000000 + 2 * offs[1], N, 0x400000000000 + 2 * offs[2], N)
    st, size = gr.gemm_relu_f16_workspace_size(*args)
    assert st == gr.GR_OK and size > 0
    ws = t.empty(size, dtype=t.uint8, device="cuda")
    dC = full_dev((M * N + offs[2] + 8,), SENTINEL)
    assert call_ws(M, N, K, to_dev(Ap), K, to_dev(Bp), N, dC, N, ws, size, path=gr.GR_PATH_TILE_PACKED,
                   offsets=offs) == gr.GR_OK
    Cflat = from_dev(dC)
    C = Cflat[offs[2]:offs[2] + M * N].reshape(M, N)
    assert_parity(C, oracle.gemm_relu_full(A, B), "packed offsets %s" % (offs,))
    assert np.all(Cflat[:offs[2]] == SENTINEL)
    assert np.all(Cflat[offs[2] + M * N:] == SENTINEL)


def test_packed_path_reuses_a_dirty_workspace():
    """Two calls in a row on one workspace, the second smaller with other
    pitches: stale copies from the first never leak into the second."""
    import torch as t
    shapes = [(1200, 1100, 700, 701, 1101, 1100), (520, 300, 90, 91, 301, 300)]
    sizes = [gr.gemm_relu_f16_workspace_size(M, N, K, 0x100000, la, 0x200000000000, lb, 0x400000000000, lc)[1]
             for M, N, K, la, lb, lc in shapes]
    ws = full_dev((max(sizes) // 2 + 128,), WS_POISON).view(t.uint8)
    for (M, N, K, la, lb, lc), size in zip(shapes, sizes):
        A, B = synth.random_operands(M, N, K, seed=M + K, lda=la, ldb=lb)
        dC = full_dev((M * lc,), SENTINEL)
        assert call_ws(M, N, K, to_dev(A), la, to_dev(B), lb, dC, lc, ws, size,
                       path=gr.GR_PATH_TILE_PACKED) == gr.GR_OK
        C = from_dev(dC).reshape(M, lc)
        assert_parity(C[:, :N], oracle.gemm_relu_full(A, B, M=M, N=N, K=K, lda=la, ldb=lb), "reuse %d" % M)


@pytest.mark.parametrize("M,N,K", [(8, 4096, 4096), (1, 640, 96), (16, 1000, 1000), (5, 128, 8200)])
def test_small_m_and_tile_paths_agree(M, N, K):
    A, B = synth.random_operands(M, N, K, seed=64, b_scale=K ** -0.5)
    Cs = window(run_full(A, B, M, N, K, path=gr.GR_PATH_SMALL_M), M, N, N)
    Ct = window(run_full(A, B, M, N, K, path=gr.GR_PATH_TILE_EDGE), M, N, N)
    ref = oracle.gemm_relu_full(A, B)
    assert_parity(Cs, ref, "small-M")
    assert_parity(Ct, ref, "tile")
    assert_parity(Cs, Ct, "small-M vs tile")


# ---- the small-M split-K path (fp32 partial sums in a workspace) -------------

SPLIT_CASES = [
    # M, N, K, lda, ldb, ldc
    (8, 16384, 8192, 8192, 16384, 16384),  # the small-M workload's shape (forced: 4 splits)
    (8, 2048, 8192, 8192, 2048, 2048),     # 8 column blocks x 32 splits
    (16, 1000, 1000, 1000, 1000, 1000),    # partial column block, K % 32 == 8
    (5, 128, 8200, 8200, 128, 128),        # one column block, 8 splits
    (1, 640, 96, 96, 640, 640),            # one row, 3 splits of one step
    (3, 4096, 4096, 4104, 4104, 4097),     # padded A and B (poisoned), odd ldc
]


@pytest.mark.parametrize("M,N,K,lda,ldb,ldc", SPLIT_CASES)
def test_small_m_split_parity(M, N, K, lda, ldb, ldc):
    """Forced split-K small-M path against the oracle (full), C's padding and
    the rows after it keep the sentinel, the workspace is not written past the
    size asked for, and the single-pass small-M kernel agrees within the
    tolerance (the two differ in fp32 summation order only)."""
    import torch as t
    st, size = gr.gemm_relu_f16_workspace_size(M, N, K, 0x100000, lda, 0x200000000000, ldb, 0x400000000000, ldc)
    st2, plan = gr.gemm_relu_f16_plan_ws(M, N, K, 0x100000, lda, 0x200000000000, ldb, 0x400000000000, ldc, size)
    log("split %dx%dx%d size=%d plan=%s" % (M, N, K, size, plan))
    if size == 0:  # the planner would not split (the single pass fills the chip): force it
        size = 64 * 4 * M * N + 256
    assert st == gr.GR_OK and st2 == gr.GR_OK
    A, B = synth.random_operands(M, N, K, seed=M * 31 + N + K, lda=lda, ldb=ldb, b_scale=K ** -0.5)
    dA, dB = to_dev(A), to_dev(B)
    extra_rows = 2
    dC = full_dev(((M + extra_rows) * ldc,), SENTINEL)
    tail = 4096
    ws = full_dev(((size + tail) // 2,), WS_POISON).view(t.uint8)
    assert call_ws(M, N, K, dA, lda, dB, ldb, dC, ldc, ws, size, path=gr.GR_PATH_SMALL_M_SPLIT) == gr.GR_OK
    C1 = from_dev(dC)
    C = C1[:M * ldc].reshape(M, ldc)
    ref = oracle.gemm_relu_full(A, B, M=M, N=N, K=K, lda=lda, ldb=ldb)
    assert_parity(C[:, :N], ref, "split %dx%dx%d" % (M, N, K))
    assert np.all(C[:, N:] == SENTINEL), "a padding column of C was written"
    assert np.all(C1[M * ldc:] == SENTINEL), "a row past M was written"
    w = ws.view(t.int16).cpu().numpy().view(np.uint16)
    assert np.all(w[size // 2:] == WS_POISON), "workspace written past the size the library asked for"
    dC2 = full_dev((M * ldc,), SENTINEL)
    assert call(M, N, K, dA, lda, dB, ldb, dC2, ldc, path=gr.GR_PATH_SMALL_M) == gr.GR_OK
    C2 = from_dev(dC2).reshape(M, ldc)
    assert_parity(C[:, :N], C2[:, :N], "split vs single pass")
    # deterministic: a second call on the dirty workspace gives the same bits
    dC3 = full_dev(((M + extra_rows) * ldc,), SENTINEL)
    assert call_ws(M, N, K, dA, lda, dB, ldb, dC3, ldc, ws, size, path=gr.GR_PATH_SMALL_M_SPLIT) == gr.GR_OK
    assert np.array_equal(C1, from_dev(dC3))


def test_ws_call_picks_split_path_for_narrow_small_m():
    """gemm_relu_f16_ws with the size the library asks for splits K when the
    single-pass kernel would leave CUs idle (8 x 2048 x 8192: 32 strips)."""
    import torch as t
    M, N, K = 8, 2048, 8192
    st, size = gr.gemm_relu_f16_workspace_size(M, N, K, 0x100000, K, 0x200000000000, N, 0x400000000000, N)
    assert gr.gemm_relu_f16_plan_ws(M, N, K, 0x100000, K, 0x200000000000, N, 0x400000000000, N,
                                    size)[1]["path"] == gr.GR_PATH_SMALL_M_SPLIT
    A, B = synth.random_operands(M, N, K, seed=77, b_scale=K ** -0.5)
    ws = t.empty(size, dtype=t.uint8, device="cuda")
    dC = full_dev((M * N,), SENTINEL)
    assert call_ws(M, N, K, to_dev(A), K, to_dev(B), N, dC, N, ws, size) == gr.GR_OK
    assert_parity(from_dev(dC).reshape(M, N), oracle.gemm_relu_full(A, B), "narrow small-M, split")


# ---- split-K on the 128 x 128 tile path --------------------------------------

TILE_SPLIT_CASES = [
    # M, N, K, lda, ldb, ldc
    (1024, 1024, 16384, 16384, 1024, 1024),  # 64 tiles x 4 splits
    (128, 128, 1024, 1024, 128, 128),        # one tile, 4 splits
    (300, 520, 4096, 4104, 520, 521),        # partial tiles, padded A, odd ldc
    (640, 1000, 2080, 2080, 1000, 1000),     # 40 tiles x 6 splits of 11 strips, the last 10 deep
    (640, 1000, 1568, 1568, 1000, 1000),     # 40 tiles x 6 splits of 9 strips, the last 4 deep
]


@pytest.mark.parametrize("M,N,K,lda,ldb,ldc", TILE_SPLIT_CASES)
def test_tile_split_parity(M, N, K, lda, ldb, ldc):
    """Forced split-K tile path against the oracle (full), padding of C and
    the rows after it untouched, workspace not written past its size, the
    unsplit kernel agrees within tolerance, and a repeat on the dirty
    workspace gives the same bits."""
    import torch as t
    st, size = gr.gemm_relu_f16_workspace_size(M, N, K, 0x100000, lda, 0x200000000000, ldb, 0x400000000000, ldc)
    st2, plan = gr.gemm_relu_f16_plan_ws(M, N, K, 0x100000, lda, 0x200000000000, ldb, 0x400000000000, ldc, size)
    log("tile split %dx%dx%d size=%d plan=%s" % (M, N, K, size, plan))
    if size == 0:  # the planner would not split this one: force it
        size = 16 * M * N * 4 + 256
    assert st == gr.GR_OK and st2 == gr.GR_OK
    A, B = synth.random_operands(M, N, K, seed=M + N + K + 9, lda=lda, ldb=ldb, b_scale=K ** -0.5)
    dA, dB = to_dev(A), to_dev(B)
    extra_rows = 2
    dC = full_dev(((M + extra_rows) * ldc,), SENTINEL)
    tail = 4096
    ws = full_dev(((size + tail) // 2,), WS_POISON).view(t.uint8)
    assert call_ws(M, N, K, dA, lda, dB, ldb, dC, ldc, ws, size, path=gr.GR_PATH_TILE_SPLIT) == gr.GR_OK
    C1 = from_dev(dC)
    C = C1[:M * ldc].reshape(M, ldc)
    assert_parity(C[:, :N], oracle.gemm_relu_full(A, B, M=M, N=N, K=K, lda=lda, ldb=ldb),
                  "tile split %dx%dx%d" % (M, N, K))
    assert np.all(C[:, N:] == SENTINEL), "a padding column of C was written"
    assert np.all(C1[M * ldc:] == SENTINEL), "a row past M was written"
    w = ws.view(t.int16).cpu().numpy().view(np.uint16)
    assert np.all(w[size // 2:] == WS_POISON), "workspace written past the size the library asked for"
    dC2 = full_dev((M * ldc,), SENTINEL)
    assert call(M, N, K, dA, lda, dB, ldb, dC2, ldc, path=gr.GR_PATH_TILE) == gr.GR_OK
    assert_parity(C[:, :N], from_dev(dC2).reshape(M, ldc)[:, :N], "split vs unsplit")
    dC3 = full_dev(((M + extra_rows) * ldc,), SENTINEL)
    assert call_ws(M, N, K, dA, lda, dB, ldb, dC3, ldc, ws, size, path=gr.GR_PATH_TILE_SPLIT) == gr.GR_OK
    assert np.array_equal(C1, from_dev(dC3))


# ---- seeded random problems across every planner decision --------------------

def _fuzz_cases(count, seed):
    """Half the cases have 16-byte rows and K % 32 == 0 (pipelined, small-M and
    split paths; some with K of 3200-6400 so that the tile path splits K),
    the others arbitrary pitches and offsets (guarded kernel, or packed with a
    workspace), some of them large enough (>= 2^30 MAC) for the planner to
    pack."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        mode = ["aligned", "aligned", "aligned", "any", "any", "big", "long", "any"][i % 8]
        M = int(rng.choice([rng.integers(1, 17), rng.integers(17, 300), rng.integers(300, 700)]))
        N = int(rng.integers(1, 700))
        if mode in ("aligned", "long"):
            K = int(32 * (rng.integers(100, 200) if mode == "long" else rng.integers(1, 40)))
            pads = [(-K) % 8 + 8 * int(rng.integers(0, 2)), (-N) % 8 + 8 * int(rng.integers(0, 2)),
                    int(rng.integers(0, 9))]
            offs = [0, 0, int(rng.choice([0, 0, rng.integers(1, 8)]))]
        else:
            K = int(rng.choice([0, rng.integers(1, 64), rng.integers(64, 700), 32 * rng.integers(1, 22)]))
            pads = [int(rng.choice([0, 0, rng.integers(1, 9), 8])) for _ in range(3)]
            offs = [int(rng.choice([0, 0, 0, rng.integers(1, 8)])) for _ in range(3)]
            if mode == "big":
                M, N, K = int(rng.integers(1000, 1300)), int(rng.integers(1000, 1300)), int(rng.integers(900, 1100))
        use_ws = bool(rng.integers(0, 2)) or mode == "big"
        cases.append((i, M, N, K, pads, offs, use_ws))
    return cases


@pytest.mark.parametrize("case", _fuzz_cases(48, 2024), ids=lambda c: "fuzz%d" % c[0])
def test_random_problems_against_oracle(case):
    """Random shapes, pitches and pointer offsets, with and without the
    workspace the library asks for: whatever path the planner picks, the
    result matches the oracle, padding of C and the bytes around it keep the
    sentinel."""
    import torch as t
    i, M, N, K, pads, offs, use_ws = case
    lda, ldb, ldc = max(K, 1) + pads[0], max(N, 1) + pads[1], N + pads[2]
    A, B = synth.random_operands(M, N, K, seed=1000 + i, lda=lda, ldb=ldb)
    Ap = np.concatenate([np.zeros(offs[0], np.uint16), A.ravel(), np.zeros(8, np.uint16)])
    Bp = np.concatenate([np.zeros(offs[1], np.uint16), B.ravel(), np.zeros(8, np.uint16)])
    dA, dB = to_dev(Ap), to_dev(Bp)
    c_elems = M * ldc + offs[2] + 8
    dC = full_dev((c_elems,), SENTINEL)
    a = dA.data_ptr() + 2 * offs[0]
    b = dB.data_ptr() + 2 * offs[1]
    c = dC.data_ptr() + 2 * offs[2]
    st, size = gr.gemm_relu_f16_workspace_size(M, N, K, a, lda, b, ldb, c, ldc)
    assert st == gr.GR_OK
    ws = t.empty(max(size, 256), dtype=t.uint8, device="cuda") if (use_ws and size) else None
    wbytes = size if ws is not None else 0
    st, plan = gr.gemm_relu_f16_plan_ws(M, N, K, a, lda, b, ldb, c, ldc, wbytes)
    log("fuzz%d M=%d N=%d K=%d ld=%d,%d,%d offs=%s ws=%d path=%s" % (i, M, N, K, lda, ldb, ldc, offs, wbytes,
                                                                    plan["path_name"]))
    assert call_ws(M, N, K, dA, lda, dB, ldb, dC, ldc, ws, wbytes, offsets=tuple(offs)) == gr.GR_OK
    Cflat = from_dev(dC)
    assert np.all(Cflat[:offs[2]] == SENTINEL)
    Cw = Cflat[offs[2]:offs[2] + M * ldc].reshape(M, ldc) if M else np.zeros((0, ldc), np.uint16)
    assert np.all(Cflat[offs[2] + M * ldc:] == SENTINEL)
    if M and N:
        ref = oracle.gemm_relu_full(A, B, M=M, N=N, K=K, lda=lda, ldb=ldb)
        assert_parity(Cw[:, :N], ref, "fuzz%d %s" % (i, plan["path_name"]))
    assert np.all(Cw[:, N:] == SENTINEL)


# ---- the small-M stream with 2 or 4 blocks of 16 rows ----------------------------

MIDM_CASES = [
    # M, N, K, lda, ldb, ldc
    (17, 512, 512, 512, 512, 512),        # two row blocks, whole strips
    (32, 4096, 1024, 1024, 4096, 4096),
    (33, 2000, 1000, 1000, 2000, 2001),   # four row blocks, guarded: N % 64 != 0, K % 32 != 0
    (48, 1000, 256, 264, 1008, 1003),     # padded pitches
    (64, 16384, 2048, 2048, 16384, 16384),  # 256 strips, four row blocks
    (24, 300, 130, 136, 300, 301),
]


@pytest.mark.parametrize("M,N,K,lda,ldb,ldc", MIDM_CASES)
def test_small_m_row_blocks(M, N, K, lda, ldb, ldc):
    """17-64 rows of A on the small-M stream (each B operand feeds 2 or 4
    row blocks): full comparison with the oracle, poisoned padding, C
    canaries, and agreement with the tile kernels within the tolerance."""
    st, plan = gr.gemm_relu_f16_plan(M, N, K, 0x100000, lda, 0x200000000000, ldb, 0x400000000000, ldc)
    assert plan["path"] in (gr.GR_PATH_SMALL_M, gr.GR_PATH_TILE_STREAM), plan
    assert plan["path"] == gr.GR_PATH_TILE_STREAM or plan["block_m"] == (32 if M <= 32 else 64), plan
    A, B = synth.random_operands(M, N, K, seed=M * 3 + N + K, lda=lda, ldb=ldb, b_scale=K ** -0.5)
    Cflat = run_full(A, B, M, N, K, lda, ldb, ldc, c_rows=M + 1, path=gr.GR_PATH_SMALL_M)
    C = Cflat[:M * ldc].reshape(M, ldc)
    assert_parity(C[:, :N], oracle.gemm_relu_full(A, B, M=M, N=N, K=K, lda=lda, ldb=ldb), "small-M rows")
    assert np.all(C[:, N:] == SENTINEL) and np.all(Cflat[M * ldc:] == SENTINEL)
    C2 = run_full(A, B, M, N, K, lda, ldb, ldc, c_rows=M + 1, path=gr.GR_PATH_TILE_EDGE)
    assert_parity(C[:, :N], C2[:M * ldc].reshape(M, ldc)[:, :N], "small-M rows vs guarded tile")


# ---- more 256 x 256 tiles than CUs ---------------------------------------------

MANY_TILE_CASES = [
    # M, N, K, lda, ldb, ldc: tiles
    (4352, 4352, 128, 128, 4352, 4352),   # 289 whole tiles, 64-deep kernel: a second round of 33
    (4100, 4400, 96, 104, 4400, 4401),    # 17 x 18 = 306 partial tiles, 32-deep kernel
    (6000, 2600, 64, 64, 2608, 2601),     # 24 x 11 = 264 partial tiles
    (8192, 8192, 64, 64, 8192, 8192),     # 1024 tiles: four rounds
]


@pytest.mark.parametrize("M,N,K,lda,ldb,ldc", MANY_TILE_CASES)
def test_more_tiles_than_compute_units(M, N, K, lda, ldb, ldc):
    """Several rounds of workgroups (and a partial last round) produce every
    tile exactly as the guarded kernel does, bit for bit, and match the
    oracle; C's padding and the rows below stay untouched."""
    st, plan = gr.gemm_relu_f16_plan(M, N, K, 0x100000, lda, 0x200000000000, ldb, 0x400000000000, ldc)
    assert plan["path"] == gr.GR_PATH_TILE and plan["block_m"] == 256 and plan["grid"] > 256, plan
    A, B = synth.random_operands(M, N, K, seed=M + N + K, lda=lda, ldb=ldb, b_scale=K ** -0.5)
    C1 = run_full(A, B, M, N, K, lda, ldb, ldc, c_rows=M + 1)
    C2 = run_full(A, B, M, N, K, lda, ldb, ldc, c_rows=M + 1, path=gr.GR_PATH_TILE_EDGE)
    assert np.array_equal(C1, C2)
    C = C1[:M * ldc].reshape(M, ldc)
    assert np.all(C[:, N:] == SENTINEL) and np.all(C1[M * ldc:] == SENTINEL)
    if M * N * K <= 4 << 30:
        assert_parity(C[:, :N], oracle.gemm_relu_full(A, B, M=M, N=N, K=K, lda=lda, ldb=ldb), "many tiles")
    else:
        ii, jj = synth.sample_indices(M, N, 4096, 7)
        assert_parity(C[ii, jj], oracle.gemm_relu_elems(A, B, ii, jj, M=M, N=N, K=K, lda=lda, ldb=ldb), "many tiles")


# ---- B given transposed (Bt, N x K) --------------------------------------------

def run_bt(A, Bt, M, N, K, lda, ldbt, ldc, path=None, c_rows=None, offsets=(0, 0, 0)):
    import torch as t
    dA, dBt = to_dev(A), to_dev(Bt)
    rows = M if c_rows is None else c_rows
    dC = full_dev((rows * ldc + offsets[2] + 8,), SENTINEL)
    a = dA.data_ptr() + 2 * offsets[0]
    b = dBt.data_ptr() + 2 * offsets[1]
    c = dC.data_ptr() + 2 * offsets[2]
    s = t.cuda.current_stream().cuda_stream
    log("bt M=%d N=%d K=%d lda=%d ldbt=%d ldc=%d path=%s offsets=%s" % (M, N, K, lda, ldbt, ldc, path, offsets))
    if path is None:
        st = gr.gemm_relu_f16_bt(M, N, K, a, lda, b, ldbt, c, ldc, s)
    else:
        st = gr.gemm_relu_f16_bt_forced(M, N, K, a, lda, b, ldbt, c, ldc, s, path)
    t.cuda.synchronize()
    assert st == gr.GR_OK, gr.gemm_relu_status_string(st)
    return from_dev(dC)


def bt_operands(M, N, K, seed, lda, ldbt, b_scale=None):
    """A (M x lda) and Bt (N x ldbt), padding poisoned, plus the K x N B the
    oracle takes (the transpose of Bt's first K columns)."""
    A, B = synth.random_operands(M, N, K, seed=seed, lda=lda, b_scale=b_scale)
    Bt = np.full((N, max(ldbt, 1)), 0x7BFF, dtype=np.uint16)
    Bt[:, :K] = B[:, :N].T
    return A, Bt, np.ascontiguousarray(Bt[:, :K].T)


BT_CASES = [
    # M, N, K, lda, ldbt, ldc, expected path
    (8, 16384, 8192, 8192, 8192, 16384, gr.GR_PATH_SMALL_M),   # the small-M workload's shape
    (16, 1000, 1000, 1000, 1000, 1000, gr.GR_PATH_SMALL_M),    # K % 32 != 0: guarded loads
    (16, 1000, 1024, 1032, 1032, 1001, gr.GR_PATH_SMALL_M),    # partial wave of columns, padding
    (1, 100, 96, 96, 96, 100, gr.GR_PATH_SMALL_M),
    (5, 4096, 256, 256, 264, 4096, gr.GR_PATH_SMALL_M),        # one 256-deep chunk, padded Bt
    (3, 64, 512, 520, 512, 65, gr.GR_PATH_SMALL_M),            # one workgroup, two chunks, odd ldc
    (12, 70, 512, 512, 520, 71, gr.GR_PATH_SMALL_M),           # 16 rows of A per slot; 3 waves past N
    (8, 130, 768, 776, 768, 130, gr.GR_PATH_SMALL_M),          # 8 rows of A per slot, 3 chunks, N % 64 = 2
    (512, 768, 224, 224, 224, 768, gr.GR_PATH_TILE),           # 128 x 128 tiles
    (4096, 2304, 512, 512, 520, 2304, gr.GR_PATH_TILE),        # 256 x 256 tiles, padded Bt
    (300, 250, 96, 104, 96, 251, gr.GR_PATH_TILE),             # partial tiles, rows of Bt clamped
    (2400, 4000, 96, 96, 96, 4001, gr.GR_PATH_TILE),           # large partial tiles
    (17, 264, 64, 72, 64, 265, gr.GR_PATH_TILE),
    (300, 270, 100, 109, 105, 273, gr.GR_PATH_TILE_EDGE),      # odd pitches
    (4352, 4352, 128, 128, 136, 4352, gr.GR_PATH_TILE),        # 289 tiles: a second round
    (4100, 4400, 96, 96, 96, 4400, gr.GR_PATH_TILE),           # 306 partial tiles
    # 256 x 256 tiles with K % 64 = 0 (A and Bt in one ring of 64-deep strips):
    (2600, 3000, 1024, 1024, 1032, 3001, gr.GR_PATH_TILE),     # partial tiles, clamped Bt rows, steady steps
    (4096, 2304, 64, 64, 64, 2304, gr.GR_PATH_TILE),           # one pair of strips
    (4096, 2304, 192, 200, 192, 2304, gr.GR_PATH_TILE),        # three pairs: no steady step
    (4096, 2304, 320, 320, 328, 2304, gr.GR_PATH_TILE),        # steady steps, then the tail
]


@pytest.mark.parametrize("M,N,K,lda,ldbt,ldc,path", BT_CASES)
def test_transposed_b_parity(M, N, K, lda, ldbt, ldc, path):
    """gemm_relu_f16_bt against the oracle on the transposed operand (full),
    with poisoned padding and C canaries; the guarded kernel on the same
    input gives the same bits as the pipelined one (same k order)."""
    st, plan = gr.gemm_relu_f16_bt_plan(M, N, K, 0x100000, lda, 0x200000000000, ldbt, 0x400000000000, ldc)
    assert st == gr.GR_OK and plan["path"] == path, plan
    A, Bt, B = bt_operands(M, N, K, seed=M + N + K + 5, lda=lda, ldbt=ldbt, b_scale=K ** -0.5)
    extra = 2
    C1 = run_bt(A, Bt, M, N, K, lda, ldbt, ldc, c_rows=M + extra)
    C = C1[:M * ldc].reshape(M, ldc)
    assert_parity(C[:, :N], oracle.gemm_relu_full(A, B, M=M, N=N, K=K, lda=lda, ldb=N),
                  "bt %dx%dx%d" % (M, N, K))
    assert np.all(C[:, N:] == SENTINEL) and np.all(C1[M * ldc:] == SENTINEL)
    if path == gr.GR_PATH_TILE:
        C2 = run_bt(A, Bt, M, N, K, lda, ldbt, ldc, c_rows=M + extra, path=gr.GR_PATH_TILE_EDGE)
        assert np.array_equal(C1, C2)


@pytest.mark.parametrize("M,N,K", [(512, 768, 224), (4096, 2304, 256), (300, 250, 96)])
def test_transposed_b_matches_plain_layout_bitwise(M, N, K):
    """The same product through B (K x N) and through Bt (N x K) gives the same
    bits: both layouts feed the same MFMA sequence on the tile kernels (the
    plain layout forced onto them: the planner gives small shapes to the
    streaming kernel, which splits K between waves)."""
    A, Bt, B = bt_operands(M, N, K, seed=K + 3, lda=K, ldbt=K)
    Cbt = run_bt(A, Bt, M, N, K, K, K, N)
    Cnn = run_full(A, B, M, N, K, path=gr.GR_PATH_TILE if N % 8 == 0 else gr.GR_PATH_TILE_EDGE)
    assert np.array_equal(Cbt[:M * N], Cnn[:M * N])


@pytest.mark.parametrize("offs", [(1, 0, 0), (0, 3, 0), (5, 7, 1)])
def test_transposed_b_unaligned_base_pointers(offs):
    M, N, K = 320, 288, 96
    A, Bt, B = bt_operands(M, N, K, seed=sum(offs), lda=K, ldbt=K)
    Ap = np.concatenate([np.zeros(offs[0], np.uint16), A.ravel(), np.zeros(8, np.uint16)])
    Btp = np.concatenate([np.zeros(offs[1], np.uint16), Bt.ravel(), np.zeros(8, np.uint16)])
    Cflat = run_bt(Ap, Btp, M, N, K, K, K, N, offsets=offs)
    C = Cflat[offs[2]:offs[2] + M * N].reshape(M, N)
    assert_parity(C, oracle.gemm_relu_full(A, B), "bt offsets %s" % (offs,))
    assert np.all(Cflat[:offs[2]] == SENTINEL) and np.all(Cflat[offs[2] + M * N:] == SENTINEL)


def test_transposed_b_tensor_wrapper():
    t = pytest.importorskip("torch")
    M, N, K = 300, 200, 128
    A, Bt, B = bt_operands(M, N, K, seed=91, lda=K, ldbt=K)
    a = to_dev(A).view(t.float16).reshape(M, K)
    bt = to_dev(Bt).view(t.float16).reshape(N, K)
    c = gr.gemm_relu_bt(a, bt)
    t.cuda.synchronize()
    assert_parity(c.view(t.int16).cpu().numpy().view(np.uint16), oracle.gemm_relu_full(A, B), "bt wrapper")


def test_runs_on_a_side_stream():
    t = pytest.importorskip("torch")
    M, N, K = 512, 512, 256
    A, B = synth.random_operands(M, N, K, seed=65)
    dA, dB = to_dev(A), to_dev(B)
    s = t.cuda.Stream()
    with t.cuda.stream(s):
        dC = full_dev((M * N,), SENTINEL)
    assert call(M, N, K, dA, K, dB, N, dC, N, stream=s) == gr.GR_OK
    assert_parity(from_dev(dC).reshape(M, N), oracle.gemm_relu_full(A, B), "side stream")


def test_tensor_convenience_wrapper():
    t = pytest.importorskip("torch")
    M, N, K = 300, 200, 100
    A, B = synth.random_operands(M, N, K, seed=66)
    a = to_dev(A).view(t.float16).reshape(M, K)
    b = to_dev(B).view(t.float16).reshape(K, N)
    c = gr.gemm_relu(a, b)
    t.cuda.synchronize()
    assert_parity(c.view(t.int16).cpu().numpy().view(np.uint16), oracle.gemm_relu_full(A, B), "wrapper")
