"""Pins for the CPU oracle, each independent of the oracle's own code.

The oracle (``oracle/``) computes C = fp16_RNE(ReLU(fp32 sum_k A.B)), the
definition the GEMM+ReLU listings set up (blog "TileLang programming basics",
section 2; "Writing high-performance kernels in TileLang", section "Writing a
GEMM"). None of these tests retypes that loop. They check it against:
  * numpy's own fp16 <-> fp32 conversions (library routines), exhaustively;
  * exact results: integer-valued inputs whose every partial sum is exact;
  * float64 results with a proven fp32 rounding bound;
  * closed forms (all-ones, identity, diagonal, powers of two);
  * invariants (non-negativity, scaling by 2, row/column permutation,
    padding independence) and the agreement of the four entry points.
A plausible slip (a dropped term, a swapped sign, a transposed operand, a
wrong pitch, truncation instead of rounding) fails at least one of them.
"""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.usefixtures("oracle_lib")

F16_MAX = 65504.0


def as_f16(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16)


def bits(x):
    return np.asarray(x, dtype=np.float16).view(np.uint16)


# --- conversions ---------------------------------------------------------


def test_f16_to_f32_exhaustive_vs_numpy():
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_to_f32(allbits)
    ref = allbits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _f16_boundary_values():
    """Every fp16 value, every midpoint between neighbours, and 1-ulp fp32
    neighbours of each midpoint (ties and near-ties for RNE)."""
    allbits = np.arange(0, 0x7C01, dtype=np.uint32).astype(np.uint16)  # +0 .. +Inf
    vals = allbits.view(np.float16).astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2  # exact in float64, representable in fp32
    mids32 = mids[np.isfinite(mids)].astype(np.float32)
    assert np.array_equal(mids32.astype(np.float64), mids[np.isfinite(mids)])
    up = np.nextafter(mids32, np.float32(np.inf))
    dn = np.nextafter(mids32, np.float32(0))
    extra = np.array([65504.0, 65519.996, 65520.0, 65520.004, 1e30, 2.0 ** -24, 2.0 ** -25,
                      2.0 ** -25 * 1.0000001, 2.0 ** -26, 2.0 ** -14, 1e-40, 0.0],
                     dtype=np.float32)
    pos = np.concatenate([vals.astype(np.float32), mids32, up, dn, extra])
    return np.concatenate([pos, -pos])


@pytest.mark.filterwarnings("ignore:overflow encountered in cast")
def test_f32_to_f16_rne_boundaries_vs_numpy():
    v = _f16_boundary_values()
    ours = oracle.f32_to_f16(v)
    ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


@pytest.mark.filterwarnings("ignore:overflow encountered in cast")
def test_f32_to_f16_rne_random_vs_numpy():
    rng = np.random.default_rng(1234)
    u = rng.integers(0, 2 ** 32, size=10_000_000, dtype=np.uint64).astype(np.uint32)
    v = u.view(np.float32)
    v = v[~np.isnan(v)]
    # also a dense sample over the fp16 range, where most rounding happens
    w = (rng.standard_normal(2_000_000) * np.exp2(rng.integers(-26, 17, 2_000_000))).astype(np.float32)
    for x in (v, w):
        assert np.array_equal(oracle.f32_to_f16(x), x.astype(np.float16).view(np.uint16))


def test_f32_to_f16_nan_stays_nan():
    x = np.array([np.nan, -np.nan], dtype=np.float32)
    assert np.all(np.isnan(as_f16(oracle.f32_to_f16(x))))


# --- exact results -------------------------------------------------------


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_tiny_integer_exact(seed):
    """Integer inputs in [-3,3], K <= 64: every partial sum is an integer below
    2^11, exact in fp16 and fp32 in any order, so the float64 result rounded
    through ReLU must match bit for bit."""
    rng = np.random.default_rng(seed)
    for _ in range(40):
        M, N, K = (int(x) for x in rng.integers(1, 9, size=3))
        if seed >= 3:
            K = int(rng.integers(9, 65))
        A, B = synth.small_int_operands(M, N, K, seed=int(rng.integers(1 << 30)))
        ref = np.maximum(as_f16(A).astype(np.float64) @ as_f16(B).astype(np.float64), 0.0)
        C = oracle.gemm_relu_full(A, B)
        assert np.array_equal(C, bits(ref)), (M, N, K)


def test_handworked_example():
    """A 2x3 by 3x2 product worked by hand.
    A = [[1, 2, 3], [-1, 0.5, -2]], B = [[1, -1], [2, 0.25], [-1, 1]]
    A.B = [[1+4-3, -1+0.5+3], [-1+1+2, 1+0.125-2]] = [[2, 2.5], [2, -0.875]]
    ReLU -> [[2, 2.5], [2, 0]]."""
    A = bits([[1, 2, 3], [-1, 0.5, -2]])
    B = bits([[1, -1], [2, 0.25], [-1, 1]])
    C = oracle.gemm_relu_full(A, B)
    assert np.array_equal(as_f16(C).astype(np.float64), [[2.0, 2.5], [2.0, 0.0]])
    assert C[1, 1] == 0x0000  # +0, not -0


@pytest.mark.parametrize("seed", range(4))
def test_random_fp16_within_proven_bound(seed):
    """Random N(0,1) fp16 inputs against float64 products.

    The sequential fp32 sum satisfies |s32 - s| <= gamma_K * sum|a b| with
    gamma_K = K u / (1 - K u), u = 2^-24 (standard forward error bound of
    recursive summation; the products themselves are exact). ReLU is
    1-Lipschitz and RNE to fp16 adds at most half an fp16 ulp of the result."""
    rng = np.random.default_rng(100 + seed)
    for _ in range(30):
        M, N = (int(x) for x in rng.integers(1, 12, size=2))
        K = int(rng.integers(1, 300))
        A, B = synth.random_operands(M, N, K, seed=int(rng.integers(1 << 30)))
        a = as_f16(A).astype(np.float64)
        b = as_f16(B).astype(np.float64)
        exact = a @ b
        mag = np.abs(a) @ np.abs(b)
        u = 2.0 ** -24
        gamma = K * u / (1 - K * u)
        r = np.maximum(exact, 0.0)
        hi = r + gamma * mag
        # half an fp16 ulp at the largest value the result could take
        e = np.floor(np.log2(np.maximum(hi, 2.0 ** -14)))
        half_ulp = 2.0 ** (e - 11)
        got = as_f16(oracle.gemm_relu_full(A, B)).astype(np.float64)
        assert np.all(np.abs(got - r) <= gamma * mag + half_ulp + 1e-300)
        assert np.all(got >= 0)


# --- closed forms --------------------------------------------------------


@pytest.mark.parametrize("M,N,K", [(3, 5, 1024), (2, 4, 4096), (4, 3, 2050), (1, 2, 8192), (7, 9, 1)])
def test_all_ones_gives_K(M, N, K):
    A = np.full((M, K), 0x3C00, dtype=np.uint16)
    B = np.full((K, N), 0x3C00, dtype=np.uint16)
    C = oracle.gemm_relu_full(A, B)
    assert np.array_equal(as_f16(C).astype(np.float64), np.full((M, N), float(K)))


def test_minus_one_times_one_gives_zero():
    A = np.full((5, 33), 0xBC00, dtype=np.uint16)  # -1
    B = np.full((33, 6), 0x3C00, dtype=np.uint16)  # +1
    C = oracle.gemm_relu_full(A, B)
    assert np.all(C == 0x0000)


def test_identity_A_gives_relu_B():
    K = 37
    A = bits(np.eye(K))
    _, B = synth.random_operands(K, 19, K, seed=7)
    C = oracle.gemm_relu_full(A, B)
    expect = np.where(as_f16(B) > 0, B, np.uint16(0))
    assert np.array_equal(C, expect)


def test_diagonal_B_pins_rounding():
    """B = diag(d): C[i,j] = RNE(ReLU(a_ij * d_j)): one exact product, one
    rounding to fp16 (numpy's float64 -> float16 cast rounds once, RNE)."""
    M, K = 64, 48
    A, _ = synth.random_operands(M, K, K, seed=11)
    rng = np.random.default_rng(12)
    d = (rng.standard_normal(K) * 3).astype(np.float16)
    B = bits(np.diag(d.astype(np.float64)))
    C = oracle.gemm_relu_full(A, B)
    prod = as_f16(A).astype(np.float64) * d.astype(np.float64)[None, :]
    assert np.array_equal(C, bits(np.maximum(prod, 0.0)))


def test_rank1_powers_of_two():
    """A[i,k] = 2^p_i, B[k,j] = 2^q_j: C = K * 2^(p_i + q_j), exact."""
    M, N, K = 6, 7, 96
    p = np.arange(M) - 3
    q = np.arange(N) - 4
    A = bits(np.repeat((2.0 ** p)[:, None], K, axis=1))
    B = bits(np.repeat((2.0 ** q)[None, :], K, axis=0))
    C = oracle.gemm_relu_full(A, B)
    assert np.array_equal(as_f16(C).astype(np.float64), K * 2.0 ** (p[:, None] + q[None, :]))


def test_overflow_rounds_to_inf_and_nan_relu_to_zero():
    A = bits([[F16_MAX, F16_MAX], [np.inf, 1.0], [-np.inf, 1.0]])
    B = bits([[F16_MAX], [0.0]])
    C = oracle.gemm_relu_full(A, B)
    assert C[0, 0] == 0x7C00  # 65504^2 is finite in fp32, above the fp16 range
    assert C[1, 0] == 0x7C00  # +Inf survives ReLU
    assert C[2, 0] == 0x0000  # -Inf -> 0
    A2 = bits([[np.inf, 1.0]])
    B2 = bits([[0.0], [1.0]])  # inf * 0 = NaN -> ReLU gives +0
    assert oracle.gemm_relu_full(A2, B2)[0, 0] == 0x0000


def test_empty_and_k_zero():
    A = np.zeros((4, 0), dtype=np.uint16)
    B = np.zeros((0, 3), dtype=np.uint16)
    C = oracle.gemm_relu_full(A, B, M=4, N=3, K=0, lda=1, ldb=3)
    assert C.shape == (4, 3) and np.all(C == 0)
    assert oracle.gemm_relu_full(np.zeros((0, 5), np.uint16), np.zeros((5, 2), np.uint16)).shape == (0, 2)


# --- invariants ----------------------------------------------------------


def _rand(M, N, K, seed, **kw):
    return synth.random_operands(M, N, K, seed=seed, **kw)


def test_nonnegative_and_relu_agrees_with_product_sign():
    A, B = _rand(40, 50, 300, seed=21)
    C = as_f16(oracle.gemm_relu_full(A, B)).astype(np.float64)
    x = as_f16(A).astype(np.float64) @ as_f16(B).astype(np.float64)
    assert np.all(C >= 0) and not np.any(np.signbit(C))
    tol = 1e-2 + 1e-2 * np.abs(x)
    assert np.all(C[x < -tol] == 0)
    pos = x > tol
    assert np.all(np.abs(C[pos] - x[pos]) <= tol[pos])


def test_c_of_a_minus_c_of_minus_a_is_product():
    A, B = _rand(30, 20, 200, seed=22)
    negA = A ^ np.uint16(0x8000)
    C1 = as_f16(oracle.gemm_relu_full(A, B)).astype(np.float64)
    C2 = as_f16(oracle.gemm_relu_full(negA, B)).astype(np.float64)
    x = as_f16(A).astype(np.float64) @ as_f16(B).astype(np.float64)
    assert np.allclose(C1 - C2, x, rtol=1e-2, atol=1e-2)
    # at most one of the two is nonzero
    assert np.all((C1 == 0) | (C2 == 0))


def test_scaling_by_two_is_bitwise_on_normals():
    A, B = _rand(32, 48, 257, seed=23)
    A2 = bits(as_f16(A).astype(np.float64) * 2)  # exact: no input overflows
    C1 = as_f16(oracle.gemm_relu_full(A, B)).astype(np.float64)
    C2 = as_f16(oracle.gemm_relu_full(A2, B)).astype(np.float64)
    normal = (C1 >= 2.0 ** -14) & np.isfinite(C1) & (C1 * 2 <= F16_MAX)
    assert np.array_equal(C2[normal], 2 * C1[normal])
    sub = (C1 < 2.0 ** -14)
    assert np.all(np.abs(C2[sub] - 2 * C1[sub]) <= 2.0 ** -24)


def test_row_and_column_permutation_bitwise():
    A, B = _rand(25, 31, 129, seed=24)
    rng = np.random.default_rng(5)
    pr = rng.permutation(25)
    pc = rng.permutation(31)
    C = oracle.gemm_relu_full(A, B)
    assert np.array_equal(oracle.gemm_relu_full(np.ascontiguousarray(A[pr]), B), C[pr])
    assert np.array_equal(oracle.gemm_relu_full(A, np.ascontiguousarray(B[:, pc])), C[:, pc])


def test_k_permutation_within_tolerance():
    A, B = _rand(20, 20, 500, seed=25)
    pk = np.random.default_rng(6).permutation(500)
    C = as_f16(oracle.gemm_relu_full(A, B)).astype(np.float64)
    Cp = as_f16(oracle.gemm_relu_full(np.ascontiguousarray(A[:, pk]), np.ascontiguousarray(B[pk]))).astype(np.float64)
    assert np.all(np.abs(C - Cp) <= 1e-2 + 1e-2 * np.abs(C))


def test_transpose_identity_within_tolerance():
    """(A.B)^T = B^T.A^T: catches an operand transposed inside the loop."""
    A, B = _rand(23, 17, 90, seed=26)
    C = as_f16(oracle.gemm_relu_full(A, B)).astype(np.float64)
    Ct = as_f16(oracle.gemm_relu_full(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T))).astype(np.float64)
    assert np.all(np.abs(C.T - Ct) <= 1e-2 + 1e-2 * np.abs(C.T))


def test_padding_is_never_read():
    """Pitched operands whose padding holds 65504 give the packed result."""
    M, N, K = 19, 21, 70
    A, B = _rand(M, N, K, seed=27, lda=K + 9, ldb=N + 5)
    C = oracle.gemm_relu_full(A, B, M=M, N=N, K=K, lda=K + 9, ldb=N + 5)
    Ap = np.ascontiguousarray(A[:, :K])
    Bp = np.ascontiguousarray(B[:, :N])
    assert np.array_equal(C, oracle.gemm_relu_full(Ap, Bp))


def test_entry_points_agree_bitwise():
    M, N, K = 37, 29, 111
    A, B = _rand(M, N, K, seed=28, lda=K + 3, ldb=N + 1)
    kw = dict(M=M, N=N, K=K, lda=K + 3, ldb=N + 1)
    C = oracle.gemm_relu_full(A, B, **kw)
    rows = [0, 5, 36]
    cols = [0, 13, 28]
    assert np.array_equal(oracle.gemm_relu_rows(A, B, rows, **kw), C[rows])
    assert np.array_equal(oracle.gemm_relu_cols(A, B, cols, **kw), C[:, cols].T)
    ii, jj = synth.sample_indices(M, N, 200, seed=3)
    assert np.array_equal(oracle.gemm_relu_elems(A, B, ii, jj, **kw), C[ii, jj])


def test_threads_do_not_change_bits():
    A, B = _rand(64, 80, 333, seed=29)
    oracle.set_threads(1)
    C1 = oracle.gemm_relu_full(A, B)
    oracle.set_threads(max(2, oracle.max_threads()))
    C2 = oracle.gemm_relu_full(A, B)
    assert np.array_equal(C1, C2)
