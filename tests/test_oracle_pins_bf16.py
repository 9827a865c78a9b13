"""Pins for the oracle's bfloat16 variant, each independent of the oracle's code.

With bfloat16 operands and result the oracle computes
C = bf16_RNE(ReLU(fp32 sum_k A.B)): the same fp32 accumulation and ReLU as the
fp16 GEMM+ReLU listings (blog "TileLang programming basics", section 2;
"Writing high-performance kernels in TileLang", section "Writing a GEMM"), the
element format swapped for bfloat16 (TileLang tutorial, section
"张量核与 CUDA core": GEMM inputs go to the matrix engines as fp16 or bf16).
The checks:
  * torch's own bfloat16 <-> fp32 conversions (library routines): every
    bfloat16 pattern, every midpoint between neighbours, random fp32 patterns;
  * exact results: integer-valued inputs whose partial sums are exact in fp32,
    rounded once to bfloat16 by torch;
  * float64 results with a proven fp32 accumulation bound plus half a bfloat16
    ulp;
  * closed forms whose rounding to bfloat16 is worked out by hand (all-ones
    sums of 257, 259 and 2050 round to 256, 260 and 2048);
  * invariants and the agreement of the four entry points.
A slip such as widening bfloat16 bits as fp16, truncating instead of rounding,
or rounding before the ReLU fails at least one of them.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.usefixtures("oracle_lib")

BF16_MAX = float(torch.finfo(torch.bfloat16).max)


def to_f64(bits):
    """bfloat16 bits -> float64 through torch."""
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def bits_from_f32(x):
    """fp32 values -> bfloat16 bits, rounded by torch (nearest, ties to even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bits_exact(x):
    """Values exactly representable in bfloat16 -> bits (asserts exactness)."""
    x = np.asarray(x, dtype=np.float64)
    b = bits_from_f32(x.astype(np.float32))
    assert np.array_equal(to_f64(b), x)
    return b


def gemm(A, B, **kw):
    return oracle.gemm_relu_full(A, B, fmt="bf16", **kw)


# --- conversions ---------------------------------------------------------


def test_bf16_to_f32_exhaustive_vs_torch():
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_to_f32(allbits)
    ref = torch.from_numpy(allbits.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f32_to_bf16_rne_boundaries_vs_torch():
    """Every finite bfloat16 value, every midpoint of neighbours (ties), and the
    fp32 neighbours of each midpoint, both signs."""
    allbits = np.arange(0, 0x7F81, dtype=np.uint32).astype(np.uint16)  # +0 .. +Inf
    vals = oracle.bf16_to_f32(allbits).astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2
    mids = mids[np.isfinite(mids)]
    mids32 = mids.astype(np.float32)
    assert np.array_equal(mids32.astype(np.float64), mids)  # midpoints fit fp32
    up = np.nextafter(mids32, np.float32(np.inf))
    dn = np.nextafter(mids32, np.float32(0))
    pos = np.concatenate([vals[np.isfinite(vals)].astype(np.float32), mids32, up, dn,
                          np.array([np.inf, np.finfo(np.float32).max, 1e-45], np.float32)])
    v = np.concatenate([pos, -pos])
    assert np.array_equal(oracle.f32_to_bf16(v), bits_from_f32(v))


def test_f32_to_bf16_rne_random_vs_torch():
    rng = np.random.default_rng(4321)
    u = rng.integers(0, 2 ** 32, size=10_000_000, dtype=np.uint64).astype(np.uint32)
    v = u.view(np.float32)
    v = v[~np.isnan(v)]
    assert np.array_equal(oracle.f32_to_bf16(v), bits_from_f32(v))


def test_f32_to_bf16_hand_cases():
    """Worked by hand: 1 + 2^-8 is the midpoint of 1 and 1 + 2^-7 (tie, even ->
    1.0 = 0x3F80); 1 + 3*2^-8 is the midpoint of 1 + 2^-7 and 1 + 2^-6 (tie,
    even -> 1 + 2^-6 = 0x3F82); anything just past the largest finite midpoint
    goes to +Inf."""
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -(1 + 2 ** -8)], np.float32)
    assert list(oracle.f32_to_bf16(x)) == [0x3F80, 0x3F82, 0x3F81, 0xBF80]
    top = np.float32(BF16_MAX + 2.0 ** (127 - 8))  # midpoint of max and the next step
    assert oracle.f32_to_bf16(np.array([top], np.float32))[0] == 0x7F80
    nan = np.array([np.nan, -np.nan], np.float32)
    assert np.all(np.isnan(oracle.bf16_to_f32(oracle.f32_to_bf16(nan))))


# --- exact results -------------------------------------------------------


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_tiny_integer_exact(seed):
    """Integer inputs in [-3,3] (exact in bfloat16), K <= 64: every partial sum
    is an integer below 2^10, exact in fp32 in any order; the result is the
    float64 product, ReLU'd and rounded once to bfloat16 (sums above 256 do
    round: bfloat16 keeps 8 significant bits)."""
    rng = np.random.default_rng(50 + seed)
    for _ in range(40):
        M, N, K = (int(x) for x in rng.integers(1, 9, size=3))
        if seed >= 3:
            K = int(rng.integers(9, 65))
        r2 = np.random.default_rng(int(rng.integers(1 << 30)))
        a = r2.integers(-3, 4, size=(M, K)).astype(np.float32)
        b = r2.integers(-3, 4, size=(K, N)).astype(np.float32)
        A, B = bits_exact(a), bits_exact(b)
        ref = np.maximum(a.astype(np.float64) @ b.astype(np.float64), 0.0)
        assert np.array_equal(gemm(A, B), bits_from_f32(ref.astype(np.float32))), (M, N, K)


def test_large_integer_sums_round_in_output_only():
    """All partial sums stay exact in fp32 while the outputs need rounding:
    A = 3 everywhere, B = 1 everywhere, K = 683: C = 2049, which bfloat16 holds
    only to 16 (2048 < 2049 < 2064), so it rounds down to 2048."""
    A = np.full((2, 683), 0x4040, dtype=np.uint16)  # 3.0
    B = np.full((683, 3), 0x3F80, dtype=np.uint16)  # 1.0
    assert np.all(to_f64(gemm(A, B)) == 2048.0)


@pytest.mark.parametrize("seed", range(4))
def test_random_bf16_within_proven_bound(seed):
    """|s32 - s| <= gamma_K sum|a b| (recursive summation, exact products) plus
    half a bfloat16 ulp (2^(e-8)) of the result for the final rounding."""
    rng = np.random.default_rng(200 + seed)
    for _ in range(30):
        M, N = (int(x) for x in rng.integers(1, 12, size=2))
        K = int(rng.integers(1, 300))
        A, B = synth.random_operands(M, N, K, seed=int(rng.integers(1 << 30)), fmt="bf16")
        a, b = to_f64(A), to_f64(B)
        exact = a @ b
        mag = np.abs(a) @ np.abs(b)
        u = 2.0 ** -24
        gamma = K * u / (1 - K * u)
        r = np.maximum(exact, 0.0)
        hi = r + gamma * mag
        e = np.floor(np.log2(np.maximum(hi, 2.0 ** -126)))
        half_ulp = 2.0 ** (e - 8)
        got = to_f64(gemm(A, B))
        assert np.all(np.abs(got - r) <= gamma * mag + half_ulp + 1e-300)
        assert np.all(got >= 0)


# --- closed forms --------------------------------------------------------


@pytest.mark.parametrize("K,expect", [(1, 1.0), (256, 256.0), (257, 256.0), (259, 260.0), (1024, 1024.0),
                                      (2050, 2048.0), (2056, 2048.0), (2057, 2064.0), (8192, 8192.0)])
def test_all_ones_sum_rounds_by_hand(K, expect):
    """sum of K ones is exactly K in fp32; bfloat16 spacing is 2 on [256, 512)
    and 16 on [2048, 4096): 257 ties to even 256, 259 ties to even 260, 2050
    rounds down, 2056 ties to even 2048, 2057 rounds up to 2064."""
    A = np.full((3, K), 0x3F80, dtype=np.uint16)
    B = np.full((K, 2), 0x3F80, dtype=np.uint16)
    assert np.all(to_f64(gemm(A, B)) == expect)


def test_bf16_bits_are_not_read_as_fp16():
    """0x4000 is 2.0 in bfloat16 but 2.0 in fp16 as well; 0x3F80 is 1.0 in
    bfloat16 and 1.875 in fp16: a format mix-up changes the result."""
    A = np.full((1, 4), 0x3F80, dtype=np.uint16)
    B = np.full((4, 1), 0x4000, dtype=np.uint16)
    assert to_f64(gemm(A, B))[0, 0] == 8.0
    assert oracle.gemm_relu_full(A, B)[0, 0] != gemm(A, B)[0, 0]


def test_identity_A_gives_relu_B():
    K = 37
    A = bits_exact(np.eye(K))
    _, B = synth.random_operands(K, 19, K, seed=7, fmt="bf16")
    expect = np.where(to_f64(B) > 0, B, np.uint16(0))
    assert np.array_equal(gemm(A, B), expect)


def test_diagonal_B_pins_rounding():
    """B = diag(d): C[i,j] = RNE(ReLU(a_ij d_j)); the product of two bfloat16
    values is exact in fp32 (16 significant bits), then rounded once by torch."""
    M, K = 64, 48
    A, _ = synth.random_operands(M, K, K, seed=11, fmt="bf16")
    rng = np.random.default_rng(13)
    d = bits_from_f32((rng.standard_normal(K) * 3).astype(np.float32))
    B = bits_exact(np.diag(to_f64(d)))
    prod = to_f64(A) * to_f64(d)[None, :]
    assert np.array_equal(gemm(A, B), bits_from_f32(np.maximum(prod, 0.0).astype(np.float32)))


def test_rank1_powers_of_two_beyond_fp16_range():
    """A[i,k] = 2^p_i, B[k,j] = 2^q_j with exponents far outside fp16's range:
    C = K 2^(p_i + q_j), exact."""
    M, N, K = 6, 7, 64
    p = np.arange(M) * 9 - 40
    q = np.arange(N) * 7 - 10
    A = bits_exact(np.repeat((2.0 ** p)[:, None], K, axis=1))
    B = bits_exact(np.repeat((2.0 ** q)[None, :], K, axis=0))
    assert np.array_equal(to_f64(gemm(A, B)), K * 2.0 ** (p[:, None] + q[None, :]))


def test_overflow_to_inf_and_nan_relu_to_zero():
    A = bits_exact([[BF16_MAX, BF16_MAX], [np.inf, 1.0], [-np.inf, 1.0]])
    B = bits_exact([[BF16_MAX], [0.0]])
    C = gemm(A, B)
    assert C[0, 0] == 0x7F80  # BF16_MAX^2 overflows fp32 -> +Inf
    assert C[1, 0] == 0x7F80
    assert C[2, 0] == 0x0000
    A2 = bits_exact([[np.inf, 1.0]])
    B2 = bits_exact([[0.0], [1.0]])  # inf * 0 = NaN -> ReLU gives +0
    assert gemm(A2, B2)[0, 0] == 0x0000


def test_tiny_negative_gives_plus_zero():
    """ReLU comes before the rounding: a tiny negative sum gives +0 (0x0000),
    not -0 (0x8000)."""
    A = bits_exact([[1.0, -1.0]])
    B = bits_exact([[2.0 ** -130], [2.0 ** -129]])
    assert gemm(A, B)[0, 0] == 0x0000


# --- invariants ----------------------------------------------------------


def test_row_and_column_permutation_bitwise():
    A, B = synth.random_operands(25, 31, 129, seed=24, fmt="bf16")
    rng = np.random.default_rng(5)
    pr = rng.permutation(25)
    pc = rng.permutation(31)
    C = gemm(A, B)
    assert np.array_equal(gemm(np.ascontiguousarray(A[pr]), B), C[pr])
    assert np.array_equal(gemm(A, np.ascontiguousarray(B[:, pc])), C[:, pc])


def test_transpose_identity_within_tolerance():
    A, B = synth.random_operands(23, 17, 90, seed=26, fmt="bf16")
    C = to_f64(gemm(A, B))
    Ct = to_f64(gemm(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T)))
    assert np.all(np.abs(C.T - Ct) <= 2e-2 + 2e-2 * np.abs(C.T))


def test_padding_is_never_read():
    M, N, K = 19, 21, 70
    A, B = synth.random_operands(M, N, K, seed=27, lda=K + 9, ldb=N + 5, fmt="bf16")
    C = gemm(A, B, M=M, N=N, K=K, lda=K + 9, ldb=N + 5)
    assert np.array_equal(C, gemm(np.ascontiguousarray(A[:, :K]), np.ascontiguousarray(B[:, :N])))


def test_entry_points_agree_bitwise():
    M, N, K = 37, 29, 111
    A, B = synth.random_operands(M, N, K, seed=28, lda=K + 3, ldb=N + 1, fmt="bf16")
    kw = dict(M=M, N=N, K=K, lda=K + 3, ldb=N + 1, fmt="bf16")
    C = oracle.gemm_relu_full(A, B, **kw)
    rows = [0, 5, 36]
    cols = [0, 13, 28]
    assert np.array_equal(oracle.gemm_relu_rows(A, B, rows, **kw), C[rows])
    assert np.array_equal(oracle.gemm_relu_cols(A, B, cols, **kw), C[:, cols].T)
    ii, jj = synth.sample_indices(M, N, 200, seed=3)
    assert np.array_equal(oracle.gemm_relu_elems(A, B, ii, jj, **kw), C[ii, jj])


def test_unknown_format_rejected():
    A, B = synth.random_operands(2, 2, 2, seed=1)
    with pytest.raises(ValueError):
        oracle.gemm_relu_full(A, B, fmt="f32")
