"""Pins for the oracle's general epilogue, C = act(A.B + bias).

The bias is a row vector broadcast down the columns and the activations are
those the elementwise pattern lists ("Tilelang Cuda Patterns", section 1:
relu, sigmoid, tanh, gelu), plus SiLU and the tanh form of GELU. None of these
tests retypes the oracle's formulas. They check it against:
  * exact results: integer inputs and an integer bias with no activation
    (the bias must land on columns, and negative sums must survive);
  * torch's own float64 activations (library routines), applied elementwise
    through A = I, where each output is one exact fp32 value x = b + bias;
  * identities of the functions (GELU(x) - GELU(-x) = x, SiLU likewise,
    sigmoid(x) + sigmoid(-x) = 1, tanh odd) and their limits;
  * the agreement of the four entry points.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.usefixtures("oracle_lib")

ACTS = ["none", "relu", "gelu", "gelu_tanh", "silu", "sigmoid", "tanh"]
F = torch.nn.functional
TORCH_ACT = {
    "none": lambda x: x,
    "relu": lambda x: torch.clamp(x, min=0.0),
    "gelu": lambda x: F.gelu(x),
    "gelu_tanh": lambda x: F.gelu(x, approximate="tanh"),
    "silu": F.silu,
    "sigmoid": torch.sigmoid,
    "tanh": torch.tanh,
}


def f16(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_f16_bits(x64):
    """float64 -> fp16, one correct rounding (numpy's direct conversion)."""
    return np.asarray(x64, dtype=np.float64).astype(np.float16).view(np.uint16)


def to_bf16_bits(x64):
    """float64 -> bfloat16, one correct rounding (normal range): scale the
    significand to 8 bits with frexp, round half to even with rint (exact in
    float64), scale back.  Going through fp32 first would round twice, and a
    sum of two bfloat16 values often sits exactly on a bfloat16 midpoint."""
    x = np.asarray(x64, dtype=np.float64)
    m, e = np.frexp(x)
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8).astype(np.float32)
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def identity_case(fmt, K=64, N=96, seed=3, scale=4.0):
    """A = I (K x K), B random, bias random: C[i][j] = act(fl32(B[i][j] + bias[j]))."""
    _, B = synth.random_operands(K, N, K, seed=seed, b_scale=scale, fmt=fmt)
    _, bias2 = synth.random_operands(1, N, 1, seed=seed + 1, b_scale=scale, fmt=fmt)
    bias = np.ascontiguousarray(bias2[0])
    one = 0x3C00 if fmt == "f16" else 0x3F80
    A = np.zeros((K, K), dtype=np.uint16)
    A[np.arange(K), np.arange(K)] = one
    wide = f16 if fmt == "f16" else bf16
    x32 = (wide(B).astype(np.float32) + wide(bias).astype(np.float32)[None, :])  # fp32 add, RNE
    return A, B, bias, x32


# --- exact results -----------------------------------------------------------


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("seed", range(4))
def test_integer_gemm_plus_bias_exact(fmt, seed):
    """No activation, integers in [-3,3] and a bias in [-50,50]: every partial
    sum is exact, so C = A.B + bias exactly (rounded once to the format), with
    its negative entries kept.  M != N, so a bias taken by row would fail."""
    rng = np.random.default_rng(300 + seed)
    for _ in range(20):
        M, N = int(rng.integers(1, 9)), int(rng.integers(1, 9))
        while N == M:
            N = int(rng.integers(1, 9))
        K = int(rng.integers(1, 40))
        a = rng.integers(-3, 4, size=(M, K)).astype(np.float64)
        b = rng.integers(-3, 4, size=(K, N)).astype(np.float64)
        bias = rng.integers(-50, 51, size=N).astype(np.float64)
        conv = to_f16_bits if fmt == "f16" else to_bf16_bits
        A, B, bb = conv(a), conv(b), conv(bias)
        C = oracle.gemm_relu_full(A, B, fmt=fmt, bias=bb, act="none")
        assert np.array_equal(C, conv(a @ b + bias[None, :])), (M, N, K)
        Cr = oracle.gemm_relu_full(A, B, fmt=fmt, bias=bb, act="relu")
        assert np.array_equal(Cr, conv(np.maximum(a @ b + bias[None, :], 0.0)))


def test_k_zero_gives_act_of_bias():
    N = 40
    bias = to_f16_bits(np.linspace(-6, 6, N))
    for act in ACTS:
        C = oracle.gemm_relu_full(np.zeros((3, 1), np.uint16), np.zeros((1, N), np.uint16), M=3, N=N, K=0,
                                  lda=1, ldb=N, bias=bias, act=act)
        ref = TORCH_ACT[act](torch.from_numpy(f16(bias))).numpy()
        assert np.array_equal(C, np.tile(to_f16_bits(ref), (3, 1))), act


# --- activations against torch's float64 implementations ----------------------


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_activation_matches_torch_float64(act, fmt):
    """Bit for bit wherever |act(x)| > 1e-6.  Below that torch's float64
    GELU forms lose their digits to the cancellation 1 + erf (1 + tanh) -> 0
    for x < -5, while the oracle keeps them; there the check is by size."""
    A, B, bias, x32 = identity_case(fmt)
    C = oracle.gemm_relu_full(A, B, fmt=fmt, bias=bias, act=act)
    y = TORCH_ACT[act](torch.from_numpy(x32.astype(np.float64))).numpy()
    ref = to_f16_bits(y) if fmt == "f16" else to_bf16_bits(y)
    if act == "relu":  # ReLU gives +0 for every x <= 0
        ref = np.where(x32 > 0, ref, np.uint16(0))
    big = np.abs(y) > 1e-6
    assert big.mean() > 0.4
    assert np.array_equal(C[big], ref[big])
    wide = f16 if fmt == "f16" else bf16
    assert np.all(np.abs(wide(C[~big])) <= 1.01e-6)


@pytest.mark.parametrize("act", ["gelu", "gelu_tanh", "silu", "sigmoid", "tanh"])
def test_activation_wide_range_and_limits(act):
    """x from -60 to 60: the limits (sigmoid -> 0 or 1, tanh -> +-1, GELU and
    SiLU -> 0 or x) round exactly as torch's float64 functions say."""
    K, N = 1, 241
    x = np.linspace(-60, 60, N)
    A = np.full((1, K), 0x3C00, np.uint16)
    B = to_f16_bits(x)[None, :].copy()
    C = oracle.gemm_relu_full(A, B, act=act)
    y = TORCH_ACT[act](torch.from_numpy(f16(B[0]))).numpy()
    assert np.array_equal(f16(C[0]), f16(to_f16_bits(y)))  # by value: -0 and +0 agree


# --- identities ----------------------------------------------------------------


def _pm(fmt="f16", act="gelu"):
    A, B, _, _ = identity_case(fmt, seed=9, scale=3.0)
    Bn = B ^ np.uint16(0x8000)
    wide = f16 if fmt == "f16" else bf16
    return (wide(oracle.gemm_relu_full(A, B, fmt=fmt, act=act)), wide(oracle.gemm_relu_full(A, Bn, fmt=fmt, act=act)),
            wide(B))


@pytest.mark.parametrize("act", ["gelu", "silu", "gelu_tanh"])
def test_odd_part_is_identity(act):
    """GELU(x) - GELU(-x) = x Phi(x) + x Phi(-x) = x; SiLU and the tanh GELU
    likewise (x s(x) + x s(-x) = x)."""
    cp, cn, x = _pm(act=act)
    assert np.all(np.abs((cp - cn) - x) <= 2e-3 * np.maximum(np.abs(x), 1.0))


def test_sigmoid_symmetry_and_tanh_odd():
    cp, cn, _ = _pm(act="sigmoid")
    assert np.all(np.abs(cp + cn - 1.0) <= 1e-3)
    tp, tn, _ = _pm(act="tanh")
    assert np.array_equal(tp, -tn)  # tanh is odd and the rounding is symmetric


def test_gelu_forms_close():
    """The tanh form approximates x Phi(x) to within 1e-3 on this range."""
    g, _, x = _pm(act="gelu")
    gt, _, _ = _pm(act="gelu_tanh")
    assert np.all(np.abs(g - gt) <= 1e-3 + 2 ** -10 * np.abs(g))


def test_zero_points():
    """act(0): GELU, SiLU, tanh, identity 0; sigmoid 1/2."""
    A = np.zeros((2, 8), np.uint16)
    B = np.zeros((8, 3), np.uint16)
    for act in ACTS:
        C = f16(oracle.gemm_relu_full(A, B, act=act))
        assert np.all(C == (0.5 if act == "sigmoid" else 0.0)), act


def test_overflow_without_activation_goes_to_inf():
    A = to_f16_bits([[60000.0, 60000.0]])
    B = to_f16_bits([[1.0], [1.0]])
    C = oracle.gemm_relu_full(A, B, act="none", bias=to_f16_bits([-1000.0]))
    assert C[0, 0] == 0x7C00  # 119000 is above the fp16 range
    C = oracle.gemm_relu_full(A * 0 + to_f16_bits([[-60000.0]]), B, act="none")
    assert C[0, 0] == 0xFC00


# --- entry points ------------------------------------------------------------------


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_entry_points_agree_bitwise(fmt):
    M, N, K = 29, 37, 91
    A, B = synth.random_operands(M, N, K, seed=41, lda=K + 5, ldb=N + 3, fmt=fmt)
    _, b2 = synth.random_operands(1, N, 1, seed=42, fmt=fmt)
    bias = np.ascontiguousarray(b2[0])
    for act in ("gelu", "silu", "none"):
        kw = dict(M=M, N=N, K=K, lda=K + 5, ldb=N + 3, fmt=fmt, bias=bias, act=act)
        C = oracle.gemm_relu_full(A, B, **kw)
        rows, cols = [0, 7, 28], [0, 19, 36]
        assert np.array_equal(oracle.gemm_relu_rows(A, B, rows, **kw), C[rows])
        assert np.array_equal(oracle.gemm_relu_cols(A, B, cols, **kw), C[:, cols].T)
        ii, jj = synth.sample_indices(M, N, 150, seed=4)
        assert np.array_equal(oracle.gemm_relu_elems(A, B, ii, jj, **kw), C[ii, jj])


def test_relu_with_zero_bias_is_the_fused_relu():
    A, B = synth.random_operands(33, 45, 70, seed=43)
    zero = np.zeros(45, np.uint16)
    assert np.array_equal(oracle.gemm_relu_full(A, B, bias=zero, act="relu"), oracle.gemm_relu_full(A, B))


def test_bad_arguments_rejected():
    A, B = synth.random_operands(2, 3, 2, seed=1)
    with pytest.raises(ValueError):
        oracle.gemm_relu_full(A, B, act="swish")
    with pytest.raises(ValueError):
        oracle.gemm_relu_full(A, B, bias=np.zeros(2, np.uint16), act="none")
    with pytest.raises(TypeError):
        oracle.gemm_relu_full(A, B, bias=np.zeros(3, np.float32), act="none")
