"""Pins for the oracle's fp8 entry points: C = act(sa * sb * (A . Bt^T) + bias)
with A and Bt in OCP fp8 E4M3 (B given transposed), fp32 accumulation.

Checked against:
  * torch's own float8_e4m3fn -> float32 conversion, all 256 codes;
  * the fp16 oracle (already pinned): every E4M3 value is exact in fp16, so
    the fp8 product with unit scales must equal, bit for bit, the fp16
    oracle on the same values with B = Bt^T (this pins the decoding, the
    transposed indexing and the accumulation together);
  * exact integer results, and power-of-two scales (exact);
  * a general scale within the proven accumulation bound of float64;
  * NaN codes: ReLU maps them to +0, the identity keeps a NaN.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.usefixtures("oracle_lib")


def e4m3_bits(x):
    """float values exactly representable in E4M3 -> bits (asserts exactness)."""
    t = torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    back = t.float().numpy()
    assert np.array_equal(back, np.asarray(x, dtype=np.float32))
    return t.view(torch.uint8).numpy()


def f16_of_e4m3(bits):
    return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.float8_e4m3fn).to(torch.float16) \
        .view(torch.int16).numpy().view(np.uint16)


def test_e4m3_decode_all_codes_vs_torch():
    b = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_to_f32(b)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


@pytest.mark.parametrize("seed", range(4))
def test_matches_fp16_oracle_bitwise(seed):
    """Unit scales, no bias: the fp8 GEMM is the fp16 GEMM of the same values."""
    rng = np.random.default_rng(400 + seed)
    for _ in range(10):
        M, N = (int(x) for x in rng.integers(1, 20, size=2))
        K = int(rng.integers(1, 200))
        A, Bt = synth.fp8_operands(M, N, K, seed=int(rng.integers(1 << 30)), scale_b=0.5)
        C8 = oracle.gemm_fp8_bt_full(A, Bt)
        A16 = f16_of_e4m3(A)
        B16 = np.ascontiguousarray(f16_of_e4m3(Bt).T)
        assert np.array_equal(C8, oracle.gemm_relu_full(A16, B16)), (M, N, K)
        for act in ("gelu", "none"):
            assert np.array_equal(oracle.gemm_fp8_bt_full(A, Bt, act=act), oracle.gemm_relu_full(A16, B16, act=act))


def test_pitched_operands_and_padding_never_read():
    M, N, K = 13, 17, 70
    A, Bt = synth.fp8_operands(M, N, K, seed=5, lda=K + 10, ldbt=K + 3)
    C = oracle.gemm_fp8_bt_full(A, Bt, M=M, N=N, K=K, lda=K + 10, ldbt=K + 3)
    Ap = np.ascontiguousarray(A[:, :K])
    Bp = np.ascontiguousarray(Bt[:, :K])
    assert np.array_equal(C, oracle.gemm_fp8_bt_full(Ap, Bp))


@pytest.mark.parametrize("sa,sb", [(1.0, 1.0), (0.5, 0.25), (4.0, 0.125)])
def test_integer_inputs_and_power_of_two_scales_exact(sa, sb):
    """Integers in [-4, 4]: partial sums exact; a power-of-two scale is exact;
    |sum * sa * sb| <= 2048 is exact in fp16, so C is the exact value."""
    rng = np.random.default_rng(7)
    for _ in range(20):
        M, N, K = (int(x) for x in rng.integers(1, 10, size=3))
        K = K * 7
        a = rng.integers(-4, 5, size=(M, K)).astype(np.float64)
        b = rng.integers(-4, 5, size=(N, K)).astype(np.float64)
        C = oracle.gemm_fp8_bt_full(e4m3_bits(a), e4m3_bits(b), sa, sb, act="none")
        ref = (a @ b.T) * sa * sb
        assert np.array_equal(C.view(np.float16).astype(np.float64), ref), (M, N, K)


def test_general_scale_within_bound():
    """sa = 0.3, sb = 1.7 (not powers of two): within the fp32 accumulation
    bound plus the two roundings of the scale and half an fp16 ulp."""
    M, N, K = 20, 30, 500
    A, Bt = synth.fp8_operands(M, N, K, seed=9)
    a = oracle.e4m3_to_f32(A).astype(np.float64)
    b = oracle.e4m3_to_f32(Bt).astype(np.float64)
    sa, sb = 0.3, 1.7
    s64 = float(np.float32(sa)) * float(np.float32(sb))
    exact = (a @ b.T) * s64
    mag = (np.abs(a) @ np.abs(b).T) * abs(s64)
    u = 2.0 ** -24
    gamma = (K + 2) * u / (1 - (K + 2) * u)
    got = oracle.gemm_fp8_bt_full(A, Bt, sa, sb, act="none").view(np.float16).astype(np.float64)
    half_ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(exact) + gamma * mag, 2.0 ** -14))) - 11)
    assert np.all(np.abs(got - exact) <= gamma * mag + half_ulp)


def test_bias_and_bf16_output():
    M, N, K = 9, 11, 64
    A, Bt = synth.fp8_operands(M, N, K, seed=10)
    A16 = f16_of_e4m3(A)
    B16 = np.ascontiguousarray(f16_of_e4m3(Bt).T)
    bias16 = np.linspace(-2, 2, N).astype(np.float16).view(np.uint16)
    got = oracle.gemm_fp8_bt_full(A, Bt, bias=bias16, act="silu")
    assert np.array_equal(got, oracle.gemm_relu_full(A16, B16, bias=bias16, act="silu"))
    # bfloat16 output of the same sums: every E4M3 value is exact in bfloat16 too
    Ab = torch.from_numpy(A).view(torch.float8_e4m3fn).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    Bb = torch.from_numpy(np.ascontiguousarray(Bt.T)).view(torch.float8_e4m3fn).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)
    biasb = torch.linspace(-2, 2, N).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got_b = oracle.gemm_fp8_bt_full(A, Bt, fmt="bf16", bias=biasb, act="gelu")
    assert np.array_equal(got_b, oracle.gemm_relu_full(Ab, Bb, fmt="bf16", bias=biasb, act="gelu"))


def test_nan_codes():
    A = np.array([[0x7F, 0x38]], dtype=np.uint8)  # NaN, 1.0
    Bt = np.array([[0x38, 0x38]], dtype=np.uint8)
    assert oracle.gemm_fp8_bt_full(A, Bt)[0, 0] == 0x0000  # ReLU(NaN) = +0
    assert np.isnan(oracle.gemm_fp8_bt_full(A, Bt, act="none").view(np.float16)[0, 0])


def test_k_zero_and_elems_agree():
    bias = np.linspace(-1, 1, 6).astype(np.float16).view(np.uint16)
    C = oracle.gemm_fp8_bt_full(np.zeros((4, 1), np.uint8), np.zeros((6, 1), np.uint8), M=4, N=6, K=0, lda=1, ldbt=1,
                                bias=bias, act="sigmoid")
    ref = torch.sigmoid(torch.from_numpy(bias.view(np.float16).astype(np.float64))).numpy().astype(np.float16)
    assert np.array_equal(C, np.tile(ref.view(np.uint16), (4, 1)))
    A, Bt = synth.fp8_operands(23, 19, 130, seed=11, lda=136, ldbt=144)
    kw = dict(M=23, N=19, K=130, lda=136, ldbt=144, scale_a=0.7, scale_b=0.9, act="tanh")
    C = oracle.gemm_fp8_bt_full(A, Bt, **kw)
    ii, jj = synth.sample_indices(23, 19, 100, seed=2)
    assert np.array_equal(oracle.gemm_fp8_bt_elems(A, Bt, ii, jj, **kw), C[ii, jj])
