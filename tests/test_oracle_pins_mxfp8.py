"""Pins for the oracle's MX fp8 entry points: C = act(sum_k a * 2^(sa-127) *
bt * 2^(sb-127) + bias), A and Bt in OCP fp8 E4M3, one E8M0 scale per 32
consecutive k of each row (OCP Microscaling formats: block size 32, scale
2^(x-127), code 255 = NaN).

Checked against:
  * Python's own power of two for all 256 scale codes;
  * brute force in float64 numpy on small-integer operands with scales in a
    narrow range, where every product and every partial sum is exact in fp32,
    so the oracle must agree bit for bit (any slip in which block, which row
    or which operand a scale belongs to changes the result);
  * block locality: raising one scale code by one doubles exactly the
    contribution of that one block of that one row;
  * unit scales (code 127): the MX product is the per-tensor fp8 product,
    itself pinned against the fp16 oracle;
  * a NaN scale poisons exactly the outputs whose sum uses it.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.usefixtures("oracle_lib")


def e4m3_bits(x):
    t = torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    assert np.array_equal(t.float().numpy(), np.asarray(x, dtype=np.float32))
    return t.view(torch.uint8).numpy()


def f16_bits(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def test_e8m0_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e8m0_to_f64(codes)
    assert math.isnan(got[255])
    for x in range(255):
        assert got[x] == 2.0 ** (x - 127), x
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and got[254] == 2.0 ** 127


def small_int_case(M, N, K, seed, lo=124, hi=130):
    """E4M3 operands drawn from the integers -4..4 and scales in [lo, hi]."""
    rng = np.random.default_rng(seed)
    a = rng.integers(-4, 5, size=(M, K)).astype(np.float32)
    b = rng.integers(-4, 5, size=(N, K)).astype(np.float32)
    sa = rng.integers(lo, hi + 1, size=(M, K // 32)).astype(np.uint8)
    sb = rng.integers(lo, hi + 1, size=(N, K // 32)).astype(np.uint8)
    return a, b, sa, sb


def brute(a, b, sa, sb):
    """float64 (sum is exact here): expand each scale over its 32 k."""
    ea = np.repeat(sa.astype(np.float64) - 127.0, 32, axis=1)
    eb = np.repeat(sb.astype(np.float64) - 127.0, 32, axis=1)
    return (a.astype(np.float64) * np.exp2(ea)) @ (b.astype(np.float64) * np.exp2(eb)).T


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (3, 5, 64), (7, 2, 96), (9, 11, 160), (4, 4, 256)])
def test_brute_force_exact(M, N, K):
    a, b, sa, sb = small_int_case(M, N, K, seed=M * 1000 + N * 10 + K)
    A, Bt = e4m3_bits(a), e4m3_bits(b)
    x = brute(a, b, sa, sb)
    # |x| <= K * 16 * 2^6 and granularity 2^-6: every partial sum is exact in fp32
    for act, ref in (("none", x), ("relu", np.maximum(x, 0.0))):
        got = oracle.gemm_mxfp8_bt_full(A, sa, Bt, sb, act=act)
        assert np.array_equal(got, f16_bits(ref)), act
    got = oracle.gemm_mxfp8_bt_full(A, sa, Bt, sb, fmt="bf16", act="none")
    ref = torch.tensor(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_pitches_and_elems():
    """Row pitches of A, Bt and both scale arrays beyond their widths; the
    single-element entry point gives the same values."""
    M, N, K = 5, 6, 128
    a, b, sa, sb = small_int_case(M, N, K, seed=7)
    lda, ldbt, ldsa, ldsb = K + 16, K + 48, K // 32 + 3, K // 32 + 1
    A = np.full((M, lda), 0x7F, np.uint8)   # NaN codes in the padding must not be read
    Bt = np.full((N, ldbt), 0x7F, np.uint8)
    SA = np.full((M, ldsa), 255, np.uint8)  # NaN scales in the padding
    SB = np.full((N, ldsb), 255, np.uint8)
    A[:, :K], Bt[:, :K], SA[:, :K // 32], SB[:, :K // 32] = e4m3_bits(a), e4m3_bits(b), sa, sb
    got = oracle.gemm_mxfp8_bt_full(A, SA, Bt, SB, act="none", M=M, N=N, K=K, lda=lda, ldsa=ldsa, ldbt=ldbt,
                                    ldsb=ldsb)
    assert np.array_equal(got, f16_bits(brute(a, b, sa, sb)))
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    e = oracle.gemm_mxfp8_bt_elems(A, SA, Bt, SB, ii.ravel(), jj.ravel(), act="none", M=M, N=N, K=K, lda=lda,
                                   ldsa=ldsa, ldbt=ldbt, ldsb=ldsb)
    assert np.array_equal(e.reshape(M, N), got)


@pytest.mark.parametrize("blk", [0, 1, 3])
def test_one_scale_scales_one_block_of_one_row(blk):
    """Only block blk of row 1 of A is non-zero; its scale code + 1 doubles
    row 1 exactly and leaves every other row at zero."""
    M, N, K = 3, 4, 128
    rng = np.random.default_rng(blk)
    a = np.zeros((M, K), np.float32)
    a[1, 32 * blk:32 * blk + 32] = rng.integers(1, 5, size=32)
    b = rng.integers(-3, 4, size=(N, K)).astype(np.float32)
    sa = np.full((M, K // 32), 127, np.uint8)
    sb = rng.integers(125, 130, size=(N, K // 32)).astype(np.uint8)
    A, Bt = e4m3_bits(a), e4m3_bits(b)
    base = oracle.gemm_mxfp8_bt_full(A, sa, Bt, sb, act="none").view(np.float16).astype(np.float64)
    sa2 = sa.copy()
    sa2[1, blk] += 1
    up = oracle.gemm_mxfp8_bt_full(A, sa2, Bt, sb, act="none").view(np.float16).astype(np.float64)
    assert np.array_equal(up[1], 2.0 * base[1]) and np.any(base[1] != 0)
    assert not np.any(up[[0, 2]]) and not np.any(base[[0, 2]])
    sa3 = sa.copy()
    sa3[1, (blk + 1) % 4] = 200          # a block of zeros: its scale changes nothing
    sa3[0, blk] = 200                    # a row of zeros
    assert np.array_equal(oracle.gemm_mxfp8_bt_full(A, sa3, Bt, sb, act="none").view(np.float16), base)


@pytest.mark.parametrize("seed", range(3))
def test_unit_scales_are_the_per_tensor_product(seed):
    rng = np.random.default_rng(900 + seed)
    M, N = (int(x) for x in rng.integers(1, 24, size=2))
    K = 32 * int(rng.integers(1, 9))
    A, Bt = synth.fp8_operands(M, N, K, seed=seed + 5)
    ones_a = np.full((M, K // 32), 127, np.uint8)
    ones_b = np.full((N, K // 32), 127, np.uint8)
    for act in ("relu", "gelu", "none"):
        assert np.array_equal(oracle.gemm_mxfp8_bt_full(A, ones_a, Bt, ones_b, act=act),
                              oracle.gemm_fp8_bt_full(A, Bt, act=act))


def test_nan_scale():
    M, N, K = 2, 3, 64
    a, b, sa, sb = small_int_case(M, N, K, seed=3, lo=126, hi=128)
    a[:] = 1.0
    sb = sb.copy()
    sb[2, 1] = 255
    got = oracle.gemm_mxfp8_bt_full(e4m3_bits(a), sa, e4m3_bits(b), sb, act="none").view(np.float16)
    assert np.all(np.isnan(got[:, 2])) and not np.any(np.isnan(got[:, :2]))
    relu = oracle.gemm_mxfp8_bt_full(e4m3_bits(a), sa, e4m3_bits(b), sb, act="relu")
    assert np.all(relu[:, 2] == 0)


def test_rejects_k_not_a_multiple_of_32():
    with pytest.raises(ValueError):
        oracle.gemm_mxfp8_bt_full(np.zeros((2, 40), np.uint8), np.zeros((2, 2), np.uint8),
                                  np.zeros((2, 40), np.uint8), np.zeros((2, 2), np.uint8))
