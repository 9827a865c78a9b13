"""Pins for the oracle's MX fp4 entry points: E2M1 elements packed two per
byte (k even in the low nibble), one E8M0 scale per 32 consecutive k of each
row (OCP Microscaling formats: E2M1 = sign, 2 exponent bits with bias 1, 1
fraction bit; block size 32).

Checked against:
  * the E2M1 value table of the format (0, 0.5, 1, 1.5, 2, 3, 4, 6 and their
    negatives), all 16 codes;
  * the MX fp8 oracle (already pinned): every E2M1 value is exact in E4M3, so
    re-encoding each element as E4M3 with torch's own encoder and keeping the
    scales must give the same result bit for bit -- this pins the unpacking,
    the k indexing and the scale indexing (per 32 elements, not per 32 bytes);
  * brute force in float64 where every partial sum is exact in fp32;
  * block locality at the k = 31 / 32 boundary, inside one byte pair.
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.usefixtures("oracle_lib")

E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def pack(codes):
    """rows x K nibble codes -> rows x K/2 bytes, k even in the low nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    return np.ascontiguousarray(codes[:, 0::2] | (codes[:, 1::2] << 4))


def code_of(v):
    """E2M1 code of a table value (sign in bit 3)."""
    mag = E2M1_TABLE.index(abs(v))
    return mag | (8 if v < 0 else 0)


def values(codes):
    """float64 values of E2M1 codes, from the table."""
    return np.array([[(-1.0 if c & 8 else 1.0) * E2M1_TABLE[int(c) & 7] for c in row] for row in codes])


def e4m3_of_codes(codes):
    vals = values(codes).astype(np.float32)
    t = torch.from_numpy(vals).to(torch.float8_e4m3fn)
    assert np.array_equal(t.float().numpy(), vals)
    return t.view(torch.uint8).numpy()


def test_e2m1_decode_all_codes():
    got = oracle.e2m1_to_f32(np.arange(16, dtype=np.uint8))
    assert list(got[:8]) == E2M1_TABLE
    assert list(got[8:]) == [-v for v in E2M1_TABLE]
    assert np.signbit(got[8]) and not np.signbit(got[0])


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (3, 4, 64), (5, 7, 160), (8, 3, 256)])
def test_matches_mxfp8_oracle_bitwise(M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    ca = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    cb = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    sa = rng.integers(110, 140, size=(M, K // 32)).astype(np.uint8)
    sb = rng.integers(110, 140, size=(N, K // 32)).astype(np.uint8)
    for act in ("relu", "none", "gelu"):
        for fmt in ("f16", "bf16"):
            got = oracle.gemm_mxfp4_bt_full(pack(ca), sa, pack(cb), sb, fmt=fmt, act=act, K=K)
            ref = oracle.gemm_mxfp8_bt_full(e4m3_of_codes(ca), sa, e4m3_of_codes(cb), sb, fmt=fmt, act=act)
            assert np.array_equal(got, ref), (act, fmt)


def test_brute_force_exact_with_pitches():
    M, N, K = 6, 5, 96
    rng = np.random.default_rng(11)
    ca = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    cb = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    sa = rng.integers(124, 131, size=(M, K // 32)).astype(np.uint8)
    sb = rng.integers(124, 131, size=(N, K // 32)).astype(np.uint8)
    a = values(ca) * np.exp2(np.repeat(sa - 127.0, 32, axis=1))
    b = values(cb) * np.exp2(np.repeat(sb - 127.0, 32, axis=1))
    x = a @ b.T  # exact: small multiples of powers of two
    lda, ldbt, ldsa, ldsb = K // 2 + 8, K // 2 + 3, K // 32 + 1, K // 32 + 2
    A = np.full((M, lda), 0x77, np.uint8)   # 6.0 in both nibbles in the padding
    Bt = np.full((N, ldbt), 0x77, np.uint8)
    SA = np.full((M, ldsa), 255, np.uint8)
    SB = np.full((N, ldsb), 255, np.uint8)
    A[:, :K // 2], Bt[:, :K // 2], SA[:, :K // 32], SB[:, :K // 32] = pack(ca), pack(cb), sa, sb
    got = oracle.gemm_mxfp4_bt_full(A, SA, Bt, SB, act="none", M=M, N=N, K=K, lda=lda, ldsa=ldsa, ldbt=ldbt,
                                    ldsb=ldsb)
    assert np.array_equal(got, x.astype(np.float16).view(np.uint16))
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    e = oracle.gemm_mxfp4_bt_elems(A, SA, Bt, SB, ii.ravel(), jj.ravel(), act="none", M=M, N=N, K=K, lda=lda,
                                   ldsa=ldsa, ldbt=ldbt, ldsb=ldsb)
    assert np.array_equal(e.reshape(M, N), got)


@pytest.mark.parametrize("k", [30, 31, 32, 33])
def test_block_boundary(k):
    """One non-zero element of A at k; the scale of block k // 32 alone
    decides the result."""
    K = 64
    ca = np.zeros((1, K), np.uint8)
    ca[0, k] = code_of(1.5)
    cb = np.full((1, K), code_of(2.0), np.uint8)
    sa = np.array([[127 + 3, 127 - 2]], np.uint8)
    sb = np.array([[127, 127]], np.uint8)
    got = oracle.gemm_mxfp4_bt_full(pack(ca), sa, pack(cb), sb, act="none", K=K).view(np.float16)[0, 0]
    assert got == 3.0 * 2.0 ** (3 if k < 32 else -2)
