"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of C = ReLU(A.B): it only draws operands. Both
the CPU oracle and the GPU path consume the very same fp16 bit patterns it
returns, as ``numpy.uint16`` arrays (row-major, packed unless a pitch is given).

Recipe (one CPU ``torch.Generator`` per workload, A drawn first, then B):
  * entries i.i.d. normal, drawn in fp32 with ``torch.randn``, as the GEMM+ReLU
    listings do with ``torch.randn(..., dtype=float16)`` (blog "TileLang
    programming basics", section 2; "Writing high-performance kernels in
    TileLang", section "Writing a GEMM");
  * for the MLP-projection and small-M shapes B is scaled by K^-1/2 in fp32;
  * each fp32 value is rounded to fp16 (round to nearest even) by torch; the
    bfloat16 variants (``fmt="bf16"``) round the same fp32 draws to bfloat16.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    seed: int
    b_scaled: bool  # B ~ N(0, 1/K) instead of N(0, 1)
    check: str      # "full" or "sampled"


# The five workloads: square 1024^3; square 4096^3 (the headline
# compute-bound case); a shape dividing no tile; an LLM MLP up-projection;
# and a GEMV-like small-M product.
WORKLOADS = {
    "square1024": Workload("square1024", 1024, 1024, 1024, 1, False, "full"),
    "square4096": Workload("square4096", 4096, 4096, 4096, 2, False, "sampled"),
    "ragged4099x3071x2050": Workload("ragged4099x3071x2050", 4099, 3071, 2050, 3, False, "full"),
    "mlp8192x28672x8192": Workload("mlp8192x28672x8192", 8192, 28672, 8192, 4, True, "sampled"),
    "smallm8x16384x8192": Workload("smallm8x16384x8192", 8, 16384, 8192, 5, True, "full"),
}


def _torch():
    import torch  # imported lazily: the oracle pins do not need it
    return torch


FORMATS = ("f16", "bf16")

# Largest finite value of each format, as bits: the default padding pattern.
LARGEST_FINITE = {"f16": 0x7BFF, "bf16": 0x7F7F}


def normal_f16(shape, gen, scale: float | None = None, fmt: str = "f16") -> np.ndarray:
    """N(0,1) (times ``scale``) drawn in fp32, rounded to fp16 (or bfloat16 with
    ``fmt="bf16"``); returns uint16 bits."""
    torch = _torch()
    if fmt not in FORMATS:
        raise ValueError("fmt must be one of %s" % (FORMATS,))
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if scale is not None:
        x.mul_(scale)
    dt = torch.bfloat16 if fmt == "bf16" else torch.float16
    return x.to(dt).view(torch.int16).numpy().view(np.uint16)


def operands(w: Workload, fmt: str = "f16"):
    """(A, B) as packed row-major uint16 arrays for workload ``w``."""
    torch = _torch()
    gen = torch.Generator().manual_seed(w.seed)
    A = normal_f16((w.M, w.K), gen, fmt=fmt)
    B = normal_f16((w.K, w.N), gen, scale=(w.K ** -0.5) if w.b_scaled else None, fmt=fmt)
    return A, B


def random_operands(M: int, N: int, K: int, seed: int, lda: int | None = None,
                    ldb: int | None = None, pad_value: int | None = None,
                    b_scale: float | None = None, fmt: str = "f16"):
    """Random N(0,1) operands with optional row pitches.

    With ``lda > K`` (``ldb > N``) the padding columns are filled with the bit
    pattern ``pad_value`` (default: the format's largest finite value, 65504
    for fp16), so a kernel that reads padding produces visibly wrong results.
    """
    torch = _torch()
    gen = torch.Generator().manual_seed(seed)
    lda = K if lda is None else lda
    ldb = N if ldb is None else ldb
    pad = LARGEST_FINITE[fmt] if pad_value is None else pad_value
    A = np.full((M, max(lda, 1)), pad, dtype=np.uint16)
    B = np.full((K, max(ldb, 1)), pad, dtype=np.uint16)
    if M and K:
        A[:, :K] = normal_f16((M, K), gen, fmt=fmt)
    if K and N:
        B[:, :N] = normal_f16((K, N), gen, scale=b_scale, fmt=fmt)
    return A, B


def small_int_operands(M: int, N: int, K: int, seed: int, lo: int = -3, hi: int = 3):
    """Integer-valued fp16 operands in [lo, hi] (every partial sum stays exact)."""
    rng = np.random.default_rng(seed)
    A = rng.integers(lo, hi + 1, size=(M, K)).astype(np.float16).view(np.uint16)
    B = rng.integers(lo, hi + 1, size=(K, N)).astype(np.float16).view(np.uint16)
    return A, B


def sample_indices(M: int, N: int, count: int, seed: int):
    """``count`` seeded (i, j) pairs, uniform over the M x N result."""
    rng = np.random.default_rng(10_000 + seed)
    return rng.integers(0, M, size=count), rng.integers(0, N, size=count)


E4M3_MAX = 448.0  # largest finite OCP fp8 E4M3 value
E4M3_LARGEST_BITS = 0x7E


def e4m3(shape, gen, scale: float = 1.0) -> np.ndarray:
    """N(0,1) * scale drawn in fp32, clamped to +-448 and rounded to OCP fp8
    E4M3 (nearest even) by torch; returns uint8 bits."""
    torch = _torch()
    x = torch.randn(*shape, generator=gen, dtype=torch.float32) * scale
    x = x.clamp(-E4M3_MAX, E4M3_MAX)
    return x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def fp8_operands(M: int, N: int, K: int, seed: int, lda: int | None = None, ldbt: int | None = None,
                 scale_a: float = 1.0, scale_b: float = 1.0, pad_value: int = E4M3_LARGEST_BITS):
    """A (M x lda) and Bt (N x ldbt) as E4M3 bits, entries N(0,1) times the
    given scales; padding columns hold ``pad_value`` (default 448)."""
    torch = _torch()
    gen = torch.Generator().manual_seed(seed)
    lda = K if lda is None else lda
    ldbt = K if ldbt is None else ldbt
    A = np.full((M, max(lda, 1)), pad_value, dtype=np.uint8)
    Bt = np.full((N, max(ldbt, 1)), pad_value, dtype=np.uint8)
    if M and K:
        A[:, :K] = e4m3((M, K), gen, scale_a)
    if N and K:
        Bt[:, :K] = e4m3((N, K), gen, scale_b)
    return A, Bt


def mx_quantize(x: np.ndarray):
    """OCP MX quantisation of a float32 matrix (rows x K, K a multiple of 32)
    to E4M3 elements with one E8M0 scale per 32 consecutive k: the shared
    exponent of a block is floor(log2(max |x|)) - 8 (8 = the largest E4M3
    exponent), the elements are x / 2^exponent rounded to E4M3 (nearest even,
    saturating at +-448).  An all-zero block gets the code 127."""
    torch = _torch()
    rows, K = x.shape
    blocks = x.reshape(rows, K // 32, 32).astype(np.float32)
    amax = np.abs(blocks).max(axis=2)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8, 0).astype(np.int64)
    e = np.clip(e, -127, 127)
    scaled = (blocks / np.exp2(e)[:, :, None].astype(np.float64)).astype(np.float32)
    scaled = np.clip(scaled, -E4M3_MAX, E4M3_MAX).reshape(rows, K)
    elems = torch.from_numpy(scaled).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return elems, (e + 127).astype(np.uint8)


def mx_operands(M: int, N: int, K: int, seed: int, lda: int | None = None, ldbt: int | None = None,
                ldsa: int | None = None, ldsb: int | None = None, spread: int = 2,
                pad_value: int = E4M3_LARGEST_BITS, pad_scale: int = 255):
    """A, SA, Bt, SB for the MX fp8 product: N(0,1) values times 2^u, u drawn
    per 32-k block from [-spread, spread] (so the scales vary from block to
    block), quantised by mx_quantize.  Padding columns hold ``pad_value``
    (448) and the scale padding ``pad_scale`` (255, the NaN code), so a read
    outside the matrices shows in the result."""
    torch = _torch()
    gen = torch.Generator().manual_seed(seed)
    kb = K // 32
    lda = K if lda is None else lda
    ldbt = K if ldbt is None else ldbt
    ldsa = max(kb, 1) if ldsa is None else ldsa
    ldsb = max(kb, 1) if ldsb is None else ldsb
    out = []
    for rows, ld, lds in ((M, lda, ldsa), (N, ldbt, ldsb)):
        E = np.full((rows, max(ld, 1)), pad_value, dtype=np.uint8)
        S = np.full((rows, max(lds, 1)), pad_scale, dtype=np.uint8)
        if rows and K:
            x = torch.randn(rows, K, generator=gen, dtype=torch.float32).numpy()
            u = torch.randint(-spread, spread + 1, (rows, kb), generator=gen).numpy()
            x = x * np.repeat(np.exp2(u), 32, axis=1).astype(np.float32)
            E[:, :K], S[:, :kb] = mx_quantize(x)
        out.append((E, S))
    (A, SA), (Bt, SB) = out
    return A, SA, Bt, SB


E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_codes(v: np.ndarray) -> np.ndarray:
    """Round to OCP fp4 E2M1 (nearest, ties to the even code, saturating at
    +-6); returns codes 0..15 (sign in bit 3)."""
    a = np.minimum(np.abs(v), 6.0)
    d = np.abs(a[..., None] - E2M1_VALUES)
    best = d.min(axis=-1, keepdims=True)
    cand = np.where(d == best, np.arange(8), 99)
    even = np.where(cand % 2 == 0, cand, 99).min(axis=-1)
    code = np.where(even < 99, even, cand.min(axis=-1)).astype(np.uint8)
    return code | np.where(np.signbit(v) & (code != 0), 8, 0).astype(np.uint8)


def mxfp4_operands(M: int, N: int, K: int, seed: int, lda: int | None = None, ldbt: int | None = None,
                   ldsa: int | None = None, ldsb: int | None = None, spread: int = 2):
    """A, SA, Bt, SB for the MX fp4 product: N(0,1) values times 2^u (u per
    32-k block from [-spread, spread]) quantised the OCP MX way -- shared
    exponent floor(log2 max|x|) - 2 per block (2 = the largest E2M1
    exponent), elements rounded to E2M1 -- and packed two per byte (k even in
    the low nibble).  lda, ldbt count bytes; padding bytes hold 0x77 (6.0
    twice), scale padding the NaN code 255."""
    torch = _torch()
    gen = torch.Generator().manual_seed(seed)
    kb = K // 32
    lda = K // 2 if lda is None else lda
    ldbt = K // 2 if ldbt is None else ldbt
    ldsa = max(kb, 1) if ldsa is None else ldsa
    ldsb = max(kb, 1) if ldsb is None else ldsb
    out = []
    for rows, ld, lds in ((M, lda, ldsa), (N, ldbt, ldsb)):
        P = np.full((rows, max(ld, 1)), 0x77, dtype=np.uint8)
        S = np.full((rows, max(lds, 1)), 255, dtype=np.uint8)
        if rows and K:
            x = torch.randn(rows, K, generator=gen, dtype=torch.float64).numpy()
            u = torch.randint(-spread, spread + 1, (rows, kb), generator=gen).numpy()
            x = x * np.repeat(np.exp2(u), 32, axis=1)
            blocks = x.reshape(rows, kb, 32)
            amax = np.abs(blocks).max(axis=2)
            with np.errstate(divide="ignore"):
                e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, 0).astype(np.int64)
            e = np.clip(e, -127, 127)
            codes = e2m1_codes((blocks / np.exp2(e)[:, :, None]).reshape(rows, K))
            P[:, :K // 2] = codes[:, 0::2] | (codes[:, 1::2] << 4)
            S[:, :kb] = (e + 127).astype(np.uint8)
        out.append((P, S))
    (A, SA), (Bt, SB) = out
    return A, SA, Bt, SB
