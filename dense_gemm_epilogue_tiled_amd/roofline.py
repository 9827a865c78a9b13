"""Algorithmic work and roofline arithmetic for C = ReLU(A.B) (host only).

The same accounting the TileLang tutorial uses in its chapters "GEMM
walkthrough and parameter derivation" (shared-memory bill of a pipelined tile,
arithmetic intensity of one tile step) and "Performance forensics" (the 4096^3
case: total work, whole-problem intensity, ideal versus per-tile traffic).
"""
from __future__ import annotations

MI355X_PEAK_SCLK_MHZ = 2400.0     # the clock of the published peaks
MI355X_MFMA_F16_TFLOPS = 2516.6   # 256 CU x 4096 FLOP/clk x 2.4 GHz (published 2.5 PFLOP/s)
MI355X_HBM_GBS = 8000.0           # published 8 TB/s
FP16_BYTES = 2


def algorithmic_flops(M: int, N: int, K: int) -> float:
    """2 M N K: one multiply and one add per (i, j, k); the ReLU is not counted."""
    return 2.0 * M * N * K


def algorithmic_bytes(M: int, N: int, K: int) -> float:
    """Each operand read once and C written once, fp16."""
    return float(FP16_BYTES * (M * K + K * N + M * N))


def whole_problem_intensity(M: int, N: int, K: int) -> float:
    return algorithmic_flops(M, N, K) / algorithmic_bytes(M, N, K)


def pipelined_tile_smem_bytes(bm: int, bn: int, bk: int, stages: int) -> int:
    """Shared memory of a tile with `stages` buffers of the A (bm x bk) and B
    (bk x bn) strips, fp16."""
    return stages * (bm * bk + bk * bn) * FP16_BYTES


def tile_step_intensity(bm: int, bn: int) -> float:
    """FLOP per byte of one K step of a bm x bn tile whose operands all come
    from off-chip: 2 bm bn bk / ((bm + bn) bk 2) = bm bn / (bm + bn)."""
    return bm * bn / (bm + bn)


def per_tile_traffic_bytes(M: int, N: int, K: int, bm: int, bn: int) -> float:
    """Operand bytes if every tile reads its A and B panels from memory."""
    tiles = -(-M // bm) * -(-N // bn)
    return float(tiles * (bm + bn) * K * FP16_BYTES)


def ideal_traffic_bytes(M: int, N: int, K: int) -> float:
    """A, B and C each touched once (the same as algorithmic_bytes)."""
    return algorithmic_bytes(M, N, K)


def ridge_flop_per_byte(peak_tflops: float, bw_tbs: float) -> float:
    return peak_tflops / bw_tbs


def time_at_peak_s(M: int, N: int, K: int, peak_tflops: float) -> float:
    return algorithmic_flops(M, N, K) / (peak_tflops * 1e12)
