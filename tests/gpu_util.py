"""Helpers for the GPU tests: device buffers, calls through the C ABI, and the
parity check against the oracle."""
from __future__ import annotations

import sys

import numpy as np

import dense_gemm_epilogue_tiled_amd as gr

RTOL = 1e-2
ATOL = 1e-2


def log(msg: str) -> None:
    print("[gpu-case] " + msg, file=sys.stderr, flush=True)


def torch():
    import torch as t
    return t


def to_dev(x: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(x).view(np.int16)).to("cuda")


def from_dev(d) -> np.ndarray:
    return d.cpu().numpy().view(np.uint16)


def full_dev(shape, value: int):
    t = torch()
    v = value - 65536 if value >= 32768 else value
    return t.full(shape, v, dtype=t.int16, device="cuda")


def call(M, N, K, dA, lda, dB, ldb, dC, ldc, path=None, stream=None, offsets=(0, 0, 0)):
    """Run the library on device tensors (element offsets allowed) and sync."""
    t = torch()
    a = dA.data_ptr() + 2 * offsets[0] if dA is not None else 0
    b = dB.data_ptr() + 2 * offsets[1] if dB is not None else 0
    c = dC.data_ptr() + 2 * offsets[2] if dC is not None else 0
    s = (stream or t.cuda.current_stream()).cuda_stream
    if path is None:
        st = gr.gemm_relu_f16(M, N, K, a, lda, b, ldb, c, ldc, s)
    else:
        st = gr.gemm_relu_f16_forced(M, N, K, a, lda, b, ldb, c, ldc, s, path)
    t.cuda.synchronize()
    return st


def call_ws(M, N, K, dA, lda, dB, ldb, dC, ldc, ws, ws_bytes, path=None, offsets=(0, 0, 0)):
    """As call(), with a device workspace (a tensor, or None) of ws_bytes bytes."""
    t = torch()
    a = dA.data_ptr() + 2 * offsets[0] if dA is not None else 0
    b = dB.data_ptr() + 2 * offsets[1] if dB is not None else 0
    c = dC.data_ptr() + 2 * offsets[2] if dC is not None else 0
    w = ws.data_ptr() if ws is not None else 0
    s = t.cuda.current_stream().cuda_stream
    if path is None:
        st = gr.gemm_relu_f16_ws(M, N, K, a, lda, b, ldb, c, ldc, w, ws_bytes, s)
    else:
        st = gr.gemm_relu_f16_forced_ws(M, N, K, a, lda, b, ldb, c, ldc, w, ws_bytes, s, path)
    t.cuda.synchronize()
    return st


def as_f64(bits, fmt: str = "f16") -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    if fmt == "bf16":  # the upper half of a binary32
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return b.view(np.float16).astype(np.float64)


# The fp8 / fp4 matrix-core instructions (v_mfma_*_f8f6f4) do not add their
# 64 products in IEEE fp32 order: measured against the exact sum, their error
# beyond the output rounding reaches 2^-17.6 of sum_k |a_k b_k| (MX fp8 with
# block magnitudes spread over 16x), 2^-19.3 with plain per-tensor fp8 (the
# fp16 instruction: 2^-27.5).  The fp8 paths are checked with this allowance
# on top of the common bar: F8_SUM_ALLOWANCE * sum_k |a_k b_k| * 1.2 (the
# steepest activation slope), where the sum is of the dequantised products.
F8_SUM_ALLOWANCE = 2.0 ** -16


def f8_extra(abs_sum):
    """Extra absolute allowance for an fp8 / MX result whose dequantised
    products have absolute sum ``abs_sum`` (array)."""
    return 1.2 * F8_SUM_ALLOWANCE * np.asarray(abs_sum, dtype=np.float64)


def parity_report(got_bits, ref_bits, fmt: str = "f16", extra=None):
    g = as_f64(got_bits, fmt)
    o = as_f64(ref_bits, fmt)
    err = np.abs(g - o)
    bound = ATOL + RTOL * np.abs(o)
    if extra is not None:
        bound = bound + extra
    bad = ~(err <= bound) | ~np.isfinite(g)
    rel = err / np.maximum(np.abs(o), 1e-30)
    rep = {
        "checked": int(g.size),
        "violations": int(bad.sum()),
        "max_abs": float(err.max()) if err.size else 0.0,
        "max_rel": float(rel[np.abs(o) > 1e-3].max()) if np.any(np.abs(o) > 1e-3) else 0.0,
        "nonfinite": int((~np.isfinite(g)).sum()),
    }
    if bad.any():
        idx = np.unravel_index(np.argmax(np.where(bad, err, -1)), g.shape)
        rep["worst"] = tuple(int(i) for i in idx)
        rep["worst_got_ref"] = (float(g[idx]), float(o[idx]))
    return rep


def assert_parity(got_bits, ref_bits, label="", fmt: str = "f16", extra=None):
    rep = parity_report(got_bits, ref_bits, fmt, extra)
    assert rep["violations"] == 0, "%s: %s" % (label, rep)
    return rep


def edge_indices(extent: int, block: int):
    """First/last index of the first, second and last tile along one axis."""
    last = block * ((extent - 1) // block)
    cand = {0, block - 1, block, last - 1, last, extent - 1}
    return sorted(i for i in cand if 0 <= i < extent)
