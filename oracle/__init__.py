"""CPU oracle for C = ReLU(A.B), fp16 in, fp32 accumulate, fp16 out (and the
same with bfloat16 operands and result, ``fmt="bf16"``).

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product
library (``dense_gemm_epilogue_tiled_amd``) never imports, links or calls it,
and this package imports nothing from the product.

The arithmetic lives in ``oracle_gemm_relu.c`` (plain C, built with gcc
``-O2 -fno-fast-math -ffp-contract=off``); this module only compiles it and
marshals numpy arrays of fp16 bit patterns (``uint16``) through ctypes.

Every function here follows the definition written out at the top of the C
file: fp32 accumulator cleared to zero, products accumulated in increasing k,
ReLU on the fp32 value, round-to-nearest-even to fp16 (TileLang tutorial,
chapter "GEMM walkthrough and parameter derivation"; blog "TileLang
programming basics", section 2, the FP16 GEMM + ReLU listing).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_gemm_relu.c")
LIB_PATH = os.path.join(_HERE, "liboracle_gemm_relu.so")
_CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra"]

_FMTS = ("f16", "bf16")

# Activation names and their codes (the library's GR_ACT_* values).
ACTS = {"none": 0, "relu": 1, "gelu": 2, "gelu_tanh": 3, "silu": 4, "sigmoid": 5, "tanh": 6}

_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle shared library with gcc; returns its path."""
    if force or not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(_SRC):
        tmp = LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(_SRC):
                build(force=True)
            lib = ctypes.CDLL(LIB_PATH)
            i64, p = ctypes.c_int64, ctypes.c_void_p
            lib.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
            lib.oracle_f16_to_f32.restype = ctypes.c_float
            lib.oracle_f32_to_f16_rne.argtypes = [ctypes.c_float]
            lib.oracle_f32_to_f16_rne.restype = ctypes.c_uint16
            lib.oracle_f16_to_f32_array.argtypes = [p, p, i64]
            lib.oracle_f16_to_f32_array.restype = None
            lib.oracle_f32_to_f16_array.argtypes = [p, p, i64]
            lib.oracle_f32_to_f16_array.restype = None
            lib.oracle_bf16_to_f32_array.argtypes = [p, p, i64]
            lib.oracle_bf16_to_f32_array.restype = None
            lib.oracle_f32_to_bf16_array.argtypes = [p, p, i64]
            lib.oracle_f32_to_bf16_array.restype = None
            lib.oracle_set_threads.argtypes = [ctypes.c_int]
            lib.oracle_set_threads.restype = None
            lib.oracle_max_threads.argtypes = []
            lib.oracle_max_threads.restype = ctypes.c_int
            for fmt in _FMTS:
                getattr(lib, "oracle_gemm_relu_%s_full" % fmt).argtypes = [i64, i64, i64, p, i64, p, i64, p, i64]
                getattr(lib, "oracle_gemm_relu_%s_rows" % fmt).argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p]
                getattr(lib, "oracle_gemm_relu_%s_cols" % fmt).argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p]
                getattr(lib, "oracle_gemm_relu_%s_elems" % fmt).argtypes = [
                    i64, i64, i64, p, i64, p, i64, p, p, i64, p]
                for name in ("full", "rows", "cols", "elems"):
                    getattr(lib, "oracle_gemm_relu_%s_%s" % (fmt, name)).restype = ctypes.c_int
            lib.oracle_gemm_epi_full.argtypes = [ctypes.c_int, p, ctypes.c_int, i64, i64, i64, p, i64, p, i64, p, i64]
            lib.oracle_gemm_epi_rows.argtypes = [ctypes.c_int, p, ctypes.c_int, i64, i64, i64, p, i64, p, i64, p,
                                                 i64, p]
            lib.oracle_gemm_epi_cols.argtypes = [ctypes.c_int, p, ctypes.c_int, i64, i64, i64, p, i64, p, i64, p,
                                                 i64, p]
            lib.oracle_gemm_epi_elems.argtypes = [ctypes.c_int, p, ctypes.c_int, i64, i64, i64, p, i64, p, i64, p, p,
                                                  i64, p]
            for name in ("full", "rows", "cols", "elems"):
                getattr(lib, "oracle_gemm_epi_" + name).restype = ctypes.c_int
            lib.oracle_e4m3_to_f32_array.argtypes = [p, p, i64]
            lib.oracle_e4m3_to_f32_array.restype = None
            f32 = ctypes.c_float
            ci = ctypes.c_int
            lib.oracle_gemm_fp8_bt_full.argtypes = [ci, p, ci, f32, f32, i64, i64, i64, p, i64, p, i64, p, i64]
            lib.oracle_gemm_fp8_bt_full.restype = ci
            lib.oracle_gemm_fp8_bt_elems.argtypes = [ci, p, ci, f32, f32, i64, i64, i64, p, i64, p, i64, p, p, i64, p]
            lib.oracle_gemm_fp8_bt_elems.restype = ci
            lib.oracle_e8m0_to_f64_array.argtypes = [p, p, i64]
            lib.oracle_e8m0_to_f64_array.restype = None
            lib.oracle_gemm_mxfp8_bt_full.argtypes = [ci, p, ci, i64, i64, i64, p, i64, p, i64, p, i64, p, i64, p, i64]
            lib.oracle_gemm_mxfp8_bt_full.restype = ci
            lib.oracle_gemm_mxfp8_bt_elems.argtypes = [ci, p, ci, i64, i64, i64, p, i64, p, i64, p, i64, p, i64, p, p,
                                                       i64, p]
            lib.oracle_gemm_mxfp8_bt_elems.restype = ci
            lib.oracle_e2m1_to_f32_array.argtypes = [p, p, i64]
            lib.oracle_e2m1_to_f32_array.restype = None
            lib.oracle_gemm_mxfp4_bt_full.argtypes = lib.oracle_gemm_mxfp8_bt_full.argtypes
            lib.oracle_gemm_mxfp4_bt_full.restype = ci
            lib.oracle_gemm_mxfp4_bt_elems.argtypes = lib.oracle_gemm_mxfp8_bt_elems.argtypes
            lib.oracle_gemm_mxfp4_bt_elems.restype = ci
            _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _check_operands(A, B, M, N, K, lda, ldb):
    if A.dtype != np.uint16 or B.dtype != np.uint16:
        raise TypeError("operands must be uint16 arrays of fp16 / bf16 bit patterns")
    if not (A.flags.c_contiguous and B.flags.c_contiguous):
        raise ValueError("operands must be C-contiguous")
    if M > 0 and K > 0 and A.size < (M - 1) * lda + K:
        raise ValueError("A too small for M, K, lda")
    if K > 0 and N > 0 and B.size < (K - 1) * ldb + N:
        raise ValueError("B too small for K, N, ldb")


def _dims(A, B, M, N, K, lda, ldb):
    if M is None:
        M, K = A.shape
    if N is None:
        N = B.shape[1]
    lda = K if lda is None else lda
    ldb = N if ldb is None else ldb
    return int(M), int(N), int(K), int(lda), int(ldb)


def f16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Element-wise binary16 -> binary32 through the oracle's own conversion."""
    lib = _load()
    flat = np.ascontiguousarray(bits, dtype=np.uint16).ravel()
    out = np.empty(flat.size, dtype=np.float32)
    lib.oracle_f16_to_f32_array(_ptr(flat), _ptr(out), flat.size)
    return out.reshape(np.shape(bits))


def f32_to_f16(vals: np.ndarray) -> np.ndarray:
    """Element-wise binary32 -> binary16 (RNE) through the oracle's own conversion."""
    lib = _load()
    flat = np.ascontiguousarray(vals, dtype=np.float32).ravel()
    out = np.empty(flat.size, dtype=np.uint16)
    lib.oracle_f32_to_f16_array(_ptr(flat), _ptr(out), flat.size)
    return out.reshape(np.shape(vals))


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Element-wise bfloat16 -> binary32 through the oracle's own conversion."""
    lib = _load()
    flat = np.ascontiguousarray(bits, dtype=np.uint16).ravel()
    out = np.empty(flat.size, dtype=np.float32)
    lib.oracle_bf16_to_f32_array(_ptr(flat), _ptr(out), flat.size)
    return out.reshape(np.shape(bits))


def f32_to_bf16(vals: np.ndarray) -> np.ndarray:
    """Element-wise binary32 -> bfloat16 (RNE) through the oracle's own conversion."""
    lib = _load()
    flat = np.ascontiguousarray(vals, dtype=np.float32).ravel()
    out = np.empty(flat.size, dtype=np.uint16)
    lib.oracle_f32_to_bf16_array(_ptr(flat), _ptr(out), flat.size)
    return out.reshape(np.shape(vals))


def _entry(lib, fmt, name, bias=None, act="relu", N=None):
    """The C routine for (fmt, name): the fused-ReLU entry points, or, with a
    bias or another activation, the general epilogue with its first three
    arguments (format, bias pointer, activation code) bound."""
    if fmt not in _FMTS:
        raise ValueError("fmt must be one of %s" % (_FMTS,))
    if act not in ACTS:
        raise ValueError("act must be one of %s" % (sorted(ACTS),))
    if bias is None and act == "relu":
        return getattr(lib, "oracle_gemm_relu_%s_%s" % (fmt, name))
    bptr = 0
    if bias is not None:
        if bias.dtype != np.uint16 or not bias.flags.c_contiguous or bias.ndim != 1:
            raise TypeError("bias must be a contiguous 1-D uint16 array of bit patterns")
        if N is not None and bias.size < N:
            raise ValueError("bias needs N values")
        bptr = _ptr(bias)
    fn = getattr(lib, "oracle_gemm_epi_" + name)
    code = _FMTS.index(fmt)

    def call(*args):
        rc = fn(code, bptr, ACTS[act], *args)
        if rc == -2:
            raise ValueError("bad format or activation")
        return rc
    return call


def gemm_relu_full(A, B, M=None, N=None, K=None, lda=None, ldb=None, threads=None, fmt="f16", bias=None, act="relu"):
    """The whole M x N result as fp16 (or bf16, fmt="bf16") bits (packed, ldc = N).

    With ``bias`` (N values, same format) and/or ``act`` (a key of ACTS) the
    result is act(A.B + bias) instead of ReLU(A.B); the same holds for the
    rows, cols and elems variants."""
    M, N, K, lda, ldb = _dims(A, B, M, N, K, lda, ldb)
    _check_operands(A, B, M, N, K, lda, ldb)
    lib = _load()
    if threads:
        lib.oracle_set_threads(int(threads))
    C = np.zeros((M, N), dtype=np.uint16)
    if M > 0 and N > 0:
        rc = _entry(lib, fmt, "full", bias, act, N)(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), N)
        if rc != 0:
            raise MemoryError("oracle allocation failed")
    return C


def gemm_relu_rows(A, B, rows, M=None, N=None, K=None, lda=None, ldb=None, threads=None, fmt="f16", bias=None, act="relu"):
    """Full rows ``rows`` of the result: array (len(rows), N) of fp16 / bf16 bits."""
    M, N, K, lda, ldb = _dims(A, B, M, N, K, lda, ldb)
    _check_operands(A, B, M, N, K, lda, ldb)
    r = np.ascontiguousarray(rows, dtype=np.int64)
    if r.size and (r.min() < 0 or r.max() >= M):
        raise IndexError("row index out of range")
    lib = _load()
    if threads:
        lib.oracle_set_threads(int(threads))
    out = np.zeros((r.size, N), dtype=np.uint16)
    if r.size and N > 0:
        rc = _entry(lib, fmt, "rows", bias, act, N)(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(r), r.size, _ptr(out))
        if rc != 0:
            raise MemoryError("oracle allocation failed")
    return out


def gemm_relu_cols(A, B, cols, M=None, N=None, K=None, lda=None, ldb=None, threads=None, fmt="f16", bias=None, act="relu"):
    """Full columns ``cols`` of the result: array (len(cols), M) of fp16 / bf16 bits."""
    M, N, K, lda, ldb = _dims(A, B, M, N, K, lda, ldb)
    _check_operands(A, B, M, N, K, lda, ldb)
    c = np.ascontiguousarray(cols, dtype=np.int64)
    if c.size and (c.min() < 0 or c.max() >= N):
        raise IndexError("column index out of range")
    lib = _load()
    if threads:
        lib.oracle_set_threads(int(threads))
    out = np.zeros((c.size, M), dtype=np.uint16)
    if c.size and M > 0:
        rc = _entry(lib, fmt, "cols", bias, act, N)(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(c), c.size, _ptr(out))
        if rc != 0:
            raise MemoryError("oracle allocation failed")
    return out


def gemm_relu_elems(A, B, ii, jj, M=None, N=None, K=None, lda=None, ldb=None, threads=None, fmt="f16", bias=None, act="relu"):
    """Single elements C[ii[e], jj[e]] as fp16 / bf16 bits."""
    M, N, K, lda, ldb = _dims(A, B, M, N, K, lda, ldb)
    _check_operands(A, B, M, N, K, lda, ldb)
    i = np.ascontiguousarray(ii, dtype=np.int64)
    j = np.ascontiguousarray(jj, dtype=np.int64)
    if i.shape != j.shape:
        raise ValueError("index arrays differ in length")
    if i.size and (i.min() < 0 or i.max() >= M or j.min() < 0 or j.max() >= N):
        raise IndexError("element index out of range")
    lib = _load()
    if threads:
        lib.oracle_set_threads(int(threads))
    out = np.zeros(i.size, dtype=np.uint16)
    if i.size:
        _entry(lib, fmt, "elems", bias, act, N)(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(i), _ptr(j), i.size, _ptr(out))
    return out


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


# ---- fp8 (OCP E4M3) operands, B given transposed --------------------------------

def e4m3_to_f32(bits: np.ndarray) -> np.ndarray:
    """Element-wise OCP fp8 E4M3 -> binary32 through the oracle's own decoding."""
    lib = _load()
    flat = np.ascontiguousarray(bits, dtype=np.uint8).ravel()
    out = np.empty(flat.size, dtype=np.float32)
    lib.oracle_e4m3_to_f32_array(_ptr(flat), _ptr(out), flat.size)
    return out.reshape(np.shape(bits))


def _fp8_args(A, Bt, bias, act, fmt, M, N, K, lda, ldbt):
    if A.dtype != np.uint8 or Bt.dtype != np.uint8:
        raise TypeError("A and Bt must be uint8 arrays of E4M3 bit patterns")
    if not (A.flags.c_contiguous and Bt.flags.c_contiguous):
        raise ValueError("operands must be C-contiguous")
    if M is None:
        M, K = A.shape
    if N is None:
        N = Bt.shape[0]
    lda = K if lda is None else lda
    ldbt = K if ldbt is None else ldbt
    if M > 0 and K > 0 and A.size < (M - 1) * lda + K:
        raise ValueError("A too small for M, K, lda")
    if N > 0 and K > 0 and Bt.size < (N - 1) * ldbt + K:
        raise ValueError("Bt too small for N, K, ldbt")
    if fmt not in _FMTS or act not in ACTS:
        raise ValueError("bad format or activation")
    bptr = 0
    if bias is not None:
        if bias.dtype != np.uint16 or not bias.flags.c_contiguous or bias.ndim != 1 or bias.size < N:
            raise TypeError("bias must be a contiguous 1-D uint16 array of N bit patterns")
        bptr = _ptr(bias)
    return int(M), int(N), int(K), int(lda), int(ldbt), bptr


def gemm_fp8_bt_full(A, Bt, scale_a=1.0, scale_b=1.0, fmt="f16", bias=None, act="relu", M=None, N=None, K=None,
                     lda=None, ldbt=None, threads=None):
    """act(scale_a * scale_b * (A . Bt^T) + bias) as fp16 (or bf16) bits, M x N."""
    M, N, K, lda, ldbt, bptr = _fp8_args(A, Bt, bias, act, fmt, M, N, K, lda, ldbt)
    lib = _load()
    if threads:
        lib.oracle_set_threads(int(threads))
    C = np.zeros((M, N), dtype=np.uint16)
    if M > 0 and N > 0:
        lib.oracle_gemm_fp8_bt_full(_FMTS.index(fmt), bptr, ACTS[act], scale_a, scale_b, M, N, K, _ptr(A), lda,
                                    _ptr(Bt), ldbt, _ptr(C), N)
    return C


def gemm_fp8_bt_elems(A, Bt, ii, jj, scale_a=1.0, scale_b=1.0, fmt="f16", bias=None, act="relu", M=None, N=None,
                      K=None, lda=None, ldbt=None, threads=None):
    """Single elements C[ii[e], jj[e]] of gemm_fp8_bt_full."""
    M, N, K, lda, ldbt, bptr = _fp8_args(A, Bt, bias, act, fmt, M, N, K, lda, ldbt)
    i = np.ascontiguousarray(ii, dtype=np.int64)
    j = np.ascontiguousarray(jj, dtype=np.int64)
    if i.shape != j.shape:
        raise ValueError("index arrays differ in length")
    if i.size and (i.min() < 0 or i.max() >= M or j.min() < 0 or j.max() >= N):
        raise IndexError("element index out of range")
    lib = _load()
    if threads:
        lib.oracle_set_threads(int(threads))
    out = np.zeros(i.size, dtype=np.uint16)
    if i.size:
        lib.oracle_gemm_fp8_bt_elems(_FMTS.index(fmt), bptr, ACTS[act], scale_a, scale_b, M, N, K, _ptr(A), lda,
                                     _ptr(Bt), ldbt, _ptr(i), _ptr(j), i.size, _ptr(out))
    return out


def e8m0_to_f64(bits: np.ndarray) -> np.ndarray:
    """Element-wise OCP MX E8M0 scale -> float64 (2^(x-127); 255 -> NaN) through the oracle."""
    lib = _load()
    flat = np.ascontiguousarray(bits, dtype=np.uint8).ravel()
    out = np.empty(flat.size, dtype=np.float64)
    lib.oracle_e8m0_to_f64_array(_ptr(flat), _ptr(out), flat.size)
    return out.reshape(np.shape(bits))


def _mx_args(A, SA, Bt, SB, bias, act, fmt, M, N, K, lda, ldsa, ldbt, ldsb):
    M, N, K, lda, ldbt, bptr = _fp8_args(A, Bt, bias, act, fmt, M, N, K, lda, ldbt)
    if K % 32:
        raise ValueError("K must be a multiple of the 32-element block")
    if SA.dtype != np.uint8 or SB.dtype != np.uint8 or not (SA.flags.c_contiguous and SB.flags.c_contiguous):
        raise TypeError("scales must be C-contiguous uint8 arrays of E8M0 codes")
    kb = K // 32
    ldsa = kb if ldsa is None else int(ldsa)
    ldsb = kb if ldsb is None else int(ldsb)
    if kb and ((M and SA.size < (M - 1) * ldsa + kb) or (N and SB.size < (N - 1) * ldsb + kb)):
        raise ValueError("scale arrays too small")
    return M, N, K, lda, ldbt, bptr, ldsa, ldsb


def gemm_mxfp8_bt_full(A, SA, Bt, SB, fmt="f16", bias=None, act="relu", M=None, N=None, K=None, lda=None,
                       ldsa=None, ldbt=None, ldsb=None, threads=None):
    """act(sum_k A[i,k] 2^(SA[i,k/32]-127) Bt[j,k] 2^(SB[j,k/32]-127) + bias) as fp16 (or bf16) bits."""
    M, N, K, lda, ldbt, bptr, ldsa, ldsb = _mx_args(A, SA, Bt, SB, bias, act, fmt, M, N, K, lda, ldsa, ldbt, ldsb)
    lib = _load()
    if threads:
        lib.oracle_set_threads(int(threads))
    C = np.zeros((M, N), dtype=np.uint16)
    if M > 0 and N > 0:
        st = lib.oracle_gemm_mxfp8_bt_full(_FMTS.index(fmt), bptr, ACTS[act], M, N, K, _ptr(A), lda, _ptr(SA), ldsa,
                                           _ptr(Bt), ldbt, _ptr(SB), ldsb, _ptr(C), N)
        assert st == 0
    return C


def gemm_mxfp8_bt_elems(A, SA, Bt, SB, ii, jj, fmt="f16", bias=None, act="relu", M=None, N=None, K=None, lda=None,
                        ldsa=None, ldbt=None, ldsb=None, threads=None):
    """Single elements C[ii[e], jj[e]] of gemm_mxfp8_bt_full."""
    M, N, K, lda, ldbt, bptr, ldsa, ldsb = _mx_args(A, SA, Bt, SB, bias, act, fmt, M, N, K, lda, ldsa, ldbt, ldsb)
    i = np.ascontiguousarray(ii, dtype=np.int64)
    j = np.ascontiguousarray(jj, dtype=np.int64)
    if i.shape != j.shape:
        raise ValueError("index arrays differ in length")
    if i.size and (i.min() < 0 or i.max() >= M or j.min() < 0 or j.max() >= N):
        raise IndexError("element index out of range")
    lib = _load()
    if threads:
        lib.oracle_set_threads(int(threads))
    out = np.zeros(i.size, dtype=np.uint16)
    if i.size:
        st = lib.oracle_gemm_mxfp8_bt_elems(_FMTS.index(fmt), bptr, ACTS[act], M, N, K, _ptr(A), lda, _ptr(SA), ldsa,
                                            _ptr(Bt), ldbt, _ptr(SB), ldsb, _ptr(i), _ptr(j), i.size, _ptr(out))
        assert st == 0
    return out


def e2m1_to_f32(nibbles: np.ndarray) -> np.ndarray:
    """Element-wise OCP fp4 E2M1 code (low 4 bits) -> binary32 through the oracle."""
    lib = _load()
    flat = np.ascontiguousarray(nibbles, dtype=np.uint8).ravel()
    out = np.empty(flat.size, dtype=np.float32)
    lib.oracle_e2m1_to_f32_array(_ptr(flat), _ptr(out), flat.size)
    return out.reshape(np.shape(nibbles))


def _mx4_args(A, SA, Bt, SB, bias, act, fmt, M, N, K, lda, ldsa, ldbt, ldsb):
    if A.dtype != np.uint8 or Bt.dtype != np.uint8 or SA.dtype != np.uint8 or SB.dtype != np.uint8:
        raise TypeError("packed E2M1 operands and E8M0 scales are uint8 arrays")
    if not all(x.flags.c_contiguous for x in (A, SA, Bt, SB)):
        raise ValueError("arrays must be C-contiguous")
    M = A.shape[0] if M is None else M
    N = Bt.shape[0] if N is None else N
    K = 2 * A.shape[1] if K is None else K
    if K % 32:
        raise ValueError("K must be a multiple of the 32-element block")
    kb = K // 32
    lda = K // 2 if lda is None else int(lda)
    ldbt = K // 2 if ldbt is None else int(ldbt)
    ldsa = max(kb, 1) if ldsa is None else int(ldsa)
    ldsb = max(kb, 1) if ldsb is None else int(ldsb)
    if K and ((M and A.size < (M - 1) * lda + K // 2) or (N and Bt.size < (N - 1) * ldbt + K // 2)):
        raise ValueError("operands too small")
    if kb and ((M and SA.size < (M - 1) * ldsa + kb) or (N and SB.size < (N - 1) * ldsb + kb)):
        raise ValueError("scale arrays too small")
    if fmt not in _FMTS or act not in ACTS:
        raise ValueError("bad format or activation")
    bptr = 0
    if bias is not None:
        if bias.dtype != np.uint16 or not bias.flags.c_contiguous or bias.ndim != 1 or bias.size < N:
            raise TypeError("bias must be a contiguous 1-D uint16 array of N bit patterns")
        bptr = _ptr(bias)
    return int(M), int(N), int(K), lda, ldbt, bptr, ldsa, ldsb


def gemm_mxfp4_bt_full(A, SA, Bt, SB, fmt="f16", bias=None, act="relu", M=None, N=None, K=None, lda=None,
                       ldsa=None, ldbt=None, ldsb=None, threads=None):
    """gemm_mxfp8_bt_full with packed E2M1 operands (two per byte, k even in
    the low nibble); lda, ldbt in bytes."""
    M, N, K, lda, ldbt, bptr, ldsa, ldsb = _mx4_args(A, SA, Bt, SB, bias, act, fmt, M, N, K, lda, ldsa, ldbt, ldsb)
    lib = _load()
    if threads:
        lib.oracle_set_threads(int(threads))
    C = np.zeros((M, N), dtype=np.uint16)
    if M > 0 and N > 0:
        st = lib.oracle_gemm_mxfp4_bt_full(_FMTS.index(fmt), bptr, ACTS[act], M, N, K, _ptr(A), lda, _ptr(SA), ldsa,
                                           _ptr(Bt), ldbt, _ptr(SB), ldsb, _ptr(C), N)
        assert st == 0
    return C


def gemm_mxfp4_bt_elems(A, SA, Bt, SB, ii, jj, fmt="f16", bias=None, act="relu", M=None, N=None, K=None, lda=None,
                        ldsa=None, ldbt=None, ldsb=None, threads=None):
    """Single elements C[ii[e], jj[e]] of gemm_mxfp4_bt_full."""
    M, N, K, lda, ldbt, bptr, ldsa, ldsb = _mx4_args(A, SA, Bt, SB, bias, act, fmt, M, N, K, lda, ldsa, ldbt, ldsb)
    i = np.ascontiguousarray(ii, dtype=np.int64)
    j = np.ascontiguousarray(jj, dtype=np.int64)
    if i.shape != j.shape:
        raise ValueError("index arrays differ in length")
    if i.size and (i.min() < 0 or i.max() >= M or j.min() < 0 or j.max() >= N):
        raise IndexError("element index out of range")
    lib = _load()
    if threads:
        lib.oracle_set_threads(int(threads))
    out = np.zeros(i.size, dtype=np.uint16)
    if i.size:
        st = lib.oracle_gemm_mxfp4_bt_elems(_FMTS.index(fmt), bptr, ACTS[act], M, N, K, _ptr(A), lda, _ptr(SA), ldsa,
                                            _ptr(Bt), ldbt, _ptr(SB), ldsb, _ptr(i), _ptr(j), i.size, _ptr(out))
        assert st == 0
    return out
