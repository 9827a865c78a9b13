"""Python binding of the gfx950 fused fp16 GEMM + ReLU library.

Thin ctypes marshalling over the C ABI declared in ``include/gemm_relu.h``:
every step of C = ReLU(A.B) runs in the HIP kernels of ``libgemm_relu.so``.
There is no fallback: if the library has not been built, every call raises.
PyTorch is only a convenience for device memory and streams
(``gemm_relu`` accepts CUDA/HIP tensors).
"""
from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgemm_relu.so")

GR_OK = 0
GR_ERR_INVALID_DIM = -1
GR_ERR_INVALID_LD = -2
GR_ERR_NULL_PTR = -3
GR_ERR_ALIAS = -4
GR_ERR_TOO_LARGE = -5
GR_ERR_NO_DEVICE = -6
GR_ERR_UNSUPPORTED_DEVICE = -7
GR_ERR_LAUNCH = -8
GR_ERR_INVALID_PATH = -9
GR_ERR_INVALID_ARG = -10
GR_ERR_SCRATCH = -11

# bytes of the static scratch behind gemm_relu_f16_noalloc (GR_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 32 << 20

GR_PATH_NONE = 0
GR_PATH_TILE = 1
GR_PATH_TILE_EDGE = 2
GR_PATH_SMALL_M = 3
GR_PATH_TILE_PACKED = 4
GR_PATH_SMALL_M_SPLIT = 5
GR_PATH_TILE_SPLIT = 6
GR_PATH_TILE_UNALIGNED = 7
GR_PATH_TILE_PERSISTENT = 8
GR_PATH_TILE_STREAM = 9
GR_READ_CONTIGUOUS = 0
GR_READ_ROW_PIECES = 1

GR_ACT_NONE = 0
GR_ACT_RELU = 1
GR_ACT_GELU = 2
GR_ACT_GELU_TANH = 3
GR_ACT_SILU = 4
GR_ACT_SIGMOID = 5
GR_ACT_TANH = 6

GR_FMT_F16 = 0
GR_FMT_BF16 = 1

ACT_CODES = {"none": GR_ACT_NONE, "relu": GR_ACT_RELU, "gelu": GR_ACT_GELU, "gelu_tanh": GR_ACT_GELU_TANH,
             "silu": GR_ACT_SILU, "sigmoid": GR_ACT_SIGMOID, "tanh": GR_ACT_TANH}

PATH_NAMES = {GR_PATH_NONE: "none", GR_PATH_TILE: "tile", GR_PATH_TILE_EDGE: "tile_edge",
              GR_PATH_SMALL_M: "small_m", GR_PATH_TILE_PACKED: "tile_packed",
              GR_PATH_SMALL_M_SPLIT: "small_m_split", GR_PATH_TILE_SPLIT: "tile_split",
              GR_PATH_TILE_UNALIGNED: "tile_unaligned", GR_PATH_TILE_PERSISTENT: "tile_persistent",
              GR_PATH_TILE_STREAM: "tile_stream"}


class gr_plan_t(ctypes.Structure):
    _fields_ = [
        ("path", ctypes.c_int32),
        ("block_m", ctypes.c_int32),
        ("block_n", ctypes.c_int32),
        ("block_k", ctypes.c_int32),
        ("stages", ctypes.c_int32),
        ("threads", ctypes.c_int32),
        ("grid", ctypes.c_int64),
        ("vec_a", ctypes.c_int32),
        ("vec_b", ctypes.c_int32),
        ("vec_c", ctypes.c_int32),
        ("group_m", ctypes.c_int32),
        ("packed", ctypes.c_int32),
        ("workspace", ctypes.c_int64),
        ("split_k", ctypes.c_int32),
        ("plain_order", ctypes.c_int32),
    ]


class GemmReluError(RuntimeError):
    def __init__(self, status: int, what: str = "gemm_relu_f16"):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (what, gemm_relu_status_string(status), status))


_lock = threading.Lock()
_lib = None


def lib() -> ctypes.CDLL:
    """The loaded C library; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    "libgemm_relu.so is not built (%s); run `python -m dense_gemm_epilogue_tiled_amd.build` "
                    "or __graft_entry__.build()" % LIB_PATH)
            # torch carries its own copy of the HIP and HSA runtimes.  When
            # torch is loaded first, this library binds to that copy (same
            # soname), so both share devices, streams and memory; loaded
            # first, the library would pull in the system copy as a second
            # runtime, which cannot use torch's streams or see its device.
            try:
                import torch  # noqa: F401
            except ImportError:
                pass
            l = ctypes.CDLL(LIB_PATH)
            i64, p, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
            l.gemm_relu_f16.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p]
            l.gemm_relu_f16.restype = i32
            l.gemm_relu_f16_forced.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p, i32]
            l.gemm_relu_f16_forced.restype = i32
            l.gemm_relu_f16_plan.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, ctypes.POINTER(gr_plan_t)]
            l.gemm_relu_f16_plan.restype = i32
            l.gemm_relu_f16_workspace_size.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64,
                                                       ctypes.POINTER(ctypes.c_int64)]
            l.gemm_relu_f16_workspace_size.restype = i32
            l.gemm_relu_f16_ws.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p, i64, p]
            l.gemm_relu_f16_ws.restype = i32
            l.gemm_relu_f16_forced_ws.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p, i64, p, i32]
            l.gemm_relu_f16_forced_ws.restype = i32
            l.gemm_relu_f16_plan_ws.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, i64,
                                                ctypes.POINTER(gr_plan_t)]
            l.gemm_relu_f16_plan_ws.restype = i32
            l.gemm_relu_f16_ta.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p]
            l.gemm_relu_f16_ta.restype = i32
            l.gemm_relu_f16_ta_forced.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p, i32]
            l.gemm_relu_f16_ta_forced.restype = i32
            l.gemm_relu_f16_ta_plan.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, ctypes.POINTER(gr_plan_t)]
            l.gemm_relu_f16_ta_plan.restype = i32
            l.gemm_relu_f16_forced_order.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p, i32, i32, i32]
            l.gemm_relu_f16_forced_order.restype = i32
            l.gemm_relu_stream_read.argtypes = [p, i64, i32, p, p]
            l.gemm_relu_stream_read.restype = i32
            l.gemm_relu_f16_noalloc.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p]
            l.gemm_relu_f16_noalloc.restype = i32
            l.gemm_relu_f16_bt.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p]
            l.gemm_relu_f16_bt.restype = i32
            l.gemm_relu_f16_bt_forced.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p, i32]
            l.gemm_relu_f16_bt_forced.restype = i32
            l.gemm_relu_f16_bt_plan.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, ctypes.POINTER(gr_plan_t)]
            l.gemm_relu_f16_bt_plan.restype = i32
            l.gemm_relu_bf16.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p]
            l.gemm_relu_bf16.restype = i32
            l.gemm_relu_bf16_forced.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p, i32]
            l.gemm_relu_bf16_forced.restype = i32
            l.gemm_relu_bf16_ws.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p, i64, p]
            l.gemm_relu_bf16_ws.restype = i32
            l.gemm_relu_bf16_forced_ws.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p, i64, p, i32]
            l.gemm_relu_bf16_forced_ws.restype = i32
            l.gemm_bias_act_ws.argtypes = [i64, i64, i64, p, i64, p, i64, p, i32, p, i64, i32, p, i64, p, i32]
            l.gemm_bias_act_ws.restype = i32
            l.gemm_bias_act_bt.argtypes = [i64, i64, i64, p, i64, p, i64, p, i32, p, i64, i32, p, i32]
            l.gemm_bias_act_bt.restype = i32
            for nm in ("gemm_bias_act_f16", "gemm_bias_act_bf16"):
                getattr(l, nm).argtypes = [i64, i64, i64, p, i64, p, i64, p, i32, p, i64, p]
                getattr(l, nm).restype = i32
                getattr(l, nm + "_forced").argtypes = [i64, i64, i64, p, i64, p, i64, p, i32, p, i64, p, i32]
                getattr(l, nm + "_forced").restype = i32
            f32 = ctypes.c_float
            l.gemm_fp8_bt.argtypes = [i64, i64, i64, p, i64, p, i64, f32, f32, p, i32, p, i64, i32, p]
            l.gemm_fp8_bt.restype = i32
            l.gemm_fp8_bt_forced.argtypes = [i64, i64, i64, p, i64, p, i64, f32, f32, p, i32, p, i64, i32, p, i32]
            l.gemm_fp8_bt_forced.restype = i32
            l.gemm_fp8_bt_plan.argtypes = [i64, i64, i64, p, i64, p, i64, p, i32, p, i64, i32,
                                           ctypes.POINTER(gr_plan_t)]
            l.gemm_fp8_bt_plan.restype = i32
            l.gemm_fp8_bt_ws.argtypes = [i64, i64, i64, p, i64, p, i64, f32, f32, p, i32, p, i64, i32, p, i64, p, i32]
            l.gemm_fp8_bt_ws.restype = i32
            l.gemm_fp8_bt_workspace_size.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64,
                                                     ctypes.POINTER(ctypes.c_int64)]
            l.gemm_fp8_bt_workspace_size.restype = i32
            l.gemm_fp8_bt_plan_ws.argtypes = [i64, i64, i64, p, i64, p, i64, p, i32, p, i64, i32, i64,
                                              ctypes.POINTER(gr_plan_t)]
            l.gemm_fp8_bt_plan_ws.restype = i32
            l.gemm_mxfp8_bt.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p, i64, p, i32, p, i64, i32, p]
            l.gemm_mxfp8_bt.restype = i32
            l.gemm_mxfp8_bt_forced.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p, i64, p, i32, p, i64, i32, p,
                                               i32]
            l.gemm_mxfp8_bt_forced.restype = i32
            l.gemm_mxfp8_bt_plan.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p, i64, p, i32, p, i64, i32,
                                             ctypes.POINTER(gr_plan_t)]
            l.gemm_mxfp8_bt_plan.restype = i32
            for nm in ("gemm_mxfp4_bt", "gemm_mxfp4_bt_forced", "gemm_mxfp4_bt_plan"):
                getattr(l, nm).argtypes = getattr(l, nm.replace("mxfp4", "mxfp8")).argtypes
                getattr(l, nm).restype = i32
            l.gemm_relu_status_string.argtypes = [i32]
            l.gemm_relu_status_string.restype = ctypes.c_char_p
            l.gemm_relu_version.argtypes = []
            l.gemm_relu_version.restype = i32
            _lib = l
    return _lib


def _ptr(x) -> int:
    return 0 if x is None else int(x)


def gemm_relu_f16(M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> int:
    """C := ReLU(A.B) on device pointers (ints); returns the C status code."""
    return lib().gemm_relu_f16(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, _ptr(stream))


def gemm_relu_f16_ta(M, N, K, At, ldat, B, ldb, C, ldc, stream=None) -> int:
    """C := ReLU(At^T B) with A given transposed (At, K x M row-major); returns the status code."""
    return lib().gemm_relu_f16_ta(M, N, K, _ptr(At), ldat, _ptr(B), ldb, _ptr(C), ldc, _ptr(stream))


def gemm_relu_f16_ta_forced(M, N, K, At, ldat, B, ldb, C, ldc, stream=None, path=GR_PATH_TILE_EDGE) -> int:
    return lib().gemm_relu_f16_ta_forced(M, N, K, _ptr(At), ldat, _ptr(B), ldb, _ptr(C), ldc, _ptr(stream), path)


def gemm_relu_f16_ta_plan(M, N, K, At, ldat, B, ldb, C, ldc):
    plan = gr_plan_t()
    st = lib().gemm_relu_f16_ta_plan(M, N, K, _ptr(At), ldat, _ptr(B), ldb, _ptr(C), ldc, ctypes.byref(plan))
    return st, _plan_dict(plan)


def gemm_relu_f16_forced_order(M, N, K, A, lda, B, ldb, C, ldc, stream=None, path=GR_PATH_TILE, group_m=4,
                               xcd_remap=1) -> int:
    """gemm_relu_f16_forced with a chosen workgroup order (test hook)."""
    return lib().gemm_relu_f16_forced_order(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, _ptr(stream), path,
                                            group_m, xcd_remap)


def gemm_relu_stream_read(src, nbytes, sink, stream=None, pattern=0) -> int:
    """Read nbytes (a multiple of 8 MiB) of device memory once: the HBM
    read-ceiling probe (pattern GR_READ_CONTIGUOUS or GR_READ_ROW_PIECES)."""
    return lib().gemm_relu_stream_read(_ptr(src), nbytes, pattern, _ptr(sink), _ptr(stream))


def gemm_relu_f16_noalloc(M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> int:
    """As gemm_relu_f16_ws with the library's static scratch as the workspace
    (no allocation; overlapping calls on one GPU race); returns the status code
    (GR_ERR_SCRATCH when the problem needs more scratch than there is)."""
    return lib().gemm_relu_f16_noalloc(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, _ptr(stream))


def gemm_relu_f16_forced(M, N, K, A, lda, B, ldb, C, ldc, stream=None, path=GR_PATH_TILE_EDGE) -> int:
    """As gemm_relu_f16 but on the given path (GR_PATH_*); returns the status code."""
    return lib().gemm_relu_f16_forced(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, _ptr(stream), path)


def _plan_dict(plan):
    d = {name: getattr(plan, name) for name, _ in gr_plan_t._fields_}
    d["path_name"] = PATH_NAMES.get(d["path"], "?")
    return d


def gemm_relu_f16_plan(M, N, K, A, lda, B, ldb, C, ldc):
    """(status, plan dict) from the pure planner; needs no GPU."""
    plan = gr_plan_t()
    st = lib().gemm_relu_f16_plan(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, ctypes.byref(plan))
    return st, _plan_dict(plan)


def gemm_relu_f16_plan_ws(M, N, K, A, lda, B, ldb, C, ldc, workspace_bytes):
    """(status, plan dict) for a call with a workspace of the given size."""
    plan = gr_plan_t()
    st = lib().gemm_relu_f16_plan_ws(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, int(workspace_bytes),
                                     ctypes.byref(plan))
    return st, _plan_dict(plan)


def gemm_relu_f16_workspace_size(M, N, K, A, lda, B, ldb, C, ldc):
    """(status, bytes): workspace that lets the problem take the packed path."""
    n = ctypes.c_int64(0)
    st = lib().gemm_relu_f16_workspace_size(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, ctypes.byref(n))
    return st, int(n.value)


def gemm_relu_f16_ws(M, N, K, A, lda, B, ldb, C, ldc, workspace, workspace_bytes, stream=None) -> int:
    """gemm_relu_f16 with a device workspace (pointer, bytes); returns the status code."""
    return lib().gemm_relu_f16_ws(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, _ptr(workspace),
                                  int(workspace_bytes), _ptr(stream))


def gemm_relu_f16_forced_ws(M, N, K, A, lda, B, ldb, C, ldc, workspace, workspace_bytes, stream=None,
                            path=GR_PATH_TILE_PACKED) -> int:
    """gemm_relu_f16_forced with a device workspace; returns the status code."""
    return lib().gemm_relu_f16_forced_ws(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, _ptr(workspace),
                                         int(workspace_bytes), _ptr(stream), path)


def gemm_relu_f16_bt(M, N, K, A, lda, Bt, ldbt, C, ldc, stream=None) -> int:
    """C := ReLU(A.Bt^T) with B given transposed (Bt is N x K); returns the status code."""
    return lib().gemm_relu_f16_bt(M, N, K, _ptr(A), lda, _ptr(Bt), ldbt, _ptr(C), ldc, _ptr(stream))


def gemm_relu_f16_bt_forced(M, N, K, A, lda, Bt, ldbt, C, ldc, stream=None, path=GR_PATH_TILE_EDGE) -> int:
    return lib().gemm_relu_f16_bt_forced(M, N, K, _ptr(A), lda, _ptr(Bt), ldbt, _ptr(C), ldc, _ptr(stream), path)


def gemm_relu_f16_bt_plan(M, N, K, A, lda, Bt, ldbt, C, ldc):
    plan = gr_plan_t()
    st = lib().gemm_relu_f16_bt_plan(M, N, K, _ptr(A), lda, _ptr(Bt), ldbt, _ptr(C), ldc, ctypes.byref(plan))
    return st, _plan_dict(plan)


def gemm_relu_bf16(M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> int:
    """C := ReLU(A.B) with bfloat16 operands and result (device pointers as ints)."""
    return lib().gemm_relu_bf16(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, _ptr(stream))


def gemm_relu_bf16_forced(M, N, K, A, lda, B, ldb, C, ldc, stream=None, path=GR_PATH_TILE_EDGE) -> int:
    """As gemm_relu_bf16 but on the given path (GR_PATH_TILE, _TILE_EDGE or _SMALL_M)."""
    return lib().gemm_relu_bf16_forced(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, _ptr(stream), path)


def gemm_bias_act_f16(M, N, K, A, lda, B, ldb, bias, act, C, ldc, stream=None) -> int:
    """C := act(A.B + bias) with fp16 operands, bias (N values or None) and result."""
    return lib().gemm_bias_act_f16(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(bias), act, _ptr(C), ldc, _ptr(stream))


def gemm_bias_act_bf16(M, N, K, A, lda, B, ldb, bias, act, C, ldc, stream=None) -> int:
    """C := act(A.B + bias) with bfloat16 operands, bias (N values or None) and result."""
    return lib().gemm_bias_act_bf16(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(bias), act, _ptr(C), ldc, _ptr(stream))


def gemm_relu_bf16_ws(M, N, K, A, lda, B, ldb, C, ldc, workspace, workspace_bytes, stream=None) -> int:
    return lib().gemm_relu_bf16_ws(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, _ptr(workspace),
                                   workspace_bytes, _ptr(stream))


def gemm_relu_bf16_forced_ws(M, N, K, A, lda, B, ldb, C, ldc, workspace, workspace_bytes, stream=None,
                             path=GR_PATH_TILE_EDGE) -> int:
    return lib().gemm_relu_bf16_forced_ws(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, _ptr(workspace),
                                          workspace_bytes, _ptr(stream), path)


def gemm_bias_act_ws(M, N, K, A, lda, B, ldb, bias, act, C, ldc, fmt, workspace, workspace_bytes, stream=None,
                     path=-1) -> int:
    """act(A.B + bias) in fmt (GR_FMT_F16 / GR_FMT_BF16) with a caller workspace; path -1 = planner."""
    return lib().gemm_bias_act_ws(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(bias), act, _ptr(C), ldc, fmt,
                                  _ptr(workspace), workspace_bytes, _ptr(stream), path)


def gemm_bias_act_bt(M, N, K, A, lda, Bt, ldbt, bias, act, C, ldc, fmt=GR_FMT_F16, stream=None, path=-1) -> int:
    """act(A.Bt^T + bias) with B given transposed (N x K), fp16 or bfloat16; path -1 = planner."""
    return lib().gemm_bias_act_bt(M, N, K, _ptr(A), lda, _ptr(Bt), ldbt, _ptr(bias), act, _ptr(C), ldc, fmt,
                                  _ptr(stream), path)


def gemm_bias_act_f16_forced(M, N, K, A, lda, B, ldb, bias, act, C, ldc, stream=None, path=GR_PATH_TILE_EDGE) -> int:
    return lib().gemm_bias_act_f16_forced(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(bias), act, _ptr(C), ldc,
                                          _ptr(stream), path)


def gemm_bias_act_bf16_forced(M, N, K, A, lda, B, ldb, bias, act, C, ldc, stream=None, path=GR_PATH_TILE_EDGE) -> int:
    return lib().gemm_bias_act_bf16_forced(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(bias), act, _ptr(C), ldc,
                                           _ptr(stream), path)


def gemm_fp8_bt(M, N, K, A, lda, Bt, ldbt, scale_a, scale_b, bias, act, C, ldc, out_fmt=GR_FMT_F16,
                stream=None) -> int:
    """C := act(scale_a * scale_b * A.Bt^T + bias), A and Bt OCP fp8 E4M3 (device pointers)."""
    return lib().gemm_fp8_bt(M, N, K, _ptr(A), lda, _ptr(Bt), ldbt, float(scale_a), float(scale_b), _ptr(bias), act,
                             _ptr(C), ldc, out_fmt, _ptr(stream))


def gemm_fp8_bt_forced(M, N, K, A, lda, Bt, ldbt, scale_a, scale_b, bias, act, C, ldc, out_fmt=GR_FMT_F16,
                       stream=None, path=GR_PATH_TILE_EDGE) -> int:
    return lib().gemm_fp8_bt_forced(M, N, K, _ptr(A), lda, _ptr(Bt), ldbt, float(scale_a), float(scale_b),
                                    _ptr(bias), act, _ptr(C), ldc, out_fmt, _ptr(stream), path)


def gemm_fp8_bt_plan(M, N, K, A, lda, Bt, ldbt, bias, act, C, ldc, out_fmt=GR_FMT_F16):
    plan = gr_plan_t()
    st = lib().gemm_fp8_bt_plan(M, N, K, _ptr(A), lda, _ptr(Bt), ldbt, _ptr(bias), act, _ptr(C), ldc, out_fmt,
                                ctypes.byref(plan))
    return st, _plan_dict(plan)


def gemm_fp8_bt_ws(M, N, K, A, lda, Bt, ldbt, scale_a, scale_b, bias, act, C, ldc, out_fmt, workspace,
                   workspace_bytes, stream=None, path=-1) -> int:
    """gemm_fp8_bt with a caller workspace (split-K for few tiles and a long K); path -1 = planner."""
    return lib().gemm_fp8_bt_ws(M, N, K, _ptr(A), lda, _ptr(Bt), ldbt, float(scale_a), float(scale_b), _ptr(bias),
                                act, _ptr(C), ldc, out_fmt, _ptr(workspace), workspace_bytes, _ptr(stream), path)


def gemm_fp8_bt_workspace_size(M, N, K, A, lda, Bt, ldbt, C, ldc):
    """(status, bytes): the workspace with which gemm_fp8_bt_ws splits K (0: never)."""
    size = ctypes.c_int64(-1)
    st = lib().gemm_fp8_bt_workspace_size(M, N, K, _ptr(A), lda, _ptr(Bt), ldbt, _ptr(C), ldc, ctypes.byref(size))
    return st, size.value


def gemm_fp8_bt_plan_ws(M, N, K, A, lda, Bt, ldbt, bias, act, C, ldc, out_fmt, workspace_bytes):
    plan = gr_plan_t()
    st = lib().gemm_fp8_bt_plan_ws(M, N, K, _ptr(A), lda, _ptr(Bt), ldbt, _ptr(bias), act, _ptr(C), ldc, out_fmt,
                                   workspace_bytes, ctypes.byref(plan))
    return st, _plan_dict(plan)


def gemm_mxfp8_bt(M, N, K, A, lda, SA, ld_sa, Bt, ldbt, SB, ld_sb, bias, act, C, ldc, out_fmt=GR_FMT_F16,
                  stream=None) -> int:
    """C := act(A~ . Bt~^T + bias): E4M3 operands, one E8M0 scale per 32 k of each row (device pointers)."""
    return lib().gemm_mxfp8_bt(M, N, K, _ptr(A), lda, _ptr(SA), ld_sa, _ptr(Bt), ldbt, _ptr(SB), ld_sb, _ptr(bias),
                               act, _ptr(C), ldc, out_fmt, _ptr(stream))


def gemm_mxfp8_bt_forced(M, N, K, A, lda, SA, ld_sa, Bt, ldbt, SB, ld_sb, bias, act, C, ldc, out_fmt=GR_FMT_F16,
                         stream=None, path=GR_PATH_TILE_EDGE) -> int:
    return lib().gemm_mxfp8_bt_forced(M, N, K, _ptr(A), lda, _ptr(SA), ld_sa, _ptr(Bt), ldbt, _ptr(SB), ld_sb,
                                      _ptr(bias), act, _ptr(C), ldc, out_fmt, _ptr(stream), path)


def gemm_mxfp8_bt_plan(M, N, K, A, lda, SA, ld_sa, Bt, ldbt, SB, ld_sb, bias, act, C, ldc, out_fmt=GR_FMT_F16):
    plan = gr_plan_t()
    st = lib().gemm_mxfp8_bt_plan(M, N, K, _ptr(A), lda, _ptr(SA), ld_sa, _ptr(Bt), ldbt, _ptr(SB), ld_sb,
                                  _ptr(bias), act, _ptr(C), ldc, out_fmt, ctypes.byref(plan))
    return st, _plan_dict(plan)


def gemm_mxfp4_bt(M, N, K, A, lda, SA, ld_sa, Bt, ldbt, SB, ld_sb, bias, act, C, ldc, out_fmt=GR_FMT_F16,
                  stream=None) -> int:
    """gemm_mxfp8_bt with packed E2M1 operands (two per byte; lda, ldbt in bytes, K in elements)."""
    return lib().gemm_mxfp4_bt(M, N, K, _ptr(A), lda, _ptr(SA), ld_sa, _ptr(Bt), ldbt, _ptr(SB), ld_sb, _ptr(bias),
                               act, _ptr(C), ldc, out_fmt, _ptr(stream))


def gemm_mxfp4_bt_forced(M, N, K, A, lda, SA, ld_sa, Bt, ldbt, SB, ld_sb, bias, act, C, ldc, out_fmt=GR_FMT_F16,
                         stream=None, path=GR_PATH_TILE_EDGE) -> int:
    return lib().gemm_mxfp4_bt_forced(M, N, K, _ptr(A), lda, _ptr(SA), ld_sa, _ptr(Bt), ldbt, _ptr(SB), ld_sb,
                                      _ptr(bias), act, _ptr(C), ldc, out_fmt, _ptr(stream), path)


def gemm_mxfp4_bt_plan(M, N, K, A, lda, SA, ld_sa, Bt, ldbt, SB, ld_sb, bias, act, C, ldc, out_fmt=GR_FMT_F16):
    plan = gr_plan_t()
    st = lib().gemm_mxfp4_bt_plan(M, N, K, _ptr(A), lda, _ptr(SA), ld_sa, _ptr(Bt), ldbt, _ptr(SB), ld_sb,
                                  _ptr(bias), act, _ptr(C), ldc, out_fmt, ctypes.byref(plan))
    return st, _plan_dict(plan)


def gemm_relu_status_string(status: int) -> str:
    return lib().gemm_relu_status_string(int(status)).decode()


def gemm_relu_version() -> int:
    return int(lib().gemm_relu_version())


def _stream_handle(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def gemm_relu_bt(a, bt, out=None, stream=None, path=None):
    """Tensor convenience: ``out = ReLU(a @ bt.T)`` with the second operand
    given transposed (``bt`` is N x K, as a linear layer's weight), 2-D fp16
    tensors on the GPU with unit column stride."""
    import torch
    if a.dtype != torch.float16 or bt.dtype != torch.float16:
        raise TypeError("a and bt must be float16")
    if a.dim() != 2 or bt.dim() != 2 or a.shape[1] != bt.shape[1]:
        raise ValueError("shapes do not form a matrix product: %s x %s^T" % (tuple(a.shape), tuple(bt.shape)))
    M, K = a.shape
    N = bt.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=a.device)
    for t in (a, bt, out):
        if t.numel() and t.stride(1) != 1:
            raise ValueError("tensors need unit column stride")
    lda = max(a.stride(0), 1) if M > 1 else max(K, 1)
    ldbt = max(bt.stride(0), 1) if N > 1 else max(K, 1)
    ldc = max(out.stride(0), 1) if M > 1 else max(N, 1)
    h = _stream_handle(stream)
    args = (M, N, K, a.data_ptr(), lda, bt.data_ptr(), ldbt, out.data_ptr(), ldc, h)
    st = gemm_relu_f16_bt(*args) if path is None else gemm_relu_f16_bt_forced(*args, path)
    if st != GR_OK:
        raise GemmReluError(st, "gemm_relu_f16_bt")
    return out


def gemm_relu(a, b, out=None, stream=None, path=None, workspace="auto"):
    """Tensor convenience: ``out = ReLU(a @ b)`` for 2-D fp16 (or bfloat16)
    tensors on the GPU.

    Row pitches are taken from the tensors' strides (unit column stride
    required). ``workspace``: "auto" allocates (from torch's caching
    allocator) the scratch the library asks for, if any; a uint8 device
    tensor is used as given; None means no workspace. Raises GemmReluError on
    a non-zero status.
    """
    import torch
    if a.dtype not in (torch.float16, torch.bfloat16) or b.dtype != a.dtype:
        raise TypeError("a and b must both be float16 or both bfloat16")
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[0]:
        raise ValueError("shapes do not form a matrix product: %s x %s" % (tuple(a.shape), tuple(b.shape)))
    M, K = a.shape
    N = b.shape[1]
    if out is None:
        out = torch.empty((M, N), dtype=a.dtype, device=a.device)
    elif out.dtype != a.dtype:
        raise TypeError("out must have the operands' dtype")
    for t in (a, b, out):
        if t.numel() and t.stride(1) != 1:
            raise ValueError("tensors need unit column stride")
    lda = max(a.stride(0), 1) if M > 1 else max(K, 1)
    ldb = max(b.stride(0), 1) if K > 1 else max(N, 1)
    ldc = max(out.stride(0), 1) if M > 1 else max(N, 1)
    args = (M, N, K, a.data_ptr(), lda, b.data_ptr(), ldb, out.data_ptr(), ldc)
    workspace = _workspace_for(torch, args, workspace, a.device, stream)
    ws_ptr, ws_bytes = (workspace.data_ptr(), workspace.numel()) if workspace is not None else (0, 0)
    h = _stream_handle(stream)
    if a.dtype == torch.bfloat16:
        if path is None:
            st = gemm_relu_bf16_ws(*args, ws_ptr, ws_bytes, h)
        else:
            st = gemm_relu_bf16_forced_ws(*args, ws_ptr, ws_bytes, h, path)
        if st != GR_OK:
            raise GemmReluError(st, "gemm_relu_bf16_ws")
        return out
    if path is None:
        st = gemm_relu_f16_ws(*args, ws_ptr, ws_bytes, h)
    else:
        st = gemm_relu_f16_forced_ws(*args, ws_ptr, ws_bytes, h, path)
    if st != GR_OK:
        raise GemmReluError(st)
    return out


def _workspace_for(torch, args, workspace, device, stream):
    """The workspace a tensor helper passes: "auto" allocates (from torch's
    caching allocator) what the library asks for, if anything; a uint8
    device tensor is used as given; None means none."""
    if not isinstance(workspace, str):
        return workspace
    if workspace != "auto":
        raise ValueError("workspace must be 'auto', None or a uint8 tensor")
    st, size = gemm_relu_f16_workspace_size(*args)  # the sizes do not depend on the element format
    if st != GR_OK:
        raise GemmReluError(st, "gemm_relu_f16_workspace_size")
    ws = torch.empty(size, dtype=torch.uint8, device=device) if size else None
    if ws is not None and stream is not None and not isinstance(stream, int):
        # the scratch block must not be handed out again before this stream is done with it
        ws.record_stream(stream)
    return ws


def gemm_bias_act(a, b, bias=None, act="gelu", out=None, stream=None, path=None, workspace="auto"):
    """Tensor convenience: ``out = act(a @ b + bias)`` for 2-D fp16 or bfloat16
    tensors on the GPU; ``bias`` is None or a 1-D tensor of N values of the
    same dtype, ``act`` a key of ACT_CODES or a GR_ACT_* code; ``workspace``
    as for gemm_relu."""
    import torch
    if a.dtype not in (torch.float16, torch.bfloat16) or b.dtype != a.dtype:
        raise TypeError("a and b must both be float16 or both bfloat16")
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[0]:
        raise ValueError("shapes do not form a matrix product: %s x %s" % (tuple(a.shape), tuple(b.shape)))
    M, K = a.shape
    N = b.shape[1]
    code = ACT_CODES[act] if isinstance(act, str) else int(act)
    if bias is not None:
        if bias.dtype != a.dtype or bias.dim() != 1 or bias.shape[0] != N or (N > 1 and bias.stride(0) != 1):
            raise ValueError("bias must be a contiguous 1-D tensor of N values of the operands' dtype")
    if out is None:
        out = torch.empty((M, N), dtype=a.dtype, device=a.device)
    elif out.dtype != a.dtype:
        raise TypeError("out must have the operands' dtype")
    for t in (a, b, out):
        if t.numel() and t.stride(1) != 1:
            raise ValueError("tensors need unit column stride")
    lda = max(a.stride(0), 1) if M > 1 else max(K, 1)
    ldb = max(b.stride(0), 1) if K > 1 else max(N, 1)
    ldc = max(out.stride(0), 1) if M > 1 else max(N, 1)
    bptr = bias.data_ptr() if bias is not None and bias.numel() else None
    h = _stream_handle(stream)
    ws = _workspace_for(torch, (M, N, K, a.data_ptr(), lda, b.data_ptr(), ldb, out.data_ptr(), ldc), workspace,
                        a.device, stream)
    ws_ptr, ws_bytes = (ws.data_ptr(), ws.numel()) if ws is not None else (0, 0)
    fmt = GR_FMT_BF16 if a.dtype == torch.bfloat16 else GR_FMT_F16
    st = gemm_bias_act_ws(M, N, K, a.data_ptr(), lda, b.data_ptr(), ldb, bptr, code, out.data_ptr(), ldc, fmt,
                          ws_ptr, ws_bytes, h, -1 if path is None else path)
    if st != GR_OK:
        raise GemmReluError(st, "gemm_bias_act_ws")
    return out


def gemm_fp8(a, bt, scale_a=1.0, scale_b=1.0, bias=None, act="relu", out_dtype=None, out=None, stream=None,
             path=None, workspace="auto"):
    """Tensor convenience: ``out = act(scale_a * scale_b * a @ bt.T + bias)``
    with ``a`` (M x K) and ``bt`` (N x K) torch.float8_e4m3fn tensors on the
    GPU (unit column stride), fp16 or bfloat16 output (``out_dtype``, default
    float16) and an optional 1-D bias of N values in the output dtype.
    ``workspace``: "auto" allocates what gemm_fp8_bt_workspace_size asks for
    (split-K for few tiles and a long K), a uint8 device tensor is used as
    given, None means none."""
    import torch
    if a.dtype != torch.float8_e4m3fn or bt.dtype != torch.float8_e4m3fn:
        raise TypeError("a and bt must be torch.float8_e4m3fn")
    if a.dim() != 2 or bt.dim() != 2 or a.shape[1] != bt.shape[1]:
        raise ValueError("shapes do not form a product: %s x %s^T" % (tuple(a.shape), tuple(bt.shape)))
    M, K = a.shape
    N = bt.shape[0]
    if out is not None:
        out_dtype = out.dtype
    out_dtype = torch.float16 if out_dtype is None else out_dtype
    if out_dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("the output is float16 or bfloat16")
    fmt = GR_FMT_BF16 if out_dtype == torch.bfloat16 else GR_FMT_F16
    if bias is not None and (bias.dtype != out_dtype or bias.dim() != 1 or bias.shape[0] != N or
                             (N > 1 and bias.stride(0) != 1)):
        raise ValueError("bias must be a contiguous 1-D tensor of N values of the output dtype")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    for t in (a, bt, out):
        if t.numel() and t.stride(1) != 1:
            raise ValueError("tensors need unit column stride")
    lda = max(a.stride(0), 1) if M > 1 else max(K, 1)
    ldbt = max(bt.stride(0), 1) if N > 1 else max(K, 1)
    ldc = max(out.stride(0), 1) if M > 1 else max(N, 1)
    code = ACT_CODES[act] if isinstance(act, str) else int(act)
    bptr = bias.data_ptr() if bias is not None and bias.numel() else None
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', None or a uint8 tensor")
        st, size = gemm_fp8_bt_workspace_size(M, N, K, a.data_ptr(), lda, bt.data_ptr(), ldbt, out.data_ptr(), ldc)
        if st != GR_OK:
            raise GemmReluError(st, "gemm_fp8_bt_workspace_size")
        workspace = torch.empty(size, dtype=torch.uint8, device=a.device) if size else None
        if workspace is not None and stream is not None and not isinstance(stream, int):
            workspace.record_stream(stream)
    ws_ptr, ws_bytes = (workspace.data_ptr(), workspace.numel()) if workspace is not None else (0, 0)
    st = gemm_fp8_bt_ws(M, N, K, a.data_ptr(), lda, bt.data_ptr(), ldbt, scale_a, scale_b, bptr, code,
                        out.data_ptr(), ldc, fmt, ws_ptr, ws_bytes, _stream_handle(stream),
                        -1 if path is None else path)
    if st != GR_OK:
        raise GemmReluError(st, "gemm_fp8_bt_ws")
    return out


def gemm_mxfp8(a, scale_a, bt, scale_b, bias=None, act="relu", out_dtype=None, out=None, stream=None, path=None):
    """Tensor convenience for the MX (block-scaled) fp8 product:
    ``out = act((a * 2^(scale_a - 127)) @ (bt * 2^(scale_b - 127)).T + bias)``
    with ``a`` (M x K) and ``bt`` (N x K) torch.float8_e4m3fn tensors and
    ``scale_a`` (M x K/32), ``scale_b`` (N x K/32) uint8 E8M0 codes (each
    expanded over its 32 consecutive k), all on the GPU with unit column
    stride; fp16 or bfloat16 output as for gemm_fp8."""
    import torch
    if a.dtype != torch.float8_e4m3fn or bt.dtype != torch.float8_e4m3fn:
        raise TypeError("a and bt must be torch.float8_e4m3fn")
    if scale_a.dtype != torch.uint8 or scale_b.dtype != torch.uint8:
        raise TypeError("scales must be uint8 E8M0 codes")
    if a.dim() != 2 or bt.dim() != 2 or a.shape[1] != bt.shape[1]:
        raise ValueError("shapes do not form a product: %s x %s^T" % (tuple(a.shape), tuple(bt.shape)))
    M, K = a.shape
    N = bt.shape[0]
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    if scale_a.dim() != 2 or tuple(scale_a.shape) != (M, K // 32) or tuple(scale_b.shape) != (N, K // 32):
        raise ValueError("scales must be M x K/32 and N x K/32")
    if out is not None:
        out_dtype = out.dtype
    out_dtype = torch.float16 if out_dtype is None else out_dtype
    if out_dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("the output is float16 or bfloat16")
    fmt = GR_FMT_BF16 if out_dtype == torch.bfloat16 else GR_FMT_F16
    if bias is not None and (bias.dtype != out_dtype or bias.dim() != 1 or bias.shape[0] != N or
                             (N > 1 and bias.stride(0) != 1)):
        raise ValueError("bias must be a contiguous 1-D tensor of N values of the output dtype")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    for t in (a, bt, scale_a, scale_b, out):
        if t.numel() and t.stride(1) != 1:
            raise ValueError("tensors need unit column stride")
    lda = max(a.stride(0), 1) if M > 1 else max(K, 1)
    ldbt = max(bt.stride(0), 1) if N > 1 else max(K, 1)
    ldsa = max(scale_a.stride(0), 1) if M > 1 else max(K // 32, 1)
    ldsb = max(scale_b.stride(0), 1) if N > 1 else max(K // 32, 1)
    ldc = max(out.stride(0), 1) if M > 1 else max(N, 1)
    code = ACT_CODES[act] if isinstance(act, str) else int(act)
    bptr = bias.data_ptr() if bias is not None and bias.numel() else None
    args = (M, N, K, a.data_ptr(), lda, scale_a.data_ptr(), ldsa, bt.data_ptr(), ldbt, scale_b.data_ptr(), ldsb, bptr,
            code, out.data_ptr(), ldc, fmt, _stream_handle(stream))
    st = gemm_mxfp8_bt(*args) if path is None else gemm_mxfp8_bt_forced(*args, path)
    if st != GR_OK:
        raise GemmReluError(st, "gemm_mxfp8_bt")
    return out


def linear(x, weight, bias=None, act="none", out=None, stream=None, path=None):
    """Tensor convenience in the layout of a linear layer:
    ``out = act(x @ weight.T + bias)`` with ``x`` (M x K) and ``weight``
    (N x K) both float16 or both bfloat16 on the GPU (unit column stride),
    ``bias`` None or N values of the same dtype, ``act`` a key of ACT_CODES
    (default: none) or a GR_ACT_* code."""
    import torch
    if x.dtype not in (torch.float16, torch.bfloat16) or weight.dtype != x.dtype:
        raise TypeError("x and weight must both be float16 or both bfloat16")
    if x.dim() != 2 or weight.dim() != 2 or x.shape[1] != weight.shape[1]:
        raise ValueError("shapes do not form x @ weight.T: %s, %s" % (tuple(x.shape), tuple(weight.shape)))
    M, K = x.shape
    N = weight.shape[0]
    code = ACT_CODES[act] if isinstance(act, str) else int(act)
    if bias is not None:
        if bias.dtype != x.dtype or bias.dim() != 1 or bias.shape[0] != N or (N > 1 and bias.stride(0) != 1):
            raise ValueError("bias must be a contiguous 1-D tensor of N values of x's dtype")
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    elif out.dtype != x.dtype:
        raise TypeError("out must have x's dtype")
    for t in (x, weight, out):
        if t.numel() and t.stride(1) != 1:
            raise ValueError("tensors need unit column stride")
    lda = max(x.stride(0), 1) if M > 1 else max(K, 1)
    ldbt = max(weight.stride(0), 1) if N > 1 else max(K, 1)
    ldc = max(out.stride(0), 1) if M > 1 else max(N, 1)
    bptr = bias.data_ptr() if bias is not None and bias.numel() else None
    fmt = GR_FMT_BF16 if x.dtype == torch.bfloat16 else GR_FMT_F16
    st = gemm_bias_act_bt(M, N, K, x.data_ptr(), lda, weight.data_ptr(), ldbt, bptr, code, out.data_ptr(), ldc, fmt,
                          _stream_handle(stream), -1 if path is None else path)
    if st != GR_OK:
        raise GemmReluError(st, "gemm_bias_act_bt")
    return out
