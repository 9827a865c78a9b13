"""gemm_relu_f16_noalloc (the library's static scratch as the workspace)
against gemm_relu_f16_ws with a caller workspace, through the C ABI.

Same plan, same kernels: the two must agree bit for bit.  Two calls in a row
on every path that uses scratch, the second with a smaller problem, so that
the second call runs on scratch the first one left dirty.
"""
import numpy as np
import pytest

import dense_gemm_epilogue_tiled_amd as gr
import synth
from gpu_util import from_dev, full_dev, log, to_dev

pytestmark = pytest.mark.gpu

SENTINEL = 0x7E5A

# (first, second): each M, N, K; the second smaller than the first
PAIRS = [
    # small-M split (fp32 partial sums): 1 MiB, then 512 KiB
    ((8, 16384, 8192), (4, 2048, 4096)),
    # 128 x 128 tile split: 16 MiB twice (4 and 16 splits)
    ((1024, 1024, 16384), (512, 512, 8192)),
    # packed copies (K % 32 != 0, too few tiles for the unaligned kernel):
    # about 6 MiB, then 4 MiB
    ((2048, 1088, 1000), (1024, 1040, 1010)),
]


def _ws_call(M, N, K, dA, dB, dC, size):
    import torch as t
    ws = t.empty(max(size, 256), dtype=t.uint8, device="cuda")
    st = gr.gemm_relu_f16_ws(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, dC.data_ptr(), N, ws.data_ptr(), size,
                             t.cuda.current_stream().cuda_stream)
    t.cuda.synchronize()
    return st


def _noalloc_call(M, N, K, dA, dB, dC):
    import torch as t
    st = gr.gemm_relu_f16_noalloc(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, dC.data_ptr(), N,
                                  t.cuda.current_stream().cuda_stream)
    t.cuda.synchronize()
    return st


@pytest.mark.parametrize("pair", PAIRS, ids=["small_m_split", "tile_split", "packed"])
def test_noalloc_matches_workspace_call_twice(pair):
    for M, N, K in pair:
        st, size = gr.gemm_relu_f16_workspace_size(M, N, K, 0x100000, K, 0x200000000000, N, 0x400000000000, N)
        assert st == gr.GR_OK and 0 < size <= gr.NOALLOC_SCRATCH_BYTES, (M, N, K, size)
        st, plan = gr.gemm_relu_f16_plan_ws(M, N, K, 0x100000, K, 0x200000000000, N, 0x400000000000, N, size)
        log("noalloc %dx%dx%d scratch=%d path=%s" % (M, N, K, size, plan["path_name"]))
        A, B = synth.random_operands(M, N, K, seed=M + 7 * N + 13 * K, b_scale=K ** -0.5)
        dA, dB = to_dev(A), to_dev(B)
        dC1 = full_dev((M * N,), SENTINEL)
        dC2 = full_dev((M * N,), SENTINEL)
        assert _noalloc_call(M, N, K, dA, dB, dC1) == gr.GR_OK
        assert _ws_call(M, N, K, dA, dB, dC2, size) == gr.GR_OK
        c1, c2 = from_dev(dC1), from_dev(dC2)
        assert not np.any((c1 & 0x7C00) == 0x7C00), "an element was left unwritten or is not finite"
        assert np.array_equal(c1, c2), (M, N, K)


def test_noalloc_in_place_problem_needs_no_scratch():
    """A problem that takes no workspace runs the in-place path through the
    no-allocation call as well (the unaligned tile path here)."""
    M, N, K = 2304, 4096, 300
    st, size = gr.gemm_relu_f16_workspace_size(M, N, K, 0x100000, K, 0x200000000000, N, 0x400000000000, N)
    assert st == gr.GR_OK and size == 0
    A, B = synth.random_operands(M, N, K, seed=5)
    dA, dB = to_dev(A), to_dev(B)
    dC1 = full_dev((M * N,), SENTINEL)
    dC2 = full_dev((M * N,), SENTINEL)
    assert _noalloc_call(M, N, K, dA, dB, dC1) == gr.GR_OK
    assert _ws_call(M, N, K, dA, dB, dC2, 0) == gr.GR_OK
    assert np.array_equal(from_dev(dC1), from_dev(dC2))
