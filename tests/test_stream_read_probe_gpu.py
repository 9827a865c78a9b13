"""GPU check of the HBM read-ceiling probe (gemm_relu_stream_read): each of
its 256 workgroups must fold every 32-bit word of its contiguous 1/256 of the
buffer into its sink entry, so the probe provably reads all the bytes it is
timed on."""
import numpy as np
import pytest

import dense_gemm_epilogue_tiled_amd as gr
from gpu_util import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mib", [8, 24])
def test_stream_read_folds_every_word(mib):
    import torch as t
    nbytes = mib << 20
    log("stream_read %d MiB" % mib)
    rng = np.random.default_rng(mib)
    host = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    src = t.from_numpy(host.view(np.int32)).to("cuda")
    sink = t.zeros(256, dtype=t.int64, device="cuda")
    st = gr.gemm_relu_stream_read(src.data_ptr(), nbytes, sink.data_ptr(), t.cuda.current_stream().cuda_stream)
    t.cuda.synchronize()
    assert st == gr.GR_OK, gr.gemm_relu_status_string(st)
    expect = np.bitwise_xor.reduce(host.reshape(256, -1), axis=1).astype(np.uint64)
    got = sink.cpu().numpy().view(np.uint64)
    assert np.array_equal(got, expect)
