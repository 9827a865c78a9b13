"""GPU check of the HBM read-ceiling probe (gemm_relu_stream_read): in both
read patterns each of its 256 workgroups must fold every 32-bit word of its
part of the buffer into its sink entry, so the probe provably reads all the
bytes it is timed on."""
import numpy as np
import pytest

import dense_gemm_epilogue_tiled_amd as gr
from gpu_util import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("pattern", [0, 1])
@pytest.mark.parametrize("mib", [8, 24])
def test_stream_read_folds_every_word(mib, pattern):
    import torch as t
    nbytes = mib << 20
    log("stream_read %d MiB pattern %d" % (mib, pattern))
    rng = np.random.default_rng(mib + 7 * pattern)
    host = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    src = t.from_numpy(host.view(np.int32)).to("cuda")
    sink = t.zeros(256, dtype=t.int64, device="cuda")
    st = gr.gemm_relu_stream_read(src.data_ptr(), nbytes, sink.data_ptr(), t.cuda.current_stream().cuda_stream,
                                  pattern=pattern)
    t.cuda.synchronize()
    assert st == gr.GR_OK, gr.gemm_relu_status_string(st)
    if pattern == gr.GR_READ_CONTIGUOUS:
        regions = host.reshape(256, -1)
    else:
        # rows of 32 KiB (8192 words); workgroup g: words 64 (g % 128) .. +63
        # of every row in half g // 128 of the rows
        rows = host.reshape(-1, 8192)
        half = rows.shape[0] // 2
        regions = [rows[(g // 128) * half:(g // 128 + 1) * half, 64 * (g % 128):64 * (g % 128) + 64].ravel()
                   for g in range(256)]
    expect = np.array([np.bitwise_xor.reduce(r) for r in regions], dtype=np.uint64)
    got = sink.cpu().numpy().view(np.uint64)
    assert np.array_equal(got, expect)
