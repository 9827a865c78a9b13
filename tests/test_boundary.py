"""The C-ABI boundary, checked without a GPU.

* the built library loads and exports every function include/gemm_relu.h
  declares;
* argument validation returns the documented codes before any HIP call;
* the pure planner picks the documented path for each workload shape;
* status strings and constants match the header.
No compute call is made here: the parity tests live in test_parity_gpu.py.
"""
import ctypes
import os
import re

import pytest

import dense_gemm_epilogue_tiled_amd as gr
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm_relu.h")

# Fake device addresses: only their values are used by validation/planning.
BASE_A = 0x7F0000000000
BASE_B = 0x7F2000000000
BASE_C = 0x7F4000000000


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", text, flags=re.M)


def header_defines():
    text = open(HEADER).read()
    return {m.group(1): int(m.group(2)) for m in re.finditer(r"#define\s+(GR_\w+)\s+(-?\d+)", text)}


def test_library_exports_every_declared_symbol():
    names = header_functions()
    assert set(names) >= {"gemm_relu_f16", "gemm_relu_f16_plan", "gemm_relu_f16_forced",
                          "gemm_relu_f16_workspace_size", "gemm_relu_f16_ws", "gemm_relu_f16_forced_ws",
                          "gemm_relu_f16_plan_ws", "gemm_relu_status_string", "gemm_relu_version"}
    lib = ctypes.CDLL(gr.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_library_shares_torchs_hip_runtime():
    """Loading the library, even before anything imports torch, leaves one
    HIP runtime in the process: a second copy would not see torch's device
    or streams.  Checked in a fresh interpreter."""
    import subprocess
    import sys
    code = ("import dense_gemm_epilogue_tiled_amd as gr; gr.lib(); "
            "m = open('/proc/self/maps').read(); "
            "print(len(set(l.split()[-1] for l in m.splitlines() if 'libamdhip64' in l)))")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert out.returncode == 0, out.stderr[-2000:]
    assert out.stdout.strip() == "1"


def test_python_constants_match_header():
    d = header_defines()
    for k, v in d.items():
        assert getattr(gr, k) == v, k


def test_plan_struct_layout_matches_header():
    text = open(HEADER).read()
    body = re.search(r"typedef struct gr_plan_t \{(.*?)\} gr_plan_t;", text, flags=re.S).group(1)
    fields = re.findall(r"(int32_t|int64_t)\s+(\w+);", body)
    assert [f for _, f in fields] == [f for f, _ in gr.gr_plan_t._fields_]
    sizes = {"int32_t": 4, "int64_t": 8}
    assert [sizes[t] for t, _ in fields] == [ctypes.sizeof(t) for _, t in gr.gr_plan_t._fields_]


def test_status_strings():
    for name, code in header_defines().items():
        if name.startswith("GR_ERR_") or name == "GR_OK":
            assert gr.gemm_relu_status_string(code) == name
    assert gr.gemm_relu_status_string(12345) == "GR_ERR_UNKNOWN"
    assert gr.gemm_relu_version() >= 100


def plan(M, N, K, lda=None, ldb=None, ldc=None, a=BASE_A, b=BASE_B, c=BASE_C):
    lda = max(K, 1) if lda is None else lda
    ldb = max(N, 1) if ldb is None else ldb
    ldc = max(N, 1) if ldc is None else ldc
    return gr.gemm_relu_f16_plan(M, N, K, a, lda, b, ldb, c, ldc)


@pytest.mark.parametrize("args,code", [
    ((-1, 4, 4), gr.GR_ERR_INVALID_DIM),
    ((4, -1, 4), gr.GR_ERR_INVALID_DIM),
    ((4, 4, -1), gr.GR_ERR_INVALID_DIM),
    ((1 << 31, 4, 4), gr.GR_ERR_TOO_LARGE),
])
def test_invalid_dims(args, code):
    st, _ = plan(*args, lda=8, ldb=8, ldc=8)
    assert st == code


def test_invalid_pitches():
    assert plan(8, 8, 8, lda=7)[0] == gr.GR_ERR_INVALID_LD
    assert plan(8, 8, 8, ldb=7)[0] == gr.GR_ERR_INVALID_LD
    assert plan(8, 8, 8, ldc=7)[0] == gr.GR_ERR_INVALID_LD
    assert plan(8, 8, 0, lda=0)[0] == gr.GR_ERR_INVALID_LD  # lda >= max(1, K)
    assert plan(8, 8, 0, lda=1)[0] == gr.GR_OK


def test_null_pointers():
    assert plan(8, 8, 8, a=0)[0] == gr.GR_ERR_NULL_PTR
    assert plan(8, 8, 8, b=0)[0] == gr.GR_ERR_NULL_PTR
    assert plan(8, 8, 8, c=0)[0] == gr.GR_ERR_NULL_PTR
    # empty operands may be NULL
    assert plan(8, 8, 0, a=0, b=0, lda=1)[0] == gr.GR_OK
    assert plan(0, 8, 8, a=0, c=0)[0] == gr.GR_OK
    assert plan(8, 0, 8, b=0, c=0, ldb=1, ldc=1)[0] == gr.GR_OK


def test_alias_detection():
    # C's bytes overlap A's
    assert plan(8, 8, 8, a=BASE_A, c=BASE_A + 64)[0] == gr.GR_ERR_ALIAS
    assert plan(8, 8, 8, b=BASE_B, c=BASE_B - 2 * 8 * 8 + 2)[0] == gr.GR_ERR_ALIAS
    # adjacent but disjoint is fine
    assert plan(8, 8, 8, a=BASE_A, c=BASE_A + 2 * 8 * 8)[0] == gr.GR_OK


def test_span_overflow_is_too_large():
    assert plan(1 << 30, 8, 8, lda=1 << 40)[0] == gr.GR_ERR_TOO_LARGE


def test_plan_for_each_workload():
    expect = {
        "square1024": gr.GR_PATH_TILE_STREAM,
        "square4096": gr.GR_PATH_TILE,
        "ragged4099x3071x2050": gr.GR_PATH_TILE_UNALIGNED,
        "mlp8192x28672x8192": gr.GR_PATH_TILE,
        "smallm8x16384x8192": gr.GR_PATH_SMALL_M,
    }
    for name, w in synth.WORKLOADS.items():
        st, p = plan(w.M, w.N, w.K)
        assert st == gr.GR_OK
        assert p["path"] == expect[name], (name, p)
        if p["path"] in (gr.GR_PATH_TILE, gr.GR_PATH_TILE_EDGE, gr.GR_PATH_TILE_UNALIGNED, gr.GR_PATH_TILE_STREAM):
            tiles = -(-w.M // p["block_m"]) * -(-w.N // p["block_n"])
            assert p["grid"] == tiles
        else:
            assert p["grid"] == -(-w.N // p["block_n"])


def test_plan_tile_stream_where_128_tiles_are_few():
    # 64 x 64 blocks on the streaming kernel where they are few (one round of
    # two per CU) and K is long enough (and M > 64: fewer rows are the small-M
    # path)
    for M, N, K in ((1024, 1024, 1024), (512, 1024, 1024), (1000, 1000, 1024), (65, 4096, 512),
                    (1024, 1024, 16384), (1024, 2048, 1024)):
        st, p = plan(M, N, K)
        assert st == gr.GR_OK and p["path"] == gr.GR_PATH_TILE_STREAM, (M, N, K, p)
        # 8 waves per block up to 256 blocks (one per CU), else 4
        assert (p["block_m"], p["block_n"], p["threads"]) == (64, 64, 512 if p["grid"] <= 256 else 256)
        assert p["grid"] == -(-M // 64) * -(-N // 64)
    # more than one round of blocks: the 128 x 128 (or 256 x 256) tile kernel
    for M, N, K in ((1088, 2048, 1024), (2048, 2048, 2048), (4096, 4096, 4096)):
        assert plan(M, N, K)[1]["path"] == gr.GR_PATH_TILE, (M, N, K)
    # up to 64 rows: the small-M path, or one row of streaming blocks where
    # they pay (more than 32 rows, or K x N large enough)
    assert plan(16, 1024, 1024)[1]["path"] == gr.GR_PATH_SMALL_M
    st, p = plan(64, 1024, 1024)
    assert (p["path"], p["grid"], p["threads"]) == (gr.GR_PATH_TILE_STREAM, 16, 512)
    # what the streaming kernel cannot take goes elsewhere: K % 32 != 0, N < 64
    assert plan(1024, 1024, 1000)[1]["path"] != gr.GR_PATH_TILE_STREAM
    assert plan(1024, 48, 1024)[1]["path"] != gr.GR_PATH_TILE_STREAM
    # rows of A or B of any alignment stay on it
    assert plan(1024, 1024, 1024, ldb=1027)[1]["path"] == gr.GR_PATH_TILE_STREAM
    assert plan(1024, 1024, 1024, lda=1028)[1]["path"] == gr.GR_PATH_TILE_STREAM
    assert plan(1024, 1024, 1024, a=BASE_A + 2)[1]["path"] == gr.GR_PATH_TILE_STREAM


def test_tile_stream_forced_checks():
    """Forcing the row-blocked streaming path checks what its kernel needs
    before any HIP call."""
    base = (0x100000, 0x200000000000, 0x400000000000)

    def forced(M, N, K, lda, ldb, ldc, a=base[0]):
        return gr.gemm_relu_f16_forced(M, N, K, a, lda, base[1], ldb, base[2], ldc, None, gr.GR_PATH_TILE_STREAM)
    assert forced(1024, 1024, 1000, 1000, 1024, 1024) == gr.GR_ERR_INVALID_PATH   # K % 32 != 0
    assert forced(1024, 63, 1024, 1024, 63, 63) == gr.GR_ERR_INVALID_PATH         # N < 64
    assert forced(4, 64, 32, (1 << 25) + 8, 64, 64) == gr.GR_ERR_INVALID_PATH      # 32-bit copy offsets
    # accepted shapes fail only at the device check here (no GPU)
    assert forced(1024, 1024, 1024, 1024, 1027, 1024) not in (gr.GR_ERR_INVALID_PATH, gr.GR_OK)
    # rows of A of any alignment too (the copies read any 2-byte address)
    assert forced(1024, 1024, 1024, 1028, 1024, 1024) not in (gr.GR_ERR_INVALID_PATH, gr.GR_OK)
    assert forced(1024, 1024, 1024, 1024, 1024, 1024, a=base[0] + 2) not in (gr.GR_ERR_INVALID_PATH, gr.GR_OK)
    assert forced(4096, 4096, 4096, 4096, 4096, 4096) not in (gr.GR_ERR_INVALID_PATH, gr.GR_OK)


def test_plan_ragged_vector_widths():
    # lda = 2050 (even): 4-byte aligned rows of A; ldb = 3071 (odd): 2-byte
    # aligned rows of B.  The unaligned path copies both with 16-byte copies;
    # C is stored with 16-byte stores at any alignment (vec_c 8) on every path.
    st, p = plan(4099, 3071, 2050)
    assert st == gr.GR_OK and p["path"] == gr.GR_PATH_TILE_UNALIGNED
    assert (p["vec_a"], p["vec_b"], p["vec_c"]) == (2, 1, 8)
    # misaligned base pointer: the streaming kernel (K % 32 == 0, few blocks),
    # else the unaligned kernel in place; where neither applies (K % 32 != 0,
    # M < 256) the guarded kernel drops to narrower loads
    assert plan(512, 512, 512, a=BASE_A + 2)[1]["path"] == gr.GR_PATH_TILE_STREAM
    st, p = plan(512, 512, 500, a=BASE_A + 2)
    assert p["path"] == gr.GR_PATH_TILE_UNALIGNED and p["vec_a"] == 1
    st, p = plan(200, 512, 500, a=BASE_A + 2)
    assert p["path"] == gr.GR_PATH_TILE_EDGE and p["vec_a"] == 1


def test_plan_partial_tiles_take_the_pipelined_kernel():
    # 16-byte rows and K % 32 == 0: partial tiles in M and N stay on the
    # pipelined kernel, whatever C's layout
    st, p = plan(4099, 3071, 2048, lda=2048, ldb=3072, ldc=3071)
    assert st == gr.GR_OK and p["path"] == gr.GR_PATH_TILE and p["grid"] == 17 * 12 and p["vec_c"] == 8
    assert plan(256, 1, 32, ldb=8)[1]["path"] == gr.GR_PATH_TILE
    # up to 64 rows of A and at most 256 column strips: the small-M stream
    # (2 or 4 row blocks); more rows: 64 x 64 blocks on the streaming kernel
    # where they beat the pipelined kernel (few blocks, K long enough; rows
    # of any alignment), else the pipelined kernel (rows past M clamped); K %
    # 32 != 0: the unaligned kernel (M, N >= 256, K > 128), else the guarded
    # kernel
    st, p = plan(17, 512, 512)
    assert p["path"] == gr.GR_PATH_SMALL_M and (p["block_m"], p["grid"]) == (32, 8)
    st, p = plan(64, 16384, 512)
    assert p["path"] == gr.GR_PATH_SMALL_M and (p["block_m"], p["grid"]) == (64, 256)
    st, p = plan(64, 16448, 512)
    assert p["path"] == gr.GR_PATH_TILE and (p["block_m"], p["grid"]) == (128, 129)
    st, p = plan(65, 512, 512)
    assert p["path"] == gr.GR_PATH_TILE_STREAM and (p["block_m"], p["grid"]) == (64, 16)
    st, p = plan(65, 16384, 512)
    assert p["path"] == gr.GR_PATH_TILE_STREAM and (p["block_m"], p["grid"]) == (64, 512)
    st, p = plan(65, 16384, 480)
    assert p["path"] == gr.GR_PATH_TILE and (p["block_m"], p["grid"]) == (128, 128)
    assert plan(512, 512, 48)[1]["path"] == gr.GR_PATH_TILE_EDGE
    assert plan(512, 500, 512)[1]["path"] == gr.GR_PATH_TILE_STREAM
    assert plan(512, 512, 512, b=BASE_B + 8)[1]["path"] == gr.GR_PATH_TILE_STREAM
    assert plan(512, 500, 512, lda=516)[1]["path"] == gr.GR_PATH_TILE_STREAM
    assert plan(512, 512, 512, a=BASE_A + 8)[1]["path"] == gr.GR_PATH_TILE_STREAM
    assert plan(512, 500, 500, lda=516)[1]["path"] == gr.GR_PATH_TILE_UNALIGNED
    assert plan(255, 512, 500, a=BASE_A + 8)[1]["path"] == gr.GR_PATH_TILE_EDGE
    assert plan(512, 512, 100, lda=130)[1]["path"] == gr.GR_PATH_TILE_EDGE


@pytest.mark.parametrize("M,N,K,stream", [
    # aligned rows: up to 256 blocks of 64 x 64 from K = 256, 512 (one round:
    # two per CU) from K = 512
    (1024, 1024, 224, False), (1024, 1024, 256, True), (65, 64, 256, True), (512, 1024, 128, False),
    (1024, 1536, 256, False), (1024, 1536, 480, False), (1024, 1536, 512, True), (1024, 2048, 512, True),
    (1088, 1856, 8192, True), (1088, 2048, 8192, False), (1536, 1536, 4096, False),
])
def test_tile_stream_thresholds(M, N, K, stream):
    st, p = plan(M, N, K)
    assert st == gr.GR_OK
    assert p["path"] == (gr.GR_PATH_TILE_STREAM if stream else gr.GR_PATH_TILE), (M, N, K, p)


@pytest.mark.parametrize("M,N,K,ws,path,asks", [
    # B's rows misaligned (odd pitch): one round at any K, with or without a
    # workspace (none is asked for); up to two rounds without one (with one:
    # the packed copy); beyond that the unaligned kernel in place
    (1024, 2048, 4096, False, gr.GR_PATH_TILE_STREAM, False),
    (1024, 2048, 4096, True, gr.GR_PATH_TILE_STREAM, False),
    (1024, 1024, 256, False, gr.GR_PATH_TILE_STREAM, False),
    (2048, 2048, 2048, False, gr.GR_PATH_TILE_STREAM, True),
    (2048, 2048, 2048, True, gr.GR_PATH_TILE_PACKED, True),
    (2048, 2048, 4096, False, gr.GR_PATH_TILE_STREAM, True),
    (2048, 2112, 1024, False, gr.GR_PATH_TILE_UNALIGNED, True),
])
def test_tile_stream_with_misaligned_b(M, N, K, ws, path, asks):
    st, size = ws_size(M, N, K, ldb=N + 1)
    assert st == gr.GR_OK and (size > 0) == asks, size
    st, p = plan_ws(M, N, K, size, ldb=N + 1) if ws else plan(M, N, K, ldb=N + 1)
    assert st == gr.GR_OK and p["path"] == path, (M, N, K, ws, p)


@pytest.mark.parametrize("N,plain", [(1024, True), (1792, True), (1856, False), (1920, False), (1984, False),
                                     (1000, True), (960, False)])
def test_tile_stream_workgroup_order(N, plain):
    # plain row-major order when the number of 64-column blocks is a multiple
    # of 4 (each XCD then holds a quarter or an eighth of B's columns), else
    # the XCD renumbering with groups of 4 row blocks
    st, p = plan(1024, N, 4096)
    assert st == gr.GR_OK and p["path"] == gr.GR_PATH_TILE_STREAM, p
    assert p["plain_order"] == (1 if plain else 0) and p["group_m"] == (1 if plain else 4), p
    # every other path keeps the XCD renumbering
    assert plan(4096, 4096, 4096)[1]["plain_order"] == 0


def ws_size(M, N, K, lda=None, ldb=None, ldc=None, a=BASE_A, b=BASE_B, c=BASE_C):
    lda = max(K, 1) if lda is None else lda
    ldb = max(N, 1) if ldb is None else ldb
    ldc = max(N, 1) if ldc is None else ldc
    return gr.gemm_relu_f16_workspace_size(M, N, K, a, lda, b, ldb, c, ldc)


def plan_ws(M, N, K, ws, lda=None, ldb=None, ldc=None, a=BASE_A, b=BASE_B, c=BASE_C):
    lda = max(K, 1) if lda is None else lda
    ldb = max(N, 1) if ldb is None else ldb
    ldc = max(N, 1) if ldc is None else ldc
    return gr.gemm_relu_f16_plan_ws(M, N, K, a, lda, b, ldb, c, ldc, ws)


def rup(x, m):
    return -(-x // m) * m


def test_unaligned_path_takes_large_misaligned_problems_in_place():
    # the ragged workload: rows of A (4100 B) and B (6142 B) misaligned, K % 32
    # == 2, 17 x 12 tiles: the pipelined kernel in place, no workspace asked for
    st, p = plan(4099, 3071, 2050)
    assert st == gr.GR_OK and p["path"] == gr.GR_PATH_TILE_UNALIGNED and p["grid"] == 17 * 12
    assert (p["block_m"], p["block_n"], p["workspace"]) == (256, 256, 0)
    assert ws_size(4099, 3071, 2050) == (gr.GR_OK, 0)
    assert plan_ws(4099, 3071, 2050, 1 << 30)[1]["path"] == gr.GR_PATH_TILE_UNALIGNED
    # only B misaligned, only A misaligned, aligned rows with K % 32 != 0
    assert plan(4096, 3071, 2048)[1]["path"] == gr.GR_PATH_TILE_UNALIGNED
    assert plan(4096, 4096, 4096, a=BASE_A + 2)[1]["path"] == gr.GR_PATH_TILE_UNALIGNED
    assert plan(4096, 4096, 4100)[1]["path"] == gr.GR_PATH_TILE_UNALIGNED
    # its limits: one tile in M and N, K > 128
    assert plan(4096, 255, 4100)[1]["path"] == gr.GR_PATH_TILE_EDGE
    assert plan(255, 65536, 4100)[1]["path"] == gr.GR_PATH_TILE_EDGE
    assert plan(4096, 4096, 127)[1]["path"] == gr.GR_PATH_TILE_EDGE
    assert plan(4096, 4096, 129)[1]["path"] == gr.GR_PATH_TILE_UNALIGNED
    # with more than 128 tiles it needs no workspace; with fewer a workspace
    # lets the operands be packed instead, and without one it runs in place
    assert ws_size(2304, 4096, 4100) == (gr.GR_OK, 0)  # 144 tiles
    st, size = ws_size(2048, 4096, 4100)  # 128 tiles
    assert st == gr.GR_OK and size > 0
    assert plan(2048, 4096, 4100)[1]["path"] == gr.GR_PATH_TILE_UNALIGNED
    assert plan_ws(2048, 4096, 4100, size)[1]["path"] == gr.GR_PATH_TILE_PACKED


def test_workspace_size_and_packed_plan():
    # 8 x 8 large tiles, too few for the unaligned kernel: the packed copy, K padded to 1024
    st, size = ws_size(2048, 2048, 1000, lda=1001, ldb=2049)
    kp = rup(1000, 64)
    assert st == gr.GR_OK and size == rup(2048 * kp * 2, 256) + kp * rup(2048, 8) * 2
    st, p = plan_ws(2048, 2048, 1000, size, lda=1001, ldb=2049)
    assert st == gr.GR_OK and p["path"] == gr.GR_PATH_TILE_PACKED and p["packed"] == 3
    assert p["workspace"] == size and p["grid"] == 16 * 16  # 128 x 128 tiles (64 large ones are too few)
    # one byte short, or no workspace: the unaligned kernel in place
    assert plan_ws(2048, 2048, 1000, size - 1, lda=1001, ldb=2049)[1]["path"] == gr.GR_PATH_TILE_UNALIGNED
    assert plan(2048, 2048, 1000, lda=1001, ldb=2049)[1]["path"] == gr.GR_PATH_TILE_UNALIGNED
    # K % 32 == 0 with only B misaligned: only B is copied, K unchanged
    st, size = ws_size(2048, 3071, 2048)
    assert size == 2048 * rup(3071, 8) * 2
    assert plan_ws(2048, 3071, 2048, size)[1]["packed"] == 2
    # only A misaligned
    st, size = ws_size(2048, 2048, 4096, a=BASE_A + 2)
    assert size == 2048 * 4096 * 2
    assert plan_ws(2048, 2048, 4096, size, a=BASE_A + 2)[1]["packed"] == 1
    # aligned K % 64 != 0 (but K % 32 != 0 too): both padded
    st, size = ws_size(1024, 1024, 1000)
    assert size == 1024 * 1024 * 2 + 1024 * 1024 * 2
    # below the size threshold the planner keeps a single-launch kernel (the
    # size still tells a forced packed call what it needs)
    st, size = ws_size(300, 300, 300)
    assert size > 0 and plan_ws(300, 300, 300, size)[1]["path"] == gr.GR_PATH_TILE_UNALIGNED
    st, size = ws_size(200, 300, 300)
    assert size > 0 and plan_ws(200, 300, 300, size)[1]["path"] == gr.GR_PATH_TILE_EDGE


def test_workspace_not_used_where_it_cannot_help():
    assert ws_size(4096, 4096, 4096) == (gr.GR_OK, 0)       # pipelined in place, fills the chip
    assert ws_size(0, 4096, 4096) == (gr.GR_OK, 0)          # empty
    assert ws_size(512, 512, 0, lda=1) == (gr.GR_OK, 0)     # K == 0
    assert plan_ws(4096, 4096, 4096, 1 << 30)[1]["path"] == gr.GR_PATH_TILE
    assert plan_ws(4096, 4096, 4096, 1 << 30)[1]["workspace"] == 0


def test_small_m_split_plan():
    # N = 4096: the single-pass kernel would run 64 workgroups; the streaming
    # split runs 32 column blocks of 128 x 8 splits of 1024 = 256 workgroups
    st, size = ws_size(8, 4096, 8192)
    assert st == gr.GR_OK and size == 8 * 8 * 4096 * 4
    st, p = plan_ws(8, 4096, 8192, size)
    assert p["path"] == gr.GR_PATH_SMALL_M_SPLIT and p["split_k"] == 8 and p["grid"] == 256
    assert p["workspace"] == size and p["block_n"] == 128
    # too small a workspace, or none: one row of 64 x 64 blocks on the
    # streaming kernel (64 blocks of 8 waves); with a shorter K the
    # single-pass small-M kernel
    assert plan_ws(8, 4096, 8192, size - 1)[1]["path"] == gr.GR_PATH_TILE_STREAM
    assert plan(8, 4096, 8192)[1]["path"] == gr.GR_PATH_TILE_STREAM
    assert plan(8, 4096, 1024)[1]["path"] == gr.GR_PATH_SMALL_M
    # the small-M workload: 128 column blocks x 2 splits (256-byte row pieces
    # over half of K each)
    st, size = ws_size(8, 16384, 8192)
    assert size == 2 * 8 * 16384 * 4
    st, p = plan_ws(8, 16384, 8192, size)
    assert (p["path"], p["split_k"], p["grid"], p["block_n"]) == (gr.GR_PATH_SMALL_M_SPLIT, 2, 256, 128)
    # 256 column blocks or more already fill the chip: no workspace asked for
    assert ws_size(8, 32768, 8192) == (gr.GR_OK, 0)
    # B needs no alignment on the streaming kernels
    assert ws_size(8, 4096, 8192, b=BASE_B + 8)[1] == 8 * 8 * 4096 * 4
    assert ws_size(8, 4096, 8192, ldb=4100)[1] == 8 * 8 * 4096 * 4
    assert plan(8, 4096, 8192, b=BASE_B + 2)[1]["path"] == gr.GR_PATH_TILE_STREAM
    assert plan(8, 4096, 1024, b=BASE_B + 2)[1]["path"] == gr.GR_PATH_SMALL_M
    # K of fewer than four 32-deep steps is not split
    assert ws_size(8, 4096, 96) == (gr.GR_OK, 0)
    # K % 32 != 0: the register-staged split (256-column blocks, 16-byte rows
    # of B), only where its single pass leaves CUs idle
    st, p = plan_ws(8, 4096, 8200, 1 << 24)
    assert p["path"] == gr.GR_PATH_SMALL_M_SPLIT and p["block_n"] == 256 and p["grid"] == 256
    assert ws_size(8, 16384, 8200) == (gr.GR_OK, 0)
    # two column blocks: up to 32 splits here, each at least four slots deep
    st, p = plan_ws(4, 256, 4096, 1 << 24)
    assert p["path"] == gr.GR_PATH_SMALL_M_SPLIT and p["split_k"] == 32 and p["grid"] == 64
    assert p["workspace"] == 32 * 4 * 256 * 4
    st, p = plan_ws(4, 256, 1024, 1 << 24)
    assert p["split_k"] == 8
    # forced without a workspace is refused
    assert gr.gemm_relu_f16_forced(8, 16384, 8192, BASE_A, 8192, BASE_B, 16384, BASE_C, 16384, None,
                                   gr.GR_PATH_SMALL_M_SPLIT) == gr.GR_ERR_INVALID_PATH


def test_tile_split_plan():
    # 1024 x 1024: 64 tiles of 128 x 128; K = 16384 -> 4 splits (256 workgroups, one per CU)
    st, size = ws_size(1024, 1024, 16384)
    assert st == gr.GR_OK and size == 4 * 1024 * 1024 * 4
    st, p = plan_ws(1024, 1024, 16384, size)
    assert p["path"] == gr.GR_PATH_TILE_SPLIT and p["split_k"] == 4 and p["grid"] == 256
    assert p["block_m"] == 128 and p["workspace"] == size
    # K = 8192: 4 splits of 2048 save 192 of 256 strips per workgroup
    assert plan_ws(1024, 1024, 8192, 1 << 30)[1]["split_k"] == 4
    # up to K = 4096 with 129-256 blocks of 64 x 64 the streaming path (8
    # waves per block, every CU) is faster: no workspace is asked for
    assert ws_size(1024, 1024, 4096) == (gr.GR_OK, 0)
    assert plan_ws(1024, 1024, 4096, 1 << 30)[1]["path"] == gr.GR_PATH_TILE_STREAM
    assert plan_ws(128, 8192, 4096, 1 << 30)[1]["path"] == gr.GR_PATH_TILE_STREAM
    assert plan_ws(512, 1024, 4096, 1 << 30)[1]["path"] == gr.GR_PATH_TILE_SPLIT  # 128 blocks
    # 128 tiles: 2 splits; at K = 4096 they save 64 of 128 strips, just enough
    assert plan_ws(256, 8192, 4096, 1 << 30)[1]["split_k"] == 2
    # at K = 2048 two splits save too little: the streaming kernel (512
    # blocks of 64 x 64, one round) instead
    assert plan_ws(256, 8192, 2048, 1 << 30)[1]["path"] == gr.GR_PATH_TILE_STREAM
    # a split must save at least 64 strips: not at 1024^3 (4 splits save 24)
    # nor 2048^3 (256 tiles); large tiles that fill the chip never split
    assert ws_size(1024, 1024, 1024) == (gr.GR_OK, 0)
    assert ws_size(2048, 2048, 2048) == (gr.GR_OK, 0)
    assert ws_size(1024, 1024, 256) == (gr.GR_OK, 0)
    assert ws_size(4096, 4096, 4096) == (gr.GR_OK, 0)
    assert plan_ws(2048, 2048, 2048, 1 << 30)[1]["path"] == gr.GR_PATH_TILE
    # without a workspace, or one too small: 64 x 64 blocks on the streaming
    # kernel (K split between the waves of each workgroup instead)
    assert plan(1024, 1024, 16384)[1]["path"] == gr.GR_PATH_TILE_STREAM
    assert plan_ws(1024, 1024, 16384, size - 1)[1]["path"] == gr.GR_PATH_TILE_STREAM
    # forced without a workspace is refused
    assert gr.gemm_relu_f16_forced(1024, 1024, 1024, BASE_A, 1024, BASE_B, 1024, BASE_C, 1024, None,
                                   gr.GR_PATH_TILE_SPLIT) == gr.GR_ERR_INVALID_PATH


def test_workspace_argument_checks():
    ws = 0x7F6000000000
    args = (4099, 3071, 2050, BASE_A, 2050, BASE_B, 3071, BASE_C, 3071)
    assert gr.gemm_relu_f16_ws(*args, ws, -1) == gr.GR_ERR_INVALID_ARG
    assert gr.gemm_relu_f16_ws(*args, 0, 1 << 20) == gr.GR_ERR_NULL_PTR
    assert gr.gemm_relu_f16_ws(*args, ws + 16, 1 << 20) == gr.GR_ERR_INVALID_ARG
    assert gr.gemm_relu_f16_ws(*args, BASE_C - 256, 1 << 20) == gr.GR_ERR_ALIAS
    assert gr.gemm_relu_f16_ws(*args, BASE_A + 4096, 256) == gr.GR_ERR_ALIAS
    # the packed path cannot be forced without a large enough workspace
    assert gr.gemm_relu_f16_forced(*args, None, gr.GR_PATH_TILE_PACKED) == gr.GR_ERR_INVALID_PATH
    assert gr.gemm_relu_f16_forced_ws(*args, ws, 4096, None, gr.GR_PATH_TILE_PACKED) == gr.GR_ERR_INVALID_PATH
    assert gr.gemm_relu_f16_forced_ws(*args, ws, 1 << 30, None, 99) == gr.GR_ERR_INVALID_PATH
    assert gr.gemm_relu_f16_plan_ws(*args, -1)[0] == gr.GR_ERR_INVALID_ARG
    n = ctypes.c_int64(0)
    assert gr.lib().gemm_relu_f16_workspace_size(*args, None) == gr.GR_ERR_INVALID_ARG
    assert gr.lib().gemm_relu_f16_workspace_size(-1, 8, 8, BASE_A, 8, BASE_B, 8, BASE_C, 8,
                                                 ctypes.byref(n)) == gr.GR_ERR_INVALID_DIM


def test_plan_tile_size_choice():
    # fewer than half a wave of 256 x 256 tiles (or M < 256): 128 x 128 tiles
    for (M, N), (bm, grid) in {(2048, 2048): (128, 256), (4096, 4096): (256, 256), (2816, 2816): (128, 484),
                               (4099, 3071): (256, 204), (2048, 4096): (128, 512),
                               (2304, 4096): (256, 144), (1088, 2048): (128, 144)}.items():
        st, p = plan(M, N, 512, ldb=rup(N, 8), ldc=rup(N, 8))
        assert st == gr.GR_OK and p["path"] == gr.GR_PATH_TILE, (M, N, p)
        assert (p["block_m"], p["block_n"], p["grid"]) == (bm, bm, grid), (M, N, p)
    # one round of 64 x 64 blocks or less (K >= 512): the streaming kernel
    for (M, N), grid in {(1024, 1024): 256, (128, 4096): 128, (200, 304): 20, (1024, 2048): 512}.items():
        st, p = plan(M, N, 512, ldb=rup(N, 8), ldc=rup(N, 8))
        assert st == gr.GR_OK and p["path"] == gr.GR_PATH_TILE_STREAM, (M, N, p)
        assert (p["block_m"], p["block_n"], p["grid"]) == (64, 64, grid), (M, N, p)


def test_plan_empty_and_k_zero():
    assert plan(0, 8, 8)[1]["path"] == gr.GR_PATH_NONE
    assert plan(8, 0, 8, ldb=1, ldc=1)[1]["path"] == gr.GR_PATH_NONE
    st, p = plan(300, 300, 0, lda=1)
    assert st == gr.GR_OK and p["path"] == gr.GR_PATH_TILE_EDGE


def test_plan_small_m_threshold():
    assert plan(16, 4096, 512)[1]["path"] == gr.GR_PATH_SMALL_M
    assert plan(17, 4096, 512)[1]["path"] == gr.GR_PATH_SMALL_M    # two row blocks
    assert plan(64, 16384, 4096)[1]["path"] == gr.GR_PATH_SMALL_M  # four row blocks, 256 of them
    assert plan(65, 4096, 4096)[1]["path"] == gr.GR_PATH_TILE_STREAM  # 64 x 64 blocks


@pytest.mark.parametrize("M,N,K,stream", [
    (16, 4096, 4096, True), (17, 4096, 4096, True), (64, 4096, 4096, True), (1, 2048, 4096, True),
    (32, 8192, 1024, True), (32, 8192, 4096, True), (32, 8192, 8192, False),  # 128 blocks: B up to 64 MiB
    (8, 1024, 2048, False), (8, 1024, 8192, True), (8, 512, 32768, False),   # K x N >= 2^23, N >= 1024
    (33, 256, 256, True), (64, 8192, 256, True), (64, 8256, 4096, False),    # more than 32 rows: 128 blocks
    (16, 4096, 4016, False), (8, 16384, 8192, False)])
def test_small_m_rows_on_the_streaming_kernel(M, N, K, stream):
    """Up to 64 rows without a split: one row of streaming blocks (8 waves
    each) where the small-M kernel's few blocks would leave CUs idle and B is
    large, else the small-M kernel; a workspace still buys the split."""
    st, p = plan(M, N, K)
    assert st == gr.GR_OK
    if stream:
        assert (p["path"], p["block_m"], p["grid"], p["threads"]) == (gr.GR_PATH_TILE_STREAM, 64, -(-N // 64), 512)
    else:
        assert p["path"] == gr.GR_PATH_SMALL_M, p
    if M <= 16:
        st, size = ws_size(M, N, K)
        if size > 0:
            assert plan_ws(M, N, K, size)[1]["path"] == gr.GR_PATH_SMALL_M_SPLIT


@pytest.mark.parametrize("M,N,K,a_off,lda_pad", [(8, 4096, 4096, 1, 1), (64, 16384, 4096, 1, 1), (32, 1024, 1024, 0, 3),
                                                 (1, 64, 32, 4, 0)])
def test_small_m_rows_misaligned_a_on_the_streaming_kernel(M, N, K, a_off, lda_pad):
    """A's rows not 16-byte aligned: the small-M kernels cannot take them,
    the streaming kernel does in place, with no workspace asked for."""
    lda = K + lda_pad
    a = BASE_A + 2 * a_off
    st, p = plan(M, N, K, a=a, lda=lda)
    assert st == gr.GR_OK and p["path"] == gr.GR_PATH_TILE_STREAM, p
    assert ws_size(M, N, K, a=a, lda=lda) == (gr.GR_OK, 0)
    assert plan(1, 1, 1)[1]["path"] == gr.GR_PATH_TILE_EDGE  # B row pitch 1: not 8-byte aligned


def test_planner_invariants_on_random_problems():
    """Seeded random shapes, pitches and alignments: the planner's choice
    respects every kernel's preconditions, the grid matches the tile count,
    and a workspace changes the path only when the library asked for one."""
    import numpy as np
    rng = np.random.default_rng(7)
    for _ in range(3000):
        M = int(rng.choice([rng.integers(0, 17), rng.integers(17, 65), rng.integers(17, 5000)]))
        N = int(rng.integers(0, 30000))
        K = int(rng.choice([0, rng.integers(1, 9000), 32 * rng.integers(1, 300)]))
        lda = max(K, 1) + int(rng.choice([0, 0, rng.integers(1, 17)]))
        ldb = max(N, 1) + int(rng.choice([0, 0, rng.integers(1, 17)]))
        ldc = max(N, 1) + int(rng.choice([0, 0, rng.integers(1, 17)]))
        a = BASE_A + 2 * int(rng.choice([0, 0, rng.integers(1, 8)]))
        b = BASE_B + 2 * int(rng.choice([0, 0, rng.integers(1, 8)]))
        c = BASE_C + 2 * int(rng.choice([0, 0, rng.integers(1, 8)]))
        st, p = gr.gemm_relu_f16_plan(M, N, K, a, lda, b, ldb, c, ldc)
        assert st == gr.GR_OK, (M, N, K)
        st, size = gr.gemm_relu_f16_workspace_size(M, N, K, a, lda, b, ldb, c, ldc)
        assert st == gr.GR_OK and size >= 0 and size % 256 == 0
        st, pw = gr.gemm_relu_f16_plan_ws(M, N, K, a, lda, b, ldb, c, ldc, size)
        assert st == gr.GR_OK
        key = (M, N, K, lda, ldb, ldc, a % 16, b % 16, c % 16)
        if M == 0 or N == 0:
            assert p["path"] == gr.GR_PATH_NONE and size == 0
            continue
        aligned = a % 16 == 0 and lda % 8 == 0 and b % 16 == 0 and ldb % 8 == 0
        if p["path"] == gr.GR_PATH_TILE:
            assert aligned and K % 32 == 0 and K > 0, key
            bm = p["block_m"]
            assert bm in (128, 256) and (bm == 128 or M >= 256), key
            assert p["grid"] == -(-M // bm) * -(-N // bm), key
        elif p["path"] == gr.GR_PATH_SMALL_M:
            assert 1 <= M <= 64 and K > 0 and p["grid"] == -(-N // 64), key
            assert M <= 16 or -(-N // 64) <= 256, key  # wider C with more rows: the tile kernel
        elif p["path"] == gr.GR_PATH_TILE_STREAM:
            assert K > 0 and K % 32 == 0 and N >= 64, key
            blocks = -(-M // 64) * -(-N // 64)
            if M <= 64 and a % 16 == 0 and lda % 8 == 0 and -(-N // 64) <= 256:
                # the small-M kernel's rows: one row of blocks, where it pays
                assert blocks <= 128 and (M > 32 or N >= 1024), key
            elif aligned:  # few blocks, K long enough to beat the 128 x 128 tiles
                assert (blocks <= 256 and K >= 256) or (blocks <= 512 and K >= 512), key
            else:  # rows misaligned: one round, or two without a workspace
                assert blocks <= 1024, key
                assert size == 0 or blocks > 512, key  # within one round no workspace is asked for
            assert p["block_m"] == 64 and p["grid"] == blocks, key
            assert p["plain_order"] == (1 if -(-N // 64) % 4 == 0 else 0), key
        elif p["path"] == gr.GR_PATH_TILE_UNALIGNED:
            assert not (aligned and K % 32 == 0), key
            assert M >= 256 and N >= 256 and K > 128, key
            tiles = -(-M // 256) * -(-N // 256)
            assert p["grid"] == tiles and p["block_m"] == 256, key
            assert tiles <= 128 or size == 0, key  # more than 128 tiles: never packed
            # the streaming kernel takes two rounds or less of what it can take
            assert tiles > 128 or not (K % 32 == 0 and N >= 64 and -(-M // 64) * -(-N // 64) <= 1024), key
        else:
            assert p["path"] == gr.GR_PATH_TILE_EDGE, key
            assert not (aligned and K % 32 == 0 and K > 0), key
            assert not (M >= 256 and N >= 256 and K > 128), key  # else the unaligned kernel
            assert not (M > 64 and K > 0 and K % 32 == 0 and N >= 64 and -(-M // 64) * -(-N // 64) <= 1024), key
        # the workspace plan differs from the plain one only where a workspace was asked for
        if size == 0:
            assert pw["path"] == p["path"] and pw["workspace"] == 0, key
        else:
            assert pw["workspace"] <= size, key
            if pw["path"] != p["path"]:
                assert pw["path"] in (gr.GR_PATH_TILE_PACKED, gr.GR_PATH_SMALL_M_SPLIT, gr.GR_PATH_TILE_SPLIT), key
                assert pw["workspace"] == size, key
            if pw["path"] == gr.GR_PATH_SMALL_M_SPLIT:
                assert pw["block_n"] in (128, 256), key
                assert pw["grid"] == -(-N // pw["block_n"]) * pw["split_k"], key
                assert pw["workspace"] >= 4 * M * N * pw["split_k"], key
            if pw["path"] == gr.GR_PATH_TILE_SPLIT:
                assert pw["block_m"] == 128 and pw["grid"] == -(-M // 128) * -(-N // 128) * pw["split_k"]
                assert pw["workspace"] >= 4 * M * N * pw["split_k"], key


def plan_bt(M, N, K, lda=None, ldbt=None, ldc=None, a=BASE_A, b=BASE_B, c=BASE_C):
    lda = max(K, 1) if lda is None else lda
    ldbt = max(K, 1) if ldbt is None else ldbt
    ldc = max(N, 1) if ldc is None else ldc
    return gr.gemm_relu_f16_bt_plan(M, N, K, a, lda, b, ldbt, c, ldc)


def test_transposed_b_planner_and_checks():
    # Bt is N x K: its pitch is checked against K, its span is N rows
    assert plan_bt(8, 8, 8, ldbt=7)[0] == gr.GR_ERR_INVALID_LD
    assert plan_bt(8, 100, 8, ldbt=8)[0] == gr.GR_OK
    assert plan_bt(8, 8, 8, b=0)[0] == gr.GR_ERR_NULL_PTR
    assert plan_bt(8, 8, 8, c=BASE_B + 2 * 8 * 7)[0] == gr.GR_ERR_ALIAS
    assert plan_bt(8, 8, 8, c=BASE_B + 2 * 8 * 8)[0] == gr.GR_OK
    # paths
    st, p = plan_bt(8, 16384, 8192)
    assert p["path"] == gr.GR_PATH_SMALL_M and p["grid"] == 16384 // 64
    st, p = plan_bt(4096, 4096, 4096)
    assert p["path"] == gr.GR_PATH_TILE and p["block_m"] == 256 and p["grid"] == 256
    # few blocks of 64 x 64 with K long enough: the streaming kernel with Bt
    # copied like A (up to 256 blocks from K = 256, 512 from K = 1024); M > 16
    st, p = plan_bt(1024, 1024, 1024)
    assert p["path"] == gr.GR_PATH_TILE_STREAM and (p["block_m"], p["block_n"], p["grid"]) == (64, 64, 256)
    assert p["plain_order"] == 1
    st, p = plan_bt(32, 4000, 4096)
    assert p["path"] == gr.GR_PATH_TILE_STREAM and p["grid"] == 63 and p["plain_order"] == 0
    st, p = plan_bt(1024, 1024, 128)
    assert p["path"] == gr.GR_PATH_TILE and p["block_m"] == 128
    assert plan_bt(1024, 1024, 256)[1]["path"] == gr.GR_PATH_TILE_STREAM
    assert plan_bt(1024, 2048, 512)[1]["path"] == gr.GR_PATH_TILE  # 512 blocks from K = 1024 only
    assert plan_bt(1024, 2048, 1024)[1]["path"] == gr.GR_PATH_TILE_STREAM
    assert plan_bt(4096, 4096, 4100)[1]["path"] == gr.GR_PATH_TILE_EDGE          # K % 32 != 0
    assert plan_bt(4096, 4096, 4096, ldbt=4100)[1]["path"] == gr.GR_PATH_TILE_STREAM  # Bt rows not 16-B
    assert plan_bt(1024, 1024, 1024, ldbt=1025)[1]["path"] == gr.GR_PATH_TILE_STREAM
    assert plan_bt(4096, 4096, 4100, ldbt=4101)[1]["path"] == gr.GR_PATH_TILE_EDGE  # K % 32 != 0
    assert plan_bt(8, 4096, 4096, b=BASE_B + 8)[1]["path"] == gr.GR_PATH_TILE_EDGE  # Bt rows not 16-B
    assert plan_bt(0, 4096, 4096)[1]["path"] == gr.GR_PATH_NONE
    # forced paths are checked
    assert gr.gemm_relu_f16_bt_forced(300, 256, 48, BASE_A, 48, BASE_B, 48, BASE_C, 256, None,
                                      gr.GR_PATH_TILE) == gr.GR_ERR_INVALID_PATH
    assert gr.gemm_relu_f16_bt_forced(64, 256, 64, BASE_A, 64, BASE_B, 64, BASE_C, 256, None,
                                      gr.GR_PATH_SMALL_M) == gr.GR_ERR_INVALID_PATH
    assert gr.gemm_relu_f16_bt_forced(8, 256, 64, BASE_A, 64, BASE_B, 64, BASE_C, 256, None,
                                      gr.GR_PATH_TILE_PACKED) == gr.GR_ERR_INVALID_PATH
    for M, N, K in ((16, 256, 64), (300, 256, 48), (300, 48, 64)):  # M <= 16, K % 32 != 0, N < 64
        assert gr.gemm_relu_f16_bt_forced(M, N, K, BASE_A, K, BASE_B, K, BASE_C, N, None,
                                          gr.GR_PATH_TILE_STREAM) == gr.GR_ERR_INVALID_PATH, (M, N, K)
    assert gr.gemm_relu_f16_bt_forced(300, 256, 64, BASE_A, 65, BASE_B + 2, 67, BASE_C, 256, None,
                                      gr.GR_PATH_TILE_STREAM) not in (gr.GR_ERR_INVALID_PATH, gr.GR_OK)


def test_bf16_argument_checks_need_no_gpu():
    """The bfloat16 entry points share the fp16 argument checks, which run
    before any HIP call; paths that need a workspace are refused."""
    f = gr.gemm_relu_bf16
    assert f(-1, 8, 8, BASE_A, 8, BASE_B, 8, BASE_C, 8) == gr.GR_ERR_INVALID_DIM
    assert f(8, 8, 8, BASE_A, 7, BASE_B, 8, BASE_C, 8) == gr.GR_ERR_INVALID_LD
    assert f(8, 8, 8, 0, 8, BASE_B, 8, BASE_C, 8) == gr.GR_ERR_NULL_PTR
    assert f(8, 8, 8, BASE_A, 8, BASE_B, 8, BASE_A + 64, 8) == gr.GR_ERR_ALIAS
    assert f(0, 8, 8, 0, 8, BASE_B, 8, 0, 8) == gr.GR_OK  # empty: nothing launched
    g = gr.gemm_relu_bf16_forced
    for path in (gr.GR_PATH_TILE_PACKED, gr.GR_PATH_SMALL_M_SPLIT, gr.GR_PATH_TILE_SPLIT, 99):
        assert g(8, 256, 64, BASE_A, 64, BASE_B, 256, BASE_C, 256, None, path) == gr.GR_ERR_INVALID_PATH
    assert g(300, 256, 48, BASE_A, 48, BASE_B, 256, BASE_C, 256, None, gr.GR_PATH_TILE) == gr.GR_ERR_INVALID_PATH
    assert g(65, 256, 64, BASE_A, 64, BASE_B, 256, BASE_C, 256, None, gr.GR_PATH_SMALL_M) == gr.GR_ERR_INVALID_PATH


def test_bias_act_argument_checks_need_no_gpu():
    """gemm_bias_act_* run the shared argument checks before any HIP call,
    then reject unknown activations and a bias that overlaps C."""
    for f, g in ((gr.gemm_bias_act_f16, gr.gemm_bias_act_f16_forced),
                 (gr.gemm_bias_act_bf16, gr.gemm_bias_act_bf16_forced)):
        bias = BASE_C + (1 << 30)
        assert f(-1, 8, 8, BASE_A, 8, BASE_B, 8, bias, gr.GR_ACT_GELU, BASE_C, 8) == gr.GR_ERR_INVALID_DIM
        assert f(8, 8, 8, BASE_A, 8, BASE_B, 7, bias, gr.GR_ACT_GELU, BASE_C, 8) == gr.GR_ERR_INVALID_LD
        assert f(8, 8, 8, BASE_A, 8, BASE_B, 8, bias, -1, BASE_C, 8) == gr.GR_ERR_INVALID_ARG
        assert f(8, 8, 8, BASE_A, 8, BASE_B, 8, bias, 7, BASE_C, 8) == gr.GR_ERR_INVALID_ARG
        # the bias's 16 bytes overlap C's last row / first row
        assert f(8, 8, 8, BASE_A, 8, BASE_B, 8, BASE_C + 2 * 8 * 7, gr.GR_ACT_SILU, BASE_C, 8) == gr.GR_ERR_ALIAS
        assert f(8, 8, 8, BASE_A, 8, BASE_B, 8, BASE_C - 14, gr.GR_ACT_SILU, BASE_C, 8) == gr.GR_ERR_ALIAS
        assert f(0, 8, 8, 0, 8, BASE_B, 8, bias, gr.GR_ACT_TANH, 0, 8) == gr.GR_OK  # empty: nothing launched
        for path in (gr.GR_PATH_TILE_PACKED, gr.GR_PATH_SMALL_M_SPLIT, gr.GR_PATH_TILE_SPLIT, 99):
            assert g(8, 256, 64, BASE_A, 64, BASE_B, 256, bias, 2, BASE_C, 256, None, path) == gr.GR_ERR_INVALID_PATH
        assert g(300, 256, 48, BASE_A, 48, BASE_B, 256, bias, 2, BASE_C, 256, None,
                 gr.GR_PATH_TILE) == gr.GR_ERR_INVALID_PATH


def test_workspace_variants_argument_checks_need_no_gpu():
    """gemm_relu_bf16_ws / _forced_ws and gemm_bias_act_ws: the shared checks,
    then the format code, the activation code and a bias overlapping the
    workspace, all before any HIP call."""
    ws = BASE_C + (1 << 32)
    bias = BASE_C + (1 << 30)
    assert gr.gemm_relu_bf16_ws(-1, 8, 8, BASE_A, 8, BASE_B, 8, BASE_C, 8, ws, 1 << 20) == gr.GR_ERR_INVALID_DIM
    assert gr.gemm_relu_bf16_ws(8, 8, 8, BASE_A, 8, BASE_B, 8, BASE_C, 8, ws, -1) == gr.GR_ERR_INVALID_ARG
    assert gr.gemm_relu_bf16_ws(8, 8, 8, BASE_A, 8, BASE_B, 8, BASE_C, 8, BASE_A, 1 << 20) == gr.GR_ERR_ALIAS
    assert gr.gemm_relu_bf16_forced_ws(8, 256, 64, BASE_A, 64, BASE_B, 256, BASE_C, 256, ws, 1 << 20, None,
                                       99) == gr.GR_ERR_INVALID_PATH
    # too small a workspace for the forced split
    assert gr.gemm_relu_bf16_forced_ws(8, 4096, 8192, BASE_A, 8192, BASE_B, 4096, BASE_C, 4096, ws, 1024, None,
                                       gr.GR_PATH_SMALL_M_SPLIT) == gr.GR_ERR_INVALID_PATH
    f = gr.gemm_bias_act_ws
    args = (8, 8, 8, BASE_A, 8, BASE_B, 8)
    assert f(*args, bias, gr.GR_ACT_GELU, BASE_C, 8, 2, ws, 1 << 20) == gr.GR_ERR_INVALID_ARG      # format
    assert f(*args, bias, gr.GR_ACT_GELU, BASE_C, 8, -1, ws, 1 << 20) == gr.GR_ERR_INVALID_ARG     # format
    assert f(*args, bias, 7, BASE_C, 8, gr.GR_FMT_F16, ws, 1 << 20) == gr.GR_ERR_INVALID_ARG       # activation
    assert f(*args, ws + 64, gr.GR_ACT_GELU, BASE_C, 8, gr.GR_FMT_BF16, ws, 1 << 20) == gr.GR_ERR_ALIAS
    assert f(*args, bias, gr.GR_ACT_GELU, BASE_C, 8, gr.GR_FMT_BF16, ws, 1 << 20, None, 99) == gr.GR_ERR_INVALID_PATH
    assert f(0, 8, 8, 0, 8, BASE_B, 8, bias, gr.GR_ACT_TANH, 0, 8, gr.GR_FMT_F16, None, 0) == gr.GR_OK


def test_fp8_split_planner_and_checks_need_no_gpu():
    """gemm_fp8_bt_ws: split-K only for at most 128 tiles of 128 x 128 and a
    long K, a workspace large enough, the small-M stream first; workspace
    checks before any HIP call."""
    def plan(M, N, K, ws_bytes=1 << 30):
        st, p = gr.gemm_fp8_bt_plan_ws(M, N, K, BASE_A, K, BASE_B, K, None, 1, BASE_C, N, gr.GR_FMT_F16, ws_bytes)
        assert st == gr.GR_OK
        return p

    def size(M, N, K):
        st, b = gr.gemm_fp8_bt_workspace_size(M, N, K, BASE_A, K, BASE_B, K, BASE_C, N)
        assert st == gr.GR_OK
        return b
    p = plan(128, 8192, 8192)
    assert (p["path"], p["split_k"], p["grid"], p["block_m"]) == (gr.GR_PATH_TILE_SPLIT, 4, 256, 128)
    assert p["workspace"] == size(128, 8192, 8192) == 4 * 128 * 8192 * 4
    assert plan(128, 8192, 8192, size(128, 8192, 8192) - 256)["path"] == gr.GR_PATH_TILE   # too small
    assert plan(128, 8192, 8192, 0)["path"] == gr.GR_PATH_TILE
    assert plan(512, 8192, 8192)["path"] == gr.GR_PATH_TILE and size(512, 8192, 8192) == 0   # 256 tiles
    assert plan(4096, 4096, 4096)["path"] == gr.GR_PATH_TILE and size(4096, 4096, 4096) == 0
    assert plan(64, 4096, 4096)["path"] == gr.GR_PATH_TILE                  # K too short to pay
    assert plan(16, 4096, 8192)["path"] == gr.GR_PATH_SMALL_M and size(16, 4096, 8192) == 0
    assert size(128, 8192, 8032) == 0                                       # K % 64 != 0: guarded kernel
    # every split non-empty and a whole number of 64-byte strips
    for (M, N, K) in ((300, 270, 8192), (17, 130, 8128), (20, 1, 16384), (128, 4096, 16384)):
        p = plan(M, N, K)
        assert p["path"] == gr.GR_PATH_TILE_SPLIT, (M, N, K)
        tiles = ((M + 127) // 128) * ((N + 127) // 128)
        assert p["grid"] == tiles * p["split_k"] and 2 <= p["split_k"] <= 16 and tiles * p["split_k"] <= 256
    f = gr.gemm_fp8_bt_ws
    ws = BASE_C + (1 << 32)
    args = (128, 8192, 8192, BASE_A, 8192, BASE_B, 8192, 1.0, 1.0)
    assert f(*args, None, 1, BASE_C, 8192, 0, ws, -1) == gr.GR_ERR_INVALID_ARG
    assert f(*args, None, 1, BASE_C, 8192, 0, ws + 16, 1 << 20) == gr.GR_ERR_INVALID_ARG        # alignment
    assert f(*args, None, 1, BASE_C, 8192, 0, 0, 1 << 20) == gr.GR_ERR_NULL_PTR
    assert f(*args, None, 1, BASE_C, 8192, 0, BASE_B, 1 << 20) == gr.GR_ERR_ALIAS              # overlaps Bt
    assert f(*args, ws + 1024, 1, BASE_C, 8192, 0, ws, 1 << 20) == gr.GR_ERR_ALIAS              # overlaps bias
    assert f(*args, None, 1, BASE_C, 8192, 0, ws, 1 << 20, None, gr.GR_PATH_SMALL_M_SPLIT) == gr.GR_ERR_INVALID_PATH
    assert f(*args, None, 1, BASE_C, 8192, 0, ws, 1024, None, gr.GR_PATH_TILE_SPLIT) == gr.GR_ERR_INVALID_PATH
    assert f(128, 8192, 8032, BASE_A, 8032, BASE_B, 8032, 1.0, 1.0, None, 1, BASE_C, 8192, 0, ws, 1 << 30, None,
             gr.GR_PATH_TILE_SPLIT) == gr.GR_ERR_INVALID_PATH
    assert f(0, 8, 8, 0, 8, BASE_B, 8, 1.0, 1.0, None, 1, 0, 8, 0, None, 0) == gr.GR_OK


def test_mxfp8_planner_and_checks_need_no_gpu():
    """gemm_mxfp8_bt: the pipelined kernel for K % 128 == 0 with 16-byte
    operand rows and 4-byte scale rows, the guarded kernel otherwise;
    argument errors before any HIP call."""
    SA, SB = BASE_C + (1 << 31), BASE_C + (1 << 32)

    def plan(M, N, K, ldsa=None, ldsb=None, sa=SA, sb=SB, lda=None):
        kb = max(K // 32, 1)
        return gr.gemm_mxfp8_bt_plan(M, N, K, BASE_A, lda or max(K, 1), sa, ldsa or kb, BASE_B, max(K, 1), sb,
                                     ldsb or kb, None, 1, BASE_C, max(N, 1), gr.GR_FMT_F16)
    st, p = plan(4096, 4096, 4096)
    assert st == gr.GR_OK and (p["path"], p["block_m"], p["grid"]) == (gr.GR_PATH_TILE, 256, 256)
    assert plan(300, 270, 384)[1]["path"] == gr.GR_PATH_TILE and plan(300, 270, 384)[1]["block_m"] == 128
    assert plan(300, 270, 96)[1]["path"] == gr.GR_PATH_TILE_EDGE            # K % 128 != 0
    assert plan(300, 270, 384, ldsa=13)[1]["path"] == gr.GR_PATH_TILE_EDGE  # scale pitch not a multiple of 4
    assert plan(300, 270, 384, sb=SB + 2)[1]["path"] == gr.GR_PATH_TILE_EDGE
    assert plan(300, 270, 384, lda=392)[1]["path"] == gr.GR_PATH_TILE_EDGE  # A rows not 16-byte aligned
    assert plan(300, 270, 100)[0] == gr.GR_ERR_INVALID_DIM                  # K % 32 != 0
    assert plan(300, 270, 384, ldsa=11)[0] == gr.GR_ERR_INVALID_LD          # pitch < K/32
    assert plan(0, 270, 384)[1]["path"] == gr.GR_PATH_NONE
    f = gr.gemm_mxfp8_bt
    assert f(8, 8, 64, BASE_A, 64, 0, 2, BASE_B, 64, SB, 2, None, 1, BASE_C, 8) == gr.GR_ERR_NULL_PTR
    assert f(8, 8, 64, BASE_A, 64, BASE_C + 4, 2, BASE_B, 64, SB, 2, None, 1, BASE_C, 8) == gr.GR_ERR_ALIAS
    assert f(8, 8, 64, BASE_A, 64, SA, 2, BASE_B, 64, SB, 2, None, 7, BASE_C, 8) == gr.GR_ERR_INVALID_ARG
    assert gr.gemm_mxfp8_bt_forced(300, 270, 96, BASE_A, 96, SA, 3, BASE_B, 96, SB, 3, None, 1, BASE_C, 270,
                                   gr.GR_FMT_F16, None, gr.GR_PATH_TILE) == gr.GR_ERR_INVALID_PATH
    assert gr.gemm_mxfp8_bt_forced(8, 8, 64, BASE_A, 64, SA, 2, BASE_B, 64, SB, 2, None, 1, BASE_C, 8,
                                   gr.GR_FMT_F16, None, gr.GR_PATH_SMALL_M) == gr.GR_ERR_INVALID_PATH
    assert f(0, 8, 64, 0, 64, 0, 2, BASE_B, 64, SB, 2, None, 1, 0, 8) == gr.GR_OK


def test_mxfp4_planner_and_checks_need_no_gpu():
    """gemm_mxfp4_bt: K counts elements, pitches count bytes (>= K/2); the
    pipelined kernel for K % 128 == 0 with 16-byte rows, else guarded."""
    SA, SB = BASE_C + (1 << 31), BASE_C + (1 << 32)

    def plan(M, N, K, lda=None, ldbt=None):
        kb = max(K // 32, 1)
        return gr.gemm_mxfp4_bt_plan(M, N, K, BASE_A, lda or max(K // 2, 1), SA, kb, BASE_B, ldbt or max(K // 2, 1),
                                     SB, kb, None, 1, BASE_C, max(N, 1), gr.GR_FMT_F16)
    st, p = plan(4096, 4096, 4096)
    assert st == gr.GR_OK and (p["path"], p["block_m"], p["grid"]) == (gr.GR_PATH_TILE, 256, 256)
    assert plan(300, 270, 384)[1]["path"] == gr.GR_PATH_TILE          # 192-byte rows
    assert plan(300, 270, 96)[1]["path"] == gr.GR_PATH_TILE_EDGE      # K % 128 != 0
    assert plan(300, 270, 384, lda=200)[1]["path"] == gr.GR_PATH_TILE_EDGE
    assert plan(300, 270, 384, lda=191)[0] == gr.GR_ERR_INVALID_LD    # fewer than K/2 bytes
    assert plan(300, 270, 100)[0] == gr.GR_ERR_INVALID_DIM            # K % 32 != 0
    assert gr.gemm_mxfp4_bt(-1, 8, 64, BASE_A, 32, SA, 2, BASE_B, 32, SB, 2, None, 1, BASE_C, 8) == \
        gr.GR_ERR_INVALID_DIM
    assert gr.gemm_mxfp4_bt_forced(300, 270, 96, BASE_A, 48, SA, 3, BASE_B, 48, SB, 3, None, 1, BASE_C, 270,
                                   gr.GR_FMT_F16, None, gr.GR_PATH_TILE) == gr.GR_ERR_INVALID_PATH


def test_bias_act_bt_argument_checks_need_no_gpu():
    """gemm_bias_act_bt: the transposed-B checks, then format, activation,
    path and a bias overlapping C, before any HIP call."""
    f = gr.gemm_bias_act_bt
    bias = BASE_C + (1 << 30)
    args = (8, 8, 8, BASE_A, 8, BASE_B, 8)
    assert f(-1, 8, 8, BASE_A, 8, BASE_B, 8, bias, 2, BASE_C, 8) == gr.GR_ERR_INVALID_DIM
    assert f(8, 8, 8, BASE_A, 8, BASE_B, 7, bias, 2, BASE_C, 8) == gr.GR_ERR_INVALID_LD  # ldbt < K
    assert f(*args, bias, 2, BASE_C, 8, 2) == gr.GR_ERR_INVALID_ARG                      # format
    assert f(*args, bias, 7, BASE_C, 8, gr.GR_FMT_BF16) == gr.GR_ERR_INVALID_ARG         # activation
    assert f(*args, BASE_C + 8, 2, BASE_C, 8, gr.GR_FMT_F16) == gr.GR_ERR_ALIAS          # bias inside C
    assert f(*args, bias, 2, BASE_C, 8, gr.GR_FMT_F16, None, gr.GR_PATH_TILE_SPLIT) == gr.GR_ERR_INVALID_PATH
    assert f(300, 256, 48, BASE_A, 48, BASE_B, 48, bias, 2, BASE_C, 256, gr.GR_FMT_F16, None,
             gr.GR_PATH_TILE) == gr.GR_ERR_INVALID_PATH                                  # K % 32 != 0
    assert f(0, 8, 8, 0, 8, BASE_B, 8, bias, 2, 0, 8) == gr.GR_OK


def test_fp8_planner_and_checks_need_no_gpu():
    """gemm_fp8_bt: the pipelined kernel for K % 64 == 0 with 16-byte rows (any
    M, N), the guarded kernel otherwise; argument errors before any HIP call."""
    def plan8(M, N, K, lda=None, ldbt=None, ldc=None, a=BASE_A, b=BASE_B, c=BASE_C, act=1, fmt=gr.GR_FMT_F16):
        lda = max(K, 1) if lda is None else lda
        ldbt = max(K, 1) if ldbt is None else ldbt
        ldc = max(N, 1) if ldc is None else ldc
        return gr.gemm_fp8_bt_plan(M, N, K, a, lda, b, ldbt, None, act, c, ldc, fmt)
    st, p = plan8(4096, 4096, 4096)
    assert st == gr.GR_OK and p["path"] == gr.GR_PATH_TILE and (p["block_m"], p["block_k"], p["grid"]) == (256, 64, 256)
    assert plan8(17, 600, 256)[1]["path"] == gr.GR_PATH_TILE                       # M < 256: rows clamped
    assert plan8(17, 600, 256)[1]["block_m"] == 128                                # few tiles: 128 x 128
    st, p = plan8(8, 16384, 8192)
    assert p["path"] == gr.GR_PATH_SMALL_M and p["grid"] == 16384 // 64          # M <= 16, K % 512 == 0
    assert plan8(8, 16384, 8000)[1]["path"] == gr.GR_PATH_TILE                     # K % 512 != 0
    assert plan8(300, 270, 96)[1]["path"] == gr.GR_PATH_TILE_EDGE                  # K % 64 != 0
    assert plan8(300, 270, 128, lda=136)[1]["path"] == gr.GR_PATH_TILE_EDGE        # lda not a multiple of 16
    assert plan8(300, 270, 128, a=BASE_A + 8)[1]["path"] == gr.GR_PATH_TILE_EDGE   # A not 16-byte aligned
    st, p = plan8(300, 270, 100)
    assert p["grid"] == 3 * 3 and p["block_m"] == 128
    assert plan8(0, 5, 5)[1]["path"] == gr.GR_PATH_NONE
    assert plan8(8, 8, 8, lda=7)[0] == gr.GR_ERR_INVALID_LD
    assert plan8(8, 8, 8, act=7)[0] == gr.GR_ERR_INVALID_ARG
    assert plan8(8, 8, 8, fmt=2)[0] == gr.GR_ERR_INVALID_ARG
    assert plan8(8, 8, 8, c=BASE_A + 4)[0] == gr.GR_ERR_ALIAS   # C's bytes overlap A (8 x 8 bytes)
    assert plan8(8, 8, 8, c=BASE_A + 64)[0] == gr.GR_OK          # A spans 64 bytes, C starts after
    assert gr.gemm_fp8_bt(8, 8, 8, BASE_A, 8, BASE_B, 8, 1.0, 1.0, BASE_C + 2, 1, BASE_C, 8) == gr.GR_ERR_ALIAS
    assert gr.gemm_fp8_bt_forced(300, 270, 96, BASE_A, 96, BASE_B, 96, 1.0, 1.0, None, 1, BASE_C, 270, 0, None,
                                 gr.GR_PATH_TILE) == gr.GR_ERR_INVALID_PATH
    assert gr.gemm_fp8_bt_forced(300, 270, 128, BASE_A, 128, BASE_B, 128, 1.0, 1.0, None, 1, BASE_C, 270, 0, None,
                                 gr.GR_PATH_SMALL_M) == gr.GR_ERR_INVALID_PATH
    assert gr.gemm_fp8_bt_forced(8, 270, 128, BASE_A, 128, BASE_B, 128, 1.0, 1.0, None, 1, BASE_C, 270, 0, None,
                                 gr.GR_PATH_TILE_SPLIT) == gr.GR_ERR_INVALID_PATH


def test_act_codes_match_the_oracle():
    import oracle
    assert gr.ACT_CODES == oracle.ACTS


def test_plan_null_output_struct():
    lib = gr.lib()
    assert lib.gemm_relu_f16_plan(8, 8, 8, BASE_A, 8, BASE_B, 8, BASE_C, 8, None) == gr.GR_ERR_INVALID_ARG


def test_calls_validate_before_touching_the_device():
    # Invalid arguments are rejected identically with or without a GPU.
    assert gr.gemm_relu_f16(-1, 8, 8, BASE_A, 8, BASE_B, 8, BASE_C, 8) == gr.GR_ERR_INVALID_DIM
    assert gr.gemm_relu_f16(8, 8, 8, BASE_A, 8, BASE_B, 8, BASE_A, 8) == gr.GR_ERR_ALIAS
    assert gr.gemm_relu_f16_forced(8, 8, 8, BASE_A, 8, BASE_B, 8, BASE_C, 8, None, 99) == gr.GR_ERR_INVALID_PATH
    # tile path forced where its conditions fail: K not a multiple of 32,
    # fewer than 256 rows, misaligned B rows
    assert gr.gemm_relu_f16_forced(300, 256, 48, BASE_A, 48, BASE_B, 256, BASE_C, 256, None,
                                   gr.GR_PATH_TILE) == gr.GR_ERR_INVALID_PATH
    assert gr.gemm_relu_f16_forced(300, 256, 64, BASE_A, 65, BASE_B, 256, BASE_C, 256, None,
                                   gr.GR_PATH_TILE) == gr.GR_ERR_INVALID_PATH
    assert gr.gemm_relu_f16_forced(300, 250, 64, BASE_A, 64, BASE_B, 250, BASE_C, 256, None,
                                   gr.GR_PATH_TILE) == gr.GR_ERR_INVALID_PATH
    # small-M forced with too many rows (the stream takes at most 64)
    assert gr.gemm_relu_f16_forced(65, 256, 64, BASE_A, 64, BASE_B, 256, BASE_C, 256, None,
                                   gr.GR_PATH_SMALL_M) == gr.GR_ERR_INVALID_PATH
    # empty problems succeed without a launch
    assert gr.gemm_relu_f16(0, 8, 8, 0, 8, BASE_B, 8, 0, 8) == gr.GR_OK


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


@pytest.mark.skipif(_gpu_visible(), reason="checks the no-device error path")
def test_no_device_error_without_gpu():
    assert gr.gemm_relu_f16(8, 8, 8, BASE_A, 8, BASE_B, 8, BASE_C, 8) == gr.GR_ERR_NO_DEVICE


def test_product_path_never_imports_the_oracle():
    """The product package and the library sources name nothing from oracle/."""
    pkg = os.path.join(ROOT, "dense_gemm_epilogue_tiled_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "oracle_gemm_relu" not in text, f


def test_no_kernel_spills_to_scratch():
    """Every kernel of the built library keeps its live values in registers.

    A spill reload inside the pipelined loops is a vector-memory load; the
    compiler, which cannot see the hand-placed copies, would then wait for
    every copy in flight.  Checked with the compiler's resource report of a
    fresh device-only build of the library sources (no GPU needed)."""
    import subprocess
    from dense_gemm_epilogue_tiled_amd import build as b
    cmd = [b.HIPCC, *b.FLAGS, "-c", "--cuda-device-only", b.SRC, "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    names = re.findall(r"Function Name: (\S+)", res.stderr)
    scratch = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", res.stderr)]
    assert names and len(names) == len(scratch)
    hot = dict(zip(names, scratch))
    assert any("gemm_relu_tile3_kernel" in n for n in hot) and any("gemm_fp8_tile_kernel" in n for n in hot), names
    # every kernel, whatever its epilogue: the other pipelined 256 x 256
    # kernels may spill a few bytes outside their steady loop; the 256 x 256
    # kernel for K % 64 == 0 (in place, unaligned and persistent), the
    # small-M and the 128 x 128 kernels must not spill at all (a reload in
    # the persistent loop would wait for the next tile's copies in flight)
    for n, s in hot.items():
        limit = 0 if ("smallm" in n or "tile128" in n or "tile322gemm_relu_tile3_kernel" in n) else 16
        assert s <= limit, (n, s)


def test_noalloc_refuses_problems_beyond_its_scratch():
    """gemm_relu_f16_noalloc checks its arguments and the scratch the problem
    needs before any HIP call: bad arguments keep their codes, a workspace
    need above the static scratch is GR_ERR_SCRATCH (no GPU needed)."""
    M, N, K = 2048, 2048, 8001
    lda = K + 1  # K % 32 != 0 and too few tiles for the in-place kernel: both operands copied
    st, need = gr.gemm_relu_f16_workspace_size(M, N, K, BASE_A, lda, BASE_B, N, BASE_C, N)
    assert st == gr.GR_OK and need > gr.NOALLOC_SCRATCH_BYTES
    assert gr.gemm_relu_f16_noalloc(M, N, K, BASE_A, lda, BASE_B, N, BASE_C, N) == gr.GR_ERR_SCRATCH
    assert gr.gemm_relu_status_string(gr.GR_ERR_SCRATCH) == "GR_ERR_SCRATCH"
    assert gr.gemm_relu_f16_noalloc(-1, N, K, BASE_A, lda, BASE_B, N, BASE_C, N) == gr.GR_ERR_INVALID_DIM
    assert gr.gemm_relu_f16_noalloc(M, N, K, BASE_A, K - 1, BASE_B, N, BASE_C, N) == gr.GR_ERR_INVALID_LD
    assert gr.gemm_relu_f16_noalloc(M, N, K, 0, lda, BASE_B, N, BASE_C, N) == gr.GR_ERR_NULL_PTR
    # an empty problem launches nothing and succeeds anywhere
    assert gr.gemm_relu_f16_noalloc(0, N, K, BASE_A, lda, BASE_B, N, BASE_C, N) == gr.GR_OK


def plan_ta(M, N, K, ldat=None, ldb=None, ldc=None, a=BASE_A, b=BASE_B, c=BASE_C):
    ldat = max(M, 1) if ldat is None else ldat
    ldb = max(N, 1) if ldb is None else ldb
    ldc = max(N, 1) if ldc is None else ldc
    return gr.gemm_relu_f16_ta_plan(M, N, K, a, ldat, b, ldb, c, ldc)


def test_transposed_a_planner_and_checks():
    # the three paths
    assert plan_ta(8, 16384, 8192)[1]["path"] == gr.GR_PATH_SMALL_M
    assert plan_ta(4096, 4096, 4096)[1]["path"] == gr.GR_PATH_TILE
    assert plan_ta(300, 520, 96, ldat=304)[1]["path"] == gr.GR_PATH_TILE
    st, p = plan_ta(4096, 4096, 4096)
    assert (p["block_m"], p["block_n"], p["block_k"], p["grid"]) == (256, 256, 32, 256)
    assert plan_ta(255, 4096, 4096)[1]["path"] == gr.GR_PATH_TILE_EDGE          # M < 256
    assert plan_ta(4096, 4096, 4100)[1]["path"] == gr.GR_PATH_TILE_EDGE         # K % 32 != 0
    assert plan_ta(4096, 4096, 4096, ldat=4100)[1]["path"] == gr.GR_PATH_TILE_EDGE  # At rows not 16-byte
    assert plan_ta(8, 32, 4096)[1]["path"] == gr.GR_PATH_TILE_EDGE              # N < 64
    assert plan_ta(8, 4096, 4096, ldat=9, b=BASE_B + 2)[1]["path"] == gr.GR_PATH_SMALL_M  # any alignment
    # argument checks: At is K x M with pitch >= M
    assert plan_ta(512, 512, 64, ldat=511)[0] == gr.GR_ERR_INVALID_LD
    assert plan_ta(-1, 512, 64)[0] == gr.GR_ERR_INVALID_DIM
    assert plan_ta(0, 512, 64)[1]["path"] == gr.GR_PATH_NONE
    assert gr.gemm_relu_f16_ta(512, 512, 64, 0, 512, BASE_B, 512, BASE_C, 512) == gr.GR_ERR_NULL_PTR
    assert gr.gemm_relu_f16_ta_forced(4096, 4096, 4100, BASE_A, 4096, BASE_B, 4096, BASE_C, 4096, None,
                                      gr.GR_PATH_TILE) == gr.GR_ERR_INVALID_PATH
    assert gr.gemm_relu_f16_ta_forced(4096, 4096, 4096, BASE_A, 4096, BASE_B, 4096, BASE_C, 4096, None,
                                      gr.GR_PATH_TILE_PACKED) == gr.GR_ERR_INVALID_PATH
    # C overlapping At
    assert plan_ta(64, 64, 64, a=BASE_A, c=BASE_A + 64)[0] == gr.GR_ERR_ALIAS


def test_stream_read_probe_checks_arguments():
    """The read-ceiling probe refuses sizes that are not whole 8 MiB granules,
    null and misaligned pointers and a sink inside the buffer before any HIP
    call (no GPU needed)."""
    g = 8 << 20
    assert gr.gemm_relu_stream_read(BASE_A, g - 16, BASE_C) == gr.GR_ERR_INVALID_ARG
    assert gr.gemm_relu_stream_read(BASE_A, 0, BASE_C) == gr.GR_ERR_INVALID_ARG
    assert gr.gemm_relu_stream_read(0, g, BASE_C) == gr.GR_ERR_NULL_PTR
    assert gr.gemm_relu_stream_read(BASE_A, g, 0) == gr.GR_ERR_NULL_PTR
    assert gr.gemm_relu_stream_read(BASE_A + 8, g, BASE_C) == gr.GR_ERR_INVALID_ARG
    assert gr.gemm_relu_stream_read(BASE_A, g, BASE_C + 4) == gr.GR_ERR_INVALID_ARG
    assert gr.gemm_relu_stream_read(BASE_A, g, BASE_A + 4096) == gr.GR_ERR_ALIAS
    assert gr.gemm_relu_stream_read(BASE_A, g, BASE_C, pattern=2) == gr.GR_ERR_INVALID_ARG
    assert gr.gemm_relu_stream_read(BASE_A, g, BASE_C, pattern=-1) == gr.GR_ERR_INVALID_ARG


def test_every_kernel_has_device_code():
    """Each kernel the host code registers (its launch stub) has a kernel
    descriptor in the embedded gfx950 code object.  A library whose device
    pass was compiled from older sources than its host pass would otherwise
    pass every CPU check and fail only at launch."""
    with open(gr.LIB_PATH, "rb") as f:
        data = f.read()
    toks = set(re.findall(rb"[A-Za-z0-9_.$]{8,}", data))
    stubs = [t for t in toks if b"__device_stub__" in t]
    assert len(stubs) > 50
    missing = []
    for s in stubs:
        # the stub's mangled name differs from the kernel's only in its
        # identifier: <n>__device_stub__name -> <n-15>name
        k = re.sub(rb"(\d+)__device_stub__", lambda m: str(int(m.group(1)) - 15).encode(), s, count=1)
        if k + b".kd" not in toks:
            missing.append(k.decode())
    assert not missing, missing[:5]


def test_persistent_path_checks():
    """The persistent tile loop takes whole tiles, K % 64 == 0 and 16-byte
    rows of A and B (C's rows may start anywhere: 16-byte stores at any
    alignment); anything else is refused before any HIP call."""
    base = (0x100000, 0x200000000000, 0x400000000000)

    def forced(M, N, K, lda, ldb, ldc, a=base[0], b=base[1], c=base[2]):
        return gr.gemm_relu_f16_forced(M, N, K, a, lda, b, ldb, c, ldc, None, gr.GR_PATH_TILE_PERSISTENT)
    assert forced(4096, 4100, 256, 256, 4100, 4100) == gr.GR_ERR_INVALID_PATH   # N not whole tiles
    assert forced(4000, 4096, 256, 256, 4096, 4096) == gr.GR_ERR_INVALID_PATH   # M not whole tiles
    assert forced(4096, 4096, 96, 96, 4096, 4096) == gr.GR_ERR_INVALID_PATH     # K % 64 != 0
    # rows of C not 16-byte aligned: accepted (no GPU here: the device check fails next)
    assert forced(4096, 4096, 256, 256, 4096, 4100) != gr.GR_ERR_INVALID_PATH
    assert forced(4096, 4096, 256, 260, 4096, 4096) == gr.GR_ERR_INVALID_PATH   # rows of A not 16-byte
