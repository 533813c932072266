"""The C-ABI library loads, exports what include/bitnet_tm.h declares, and rejects
bad arguments on the host.  No compute call is made, so this runs without a GPU:
every case below fails validation before the library touches the device."""
import ctypes
import os
import re

import pytest

from ternary_weight_decoder_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitnet_tm.h")

ERR = {"NULL": 1, "SHAPE": 2, "ALIGN": 3, "WORKSPACE": 4, "ALIAS": 7}


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|size_t|bitnet_status)\s*\*?\s*"
                                 r"(bitnet_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_build.LIB_PATH):
        _build.build()
    lib = ctypes.CDLL(_build.LIB_PATH)
    p, i64, sz, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int32
    lib.bitnet_status_string.restype = ctypes.c_char_p
    lib.bitnet_status_string.argtypes = [i32]
    lib.bitnet_packed_bytes.restype = sz
    lib.bitnet_packed_bytes.argtypes = [i64, i64]
    lib.bitnet_matmul_workspace_bytes.restype = sz
    lib.bitnet_matmul_workspace_bytes.argtypes = [i64, i64]
    lib.bitnet_ternarize_workspace_bytes.restype = sz
    lib.bitnet_ternarize_workspace_bytes.argtypes = [i64]
    lib.bitnet_ternary_matmul.argtypes = [i64, i64, i64, p, p, p, p, p, sz, p, p, p, p]
    lib.bitnet_ternary_matmul.restype = i32
    lib.bitnet_ternarize_pack.argtypes = [p, i64, i64, p, p, p, sz, p]
    lib.bitnet_ternarize_pack.restype = i32
    lib.bitnet_quant_act.argtypes = [p, i64, i64, p, p, p]
    lib.bitnet_quant_act.restype = i32
    lib.bitnet_ternary_matmul_q8.argtypes = [i64, i64, i64, p, p, p, p, p, p, sz, p, p]
    lib.bitnet_ternary_matmul_q8.restype = i32
    lib.bitnet_ternary_matmul_grouped.argtypes = [i64, p, i32, p, p, sz, p]
    lib.bitnet_ternary_matmul_grouped.restype = i32
    return lib


def test_header_declares_the_three_named_entry_points():
    fns = declared_functions()
    for name in ("bitnet_ternarize_pack", "bitnet_quant_act", "bitnet_ternary_matmul"):
        assert name in fns


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_library_has_gfx950_code_object():
    data = open(_build.LIB_PATH, "rb").read()
    assert b"gfx950" in data


def test_size_helpers(L):
    assert L.bitnet_packed_bytes(1536, 1536) == 589824
    assert L.bitnet_packed_bytes(8960, 1536) == 3440640
    assert L.bitnet_ternarize_workspace_bytes(8960) == 8960 * 8
    ws = L.bitnet_matmul_workspace_bytes(1800, 1536)
    assert ws >= 1800 * 1536 + 2 * 4 * 1800 and ws % 256 == 0
    for s in range(0, 7):
        assert L.bitnet_status_string(s)


# Fake, never-dereferenced device addresses: validation rejects before any use.
A = 0x7f0000000000   # 256-byte aligned
NULL = None


def test_matmul_shape_limits(L):
    """The largest shapes the size rules allow (each bound within a few hundred
    elements of 2^31; the GPU tests run them) pass the shape check and stop at
    the workspace check here, and one more row or column is a shape error."""
    f = L.bitnet_ternary_matmul
    at_limit = ((1398101, 256, 1536),    # M*K
                (1800, 278460, 128),     # (M + 128)*N*4
                (16, 239674, 8960))      # N*K
    over = ((1398102, 256, 1536), (1800, 278461, 128), (16, 239675, 8960))
    for M, N, K in at_limit:
        assert M * K < 1 << 31 and N * K < 1 << 31 and (M + 128) * N * 4 < 1 << 31
        assert f(M, N, K, A, A, A, A, A, 0, NULL, NULL, NULL, NULL) == ERR["WORKSPACE"]
    for M, N, K in over:
        assert f(M, N, K, A, A, A, A, A, 0, NULL, NULL, NULL, NULL) == ERR["SHAPE"]


def test_matmul_validation(L):
    ws_ok = L.bitnet_matmul_workspace_bytes(1, 1536)
    f = L.bitnet_ternary_matmul
    assert f(1, 1536, 1536, NULL, A, A, A, A, ws_ok, NULL, NULL, NULL, NULL) == ERR["NULL"]
    assert f(1, 1536, 1536, A, NULL, A, A, A, ws_ok, NULL, NULL, NULL, NULL) == ERR["NULL"]
    assert f(1, 1536, 1000, A, A, A, A, A, ws_ok, NULL, NULL, NULL, NULL) == ERR["SHAPE"]
    assert f(0, 1536, 1536, A, A, A, A, A, ws_ok, NULL, NULL, NULL, NULL) == ERR["SHAPE"]
    assert f(1, 0, 1536, A, A, A, A, A, ws_ok, NULL, NULL, NULL, NULL) == ERR["SHAPE"]
    assert f(1, 1 << 31, 128, A, A, A, A, A, ws_ok, NULL, NULL, NULL, NULL) == ERR["SHAPE"]
    assert f(1 << 20, 1 << 12, 128, A, A, A, A, A, ws_ok, NULL, NULL, NULL, NULL) == ERR["SHAPE"]
    assert f(1, 1536, 1536, A + 4, A, A, A, A, ws_ok, NULL, NULL, NULL, NULL) == ERR["ALIGN"]
    assert f(1, 1536, 1536, A, A + 8, A, A, A, ws_ok, NULL, NULL, NULL, NULL) == ERR["ALIGN"]
    assert f(1, 1536, 1536, A, A, A, A + 2, A, ws_ok, NULL, NULL, NULL, NULL) == ERR["ALIGN"]
    assert f(1, 1536, 1536, A, A, A, A, A, ws_ok, A + 4, NULL, NULL, NULL) == ERR["ALIGN"]
    assert f(1, 1536, 1536, A, A, A, A, A, ws_ok - 1, NULL, NULL, NULL, NULL) == ERR["WORKSPACE"]
    assert f(1, 1536, 1536, A, A, A, A, NULL, ws_ok, NULL, NULL, NULL, NULL) == ERR["WORKSPACE"]
    assert f(1, 1536, 1536, A, A, A, A, A + 16, ws_ok, NULL, NULL, NULL, NULL) == ERR["ALIGN"]


def test_ternarize_and_quant_validation(L):
    ws = L.bitnet_ternarize_workspace_bytes(64)
    t = L.bitnet_ternarize_pack
    assert t(NULL, 64, 128, A, A, A, ws, NULL) == ERR["NULL"]
    assert t(A, 64, 100, A, A, A, ws, NULL) == ERR["SHAPE"]
    assert t(A + 4, 64, 128, A, A, A, ws, NULL) == ERR["ALIGN"]
    assert t(A, 64, 128, A, A, A, ws - 8, NULL) == ERR["WORKSPACE"]
    assert t(A, 64, 128, A, A, NULL, ws, NULL) == ERR["WORKSPACE"]
    q = L.bitnet_quant_act
    assert q(NULL, 4, 128, A, A, NULL) == ERR["NULL"]
    assert q(A, 4, 130, A, A, NULL) == ERR["SHAPE"]
    assert q(A, 4, 128, A + 1, A, NULL) == ERR["ALIGN"]
    q8 = L.bitnet_ternary_matmul_q8
    wsm = L.bitnet_matmul_workspace_bytes(4, 128)
    assert q8(4, 8, 128, NULL, A, A, A, A, A, wsm, NULL, NULL) == ERR["NULL"]
    assert q8(4, 8, 128, A, A, A, A, A, A, wsm - 1, NULL, NULL) == ERR["WORKSPACE"]


def test_grouped_validation(L):
    from ternary_weight_decoder_amd.binding import bitnet_problem
    arr = (bitnet_problem * 2)()
    arr[0] = bitnet_problem(A, A, A, A, 1536, 1536)
    arr[1] = bitnet_problem(A, A, A, A, 256, 1000)
    g = L.bitnet_ternary_matmul_grouped
    ref = ctypes.cast(ctypes.byref(arr), ctypes.c_void_p)
    assert g(1, NULL, 2, ref, A, 1 << 30, NULL) == ERR["NULL"]
    assert g(1, A, 0, ref, A, 1 << 30, NULL) == ERR["SHAPE"]
    assert g(1, A, 257, ref, A, 1 << 30, NULL) == ERR["SHAPE"]
    assert g(1, A, 2, ref, A, 1 << 30, NULL) == ERR["SHAPE"]   # K = 1000
    arr[1] = bitnet_problem(A, A, NULL, A, 256, 1536)
    assert g(1, A, 2, ref, A, 1 << 30, NULL) == ERR["NULL"]
    arr[1] = bitnet_problem(A, A, A, A, 256, 1536)
    assert g(1, A, 2, ref, A, 16, NULL) == ERR["WORKSPACE"]


def test_grouped_workspace_shares_inputs(L):
    """Problems with the same x pointer and K take one workspace region; the
    same pointer with another K (other rows) takes its own."""
    from ternary_weight_decoder_amd.binding import BITNET_MAX_GROUP, bitnet_problem
    f = L.bitnet_grouped_workspace_bytes
    f.restype = ctypes.c_size_t
    f.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32]
    X1, X2 = A, A + (1 << 30)

    def ws(probs, M=40, count=None):
        arr = (bitnet_problem * len(probs))(*[bitnet_problem(x, A, A, A, n, k)
                                              for x, n, k in probs])
        return f(M, ctypes.addressof(arr), len(probs) if count is None else count)

    one = ws([(X1, 1536, 1536)])
    assert one > 0
    assert ws([(X1, 1536, 1536), (X1, 256, 1536), (X1, 256, 1536)]) == one   # q, k, v
    assert ws([(X1, 1536, 1536), (X2, 256, 1536)]) == 2 * one
    assert ws([(X1, 1536, 1536), (X1, 1536, 128)]) == one + ws([(X1, 1536, 128)])
    assert ws([(X1, 1536, 1536), (X2, 1536, 1536), (X1, 8960, 1536), (X2, 72, 1536)]) == 2 * one
    assert ws([(X1, 1536, 1536)], count=BITNET_MAX_GROUP + 1) == 0
    assert ws([(X1, 1536, 1536)], count=0) == 0


def test_stages_validation(L):
    """Argument checks of the staged call; every case fails before any device
    work (the addresses are never dereferenced)."""
    from ternary_weight_decoder_amd.binding import bitnet_problem
    p, i64, sz, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int32
    L.bitnet_ternary_matmul_stages.argtypes = [i64, p, i32, p, i32, p, p, sz, p]
    L.bitnet_ternary_matmul_stages.restype = i32
    L.bitnet_stages_workspace_bytes.argtypes = [i64, p, i32]
    L.bitnet_stages_workspace_bytes.restype = sz
    MB = 1 << 20
    X0, YQ, YK, YV, YO = (A + i * MB for i in range(5))

    def problems(*rows):
        arr = (bitnet_problem * len(rows))()
        for i, r in enumerate(rows):
            arr[i] = bitnet_problem(*r)
        return arr, ctypes.cast(ctypes.byref(arr), ctypes.c_void_p)

    def ends(*e):
        arr = (i32 * len(e))(*e)
        return arr, ctypes.cast(ctypes.byref(arr), ctypes.c_void_p)

    # q, k, v read X0; o reads q's output.
    chain = [(X0, A, A, YQ, 1536, 1536), (X0, A, A, YK, 256, 1536), (X0, A, A, YV, 256, 1536),
             (YQ, A, A, YO, 1536, 1536)]
    arr, ref = problems(*chain)
    e, eref = ends(3, 4)
    wsb = L.bitnet_stages_workspace_bytes(1, ref, 4)
    # header + one tagged (value, counter) pair per output, each region 256-aligned
    assert wsb == 256 + 2 * 1536 * 8 + 2 * 256 * 8
    assert L.bitnet_stages_workspace_bytes(17, ref, 4) == 0
    assert L.bitnet_stages_workspace_bytes(1, ref, 0) == 0
    g = L.bitnet_ternary_matmul_stages
    assert g(1, NULL, 4, eref, 2, ref, A, wsb, NULL) == ERR["NULL"]
    assert g(1, A, 4, NULL, 2, ref, A, wsb, NULL) == ERR["NULL"]
    assert g(1, A, 0, eref, 2, ref, A, wsb, NULL) == ERR["SHAPE"]
    assert g(17, A, 4, eref, 2, ref, A, wsb, NULL) == ERR["SHAPE"]      # M > 16
    big, bref = problems((X0, A, A, YQ, 1536, 8960))
    one, oref = ends(1)
    assert g(2, A, 1, oref, 1, bref, A, 1 << 30, NULL) == ERR["SHAPE"]  # 2 x 8960 > one row
    bad, badref = ends(2, 2)                                             # not increasing
    assert g(1, A, 4, badref, 2, ref, A, wsb, NULL) == ERR["SHAPE"]
    short, sref = ends(1, 3)                                             # does not end at count
    assert g(1, A, 4, sref, 2, ref, A, wsb, NULL) == ERR["SHAPE"]
    assert g(1, A, 4, eref, 2, ref, A, wsb - 4, NULL) == ERR["WORKSPACE"]
    assert g(1, A, 4, eref, 2, ref, A + 16, wsb, NULL) == ERR["ALIGN"]
    # A reader's K must equal its producer's N.
    arr2, ref2 = problems(*chain[:3], (YQ, A, A, YO, 1536, 1024))
    assert g(1, A, 4, eref, 2, ref2, A, 1 << 30, NULL) == ERR["SHAPE"]
    # Overlapping outputs.
    arr3, ref3 = problems(chain[0], (X0, A, A, YQ + 256, 256, 1536), *chain[2:])
    assert g(1, A, 4, eref, 2, ref3, A, 1 << 30, NULL) == ERR["ALIAS"]
    # An input that a later stage overwrites (v reads o's output buffer).
    arr4, ref4 = problems(*chain[:2], (YO, A, A, YV, 256, 1536), chain[3])
    assert g(1, A, 4, eref, 2, ref4, A, 1 << 30, NULL) == ERR["ALIAS"]
    # A reader in the same stage as its producer (k reads q's output).
    arr5, ref5 = problems(chain[0], (YQ, A, A, YK, 256, 1536), *chain[2:])
    assert g(1, A, 4, eref, 2, ref5, A, 1 << 30, NULL) == ERR["ALIAS"]


def test_table_entry_points_validation(L):
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    L.bitnet_i8_quant_weights_rows.argtypes = [p, i64, i64, p, p, p]
    L.bitnet_i8_quant_weights_rows.restype = i32
    L.bitnet_embed_lookup.argtypes = [p, i64, p, p, i64, i64, p, p]
    L.bitnet_embed_lookup.restype = i32
    L.bitnet_lm_head.argtypes = [i64, i64, i64, p, p, p, p, p, p, p, p]
    L.bitnet_lm_head.restype = i32
    L.bitnet_table_bytes.argtypes = [i64, i64]
    L.bitnet_table_bytes.restype = ctypes.c_size_t
    L.bitnet_table_quant.argtypes = [p, i64, i64, p, p, p]
    L.bitnet_table_quant.restype = i32
    assert L.bitnet_table_bytes(151936, 1536) == 151936 * 1536
    assert L.bitnet_table_bytes(40, 1536) == 48 * 1536
    assert L.bitnet_table_bytes(17, 320) == 32 * 512
    assert L.bitnet_table_bytes(8, 100) == 0
    tq = L.bitnet_table_quant
    assert tq(NULL, 8, 64, A, A, NULL) == ERR["NULL"]
    assert tq(A, 8, 96, A, A, NULL) == ERR["SHAPE"]
    assert tq(A, 8, 64, A, A + 2, NULL) == ERR["ALIGN"]
    rq = L.bitnet_i8_quant_weights_rows
    assert rq(NULL, 8, 64, A, A, NULL) == ERR["NULL"]
    assert rq(A, 8, 96, A, A, NULL) == ERR["SHAPE"]
    assert rq(A, 0, 64, A, A, NULL) == ERR["SHAPE"]
    assert rq(A, 8, 64, A + 4, A, NULL) == ERR["ALIGN"]
    e = L.bitnet_embed_lookup
    assert e(NULL, 0, NULL, NULL, 8, 64, NULL, NULL) == 0          # no tokens: nothing to do
    assert e(A, 4, NULL, A, 8, 64, A, NULL) == ERR["NULL"]
    assert e(A, -1, A, A, 8, 64, A, NULL) == ERR["SHAPE"]
    assert e(A, 4, A, A, 8, 100, A, NULL) == ERR["SHAPE"]
    assert e(A + 2, 4, A, A, 8, 64, A, NULL) == ERR["ALIGN"]
    assert e(A, 4, A, A, 8, 64, A + 4, NULL) == ERR["ALIGN"]
    h = L.bitnet_lm_head
    assert h(1, 151936, 1536, NULL, A, A, A, NULL, NULL, NULL, NULL) == ERR["NULL"]
    assert h(17, 151936, 1536, A, A, A, A, NULL, NULL, NULL, NULL) == ERR["SHAPE"]   # M > 16
    assert h(0, 151936, 1536, A, A, A, A, NULL, NULL, NULL, NULL) == ERR["SHAPE"]
    assert h(1, 151936, 1500, A, A, A, A, NULL, NULL, NULL, NULL) == ERR["SHAPE"]
    assert h(16, 100, 4096, A, A, A, A, NULL, NULL, NULL, NULL) == ERR["SHAPE"]     # LDS
    assert h(1, 151936, 1536, A + 4, A, A, A, NULL, NULL, NULL, NULL) == ERR["ALIGN"]
    assert h(1, 151936, 1536, A, A, A, A, A + 4, NULL, NULL, NULL) == ERR["ALIGN"]


def test_noalloc_validation(L):
    p, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    L.bitnet_scratch_bytes.argtypes = []
    L.bitnet_scratch_bytes.restype = sz
    L.bitnet_ternary_matmul_noalloc.argtypes = [i64, i64, i64, p, p, p, p, p, p, p, p]
    L.bitnet_ternary_matmul_noalloc.restype = i32
    assert L.bitnet_scratch_bytes() == 32 << 20
    f = L.bitnet_ternary_matmul_noalloc
    assert f(1, 1536, 1536, NULL, A, A, A, NULL, NULL, NULL, NULL) == ERR["NULL"]
    assert f(1, 1536, 1000, A, A, A, A, NULL, NULL, NULL, NULL) == ERR["SHAPE"]
    assert f(1, 1536, 1536, A + 4, A, A, A, NULL, NULL, NULL, NULL) == ERR["ALIGN"]
    # beyond the built-in scratch: rejected on the host, nothing launched
    assert L.bitnet_matmul_workspace_bytes(1800, 18688) > L.bitnet_scratch_bytes()
    assert L.bitnet_matmul_workspace_bytes(1800, 18560) <= L.bitnet_scratch_bytes()
    assert f(1800, 64, 18688, A, A, A, A, NULL, NULL, NULL, NULL) == 8


def test_dwconv_validation(L):
    p, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    L.bitnet_i8_dwconv_workspace_bytes.argtypes = [i64, i64, i64]
    L.bitnet_i8_dwconv_workspace_bytes.restype = sz
    L.bitnet_i8_dwconv.argtypes = [i64, i64, i64, i64, p, p, p, p, i32, p, p, sz, p, p, p]
    L.bitnet_i8_dwconv.restype = i32
    wsb = L.bitnet_i8_dwconv_workspace_bytes
    assert wsb(1, 8192, 512) == 64 * 512 * 4 and wsb(2, 129, 64) == 2 * 2 * 64 * 4
    assert wsb(1, 10, 100) == 0
    f = L.bitnet_i8_dwconv
    ws = wsb(1, 100, 64)
    assert f(1, 100, 64, 7, NULL, A, A, NULL, 0, A, A, ws, NULL, NULL, NULL) == ERR["NULL"]
    assert f(1, 100, 96, 7, A, A, A, NULL, 0, A, A, ws, NULL, NULL, NULL) == ERR["SHAPE"]
    assert f(1, 100, 64, 65, A, A, A, NULL, 0, A, A, ws, NULL, NULL, NULL) == ERR["SHAPE"]
    assert f(1, 100, 64, 0, A, A, A, NULL, 0, A, A, ws, NULL, NULL, NULL) == ERR["SHAPE"]
    assert f(1, 100, 64, 7, A + 4, A, A, NULL, 0, A, A, ws, NULL, NULL, NULL) == ERR["ALIGN"]
    assert f(1, 100, 64, 7, A, A, A, NULL, 0, A, A, ws - 4, NULL, NULL, NULL) == ERR["WORKSPACE"]
