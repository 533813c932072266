"""Python handle on the plain CPU oracle (``bitnet_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may use this package; the product library never does.  It
shares no code with the HIP path: inputs come from the seeded generators and
results are compared element by element.

All arrays are numpy, C-contiguous.  See ``bitnet_oracle.c`` for what each
function computes and which passage of the pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bitnet_oracle.c")
# BITNET_ORACLE_LIB points the tests at a deliberately broken build (mutant
# checks of the pins); it is never set in normal use.
DEFAULT_LIB_PATH = os.path.join(_HERE, "libbitnet_oracle.so")
LIB_PATH = os.environ.get("BITNET_ORACLE_LIB") or DEFAULT_LIB_PATH

CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
          "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/libbitnet_oracle.so``."""
    if force or not os.path.exists(DEFAULT_LIB_PATH):
        tmp = DEFAULT_LIB_PATH + ".tmp"
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, DEFAULT_LIB_PATH)
    return DEFAULT_LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=True)
        L = ctypes.CDLL(LIB_PATH)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        f32 = ctypes.c_float
        L.oracle_absmean.argtypes = [p, i64, i64]
        L.oracle_absmean.restype = f32
        L.oracle_ternarize.argtypes = [p, i64, i64, p, p]
        L.oracle_pack.argtypes = [p, i64, i64, p]
        L.oracle_unpack.argtypes = [p, i64, i64, p]
        L.oracle_unpack.restype = i64
        L.oracle_code_at.argtypes = [p, i64, i64, i64]
        L.oracle_code_at.restype = ctypes.c_int
        L.oracle_ternarize_pack.argtypes = [p, i64, i64, p, p]
        L.oracle_quant_act.argtypes = [p, i64, i64, p, p]
        L.oracle_matmul_i32.argtypes = [p, p, i64, i64, i64, p]
        L.oracle_dequant.argtypes = [p, f32, p, i64, i64, p]
        L.oracle_ternary_matmul.argtypes = [i64, i64, i64, p, p, f32, p, p, p, p]
        L.oracle_matmul_sampled.argtypes = [i64, i64, p, p, p, f32, p, p, i64, p, p]
        L.oracle_i8_quant_weights.argtypes = [p, i64, i64, p, p]
        L.oracle_i8_matmul.argtypes = [p, p, i64, i64, i64, p]
        L.oracle_i8_linear.argtypes = [i64, i64, i64, p, p, f32, p, ctypes.c_int, p, p, p, p]
        L.oracle_i8_linear_sampled.argtypes = [i64, i64, p, p, p, f32, p, ctypes.c_int, p, p,
                                               i64, p, p, p]
        L.oracle_rowq_quant_weights.argtypes = [p, i64, i64, p, p]
        L.oracle_rowq_embed.argtypes = [p, i64, p, p, i64, i64, p]
        L.oracle_rowq_linear.argtypes = [i64, i64, i64, p, p, p, p, p, p, p]
        L.oracle_rowq_linear_sampled.argtypes = [i64, p, p, p, p, p, p, i64, p, p]
        L.oracle_i8_linear_rows.argtypes = [i64, i64, i64, p, p, p, p, ctypes.c_int, p, p, p, p]
        L.oracle_i8_linear_rows_sampled.argtypes = [i64, p, p, p, p, p, ctypes.c_int, p, p, i64,
                                                    p, p, p]
        L.oracle_table_bytes.argtypes = [i64, i64]
        L.oracle_table_bytes.restype = i64
        L.oracle_table_pack.argtypes = [p, i64, i64, p]
        L.oracle_table_unpack.argtypes = [p, i64, i64, p]
        L.oracle_table_unpack.restype = i64
        L.oracle_i8_col_quant.argtypes = [p, i64, i64, i64, p, p]
        L.oracle_i8_dwconv.argtypes = [i64, i64, i64, i64, p, p, p, p, ctypes.c_int, p, p, p, p]
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_set_num_threads.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_num_threads(n: int) -> None:
    lib().oracle_set_num_threads(int(n))


def absmean(W: np.ndarray) -> np.float32:
    W = _c(W, np.float32)
    N, K = W.shape
    return np.float32(lib().oracle_absmean(_ptr(W), N, K))


def ternarize(W: np.ndarray):
    """-> (codes int8 [N,K] in {-1,0,1}, w_scale float32 = mean|W|)."""
    W = _c(W, np.float32)
    N, K = W.shape
    q = np.empty((N, K), np.int8)
    s = np.zeros(1, np.float32)
    lib().oracle_ternarize(_ptr(W), N, K, _ptr(q), _ptr(s))
    return q, np.float32(s[0])


def pack(q: np.ndarray) -> np.ndarray:
    q = _c(q, np.int8)
    N, K = q.shape
    assert K % 128 == 0
    out = np.empty(N * K // 4, np.uint8)
    lib().oracle_pack(_ptr(q), N, K, _ptr(out))
    return out


def unpack(packed: np.ndarray, N: int, K: int):
    """-> (codes int8 [N,K], number of invalid 2-bit fields)."""
    packed = _c(packed, np.uint8)
    assert packed.size == N * K // 4
    q = np.empty((N, K), np.int8)
    bad = lib().oracle_unpack(_ptr(packed), N, K, _ptr(q))
    return q, int(bad)


def code_at(packed: np.ndarray, N: int, n: int, k: int) -> int:
    packed = _c(packed, np.uint8)
    return int(lib().oracle_code_at(_ptr(packed), N, n, k))


def ternarize_pack(W: np.ndarray):
    """-> (packed uint8 [N*K/4], w_scale float32)."""
    W = _c(W, np.float32)
    N, K = W.shape
    out = np.empty(N * K // 4, np.uint8)
    s = np.zeros(1, np.float32)
    lib().oracle_ternarize_pack(_ptr(W), N, K, _ptr(out), _ptr(s))
    return out, np.float32(s[0])


def quant_act(x: np.ndarray):
    """-> (xq int8 [M,K], x_scale float32 [M])."""
    x = _c(x, np.float32)
    M, K = x.shape
    xq = np.empty((M, K), np.int8)
    xs = np.empty(M, np.float32)
    lib().oracle_quant_act(_ptr(x), M, K, _ptr(xq), _ptr(xs))
    return xq, xs


def matmul_i32(xq: np.ndarray, q: np.ndarray) -> np.ndarray:
    xq = _c(xq, np.int8)
    q = _c(q, np.int8)
    M, K = xq.shape
    N, K2 = q.shape
    assert K == K2
    acc = np.empty((M, N), np.int32)
    lib().oracle_matmul_i32(_ptr(xq), _ptr(q), M, N, K, _ptr(acc))
    return acc


def dequant(acc: np.ndarray, w_scale, x_scale: np.ndarray) -> np.ndarray:
    acc = _c(acc, np.int32)
    xs = _c(x_scale, np.float32)
    M, N = acc.shape
    y = np.empty((M, N), np.float32)
    lib().oracle_dequant(_ptr(acc), float(np.float32(w_scale)), _ptr(xs), M, N, _ptr(y))
    return y


def ternary_matmul(x: np.ndarray, packed: np.ndarray, w_scale, N: int):
    """Whole projection -> dict(y, xq, x_scale, acc)."""
    x = _c(x, np.float32)
    packed = _c(packed, np.uint8)
    M, K = x.shape
    y = np.empty((M, N), np.float32)
    xq = np.empty((M, K), np.int8)
    xs = np.empty(M, np.float32)
    acc = np.empty((M, N), np.int32)
    lib().oracle_ternary_matmul(M, N, K, _ptr(x), _ptr(packed), float(np.float32(w_scale)),
                                _ptr(y), _ptr(xq), _ptr(xs), _ptr(acc))
    return {"y": y, "xq": xq, "x_scale": xs, "acc": acc}


def matmul_sampled(xq: np.ndarray, x_scale: np.ndarray, packed: np.ndarray, w_scale,
                   N: int, ms: np.ndarray, ns: np.ndarray):
    """acc and y at the selected (m, n) pairs only."""
    xq = _c(xq, np.int8)
    xs = _c(x_scale, np.float32)
    packed = _c(packed, np.uint8)
    ms = _c(ms, np.int64)
    ns = _c(ns, np.int64)
    M, K = xq.shape
    cnt = ms.size
    acc = np.empty(cnt, np.int32)
    y = np.empty(cnt, np.float32)
    lib().oracle_matmul_sampled(N, K, _ptr(xq), _ptr(xs), _ptr(packed),
                                float(np.float32(w_scale)), _ptr(ms), _ptr(ns), cnt,
                                _ptr(acc), _ptr(y))
    return acc, y


# ---- I8_S: int8 weights x int8 activations --------------------------------

def i8_quant_weights(W: np.ndarray):
    """fp32 [N,K] -> (q int8 [N,K], w_scale float32): one absmax scale per tensor."""
    W = _c(W, np.float32)
    N, K = W.shape
    q = np.empty((N, K), np.int8)
    s = np.zeros(1, np.float32)
    lib().oracle_i8_quant_weights(_ptr(W), N, K, _ptr(q), _ptr(s))
    return q, np.float32(s[0])


def i8_matmul(xq: np.ndarray, q: np.ndarray) -> np.ndarray:
    xq = _c(xq, np.int8)
    q = _c(q, np.int8)
    M, K = xq.shape
    N, K2 = q.shape
    assert K == K2
    acc = np.empty((M, N), np.int32)
    lib().oracle_i8_matmul(_ptr(xq), _ptr(q), M, N, K, _ptr(acc))
    return acc


def i8_linear(x: np.ndarray, q: np.ndarray, w_scale, bias=None, relu: bool = False):
    """Whole I8_S layer -> dict(y, xq, x_scale, acc)."""
    x = _c(x, np.float32)
    q = _c(q, np.int8)
    M, K = x.shape
    N = q.shape[0]
    b = None if bias is None else _c(bias, np.float32)
    y = np.empty((M, N), np.float32)
    xq = np.empty((M, K), np.int8)
    xs = np.empty(M, np.float32)
    acc = np.empty((M, N), np.int32)
    lib().oracle_i8_linear(M, N, K, _ptr(x), _ptr(q), float(np.float32(w_scale)),
                           None if b is None else _ptr(b), int(bool(relu)), _ptr(y), _ptr(xq),
                           _ptr(xs), _ptr(acc))
    return {"y": y, "xq": xq, "x_scale": xs, "acc": acc}


def i8_linear_sampled(xq, x_scale, q, w_scale, bias, relu, ms, ns):
    """acc, d = acc * w_scale / x_scale (fp64) and y at the selected (m, n) pairs."""
    xq = _c(xq, np.int8)
    xs = _c(x_scale, np.float32)
    q = _c(q, np.int8)
    N, K = q.shape
    ms = _c(ms, np.int64)
    ns = _c(ns, np.int64)
    b = None if bias is None else _c(bias, np.float32)
    acc = np.empty(ms.size, np.int32)
    d = np.empty(ms.size, np.float64)
    y = np.empty(ms.size, np.float32)
    lib().oracle_i8_linear_sampled(N, K, _ptr(xq), _ptr(xs), _ptr(q), float(np.float32(w_scale)),
                                   None if b is None else _ptr(b), int(bool(relu)), _ptr(ms),
                                   _ptr(ns), ms.size, _ptr(acc), _ptr(d), _ptr(y))
    return acc, d, y


# ---- 8-bit weights, one scale per row: embeddings and lm_head ---------------

def rowq_quant_weights(W: np.ndarray):
    """fp32 [N,K] -> (q int8 [N,K], w_scale float32 [N]): one absmax scale per row."""
    W = _c(W, np.float32)
    N, K = W.shape
    q = np.empty((N, K), np.int8)
    s = np.empty(N, np.float32)
    lib().oracle_rowq_quant_weights(_ptr(W), N, K, _ptr(q), _ptr(s))
    return q, s


def rowq_embed(ids: np.ndarray, q: np.ndarray, w_scale: np.ndarray) -> np.ndarray:
    """Embedding rows of the int8 table for the token ids -> fp32 [T, K]."""
    ids = _c(ids, np.int32)
    q = _c(q, np.int8)
    s = _c(w_scale, np.float32)
    N, K = q.shape
    out = np.empty((ids.size, K), np.float32)
    lib().oracle_rowq_embed(_ptr(ids), ids.size, _ptr(q), _ptr(s), N, K, _ptr(out))
    return out


def rowq_linear(x: np.ndarray, q: np.ndarray, w_scale: np.ndarray):
    """lm_head over the int8 table -> dict(y, xq, x_scale, acc)."""
    x = _c(x, np.float32)
    q = _c(q, np.int8)
    s = _c(w_scale, np.float32)
    M, K = x.shape
    N = q.shape[0]
    y = np.empty((M, N), np.float32)
    xq = np.empty((M, K), np.int8)
    xs = np.empty(M, np.float32)
    acc = np.empty((M, N), np.int32)
    lib().oracle_rowq_linear(M, N, K, _ptr(x), _ptr(q), _ptr(s), _ptr(y), _ptr(xq), _ptr(xs),
                             _ptr(acc))
    return {"y": y, "xq": xq, "x_scale": xs, "acc": acc}


def rowq_linear_sampled(xq, x_scale, q, w_scale, ms, ns):
    """acc and y of the lm_head at the selected (m, n) pairs only."""
    xq = _c(xq, np.int8)
    xs = _c(x_scale, np.float32)
    q = _c(q, np.int8)
    s = _c(w_scale, np.float32)
    ms = _c(ms, np.int64)
    ns = _c(ns, np.int64)
    K = q.shape[1]
    acc = np.empty(ms.size, np.int32)
    y = np.empty(ms.size, np.float32)
    lib().oracle_rowq_linear_sampled(K, _ptr(xq), _ptr(xs), _ptr(q), _ptr(s), _ptr(ms),
                                     _ptr(ns), ms.size, _ptr(acc), _ptr(y))
    return acc, y


# ---- I8_S with one weight scale per output channel ---------------------------

def i8_linear_rows(x: np.ndarray, q: np.ndarray, w_scale: np.ndarray, bias=None,
                   relu: bool = False):
    """I8_S layer with per-channel weight scales (q, w_scale from
    rowq_quant_weights) -> dict(y, xq, x_scale, acc)."""
    x = _c(x, np.float32)
    q = _c(q, np.int8)
    s = _c(w_scale, np.float32)
    M, K = x.shape
    N = q.shape[0]
    b = None if bias is None else _c(bias, np.float32)
    y = np.empty((M, N), np.float32)
    xq = np.empty((M, K), np.int8)
    xs = np.empty(M, np.float32)
    acc = np.empty((M, N), np.int32)
    lib().oracle_i8_linear_rows(M, N, K, _ptr(x), _ptr(q), _ptr(s),
                                None if b is None else _ptr(b), int(bool(relu)), _ptr(y),
                                _ptr(xq), _ptr(xs), _ptr(acc))
    return {"y": y, "xq": xq, "x_scale": xs, "acc": acc}


def i8_linear_rows_sampled(xq, x_scale, q, w_scale, bias, relu, ms, ns):
    """acc, d = acc * w_scale[n] / x_scale[m] (fp64) and y at the (m, n) pairs."""
    xq = _c(xq, np.int8)
    xs = _c(x_scale, np.float32)
    q = _c(q, np.int8)
    s = _c(w_scale, np.float32)
    K = q.shape[1]
    ms = _c(ms, np.int64)
    ns = _c(ns, np.int64)
    b = None if bias is None else _c(bias, np.float32)
    acc = np.empty(ms.size, np.int32)
    d = np.empty(ms.size, np.float64)
    y = np.empty(ms.size, np.float32)
    lib().oracle_i8_linear_rows_sampled(K, _ptr(xq), _ptr(xs), _ptr(q), _ptr(s),
                                        None if b is None else _ptr(b), int(bool(relu)),
                                        _ptr(ms), _ptr(ns), ms.size, _ptr(acc), _ptr(d), _ptr(y))
    return acc, d, y


# ---- storage layout of the 8-bit table ----------------------------------------

def table_bytes(V: int, K: int) -> int:
    return int(lib().oracle_table_bytes(V, K))


def table_pack(q: np.ndarray) -> np.ndarray:
    """int8 codes [V,K] (row-major) -> the table's tiled bytes (int8, padded)."""
    q = _c(q, np.int8)
    V, K = q.shape
    out = np.empty(table_bytes(V, K), np.int8)
    lib().oracle_table_pack(_ptr(q), V, K, _ptr(out))
    return out


def table_unpack(table: np.ndarray, V: int, K: int):
    """Tiled table bytes -> (codes int8 [V,K], number of nonzero padding bytes)."""
    table = _c(table, np.int8)
    assert table.size == table_bytes(V, K)
    q = np.empty((V, K), np.int8)
    bad = lib().oracle_table_unpack(_ptr(table), V, K, _ptr(q))
    return q, int(bad)


# ---- I8_S depthwise convolution over time --------------------------------------

def i8_col_quant(x: np.ndarray):
    """fp32 x [B,T,C] -> (xq int8 [B,T,C], x_scale float32 [B,C]): one absmax
    scale per (sequence, channel)."""
    x = _c(x, np.float32)
    B, T, C = x.shape
    xq = np.empty((B, T, C), np.int8)
    xs = np.empty((B, C), np.float32)
    lib().oracle_i8_col_quant(_ptr(x), B, T, C, _ptr(xq), _ptr(xs))
    return xq, xs


def i8_dwconv(x: np.ndarray, q: np.ndarray, w_scale: np.ndarray, bias=None, relu=False):
    """Causal depthwise convolution over frames: x [B,T,C], int8 kernel q [C,k]
    with per-channel scales -> dict(y [B,T,C], xq, x_scale [B,C], acc)."""
    x = _c(x, np.float32)
    q = _c(q, np.int8)
    s = _c(w_scale, np.float32)
    B, T, C = x.shape
    k = q.shape[1]
    b = None if bias is None else _c(bias, np.float32)
    y = np.empty((B, T, C), np.float32)
    xq = np.empty((B, T, C), np.int8)
    xs = np.empty((B, C), np.float32)
    acc = np.empty((B, T, C), np.int32)
    lib().oracle_i8_dwconv(B, T, C, k, _ptr(x), _ptr(q), _ptr(s),
                           None if b is None else _ptr(b), int(bool(relu)), _ptr(y), _ptr(xq),
                           _ptr(xs), _ptr(acc))
    return {"y": y, "xq": xq, "x_scale": xs, "acc": acc}
