"""Thin Python binding over the C ABI in include/bitnet_tm.h.

Argument marshalling only: every step of the projection runs in the gfx950 HIP
kernels of ``libbitnet_tm.so``.  torch supplies device memory and the current
stream; no torch type crosses the ABI.  If the library is missing or the device
is not a gfx950, calls raise -- there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import _build

LIB_PATH = _build.LIB_PATH

BITNET_OK = 0
BITNET_MAX_GROUP = 256
UNIT = 128

_c = ctypes
_p = _c.c_void_p
_i64 = _c.c_int64
_i32 = _c.c_int32
_sz = _c.c_size_t


class BitnetError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__(f"{fn}: status {status} ({status_string(status)})")


class bitnet_problem(ctypes.Structure):
    _fields_ = [("x", _p), ("packed", _p), ("w_scale", _p), ("y", _p),
                ("N", _i64), ("K", _i64)]


EXPORTS = (
    "bitnet_status_string", "bitnet_packed_bytes", "bitnet_ternarize_workspace_bytes",
    "bitnet_ternarize_pack", "bitnet_quant_act", "bitnet_matmul_workspace_bytes",
    "bitnet_ternary_matmul", "bitnet_ternary_matmul_q8", "bitnet_grouped_workspace_bytes",
    "bitnet_ternary_matmul_grouped", "bitnet_stages_workspace_bytes",
    "bitnet_ternary_matmul_stages", "bitnet_ternary_matmul_lut_grouped",
    "bitnet_i8_quant_workspace_bytes", "bitnet_i8_quant_weights",
    "bitnet_i8_linear_workspace_bytes", "bitnet_i8_linear",
)

_lib = None


def lib():
    """Load libbitnet_tm.so (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"HIP library {LIB_PATH} is not built; run __graft_entry__.build() "
                "(python -m ternary_weight_decoder_amd._build)")
        L = ctypes.CDLL(LIB_PATH)
        L.bitnet_status_string.argtypes = [_i32]
        L.bitnet_status_string.restype = _c.c_char_p
        L.bitnet_packed_bytes.argtypes = [_i64, _i64]
        L.bitnet_packed_bytes.restype = _sz
        L.bitnet_ternarize_workspace_bytes.argtypes = [_i64]
        L.bitnet_ternarize_workspace_bytes.restype = _sz
        L.bitnet_ternarize_pack.argtypes = [_p, _i64, _i64, _p, _p, _p, _sz, _p]
        L.bitnet_ternarize_pack.restype = _i32
        L.bitnet_quant_act.argtypes = [_p, _i64, _i64, _p, _p, _p]
        L.bitnet_quant_act.restype = _i32
        L.bitnet_matmul_workspace_bytes.argtypes = [_i64, _i64]
        L.bitnet_matmul_workspace_bytes.restype = _sz
        L.bitnet_ternary_matmul.argtypes = [_i64, _i64, _i64, _p, _p, _p, _p, _p, _sz, _p, _p,
                                            _p, _p]
        L.bitnet_ternary_matmul.restype = _i32
        L.bitnet_ternary_matmul_q8.argtypes = [_i64, _i64, _i64, _p, _p, _p, _p, _p, _p, _sz,
                                               _p, _p]
        L.bitnet_ternary_matmul_q8.restype = _i32
        L.bitnet_grouped_workspace_bytes.argtypes = [_i64, _p, _i32]
        L.bitnet_grouped_workspace_bytes.restype = _sz
        L.bitnet_ternary_matmul_grouped.argtypes = [_i64, _p, _i32, _p, _p, _sz, _p]
        L.bitnet_ternary_matmul_grouped.restype = _i32
        L.bitnet_stages_workspace_bytes.argtypes = [_i64, _p, _i32]
        L.bitnet_stages_workspace_bytes.restype = _sz
        L.bitnet_ternary_matmul_stages.argtypes = [_i64, _p, _i32, _p, _i32, _p, _p, _sz, _p]
        L.bitnet_ternary_matmul_stages.restype = _i32
        L.bitnet_ternary_matmul_lut_grouped.argtypes = [_p, _i32, _p, _p]
        L.bitnet_ternary_matmul_lut_grouped.restype = _i32
        L.bitnet_i8_quant_workspace_bytes.argtypes = []
        L.bitnet_i8_quant_workspace_bytes.restype = _sz
        L.bitnet_i8_quant_weights.argtypes = [_p, _i64, _i64, _p, _p, _p, _sz, _p]
        L.bitnet_i8_quant_weights.restype = _i32
        L.bitnet_i8_linear_workspace_bytes.argtypes = [_i64, _i64]
        L.bitnet_i8_linear_workspace_bytes.restype = _sz
        L.bitnet_i8_linear.argtypes = [_i64, _i64, _i64, _p, _p, _p, _p, _i32, _p, _p, _sz, _p,
                                       _p]
        L.bitnet_i8_linear.restype = _i32
        L.bitnet_scratch_bytes.argtypes = []
        L.bitnet_scratch_bytes.restype = _sz
        L.bitnet_ternary_matmul_noalloc.argtypes = [_i64, _i64, _i64, _p, _p, _p, _p, _p, _p,
                                                    _p, _p]
        L.bitnet_ternary_matmul_noalloc.restype = _i32
        L.bitnet_i8_linear_rows.argtypes = [_i64, _i64, _i64, _p, _p, _p, _p, _i32, _p, _p, _sz,
                                            _p, _p]
        L.bitnet_i8_linear_rows.restype = _i32
        L.bitnet_ternary_matmul_grouped_overlap.argtypes = [_i64, _p, _i32, _p, _i32, _p, _sz, _p,
                                                            _p]
        L.bitnet_ternary_matmul_grouped_overlap.restype = _i32
        L.bitnet_i8_dwconv_quant_weights.argtypes = [_p, _i64, _i64, _p, _p, _p]
        L.bitnet_i8_dwconv_quant_weights.restype = _i32
        L.bitnet_i8_dwconv_workspace_bytes.argtypes = [_i64, _i64, _i64]
        L.bitnet_i8_dwconv_workspace_bytes.restype = _sz
        L.bitnet_i8_dwconv.argtypes = [_i64, _i64, _i64, _i64, _p, _p, _p, _p, _i32, _p, _p, _sz,
                                       _p, _p, _p]
        L.bitnet_i8_dwconv.restype = _i32
        L.bitnet_table_bytes.argtypes = [_i64, _i64]
        L.bitnet_table_bytes.restype = _sz
        L.bitnet_table_quant.argtypes = [_p, _i64, _i64, _p, _p, _p]
        L.bitnet_table_quant.restype = _i32
        L.bitnet_i8_quant_weights_rows.argtypes = [_p, _i64, _i64, _p, _p, _p]
        L.bitnet_i8_quant_weights_rows.restype = _i32
        L.bitnet_embed_lookup.argtypes = [_p, _i64, _p, _p, _i64, _i64, _p, _p]
        L.bitnet_embed_lookup.restype = _i32
        L.bitnet_lm_head.argtypes = [_i64, _i64, _i64, _p, _p, _p, _p, _p, _p, _p, _p]
        L.bitnet_lm_head.restype = _i32
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().bitnet_status_string(int(status)).decode()


def _check(status: int, fn: str) -> None:
    if status != BITNET_OK:
        raise BitnetError(status, fn)


def _ptr(t):
    return None if t is None else _p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return _p(s.cuda_stream)


def _dev(t: torch.Tensor, dtype, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# ---------------------------------------------------------------------------
# Raw entry points: same names and arguments as the C ABI (tensors stand in for
# device pointers).  They allocate nothing.
# ---------------------------------------------------------------------------

def bitnet_packed_bytes(N: int, K: int) -> int:
    return int(lib().bitnet_packed_bytes(N, K))


def bitnet_ternarize_workspace_bytes(N: int) -> int:
    return int(lib().bitnet_ternarize_workspace_bytes(N))


def bitnet_matmul_workspace_bytes(M: int, K: int) -> int:
    return int(lib().bitnet_matmul_workspace_bytes(M, K))


def bitnet_ternarize_pack_into(W, N, K, packed, w_scale, workspace, stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().bitnet_ternarize_pack(_ptr(W), N, K, _ptr(packed), _ptr(w_scale),
                                       _ptr(workspace), ws_bytes, _stream(stream)),
           "bitnet_ternarize_pack")


def bitnet_quant_act_into(x, M, K, xq, x_scale, stream=None) -> None:
    _check(lib().bitnet_quant_act(_ptr(x), M, K, _ptr(xq), _ptr(x_scale), _stream(stream)),
           "bitnet_quant_act")


def bitnet_ternary_matmul_into(M, N, K, x, packed, w_scale, y, workspace, xq_out=None,
                               x_scale_out=None, acc_out=None, stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().bitnet_ternary_matmul(M, N, K, _ptr(x), _ptr(packed), _ptr(w_scale), _ptr(y),
                                       _ptr(workspace), ws_bytes, _ptr(xq_out),
                                       _ptr(x_scale_out), _ptr(acc_out), _stream(stream)),
           "bitnet_ternary_matmul")


def bitnet_ternary_matmul_q8_into(M, N, K, xq, x_scale, packed, w_scale, y, workspace,
                                  acc_out=None, stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().bitnet_ternary_matmul_q8(M, N, K, _ptr(xq), _ptr(x_scale), _ptr(packed),
                                          _ptr(w_scale), _ptr(y), _ptr(workspace), ws_bytes,
                                          _ptr(acc_out), _stream(stream)),
           "bitnet_ternary_matmul_q8")


# ---------------------------------------------------------------------------
# Convenience forms that allocate their outputs with torch (plumbing only).
# ---------------------------------------------------------------------------

def bitnet_scratch_bytes() -> int:
    return int(lib().bitnet_scratch_bytes())


def bitnet_ternary_matmul_noalloc_into(M, N, K, x, packed, w_scale, y, xq_out=None,
                                       x_scale_out=None, acc_out=None, stream=None) -> None:
    """The projection with the library's built-in scratch instead of a workspace."""
    _check(lib().bitnet_ternary_matmul_noalloc(M, N, K, _ptr(x), _ptr(packed), _ptr(w_scale),
                                               _ptr(y), _ptr(xq_out), _ptr(x_scale_out),
                                               _ptr(acc_out), _stream(stream)),
           "bitnet_ternary_matmul_noalloc")


def bitnet_ternarize_pack(W: torch.Tensor, stream=None):
    """fp32 W [N,K] -> (packed uint8 [N*K/4], w_scale fp32 [1]) on W's device."""
    _dev(W, torch.float32, "W")
    N, K = W.shape
    packed = torch.empty(max(N * K // 4, 1), dtype=torch.uint8, device=W.device)
    w_scale = torch.empty(1, dtype=torch.float32, device=W.device)
    ws = torch.empty(max(bitnet_ternarize_workspace_bytes(N), 16), dtype=torch.uint8,
                     device=W.device)
    bitnet_ternarize_pack_into(W, N, K, packed, w_scale, ws, stream)
    return packed, w_scale


def bitnet_quant_act(x: torch.Tensor, stream=None):
    """fp32 x [M,K] -> (xq int8 [M,K], x_scale fp32 [M])."""
    _dev(x, torch.float32, "x")
    M, K = x.shape
    xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    xs = torch.empty(M, dtype=torch.float32, device=x.device)
    bitnet_quant_act_into(x, M, K, xq, xs, stream)
    return xq, xs


def bitnet_ternary_matmul(x: torch.Tensor, packed: torch.Tensor, w_scale: torch.Tensor,
                          N: int, *, return_parts: bool = False, stream=None):
    """y [M,N] fp32; with return_parts also xq, x_scale and the int32 accumulators."""
    _dev(x, torch.float32, "x")
    _dev(packed, torch.uint8, "packed")
    _dev(w_scale, torch.float32, "w_scale")
    M, K = x.shape
    y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    ws = torch.empty(bitnet_matmul_workspace_bytes(M, K), dtype=torch.uint8, device=x.device)
    if return_parts:
        xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
        xs = torch.empty(M, dtype=torch.float32, device=x.device)
        acc = torch.empty((M, N), dtype=torch.int32, device=x.device)
        bitnet_ternary_matmul_into(M, N, K, x, packed, w_scale, y, ws, xq, xs, acc, stream)
        return {"y": y, "xq": xq, "x_scale": xs, "acc": acc}
    bitnet_ternary_matmul_into(M, N, K, x, packed, w_scale, y, ws, stream=stream)
    return y


def bitnet_ternary_matmul_q8(xq: torch.Tensor, x_scale: torch.Tensor, packed: torch.Tensor,
                             w_scale: torch.Tensor, N: int, *, return_acc: bool = False,
                             stream=None):
    _dev(xq, torch.int8, "xq")
    M, K = xq.shape
    y = torch.empty((M, N), dtype=torch.float32, device=xq.device)
    ws = torch.empty(bitnet_matmul_workspace_bytes(M, K), dtype=torch.uint8, device=xq.device)
    acc = torch.empty((M, N), dtype=torch.int32, device=xq.device) if return_acc else None
    bitnet_ternary_matmul_q8_into(M, N, K, xq, x_scale, packed, w_scale, y, ws, acc, stream)
    return (y, acc) if return_acc else y


class GroupedPlan:
    """A fixed set of independent projections with the same M, launched together.

    Holds the host and device copies of the problem array and the workspace, so
    that run() is a single C call with no allocation.
    """

    def __init__(self, M: int, xs, packeds, w_scales, ys, Ns, Ks, device=None):
        count = len(xs)
        if not 1 <= count <= BITNET_MAX_GROUP:
            raise ValueError(f"group size must be 1..{BITNET_MAX_GROUP}")
        self.M = int(M)
        self.count = count
        arr = (bitnet_problem * count)()
        for i in range(count):
            arr[i] = bitnet_problem(xs[i].data_ptr(), packeds[i].data_ptr(),
                                    w_scales[i].data_ptr(), ys[i].data_ptr(), int(Ns[i]),
                                    int(Ks[i]))
        self._keep = (list(xs), list(packeds), list(w_scales), list(ys))
        self.host = arr
        dev = device if device is not None else xs[0].device
        raw = torch.frombuffer(bytearray(bytes(arr)), dtype=torch.uint8)
        self.dev = raw.to(dev)
        nbytes = int(lib().bitnet_grouped_workspace_bytes(self.M, _c.byref(arr), count))
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
        self.ws_bytes = nbytes

    def run(self, stream=None) -> None:
        bitnet_ternary_matmul_grouped(self.M, self.dev, self.count, self.host, self.workspace,
                                      stream)

    def run_overlap(self, aux_stream, nchunks: int, stream=None) -> None:
        """The same call with the quantization of later chunks on aux_stream,
        overlapping the contraction of earlier ones (prefill, M > 16)."""
        bitnet_ternary_matmul_grouped_overlap(self.M, self.dev, self.count, self.host, nchunks,
                                              self.workspace, stream, aux_stream)


def bitnet_ternary_matmul_grouped_overlap(M, problems_dev, count, problems_host, nchunks,
                                          workspace, stream=None, aux_stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().bitnet_ternary_matmul_grouped_overlap(M, _ptr(problems_dev), count,
                                                       _c.byref(problems_host), int(nchunks),
                                                       _ptr(workspace), ws_bytes,
                                                       _stream(stream), _stream(aux_stream)),
           "bitnet_ternary_matmul_grouped_overlap")


def bitnet_grouped_workspace_bytes(M: int, problems_host, count: int) -> int:
    return int(lib().bitnet_grouped_workspace_bytes(M, _c.byref(problems_host), count))


def bitnet_ternary_matmul_grouped(M, problems_dev, count, problems_host, workspace,
                                  stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().bitnet_ternary_matmul_grouped(M, _ptr(problems_dev), count,
                                               _c.byref(problems_host), _ptr(workspace),
                                               ws_bytes, _stream(stream)),
           "bitnet_ternary_matmul_grouped")


def bitnet_i8_quant_weights_into(W, N, K, q, w_scale, workspace, stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().bitnet_i8_quant_weights(_ptr(W), N, K, _ptr(q), _ptr(w_scale), _ptr(workspace),
                                         ws_bytes, _stream(stream)),
           "bitnet_i8_quant_weights")


def bitnet_i8_quant_weights(W: torch.Tensor, stream=None):
    """fp32 W [N,K] -> (q int8 [N,K], w_scale fp32 [1]) on W's device (I8_S)."""
    _dev(W, torch.float32, "W")
    N, K = W.shape
    q = torch.empty((N, K), dtype=torch.int8, device=W.device)
    w_scale = torch.empty(1, dtype=torch.float32, device=W.device)
    ws = torch.empty(int(lib().bitnet_i8_quant_workspace_bytes()), dtype=torch.uint8,
                     device=W.device)
    bitnet_i8_quant_weights_into(W, N, K, q, w_scale, ws, stream)
    return q, w_scale


def bitnet_i8_linear_workspace_bytes(M: int, K: int) -> int:
    return int(lib().bitnet_i8_linear_workspace_bytes(M, K))


def bitnet_i8_linear_into(M, N, K, x, q, w_scale, bias, relu, y, workspace, acc_out=None,
                          stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().bitnet_i8_linear(M, N, K, _ptr(x), _ptr(q), _ptr(w_scale), _ptr(bias),
                                  int(bool(relu)), _ptr(y), _ptr(workspace), ws_bytes,
                                  _ptr(acc_out), _stream(stream)),
           "bitnet_i8_linear")


def bitnet_i8_linear(x: torch.Tensor, q: torch.Tensor, w_scale: torch.Tensor, bias=None,
                     relu: bool = False, return_acc: bool = False, stream=None):
    """I8_S layer: fp32 x [M,K], int8 q [N,K] -> fp32 y [M,N] (and int32 acc)."""
    _dev(x, torch.float32, "x")
    _dev(q, torch.int8, "q")
    M, K = x.shape
    N = q.shape[0]
    y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    ws = torch.empty(bitnet_i8_linear_workspace_bytes(M, K), dtype=torch.uint8, device=x.device)
    acc = torch.empty((M, N), dtype=torch.int32, device=x.device) if return_acc else None
    bitnet_i8_linear_into(M, N, K, x, q, w_scale, bias, relu, y, ws, acc, stream)
    return (y, acc) if return_acc else y


# ---- the 8-bit table with one scale per row: embeddings and lm_head ---------

def bitnet_i8_quant_weights_rows_into(W, N, K, q, w_scale, stream=None) -> None:
    _check(lib().bitnet_i8_quant_weights_rows(_ptr(W), N, K, _ptr(q), _ptr(w_scale),
                                              _stream(stream)),
           "bitnet_i8_quant_weights_rows")


def bitnet_i8_quant_weights_rows(W: torch.Tensor, stream=None):
    """fp32 W [N,K] -> (q int8 [N,K], w_scale fp32 [N]): one absmax scale per row."""
    _dev(W, torch.float32, "W")
    N, K = W.shape
    q = torch.empty((N, K), dtype=torch.int8, device=W.device)
    w_scale = torch.empty(N, dtype=torch.float32, device=W.device)
    bitnet_i8_quant_weights_rows_into(W, N, K, q, w_scale, stream)
    return q, w_scale


def bitnet_table_bytes(V: int, K: int) -> int:
    return int(lib().bitnet_table_bytes(V, K))


def bitnet_table_quant_into(W, V, K, table, w_scale, stream=None) -> None:
    _check(lib().bitnet_table_quant(_ptr(W), V, K, _ptr(table), _ptr(w_scale), _stream(stream)),
           "bitnet_table_quant")


def bitnet_table_quant(W: torch.Tensor, stream=None):
    """fp32 W [V,K] -> (table int8 [bitnet_table_bytes(V, K)] in the library's
    storage order, w_scale fp32 [V])."""
    _dev(W, torch.float32, "W")
    V, K = W.shape
    table = torch.empty(bitnet_table_bytes(V, K), dtype=torch.int8, device=W.device)
    w_scale = torch.empty(V, dtype=torch.float32, device=W.device)
    bitnet_table_quant_into(W, V, K, table, w_scale, stream)
    return table, w_scale


def bitnet_embed_lookup_into(ids, T, table, w_scale, V, K, out, stream=None) -> None:
    _check(lib().bitnet_embed_lookup(_ptr(ids), T, _ptr(table), _ptr(w_scale), V, K, _ptr(out),
                                     _stream(stream)),
           "bitnet_embed_lookup")


def bitnet_embed_lookup(ids: torch.Tensor, table: torch.Tensor, w_scale: torch.Tensor, K: int,
                        stream=None):
    """int32 token ids [T] -> fp32 embedding rows [T, K] of the table (V = w_scale.numel())."""
    _dev(ids, torch.int32, "ids")
    _dev(table, torch.int8, "table")
    V = w_scale.numel()
    T = ids.numel()
    out = torch.empty((T, K), dtype=torch.float32, device=table.device)
    bitnet_embed_lookup_into(ids, T, table, w_scale, V, K, out, stream)
    return out


def bitnet_lm_head_into(M, V, K, x, table, w_scale, y, xq_out=None, x_scale_out=None,
                        acc_out=None, stream=None) -> None:
    _check(lib().bitnet_lm_head(M, V, K, _ptr(x), _ptr(table), _ptr(w_scale), _ptr(y),
                                _ptr(xq_out), _ptr(x_scale_out), _ptr(acc_out), _stream(stream)),
           "bitnet_lm_head")


def bitnet_lm_head(x: torch.Tensor, table: torch.Tensor, w_scale: torch.Tensor,
                   return_parts: bool = False, stream=None):
    """lm_head over the table: fp32 x [M,K] (M <= 16) -> fp32 logits [M, V]
    (V = w_scale.numel()); with return_parts, a dict that also holds xq,
    x_scale and the int32 acc."""
    _dev(x, torch.float32, "x")
    _dev(table, torch.int8, "table")
    M, K = x.shape
    V = w_scale.numel()
    y = torch.empty((M, V), dtype=torch.float32, device=x.device)
    if not return_parts:
        bitnet_lm_head_into(M, V, K, x, table, w_scale, y, stream=stream)
        return y
    xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    xs = torch.empty(M, dtype=torch.float32, device=x.device)
    acc = torch.empty((M, V), dtype=torch.int32, device=x.device)
    bitnet_lm_head_into(M, V, K, x, table, w_scale, y, xq, xs, acc, stream)
    return {"y": y, "xq": xq, "x_scale": xs, "acc": acc}


def bitnet_i8_linear_rows_into(M, N, K, x, q, w_scale, bias, relu, y, workspace, acc_out=None,
                               stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().bitnet_i8_linear_rows(M, N, K, _ptr(x), _ptr(q), _ptr(w_scale), _ptr(bias),
                                       int(bool(relu)), _ptr(y), _ptr(workspace), ws_bytes,
                                       _ptr(acc_out), _stream(stream)),
           "bitnet_i8_linear_rows")


def bitnet_i8_linear_rows(x: torch.Tensor, q: torch.Tensor, w_scale: torch.Tensor, bias=None,
                          relu: bool = False, return_acc: bool = False, stream=None):
    """I8_S layer with per-channel weight scales: fp32 x [M,K], int8 q [N,K],
    fp32 w_scale [N] -> fp32 y [M,N] (and int32 acc)."""
    _dev(x, torch.float32, "x")
    _dev(q, torch.int8, "q")
    M, K = x.shape
    N = q.shape[0]
    y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    ws = torch.empty(bitnet_i8_linear_workspace_bytes(M, K), dtype=torch.uint8, device=x.device)
    acc = torch.empty((M, N), dtype=torch.int32, device=x.device) if return_acc else None
    bitnet_i8_linear_rows_into(M, N, K, x, q, w_scale, bias, relu, y, ws, acc, stream)
    return (y, acc) if return_acc else y


# ---- I8_S causal depthwise convolution ---------------------------------------

def bitnet_i8_dwconv_quant_weights(W: torch.Tensor, stream=None):
    """fp32 kernel W [C,k] -> (q int8 [C,k], w_scale fp32 [C]), per channel."""
    _dev(W, torch.float32, "W")
    C, k = W.shape
    q = torch.empty((C, k), dtype=torch.int8, device=W.device)
    s = torch.empty(C, dtype=torch.float32, device=W.device)
    _check(lib().bitnet_i8_dwconv_quant_weights(_ptr(W), C, k, _ptr(q), _ptr(s), _stream(stream)),
           "bitnet_i8_dwconv_quant_weights")
    return q, s


def bitnet_i8_dwconv_workspace_bytes(B: int, T: int, C: int) -> int:
    return int(lib().bitnet_i8_dwconv_workspace_bytes(B, T, C))


def bitnet_i8_dwconv_into(B, T, C, k, x, q, w_scale, bias, relu, y, workspace, acc_out=None,
                          x_scale_out=None, stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().bitnet_i8_dwconv(B, T, C, k, _ptr(x), _ptr(q), _ptr(w_scale), _ptr(bias),
                                  int(bool(relu)), _ptr(y), _ptr(workspace), ws_bytes,
                                  _ptr(acc_out), _ptr(x_scale_out), _stream(stream)),
           "bitnet_i8_dwconv")


def bitnet_i8_dwconv(x: torch.Tensor, q: torch.Tensor, w_scale: torch.Tensor, bias=None,
                     relu: bool = False, return_parts: bool = False, stream=None):
    """Causal depthwise convolution over frames: fp32 x [B,T,C], int8 q [C,k] ->
    fp32 y [B,T,C] (with return_parts, a dict that also holds acc and x_scale)."""
    _dev(x, torch.float32, "x")
    _dev(q, torch.int8, "q")
    B, T, C = x.shape
    k = q.shape[1]
    y = torch.empty((B, T, C), dtype=torch.float32, device=x.device)
    ws = torch.empty(bitnet_i8_dwconv_workspace_bytes(B, T, C), dtype=torch.uint8,
                     device=x.device)
    if not return_parts:
        bitnet_i8_dwconv_into(B, T, C, k, x, q, w_scale, bias, relu, y, ws, stream=stream)
        return y
    acc = torch.empty((B, T, C), dtype=torch.int32, device=x.device)
    xs = torch.empty((B, C), dtype=torch.float32, device=x.device)
    bitnet_i8_dwconv_into(B, T, C, k, x, q, w_scale, bias, relu, y, ws, acc, xs, stream)
    return {"y": y, "acc": acc, "x_scale": xs}


def bitnet_ternary_matmul_lut_grouped(problems_dev, count, problems_host, stream=None) -> None:
    _check(lib().bitnet_ternary_matmul_lut_grouped(_ptr(problems_dev), count,
                                                   _c.byref(problems_host), _stream(stream)),
           "bitnet_ternary_matmul_lut_grouped")


class LutPlan:
    """Independent single-row projections run by the lookup-table kernel in one
    launch (the comparison variant of the grouped decode call at M = 1)."""

    def __init__(self, xs, packeds, w_scales, ys, Ns, Ks, device=None):
        count = len(xs)
        if not 1 <= count <= BITNET_MAX_GROUP:
            raise ValueError(f"group size must be 1..{BITNET_MAX_GROUP}")
        arr = (bitnet_problem * count)()
        for i in range(count):
            arr[i] = bitnet_problem(xs[i].data_ptr(), packeds[i].data_ptr(),
                                    w_scales[i].data_ptr(), ys[i].data_ptr(), int(Ns[i]),
                                    int(Ks[i]))
        self._keep = (list(xs), list(packeds), list(w_scales), list(ys))
        self.host, self.count = arr, count
        dev = device if device is not None else xs[0].device
        self.dev = torch.frombuffer(bytearray(bytes(arr)), dtype=torch.uint8).to(dev)

    def run(self, stream=None) -> None:
        bitnet_ternary_matmul_lut_grouped(self.dev, self.count, self.host, stream)


def bitnet_stages_workspace_bytes(M: int, problems_host, count: int) -> int:
    return int(lib().bitnet_stages_workspace_bytes(M, _c.byref(problems_host), count))


def bitnet_ternary_matmul_stages(M, problems_dev, count, stage_end_host, nstages, problems_host,
                                 workspace, stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().bitnet_ternary_matmul_stages(M, _ptr(problems_dev), count,
                                              _c.byref(stage_end_host), nstages,
                                              _c.byref(problems_host), _ptr(workspace), ws_bytes,
                                              _stream(stream)),
           "bitnet_ternary_matmul_stages")


class StagedPlan:
    """A fixed sequence of dependent stages of decode projections (for example
    one token through a decoder: q,k,v | o | gate,up | down per layer), run by
    one call.  stages: list of lists of (x, packed, w_scale, y, N, K) tuples; a
    problem whose x is the y tensor of a problem of an earlier stage reads that
    output.  The workspace is zero-filled here, once."""

    def __init__(self, M: int, stages, device=None):
        flat = [pr for st in stages for pr in st]
        count = len(flat)
        if not 1 <= count <= BITNET_MAX_GROUP:
            raise ValueError(f"at most {BITNET_MAX_GROUP} problems")
        self.M, self.count, self.nstages = int(M), count, len(stages)
        arr = (bitnet_problem * count)()
        for i, (x, pk, ws, y, N, K) in enumerate(flat):
            arr[i] = bitnet_problem(x.data_ptr(), pk.data_ptr(), ws.data_ptr(), y.data_ptr(),
                                    int(N), int(K))
        ends = (_i32 * self.nstages)()
        e = 0
        for s, st in enumerate(stages):
            e += len(st)
            ends[s] = e
        self._keep = flat
        self.host, self.ends = arr, ends
        dev = device if device is not None else flat[0][0].device
        self.dev = torch.frombuffer(bytearray(bytes(arr)), dtype=torch.uint8).to(dev)
        nbytes = bitnet_stages_workspace_bytes(self.M, arr, count)
        if nbytes == 0:
            raise ValueError("invalid staged problem list")
        self.workspace = torch.zeros(nbytes, dtype=torch.uint8, device=dev)

    def run(self, stream=None) -> None:
        bitnet_ternary_matmul_stages(self.M, self.dev, self.count, self.ends, self.nstages,
                                     self.host, self.workspace, stream)

    def timed_out(self) -> bool:
        """After the call has completed: did a wait between stages run out?"""
        return int(self.workspace[4:8].view(torch.int32).item()) != 0

    def timeouts_total(self) -> int:
        """Calls with a wait that ran out, since the workspace was zero-filled."""
        return int(self.workspace[8:12].view(torch.int32).item())
