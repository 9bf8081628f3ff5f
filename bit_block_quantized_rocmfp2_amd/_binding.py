"""ctypes binding of libqmoe (include/qmoe.h): argument marshalling only.

Every compute step runs in the HIP library; this module only converts numpy
arrays and torch tensors to pointers and sizes, and turns status codes into
exceptions. Importing it raises if the built library is missing: there is no
CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_double, c_int, c_int32, c_int64, c_size_t, c_uint16, c_void_p

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqmoe.so")
LIB_DEBUG_PATH = os.path.join(_HERE, "libqmoe_debug.so")   # launcher bounds checks compiled in

QMOE_OK = 0
FP2, FP3, FP4 = 2, 3, 4


class QmoeError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({strerror(status)}): {detail}")


class qmoe_layer(ctypes.Structure):
    _fields_ = [
        ("hidden", c_int32), ("inter", c_int32), ("n_experts", c_int32), ("topk", c_int32),
        ("fmt_gate", c_int32), ("fmt_up", c_int32), ("fmt_down", c_int32),
        ("rot_gateup", c_int32), ("rot_down", c_int32),
        ("w_router", c_void_p), ("w_router_bytes", c_size_t),
        ("router_bias", c_void_p),
        ("gate", c_void_p), ("gate_bytes", c_size_t),
        ("up", c_void_p), ("up_bytes", c_size_t),
        ("down", c_void_p), ("down_bytes", c_size_t),
        ("cb_gate", c_void_p), ("cb_gate_bytes", c_size_t),
        ("cb_up", c_void_p), ("cb_up_bytes", c_size_t),
        ("cb_down", c_void_p), ("cb_down_bytes", c_size_t),
    ]


class qmoe_matvec_item(ctypes.Structure):
    _fields_ = [
        ("fmt", c_int32), ("rot", c_int32), ("rows", c_int64), ("k", c_int64),
        ("w", c_void_p), ("w_bytes", c_size_t), ("cb", c_void_p), ("x", c_void_p), ("y", c_void_p),
    ]


class qmoe_ws_layout(ctypes.Structure):
    _fields_ = [(n, c_size_t) for n in
                ("xq", "dx", "idx", "gw", "logits", "plan", "hq", "dh", "group", "ypair", "total")]


def load_library(path=None):
    """The library at `path` (default libqmoe.so) with every entry point's
    signature set: the bounds-checked build (LIB_DEBUG_PATH) loads the same way."""
    # When torch is present it must load its HIP runtime first: libqmoe then binds
    # to that already-loaded libamdhip64.so.7 instead of a second runtime copy,
    # so device pointers and streams from torch are valid in the library.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise ImportError(f"libqmoe is not built ({path} missing); run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    sig = {
        "qmoe_strerror": (c_char_p, [c_int]),
        "qmoe_last_error": (c_char_p, []),
        "qmoe_version": (c_int, []),
        "qmoe_block_bytes": (c_size_t, [c_int]),
        "qmoe_packed_bytes": (c_size_t, [c_int, c_int64, c_int64]),
        "qmoe_pack": (c_int, [c_int, c_int64, c_int64, c_void_p, c_void_p, c_void_p, c_size_t]),
        "qmoe_unpack": (c_int, [c_int, c_int64, c_int64, c_void_p, c_size_t, c_void_p, c_void_p]),
        "qmoe_layer_check": (c_int, [POINTER(qmoe_layer)]),
        "qmoe_workspace_bytes": (c_size_t, [POINTER(qmoe_layer), c_int32]),
        "qmoe_workspace_layout": (c_int, [POINTER(qmoe_layer), c_int32, POINTER(qmoe_ws_layout)]),
        "qmoe_route": (c_int, [POINTER(qmoe_layer), c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_size_t,
                               c_void_p]),
        "qmoe_decode_layer": (c_int, [POINTER(qmoe_layer), c_void_p, c_int32, c_void_p, c_void_p, c_size_t,
                                      c_void_p]),
        "qmoe_decode_layer_mfma": (c_int, [POINTER(qmoe_layer), c_void_p, c_int32, c_void_p, c_void_p, c_size_t,
                                           c_void_p]),
        "qmoe_decode_noalloc_max_bytes": (c_size_t, []),
        "qmoe_decode_layer_noalloc": (c_int, [POINTER(qmoe_layer), c_void_p, c_int32, c_void_p, c_void_p]),
        "qmoe_prefill_layer": (c_int, [POINTER(qmoe_layer), c_void_p, c_int32, c_void_p, c_void_p, c_size_t,
                                       c_void_p]),
        "qmoe_prefill_layer_ex": (c_int, [POINTER(qmoe_layer), c_void_p, c_int32, c_void_p, c_void_p, c_size_t,
                                          c_int32, c_void_p]),
        "qmoe_matvec_workspace_bytes": (c_size_t, [c_int64, c_int32]),
        "qmoe_matvec_group_workspace_bytes": (c_size_t, [POINTER(qmoe_matvec_item), c_int32, c_int32]),
        "qmoe_matvec_group": (c_int, [POINTER(qmoe_matvec_item), c_int32, c_int32, c_void_p, c_size_t, c_void_p]),
        "qmoe_matvec": (c_int, [c_int, c_int64, c_int64, c_void_p, c_size_t, c_void_p, c_int32, c_void_p, c_int32,
                                c_void_p, c_void_p, c_size_t, c_void_p]),
        "qmoe_matvec_expanded_workspace_bytes": (c_size_t, [c_int64, c_int64, c_int32]),
        "qmoe_matvec_expanded": (c_int, [c_int, c_int64, c_int64, c_void_p, c_size_t, c_void_p, c_int32, c_void_p,
                                         c_int32, c_void_p, c_void_p, c_size_t, c_void_p]),
        "qmoe_quant_act": (c_int, [c_void_p, c_int64, c_int64, c_int32, c_void_p, c_void_p, c_void_p]),
        "qmoe_block_dots": (c_int, [c_int, c_int64, c_int64, c_void_p, c_size_t, c_void_p, c_void_p, c_void_p,
                                    c_void_p]),
        "qmoe_block_dots_mfma": (c_int, [c_int, c_int64, c_int64, c_void_p, c_size_t, c_void_p, c_void_p, c_int32,
                                         c_void_p, c_void_p]),
        "qmoe_probe_read": (c_int, [c_void_p, c_size_t, c_int32, c_void_p, c_void_p]),
        "qmoe_probe_mfma": (c_int, [c_int32, c_int32, c_int32, c_void_p, c_void_p]),
        "qmoe_probe_valu": (c_int, [c_int32, c_int32, c_void_p, c_void_p]),
        "qmoe_quantize_workspace_bytes": (c_size_t, [c_int32, c_int64, c_int64]),
        "qmoe_quantize": (c_int, [c_int, c_int32, c_int64, c_int64, c_void_p, c_int32, c_void_p, c_size_t, c_void_p,
                                  c_void_p, c_size_t, c_void_p]),
        "qmoe_timing_enable": (c_int, [c_int]),
        "qmoe_timing_read": (c_int, [c_char_p, POINTER(c_double), POINTER(c_int)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


LIB = load_library()

EXPORTED = (
    "qmoe_strerror", "qmoe_last_error", "qmoe_version", "qmoe_block_bytes", "qmoe_packed_bytes", "qmoe_pack",
    "qmoe_unpack", "qmoe_layer_check", "qmoe_workspace_bytes", "qmoe_workspace_layout", "qmoe_route",
    "qmoe_decode_layer", "qmoe_decode_layer_mfma", "qmoe_decode_noalloc_max_bytes", "qmoe_decode_layer_noalloc", "qmoe_prefill_layer", "qmoe_prefill_layer_ex",
    "qmoe_matvec_workspace_bytes", "qmoe_matvec_group_workspace_bytes", "qmoe_matvec_group", "qmoe_matvec", "qmoe_quant_act",
    "qmoe_block_dots", "qmoe_block_dots_mfma", "qmoe_matvec_expanded_workspace_bytes", "qmoe_matvec_expanded",
    "qmoe_quantize_workspace_bytes", "qmoe_quantize", "qmoe_timing_enable", "qmoe_timing_read", "qmoe_probe_read",
    "qmoe_probe_mfma", "qmoe_probe_valu",
)


def strerror(status: int) -> str:
    return LIB.qmoe_strerror(status).decode()


def _check(status: int, where: str):
    if status != QMOE_OK:
        raise QmoeError(status, where, LIB.qmoe_last_error().decode())


def _ptr(a) -> int:
    """Address of a numpy array or a torch tensor (None -> NULL)."""
    if a is None:
        return None
    if isinstance(a, np.ndarray):
        return a.ctypes.data
    return a.data_ptr()


def _nbytes(a) -> int:
    if a is None:
        return 0
    if isinstance(a, np.ndarray):
        return a.nbytes
    return a.numel() * a.element_size()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


# ------------------------------------------------------------------ host calls

def qmoe_block_bytes(fmt: int) -> int:
    return LIB.qmoe_block_bytes(fmt)


def qmoe_packed_bytes(fmt: int, rows: int, k: int) -> int:
    return LIB.qmoe_packed_bytes(fmt, rows, k)


def qmoe_pack(fmt: int, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Host pack: codes uint8 [rows, k], scales uint16 (fp16 bits) or uint8 (E8M0)
    [rows, k/32] -> uint8 [rows, row_bytes]."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    rows, k = codes.shape
    scales = np.ascontiguousarray(scales, dtype=np.uint8 if fmt == FP4 else np.uint16)
    if scales.size != rows * (k // 32):
        raise ValueError("scales shape does not match codes")
    nbytes = qmoe_packed_bytes(fmt, rows, k)
    out = np.empty((rows, nbytes // rows if rows else 0), dtype=np.uint8)
    _check(LIB.qmoe_pack(fmt, rows, k, _ptr(codes), _ptr(scales), _ptr(out), out.nbytes), "qmoe_pack")
    return out


def qmoe_unpack(fmt: int, packed: np.ndarray, rows: int, k: int):
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    codes = np.empty((rows, k), dtype=np.uint8)
    scales = np.empty((rows, k // 32), dtype=np.uint8 if fmt == FP4 else np.uint16)
    _check(LIB.qmoe_unpack(fmt, rows, k, _ptr(packed), packed.nbytes, _ptr(codes), _ptr(scales)), "qmoe_unpack")
    return codes, scales


def make_layer(hidden, inter, n_experts, topk, fmt_gate, fmt_up, fmt_down, rot_gateup, rot_down,
               w_router, router_bias, gate, up, down, cb_gate, cb_up, cb_down) -> qmoe_layer:
    """Descriptor from device tensors (or numpy arrays for host-only checks)."""
    return qmoe_layer(
        hidden, inter, n_experts, topk, fmt_gate, fmt_up, fmt_down, rot_gateup, rot_down,
        _ptr(w_router), _nbytes(w_router), _ptr(router_bias),
        _ptr(gate), _nbytes(gate), _ptr(up), _nbytes(up), _ptr(down), _nbytes(down),
        _ptr(cb_gate), _nbytes(cb_gate), _ptr(cb_up), _nbytes(cb_up), _ptr(cb_down), _nbytes(cb_down))


def qmoe_layer_check(L: qmoe_layer) -> None:
    _check(LIB.qmoe_layer_check(ctypes.byref(L)), "qmoe_layer_check")


def qmoe_workspace_bytes(L: qmoe_layer, max_tokens: int) -> int:
    n = LIB.qmoe_workspace_bytes(ctypes.byref(L), max_tokens)
    if n == 0:
        _check(LIB.qmoe_layer_check(ctypes.byref(L)), "qmoe_workspace_bytes")
    return n


def qmoe_workspace_layout(L: qmoe_layer, max_tokens: int) -> dict:
    lay = qmoe_ws_layout()
    _check(LIB.qmoe_workspace_layout(ctypes.byref(L), max_tokens, ctypes.byref(lay)), "qmoe_workspace_layout")
    return {name: getattr(lay, name) for name, _ in qmoe_ws_layout._fields_}


def qmoe_matvec_workspace_bytes(k: int, ncols: int) -> int:
    return LIB.qmoe_matvec_workspace_bytes(k, ncols)


# ------------------------------------------------------------------ device calls (torch tensors)

def qmoe_route(L, x, idx, gate_w, ws, stream=None) -> None:
    _check(LIB.qmoe_route(ctypes.byref(L), _ptr(x), x.shape[0], _ptr(idx), _ptr(gate_w), _ptr(ws), _nbytes(ws),
                          _stream(stream)), "qmoe_route")


def qmoe_decode_layer(L, x, out, ws, stream=None) -> None:
    _check(LIB.qmoe_decode_layer(ctypes.byref(L), _ptr(x), x.shape[0], _ptr(out), _ptr(ws), _nbytes(ws),
                                 _stream(stream)), "qmoe_decode_layer")


def qmoe_decode_layer_mfma(L, x, out, ws, stream=None) -> None:
    _check(LIB.qmoe_decode_layer_mfma(ctypes.byref(L), _ptr(x), x.shape[0], _ptr(out), _ptr(ws), _nbytes(ws),
                                      _stream(stream)), "qmoe_decode_layer_mfma")


def qmoe_decode_layer_noalloc(L, x, out, stream=None) -> None:
    _check(LIB.qmoe_decode_layer_noalloc(ctypes.byref(L), _ptr(x), x.shape[0], _ptr(out), _stream(stream)),
           "qmoe_decode_layer_noalloc")


def qmoe_prefill_layer(L, x, out, ws, stream=None) -> None:
    _check(LIB.qmoe_prefill_layer(ctypes.byref(L), _ptr(x), x.shape[0], _ptr(out), _ptr(ws), _nbytes(ws),
                                  _stream(stream)), "qmoe_prefill_layer")


# QMOE_PREFILL_SMALL_DEFAULT of qmoe.h: the small-expert threshold of qmoe_prefill_layer
PREFILL_SMALL_DEFAULT = 2


def qmoe_prefill_layer_ex(L, x, out, ws, small_pairs, stream=None) -> None:
    _check(LIB.qmoe_prefill_layer_ex(ctypes.byref(L), _ptr(x), x.shape[0], _ptr(out), _ptr(ws), _nbytes(ws),
                                     small_pairs, _stream(stream)), "qmoe_prefill_layer_ex")


def matvec_items(items):
    """ctypes array of qmoe_matvec_item from (fmt, rows, k, w, cb, rot, x, y) tuples."""
    arr = (qmoe_matvec_item * len(items))()
    for a, (fmt, rows, k, w, cb, rot, x, y) in zip(arr, items):
        a.fmt, a.rot, a.rows, a.k = fmt, rot, rows, k
        a.w, a.w_bytes, a.cb, a.x, a.y = _ptr(w), _nbytes(w), _ptr(cb), _ptr(x), _ptr(y)
    return arr


def qmoe_matvec_group_workspace_bytes(items, ncols: int) -> int:
    arr = matvec_items(items)
    return LIB.qmoe_matvec_group_workspace_bytes(arr, len(items), ncols)


def qmoe_matvec_group(items, ncols, ws, stream=None) -> None:
    """items: (fmt, rows, k, w, cb, rot, x, y) per matrix (device tensors). The
    first 16 bytes of ws must be zero before its first use (torch.zeros)."""
    arr = matvec_items(items)
    _check(LIB.qmoe_matvec_group(arr, len(items), ncols, _ptr(ws), _nbytes(ws), _stream(stream)),
           "qmoe_matvec_group")


def qmoe_matvec(fmt, rows, k, w, cb, rot, x, y, ws, stream=None) -> None:
    _check(LIB.qmoe_matvec(fmt, rows, k, _ptr(w), _nbytes(w), _ptr(cb), rot, _ptr(x), x.shape[0], _ptr(y),
                           _ptr(ws), _nbytes(ws), _stream(stream)), "qmoe_matvec")


def qmoe_matvec_expanded_workspace_bytes(rows: int, k: int, ncols: int) -> int:
    return LIB.qmoe_matvec_expanded_workspace_bytes(rows, k, ncols)


def qmoe_matvec_expanded(fmt, rows, k, w, cb, rot, x, y, ws, stream=None) -> None:
    _check(LIB.qmoe_matvec_expanded(fmt, rows, k, _ptr(w), _nbytes(w), _ptr(cb), rot, _ptr(x), x.shape[0], _ptr(y),
                                    _ptr(ws), _nbytes(ws), _stream(stream)), "qmoe_matvec_expanded")


def qmoe_quant_act(x, rot, xq, dx, stream=None) -> None:
    n_vec, k = x.shape
    _check(LIB.qmoe_quant_act(_ptr(x), n_vec, k, rot, _ptr(xq), _ptr(dx), _stream(stream)), "qmoe_quant_act")


def qmoe_block_dots(fmt, rows, k, w, cb, xq, P, stream=None) -> None:
    _check(LIB.qmoe_block_dots(fmt, rows, k, _ptr(w), _nbytes(w), _ptr(cb), _ptr(xq), _ptr(P), _stream(stream)),
           "qmoe_block_dots")


def qmoe_block_dots_mfma(fmt, rows, k, w, cb, xq, P, stream=None) -> None:
    """xq: int8 [ncols, k]; P: int32 [ncols, rows, k/32]."""
    _check(LIB.qmoe_block_dots_mfma(fmt, rows, k, _ptr(w), _nbytes(w), _ptr(cb), _ptr(xq), xq.shape[0], _ptr(P),
                                    _stream(stream)), "qmoe_block_dots_mfma")


def qmoe_probe_read(buf, grid, sink, stream=None) -> None:
    _check(LIB.qmoe_probe_read(_ptr(buf), _nbytes(buf), grid, _ptr(sink), _stream(stream)), "qmoe_probe_read")


def qmoe_probe_mfma(kind, iters, grid, sink, stream=None) -> None:
    _check(LIB.qmoe_probe_mfma(kind, iters, grid, _ptr(sink), _stream(stream)), "qmoe_probe_mfma")


def qmoe_probe_valu(iters, grid, sink, stream=None) -> None:
    _check(LIB.qmoe_probe_valu(iters, grid, _ptr(sink), _stream(stream)), "qmoe_probe_valu")


def qmoe_quantize_workspace_bytes(n: int, rows: int, k: int) -> int:
    return LIB.qmoe_quantize_workspace_bytes(n, rows, k)


def qmoe_quantize(fmt, w, iters, out, cb, ws, stream=None) -> None:
    """w: fp32 [n, rows, k]; out: uint8 [n, rows, row_bytes]; cb: int8 [n, 2^bits]."""
    n, rows, k = w.shape
    _check(LIB.qmoe_quantize(fmt, n, rows, k, _ptr(w), iters, _ptr(out), _nbytes(out), _ptr(cb), _ptr(ws),
                             _nbytes(ws), _stream(stream)), "qmoe_quantize")


def qmoe_timing_enable(on: bool) -> None:
    _check(LIB.qmoe_timing_enable(1 if on else 0), "qmoe_timing_enable")


def qmoe_timing_read(name: str):
    """-> (total_ms, count) of the recorded launches of kernel ``name``."""
    ms = c_double()
    n = c_int()
    _check(LIB.qmoe_timing_read(name.encode(), ctypes.byref(ms), ctypes.byref(n)), "qmoe_timing_read")
    return ms.value, n.value
