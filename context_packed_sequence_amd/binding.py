"""ctypes binding of libthdcp (include/thd_cp.h).

Argument marshalling only: every step of the route build, the swap and the
label roll runs in the library's HIP kernels.  Torch is used for device
memory and streams: tensors are passed as their ``data_ptr()``, streams as
``torch.cuda.current_stream().cuda_stream`` unless one is given.

The functions keep the C names.  Negative return codes raise ``ThdError``;
``thd_swap`` returns ``THD_IDENTITY`` (1) when nothing was written.

Importing this module loads ``libthdcp.so`` from the package directory and
raises ImportError if it has not been built: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libthdcp.so")

THD_OK = 0
THD_IDENTITY = 1
THD_ERR_ARG = -1
THD_ERR_DIRECTION = -2
THD_ERR_NOT_BUILT = -3
THD_ERR_ALIAS = -4
THD_ERR_CAPACITY = -5
THD_ERR_SHAPE = -6
THD_ERR_HIP = -7
THD_ERR_DEVICE = -8
THD_ERR_CU_START = -10
THD_ERR_CU_MONOTONE = -11
THD_ERR_CU_TOTAL = -12
THD_ERR_CU_DIVISIBLE = -13
THD_ERR_REAL_GT_PADDED = -14
THD_ERR_INTEGRITY = -15
THD_ERR_PACK_DOCS = -16
THD_ERR_PACK_CAPACITY = -17

THD_ZIGZAG_TO_CONTIGUOUS = 0
THD_CONTIGUOUS_TO_ZIGZAG = 1
THD_MAX_CP = 1024
THD_MAX_SHIFT = 8
THD_MAX_BATCH = 16
THD_PACK_MAX_SEQ = 2147479552
THD_PACK_STATIC_BYTES = 1048576

EXPORTS = (
    "thd_route_create", "thd_route_destroy", "thd_build_route", "thd_swap", "thd_roll_labels",
    "thd_route_status", "thd_route_copy_out", "thd_route_info", "thd_strerror",
    "thd_swap_batch", "thd_roll_labels_zigzag", "thd_pack_workspace_bytes", "thd_pack", "thd_copy",
    "thd_route_launch_shape", "thd_read_stream", "thd_write_stream", "thd_pack_noalloc",
)


class ThdError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = int(code)
        super().__init__(f"{where}: {_strerror(code)} ({code})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python context_packed_sequence_amd/build_lib.py` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    c_i32, c_i64, c_p = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    sig = {
        "thd_route_create": (ctypes.c_int, [c_i32, c_i32, c_i64, ctypes.POINTER(c_p)]),
        "thd_route_destroy": (None, [c_p]),
        "thd_build_route": (ctypes.c_int, [c_p, c_p, c_i32, c_i32, c_i64, c_p]),
        "thd_swap": (ctypes.c_int, [c_p, c_i32, c_p, c_p, c_i64, c_i64, c_p]),
        "thd_roll_labels": (ctypes.c_int, [c_p, c_p, c_p, c_i32, c_i64, c_i32, c_i64, c_p, c_p, c_p, c_p]),
        "thd_route_status": (ctypes.c_int, [c_p, c_p, ctypes.POINTER(c_i32)]),
        "thd_route_copy_out": (ctypes.c_int, [c_p, c_p, ctypes.POINTER(c_i32), c_i32, c_p, c_p, c_p]),
        "thd_route_info": (ctypes.c_int, [c_p, ctypes.POINTER(c_i32), ctypes.POINTER(c_i64),
                                          ctypes.POINTER(c_i32), ctypes.POINTER(c_i32)]),
        "thd_strerror": (ctypes.c_char_p, [c_i32]),
        "thd_swap_batch": (ctypes.c_int, [c_p, c_i32, c_i32, ctypes.POINTER(c_p), ctypes.POINTER(c_p),
                                          ctypes.POINTER(c_i64), c_i64, c_p]),
        "thd_roll_labels_zigzag": (ctypes.c_int, [c_p, c_p, c_p, c_p, c_i32, c_i64, c_i32, c_i64, c_p, c_p, c_p,
                                                  c_p]),
        "thd_pack_workspace_bytes": (ctypes.c_int64, [c_i32, c_i32]),
        "thd_copy": (ctypes.c_int, [c_p, c_p, c_i64, c_p]),
        "thd_route_launch_shape": (ctypes.c_int, [c_p, c_i64, c_i32, c_i32, c_i32]),
        "thd_read_stream": (ctypes.c_int, [c_p, c_i64, c_p, c_p, c_p]),
        "thd_write_stream": (ctypes.c_int, [c_p, c_i64, ctypes.c_uint32, c_p]),
        "thd_pack": (ctypes.c_int, [c_p, c_i32, c_i32, c_i64, c_i64, c_i32, c_i64, c_i32, c_i64, c_p, c_i64, c_p,
                                    c_p, c_p, c_p, c_p]),
        "thd_pack_noalloc": (ctypes.c_int, [c_p, c_i32, c_i32, c_i64, c_i64, c_i32, c_i64, c_i32, c_i64, c_p, c_p,
                                            c_p, c_p, c_p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def _strerror(code: int) -> str:
    return _lib.thd_strerror(int(code)).decode()


def _ptr(x) -> int | None:
    """Device address of a tensor (must be contiguous) or a raw integer address."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_contiguous():
        raise ValueError("tensors passed to libthdcp must be contiguous")
    if not x.is_cuda:
        raise ValueError("tensors passed to libthdcp must live on the GPU")
    return x.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(code: int, where: str) -> int:
    if code < 0:
        raise ThdError(code, where)
    return code


# ---- the C entry points, same names ------------------------------------------

def thd_strerror(code: int) -> str:
    return _strerror(code)


def thd_route_create(max_slots: int, max_cp: int, max_tokens: int) -> int:
    h = ctypes.c_void_p()
    _check(_lib.thd_route_create(max_slots, max_cp, max_tokens, ctypes.byref(h)), "thd_route_create")
    return h.value


def thd_route_destroy(route: int) -> None:
    _lib.thd_route_destroy(route)


def thd_build_route(route: int, cu_seqlens_padded, n_slots: int, cp_size: int, total_tokens: int,
                    stream=None) -> int:
    return _check(_lib.thd_build_route(route, _ptr(cu_seqlens_padded), n_slots, cp_size, total_tokens,
                                       _stream(stream)), "thd_build_route")


def thd_swap(route: int, direction: int, x, out, rows: int, row_bytes: int, stream=None) -> int:
    return _check(_lib.thd_swap(route, direction, _ptr(x), _ptr(out), rows, row_bytes, _stream(stream)),
                  "thd_swap")


def thd_roll_labels(ids, cu_seqlens_padded, cu_seqlens, n_slots: int, total_tokens: int, max_shift: int,
                    fill: int, shifted, mask, status, stream=None) -> int:
    return _check(_lib.thd_roll_labels(_ptr(ids), _ptr(cu_seqlens_padded), _ptr(cu_seqlens), n_slots,
                                       total_tokens, max_shift, fill, _ptr(shifted), _ptr(mask), _ptr(status),
                                       _stream(stream)), "thd_roll_labels")


def thd_swap_batch(route: int, direction: int, ins, outs, row_bytes, rows: int, stream=None) -> int:
    n = len(ins)
    arr_in = (ctypes.c_void_p * n)(*[_ptr(t) for t in ins])
    arr_out = (ctypes.c_void_p * n)(*[_ptr(t) for t in outs])
    arr_rb = (ctypes.c_int64 * n)(*[int(b) for b in row_bytes])
    return _check(_lib.thd_swap_batch(route, direction, n, arr_in, arr_out, arr_rb, rows, _stream(stream)),
                  "thd_swap_batch")


def thd_roll_labels_zigzag(route: int, ids, cu_seqlens_padded, cu_seqlens, n_slots: int, total_tokens: int,
                           max_shift: int, fill: int, shifted, mask, status, stream=None) -> int:
    return _check(_lib.thd_roll_labels_zigzag(route, _ptr(ids), _ptr(cu_seqlens_padded), _ptr(cu_seqlens),
                                              n_slots, total_tokens, max_shift, fill, _ptr(shifted), _ptr(mask),
                                              _ptr(status), _stream(stream)), "thd_roll_labels_zigzag")


def thd_pack_workspace_bytes(batch: int, seq: int) -> int:
    return int(_lib.thd_pack_workspace_bytes(batch, seq))


def thd_pack(tokens, batch: int, seq: int, pad_id: int, eod_id: int, align: int, capacity: int, max_docs: int,
             pad_value: int, workspace, workspace_bytes: int, packed, cu_seqlens, cu_seqlens_padded, status,
             stream=None) -> int:
    return _check(_lib.thd_pack(_ptr(tokens), batch, seq, pad_id, eod_id, align, capacity, max_docs, pad_value,
                                _ptr(workspace), workspace_bytes, _ptr(packed), _ptr(cu_seqlens),
                                _ptr(cu_seqlens_padded), _ptr(status), _stream(stream)), "thd_pack")


def thd_pack_noalloc(tokens, batch: int, seq: int, pad_id: int, eod_id: int, align: int, capacity: int,
                     max_docs: int, pad_value: int, packed, cu_seqlens, cu_seqlens_padded, status,
                     stream=None) -> int:
    return _check(_lib.thd_pack_noalloc(_ptr(tokens), batch, seq, pad_id, eod_id, align, capacity, max_docs,
                                        pad_value, _ptr(packed), _ptr(cu_seqlens), _ptr(cu_seqlens_padded),
                                        _ptr(status), _stream(stream)), "thd_pack_noalloc")


def thd_copy(x, out, nbytes: int, stream=None) -> int:
    return _check(_lib.thd_copy(_ptr(x), _ptr(out), nbytes, _stream(stream)), "thd_copy")


def thd_read_stream(x, nbytes: int, key: bytes, count, stream=None) -> int:
    """Add to count (device uint32) the number of 16-byte words of x equal to key (16 bytes)."""
    if len(key) != 16:
        raise ValueError("key must be 16 bytes")
    k = ctypes.create_string_buffer(bytes(key), 16)
    return _check(_lib.thd_read_stream(_ptr(x), nbytes, k, _ptr(count), _stream(stream)), "thd_read_stream")


def thd_write_stream(out, nbytes: int, seed: int, stream=None) -> int:
    return _check(_lib.thd_write_stream(_ptr(out), nbytes, seed & 0xFFFFFFFF, _stream(stream)), "thd_write_stream")


def thd_route_status(route: int, stream=None) -> int:
    v = ctypes.c_int32()
    _check(_lib.thd_route_status(route, _stream(stream), ctypes.byref(v)), "thd_route_status")
    return v.value


def thd_route_copy_out(route: int, stream=None):
    """Return (runs_by_src [n,3], runs_by_dst [n,3], split [cp,cp]) as numpy int32."""
    n = ctypes.c_int32()
    code = _lib.thd_route_copy_out(route, _stream(stream), ctypes.byref(n), 0, None, None, None)
    if code not in (THD_OK, THD_ERR_CAPACITY):
        _check(code, "thd_route_copy_out")
    cp = thd_route_info(route)["cp_size"]
    a = np.zeros((max(n.value, 1), 3), np.int32)
    b = np.zeros((max(n.value, 1), 3), np.int32)
    split = np.zeros((max(cp, 1), max(cp, 1)), np.int32)
    _check(_lib.thd_route_copy_out(route, _stream(stream), ctypes.byref(n), a.shape[0],
                                   a.ctypes.data, b.ctypes.data, split.ctypes.data), "thd_route_copy_out")
    return a[:n.value], b[:n.value], split[:cp, :cp]


def thd_route_info(route: int) -> dict:
    cp, total, n_slots, built = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32()
    _check(_lib.thd_route_info(route, ctypes.byref(cp), ctypes.byref(total), ctypes.byref(n_slots),
                               ctypes.byref(built)), "thd_route_info")
    return {"cp_size": cp.value, "total_tokens": total.value, "n_slots": n_slots.value, "built": bool(built.value)}


def thd_route_launch_shape(route: int, tile_bytes: int = 0, nontemporal: int = 1, block_threads: int = 0,
                           tile_order: int = 0) -> None:
    """Override the launch shape of later swaps on one route (0 = built-in
    choice); no shape arguments restore the defaults (include/thd_cp_bench.h)."""
    _check(_lib.thd_route_launch_shape(route, tile_bytes, nontemporal, block_threads, tile_order),
           "thd_route_launch_shape")


def library():
    """The loaded CDLL (for symbol checks)."""
    return _lib
