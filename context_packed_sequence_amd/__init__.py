"""THD context-parallel layout transform on MI355X (gfx950).

Low level: the C entry points of libthdcp under their own names
(``thd_build_route``, ``thd_swap``, ``thd_roll_labels``, ...), see
``binding.py`` and ``include/thd_cp.h``.

High level: ``Route`` (one per micro-batch: build once, swap many times) and
``roll_labels``.  Both only allocate output tensors with torch and hand
pointers to the library; the work runs in the library's HIP kernels.
"""

from __future__ import annotations

from .binding import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    THD_CONTIGUOUS_TO_ZIGZAG,
    THD_PACK_STATIC_BYTES,
    THD_ERR_ALIAS,
    THD_ERR_ARG,
    THD_ERR_CAPACITY,
    THD_ERR_CU_DIVISIBLE,
    THD_ERR_CU_MONOTONE,
    THD_ERR_CU_START,
    THD_ERR_CU_TOTAL,
    THD_ERR_DEVICE,
    THD_ERR_DIRECTION,
    THD_ERR_HIP,
    THD_ERR_INTEGRITY,
    THD_ERR_NOT_BUILT,
    THD_ERR_PACK_CAPACITY,
    THD_ERR_PACK_DOCS,
    THD_ERR_REAL_GT_PADDED,
    THD_ERR_SHAPE,
    THD_IDENTITY,
    THD_MAX_BATCH,
    THD_PACK_MAX_SEQ,
    THD_MAX_CP,
    THD_MAX_SHIFT,
    THD_OK,
    THD_ZIGZAG_TO_CONTIGUOUS,
    ThdError,
    thd_build_route,
    thd_copy,
    thd_read_stream,
    thd_write_stream,
    thd_pack,
    thd_pack_noalloc,
    thd_pack_workspace_bytes,
    thd_roll_labels,
    thd_roll_labels_zigzag,
    thd_route_copy_out,
    thd_route_create,
    thd_route_destroy,
    thd_route_info,
    thd_route_status,
    thd_strerror,
    thd_swap,
    thd_route_launch_shape,
    thd_swap_batch,
)

Z2C = THD_ZIGZAG_TO_CONTIGUOUS
C2Z = THD_CONTIGUOUS_TO_ZIGZAG


def _need(t, name, dtype=None, numel=None, device=None):
    """Shape/dtype checks the C ABI cannot make: it sees only pointers, so a
    too-small or wrongly typed buffer would be read or written out of bounds."""
    if t is None:
        raise ValueError(f"{name} is required")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


class Route:
    """A device-resident zigzag <-> contiguous route.

    ``Route(max_slots, max_cp, max_tokens)`` allocates the workspace once;
    ``build(cu_seqlens_padded, cp_size, total_tokens)`` rebuilds it for a new
    micro-batch without waiting for the GPU; ``swap(x, direction)`` moves the
    rows of ``x`` ([T, ...], token dimension first) and returns a new tensor,
    or ``x`` itself when the route is the identity.
    """

    def __init__(self, max_slots: int, max_cp: int, max_tokens: int):
        self.handle = thd_route_create(max_slots, max_cp, max_tokens)
        self.total = 0

    def close(self):
        if getattr(self, "handle", None):
            thd_route_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def build(self, cu_seqlens_padded, cp_size: int, total_tokens: int, stream=None) -> "Route":
        """total_tokens is passed in because the boundaries stay on the device."""
        import torch
        _need(cu_seqlens_padded, "cu_seqlens_padded", torch.int32)
        n_slots = int(cu_seqlens_padded.numel()) - 1
        thd_build_route(self.handle, cu_seqlens_padded, n_slots, cp_size, total_tokens, stream)
        self.total = int(total_tokens)
        return self

    def swap(self, x, direction: int, out=None, stream=None):
        import torch
        if x.dim() == 0:
            raise ValueError("x needs a token dimension")
        _need(x, "x")
        if out is None:
            out = torch.empty_like(x, memory_format=torch.contiguous_format)
        _need(out, "out", x.dtype, x.numel(), x.device)
        rows = x.shape[0]
        row_bytes = x.element_size() * (x.numel() // rows if rows else 1)
        code = thd_swap(self.handle, direction, x, out, rows, max(row_bytes, 1), stream)
        return x if code == THD_IDENTITY else out

    def swap_many(self, xs, direction: int, outs=None, stream=None):
        """Swap several tensors (same token count) in one launch; returns the
        outputs, or the inputs themselves when the route is the identity."""
        import torch
        if not xs:
            raise ValueError("swap_many needs at least one tensor")
        rows = xs[0].shape[0]
        for i, x in enumerate(xs):
            if x.dim() == 0 or x.shape[0] != rows:
                raise ValueError(f"tensor {i} does not have {rows} rows")
            _need(x, f"xs[{i}]")
        if outs is None:
            outs = [torch.empty_like(x, memory_format=torch.contiguous_format) for x in xs]
        if len(outs) != len(xs):
            raise ValueError("outs and xs differ in length")
        for i, (x, o) in enumerate(zip(xs, outs)):
            _need(o, f"outs[{i}]", x.dtype, x.numel(), x.device)
        row_bytes = [max(1, x.element_size() * (x.numel() // rows if rows else 1)) for x in xs]
        code = thd_swap_batch(self.handle, direction, xs, outs, row_bytes, rows, stream)
        return list(xs) if code == THD_IDENTITY else outs

    def roll_labels_zigzag(self, ids, cu_seqlens_padded, cu_seqlens=None, max_shift: int = 1, fill: int = 0,
                           stream=None):
        """Label shift / MTP roll / valid mask written in this route's zigzag
        order: shifted [max_shift, T] int64, mask [max_shift + 1, T] uint8,
        status int32 [1]."""
        import torch
        _check_roll_inputs(ids, cu_seqlens_padded, cu_seqlens)
        total = int(ids.numel())
        shifted = torch.empty((max_shift, total), dtype=torch.int64, device=ids.device)
        mask = torch.empty((max_shift + 1, total), dtype=torch.uint8, device=ids.device)
        status = torch.empty(1, dtype=torch.int32, device=ids.device)
        n_slots = int(cu_seqlens_padded.numel()) - 1
        thd_roll_labels_zigzag(self.handle, ids, cu_seqlens_padded, cu_seqlens, n_slots, total, max_shift, fill,
                               shifted, mask, status, stream)
        return shifted, mask, status

    def status(self, stream=None) -> int:
        return thd_route_status(self.handle, stream)

    def copy_out(self, stream=None):
        return thd_route_copy_out(self.handle, stream)

    def info(self) -> dict:
        return thd_route_info(self.handle)


def _check_roll_inputs(ids, cu_seqlens_padded, cu_seqlens):
    import torch
    _need(ids, "ids", torch.int64)
    _need(cu_seqlens_padded, "cu_seqlens_padded", torch.int32, device=ids.device)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, cu_seqlens_padded.numel(), ids.device)


def roll_labels(ids, cu_seqlens_padded, cu_seqlens=None, max_shift: int = 1, fill: int = 0, stream=None,
                with_status: bool = True):
    """Shifted label streams [max_shift, T] (int64), masks [max_shift + 1, T]
    (uint8) and, if asked, a device status word (int32 [1])."""
    import torch
    _check_roll_inputs(ids, cu_seqlens_padded, cu_seqlens)
    total = int(ids.numel())
    shifted = torch.empty((max_shift, total), dtype=torch.int64, device=ids.device)
    mask = torch.empty((max_shift + 1, total), dtype=torch.uint8, device=ids.device)
    status = torch.empty(1, dtype=torch.int32, device=ids.device) if with_status else None
    n_slots = int(cu_seqlens_padded.numel()) - 1
    thd_roll_labels(ids, cu_seqlens_padded, cu_seqlens, n_slots, total, max_shift, fill, shifted, mask, status,
                    stream)
    return shifted, mask, status


def pack(tokens, pad_id: int, eod_id: int, align: int, capacity: int, max_docs: int, pad_value: int = 0,
         stream=None):
    """Pack [batch, seq] int64 token rows on the device.  Returns (packed
    [capacity] int64, cu_seqlens [max_docs + 2] int32, cu_seqlens_padded
    [max_docs + 2] int32, status int32 [1]); the route and the roll take
    n_slots = max_docs + 1 and total_tokens = capacity."""
    import torch
    _need(tokens, "tokens", torch.int64)
    if tokens.dim() > 2:
        raise ValueError("tokens must be [batch, seq] or [seq]")
    batch, seq = (int(tokens.shape[0]), int(tokens.shape[1])) if tokens.dim() == 2 else (1, int(tokens.numel()))
    dev = tokens.device
    nbytes = thd_pack_workspace_bytes(batch, seq)
    workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    packed = torch.empty(capacity, dtype=torch.int64, device=dev)
    cu_real = torch.empty(max_docs + 2, dtype=torch.int32, device=dev)
    cu_pad = torch.empty(max_docs + 2, dtype=torch.int32, device=dev)
    status = torch.empty(1, dtype=torch.int32, device=dev)
    thd_pack(tokens, batch, seq, pad_id, eod_id, align, capacity, max_docs, pad_value, workspace, nbytes, packed,
             cu_real, cu_pad, status, stream)
    return packed, cu_real, cu_pad, status
