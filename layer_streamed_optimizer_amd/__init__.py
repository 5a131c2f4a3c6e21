"""Per-layer mixed-precision Adam on MI355X (gfx950), HBM-resident or
layer-streamed from host memory or files.

A thin binding over liblso.so (include/lso.h): it marshals descriptor tables
and stream handles; every step of the update runs in the HIP library.
PyTorch, where used, only provides device memory and streams.

    table = BlockTable.from_rows([...])       # one dict per block
    table.set_step(t)                         # the caller owns t
    adam_step(table, stream)                  # one kernel launch

    ls = LayerStream(max_layer_bytes, max_layer_params, grad_fn, user)
    ls.stream_layers(host_layers)             # H2D / update / D2H, double-buffered
    ls.stream_files(file_layers)              # the disk tier (see disk.LayerFiles)
"""
from __future__ import annotations

import ctypes
from typing import Iterable

import numpy as np

from . import _native
from ._native import (LSO_DT_BF16, LSO_DT_F32, LSO_DT_NONE, LSO_FILE_SHADOW, LSO_FILE_SYNC,
                      LSO_LAYOUT_PLANAR, LSO_LAYOUT_TILED, LSO_OPT_ADAM, LSO_OPT_SGD,
                      LSO_SHADOW_HEADER_BYTES, LSO_TILE_ELEMS, LsoBlock, LsoError, LsoFileLayer,
                      LsoHostLayer)

BLOCK_DTYPE = np.dtype(LsoBlock)
HOST_LAYER_DTYPE = np.dtype(LsoHostLayer)
FILE_LAYER_DTYPE = np.dtype(LsoFileLayer)

__all__ = ["BlockTable", "adam_step", "adam_step_noalloc", "adam_step_norms", "launch_count", "norm_workspace_bytes", "validate",
           "block_constants", "LayerStream", "HostBuffer", "host_alloc", "LsoError", "LSO_OPT_ADAM",
           "LSO_OPT_SGD", "LSO_DT_BF16", "LSO_DT_NONE", "LSO_DT_F32", "LSO_LAYOUT_PLANAR",
           "LSO_LAYOUT_TILED", "LSO_TILE_ELEMS", "BLOCK_DTYPE", "HOST_LAYER_DTYPE", "FILE_LAYER_DTYPE",
           "LSO_FILE_SYNC", "LSO_FILE_SHADOW", "LSO_SHADOW_HEADER_BYTES", "shadow_format",
           "shadow_state", "shadow_commit", "stream_handle", "tiled_state_bytes", "tiled_pack", "tiled_unpack"]


def stream_handle(stream=None) -> int:
    """hipStream_t of a torch stream, an int handle, or torch's current stream."""
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _addr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


class BlockTable:
    """A reusable lso_block table (numpy structured array in the C layout)."""

    def __init__(self, n: int):
        self.arr = np.zeros(n, BLOCK_DTYPE)
        self._ptr = self.arr.ctypes.data      # the array is never reallocated

    def __len__(self) -> int:
        return len(self.arr)

    @classmethod
    def from_array(cls, arr: np.ndarray) -> "BlockTable":
        """A table holding a copy of an lso_block structured array."""
        if arr.dtype != BLOCK_DTYPE:
            raise TypeError("need a BLOCK_DTYPE array")
        tab = cls(len(arr))
        tab.arr[:] = arr
        return tab

    @classmethod
    def from_rows(cls, rows: Iterable[dict]) -> "BlockTable":
        rows = list(rows)
        tab = cls(len(rows))
        for i, r in enumerate(rows):
            tab.set_row(i, **r)
        return tab

    def set_row(self, i: int, *, n: int, master, grad, m=None, v=None, weight=None, t: int = 1,
                lr: float = 1e-3, beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8,
                opt: int = LSO_OPT_ADAM, base: int = 0, layout: int = LSO_LAYOUT_PLANAR,
                grad_dtype: int = LSO_DT_BF16) -> None:
        """Arrays are torch tensors (their data_ptr) or integer device
        addresses; with base != 0 the integers are offsets from base.  With
        layout = LSO_LAYOUT_TILED, master is the tiled state region and m, v
        are not used."""
        row = self.arr[i]
        row["base"] = base
        row["n"] = n
        row["off_master"] = _addr(master)
        row["off_m"] = _addr(m)
        row["off_v"] = _addr(v)
        row["off_grad"] = _addr(grad)
        row["off_weight"] = _addr(weight)
        row["grad_dtype"] = grad_dtype
        row["weight_dtype"] = LSO_DT_BF16 if weight is not None else LSO_DT_NONE
        row["opt"] = opt
        row["layout"] = layout
        row["t"] = t
        row["lr"], row["beta1"], row["beta2"], row["eps"] = lr, beta1, beta2, eps

    def set_step(self, t: int) -> None:
        self.arr["t"] = t

    @property
    def ptr(self) -> int:
        return self._ptr


_step_fn = None


def adam_step(table: BlockTable, stream=None) -> None:
    """One fused update of every block in the table, enqueued on stream
    (one kernel launch).  Asynchronous."""
    global _step_fn
    if _step_fn is None:
        _step_fn = _native.lib().lso_adam_step
    st = _step_fn(table._ptr, len(table.arr), stream if type(stream) is int else stream_handle(stream))
    if st:
        _native.check(st, "lso_adam_step")


def adam_step_noalloc(table: BlockTable, stream=None) -> None:
    """adam_step for callers that cannot allocate device memory: the same
    update, with the block table kept in the library's fixed per-device
    scratch array (at most LSO_NOALLOC_MAX_BLOCKS entries per call).  Calls
    that overlap on one GPU race on that array."""
    st = _native.lib().lso_adam_step_noalloc(table.ptr, len(table), stream_handle(stream))
    if st:
        _native.check(st, "lso_adam_step_noalloc")


def norm_workspace_bytes(table: BlockTable) -> int:
    """Device workspace adam_step_norms needs for this table."""
    return int(_native.lib().lso_norm_workspace_bytes(table.ptr, len(table)))


def adam_step_norms(table: BlockTable, sq_norms, workspace, workspace_bytes: int, stream=None) -> None:
    """adam_step plus sq_norms[i] = sum of g^2 of block i (FP64, device
    array of len(table) doubles), from the same pass over the gradients.
    workspace: device memory of at least norm_workspace_bytes(table) bytes."""
    st = _native.lib().lso_adam_step_norms(table.ptr, len(table), _addr(sq_norms), _addr(workspace),
                                           int(workspace_bytes), stream_handle(stream))
    _native.check(st, "lso_adam_step_norms")


def launch_count() -> int:
    """Fused-update kernel launches this process has enqueued (host counter)."""
    return int(_native.lib().lso_kernel_launches())


def validate(table: BlockTable) -> int:
    """The host-side checks of lso_adam_step; returns the status (0 = ok)."""
    return _native.lib().lso_validate_blocks(table.ptr, len(table))


def tiled_state_bytes(n: int) -> int:
    """Bytes of the tiled [master | m | v] state region of n parameters."""
    return int(_native.lib().lso_tiled_state_bytes(n))


def tiled_pack(state, master, m=None, v=None, *, n: int, stream=None) -> None:
    """Planar FP32 master (and m, v, else zeros) -> tiled state region
    (device addresses or tensors); asynchronous on stream."""
    st = _native.lib().lso_tiled_pack(_addr(state), _addr(master), _addr(m) or None,
                                      _addr(v) or None, n, stream_handle(stream))
    _native.check(st, "lso_tiled_pack")


def tiled_unpack(state, master=None, m=None, v=None, *, n: int, stream=None) -> None:
    """Tiled state region -> planar FP32 arrays (None skips one)."""
    st = _native.lib().lso_tiled_unpack(_addr(state), _addr(master) or None, _addr(m) or None,
                                        _addr(v) or None, n, stream_handle(stream))
    _native.check(st, "lso_tiled_unpack")


def shadow_format(fd: int, file_offset: int, nbytes: int, t0: int = 0) -> None:
    """Format a crash-consistent shadow region (host only)."""
    _native.check(_native.lib().lso_shadow_format(fd, file_offset, nbytes, t0), "lso_shadow_format")


def shadow_state(fd: int, file_offset: int, nbytes: int) -> tuple[int, int, int]:
    """(epoch, t, data_offset) of a shadow region's committed state (host only)."""
    e, t, off = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint64()
    _native.check(_native.lib().lso_shadow_state(fd, file_offset, nbytes, ctypes.byref(e),
                                                 ctypes.byref(t), ctypes.byref(off)), "lso_shadow_state")
    return int(e.value), int(t.value), int(off.value)


def shadow_commit(fd: int, file_offset: int, nbytes: int, epoch: int, t: int) -> None:
    """Write and flush the header copy that commits `epoch` (host only)."""
    _native.check(_native.lib().lso_shadow_commit(fd, file_offset, nbytes, epoch, t), "lso_shadow_commit")


def last_error() -> str:
    return _native.lib().lso_last_error().decode(errors="replace")


def block_constants(*, t: int, lr: float = 1e-3, beta1: float = 0.9, beta2: float = 0.999,
                    eps: float = 1e-8, opt: int = LSO_OPT_ADAM) -> np.ndarray:
    """The FP32 constants the kernel uses for one block (host computation)."""
    b = LsoBlock()
    b.n, b.grad_dtype, b.weight_dtype, b.opt, b.t = 1, LSO_DT_BF16, LSO_DT_NONE, opt, t
    b.lr, b.beta1, b.beta2, b.eps = lr, beta1, beta2, eps
    out = (ctypes.c_float * 8)()
    _native.check(_native.lib().lso_block_constants(ctypes.byref(b), out), "lso_block_constants")
    return np.array(out, dtype=np.float32)


class HostBuffer:
    """Pinned host memory from lso_host_alloc (page aligned)."""

    def __init__(self, nbytes: int):
        p = ctypes.c_void_p()
        _native.check(_native.lib().lso_host_alloc(nbytes, ctypes.byref(p)), "lso_host_alloc")
        self.ptr = int(p.value)
        self.nbytes = nbytes
        self._closed = False

    def view(self, dtype=np.uint8, offset: int = 0, count: int | None = None) -> np.ndarray:
        dt = np.dtype(dtype)
        if count is None:
            count = (self.nbytes - offset) // dt.itemsize
        if offset + count * dt.itemsize > self.nbytes:
            raise ValueError("view past the end of the buffer")
        raw = (ctypes.c_char * (count * dt.itemsize)).from_address(self.ptr + offset)
        return np.frombuffer(raw, dtype=dt, count=count)

    def close(self) -> None:
        if not self._closed:
            _native.check(_native.lib().lso_host_free(self.ptr), "lso_host_free")
            self._closed = True

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def host_alloc(nbytes: int) -> HostBuffer:
    return HostBuffer(nbytes)


class LayerStream:
    """lso_stream_create / lso_stream_layers / lso_stream_destroy.

    grad_fn: a C function pointer (int) with the lso_grad_fn signature, or a
    Python callable (layer, dev_grad_ptr, n, stream_handle) -> int that only
    enqueues work on the given stream."""

    def __init__(self, max_layer_bytes: int, max_layer_params: int, grad_fn, user: int = 0,
                 device: int = 0):
        if callable(grad_fn):
            py = grad_fn
            self._cb = _native.GRAD_FN(lambda u, layer, g, n, s: int(py(layer, g, n, s)))
            fn_ptr = ctypes.cast(self._cb, ctypes.c_void_p).value
        else:
            self._cb = None
            fn_ptr = int(grad_fn)
        self._user = user
        ctx = ctypes.c_void_p()
        st = _native.lib().lso_stream_create(max_layer_bytes, max_layer_params, fn_ptr, user,
                                              device, ctypes.byref(ctx))
        _native.check(st, "lso_stream_create")
        self.ctx = int(ctx.value)

    @staticmethod
    def layers(n: int) -> np.ndarray:
        return np.zeros(n, HOST_LAYER_DTYPE)

    def stream_layers(self, host_layers: np.ndarray) -> None:
        _native.check(self.stream_layers_status(host_layers), "lso_stream_layers")

    def stream_layers_status(self, host_layers: np.ndarray) -> int:
        if host_layers.dtype != HOST_LAYER_DTYPE or not host_layers.flags.c_contiguous:
            raise TypeError("host_layers must be a contiguous HOST_LAYER_DTYPE array")
        return _native.lib().lso_stream_layers(self.ctx, host_layers.ctypes.data, len(host_layers))

    @staticmethod
    def file_layers(n: int) -> np.ndarray:
        return np.zeros(n, FILE_LAYER_DTYPE)

    def stream_files(self, file_layers: np.ndarray) -> None:
        """lso_stream_files: the disk tier (blocks held in file regions)."""
        st = self.stream_files_status(file_layers)
        _native.check(st, "lso_stream_files")

    def stream_files_status(self, file_layers: np.ndarray) -> int:
        if file_layers.dtype != FILE_LAYER_DTYPE or not file_layers.flags.c_contiguous:
            raise TypeError("file_layers must be a contiguous FILE_LAYER_DTYPE array")
        return _native.lib().lso_stream_files(self.ctx, file_layers.ctypes.data, len(file_layers))

    def slot_weight(self, slot: int) -> int:
        return int(_native.lib().lso_stream_slot_weight(self.ctx, slot) or 0)

    def copy_mode(self) -> dict:
        """lso_stream_copy_mode: how the context moves blocks over the link
        (name and code), and the SDMA engine masks in the sdma-pair mode."""
        h, d = ctypes.c_uint32(), ctypes.c_uint32()
        code = _native.lib().lso_stream_copy_mode(self.ctx, ctypes.byref(h), ctypes.byref(d))
        return dict(mode=_native.COPY_MODE_NAMES.get(code, code), code=code, h2d_engine=h.value,
                    d2h_engine=d.value)

    def stats(self) -> dict:
        """lso_stream_stats: pieces moved by the last call, the host loop's
        wake-ups during it, and whether each H2D was chained on the engine."""
        out = (ctypes.c_uint64 * 3)()
        if _native.lib().lso_stream_stats(self.ctx, out) != 0:
            raise RuntimeError("lso_stream_stats failed")
        return dict(pieces=int(out[0]), host_waits=int(out[1]), chained=bool(out[2]))

    def close(self) -> None:
        if self.ctx:
            _native.lib().lso_stream_destroy(self.ctx)
            self.ctx = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
