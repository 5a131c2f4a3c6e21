"""ctypes view of include/lso.h (argument marshalling only).

Every step of the update runs in liblso.so.  If the library is missing the
import still works (so host-side code can be inspected), but every call
raises: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

from . import build as _build

LSO_OK, LSO_E_INVALID, LSO_E_ALIGN, LSO_E_DTYPE, LSO_E_OVERLAP = 0, 1, 2, 3, 4
LSO_E_NOMEM, LSO_E_HIP, LSO_E_CALLBACK, LSO_E_IO = 5, 6, 7, 8
LSO_DT_NONE, LSO_DT_F32, LSO_DT_BF16 = 0, 1, 2
LSO_OPT_ADAM, LSO_OPT_SGD = 0, 1
LSO_LAYOUT_PLANAR, LSO_LAYOUT_TILED = 0, 1
LSO_TILE_ELEMS = 8192
LSO_FILE_SYNC = 1
LSO_FILE_SHADOW = 2
LSO_SHADOW_HEADER_BYTES = 8192
LSO_NOALLOC_MAX_BLOCKS = 4096
LSO_COPY_SDMA_PAIR, LSO_COPY_DMA_IN, LSO_COPY_KERNELS, LSO_COPY_DMA = 0, 1, 2, 3
COPY_MODE_NAMES = {LSO_COPY_SDMA_PAIR: "sdma-pair", LSO_COPY_DMA_IN: "dma-in", LSO_COPY_KERNELS: "kernel",
                   LSO_COPY_DMA: "dma"}

STATUS_NAMES = {0: "LSO_OK", 1: "LSO_E_INVALID", 2: "LSO_E_ALIGN", 3: "LSO_E_DTYPE",
                4: "LSO_E_OVERLAP", 5: "LSO_E_NOMEM", 6: "LSO_E_HIP", 7: "LSO_E_CALLBACK",
                8: "LSO_E_IO"}


class LsoBlock(ctypes.Structure):
    _fields_ = [
        ("base", ctypes.c_void_p),
        ("n", ctypes.c_uint64),
        ("off_master", ctypes.c_uint64),
        ("off_m", ctypes.c_uint64),
        ("off_v", ctypes.c_uint64),
        ("off_grad", ctypes.c_uint64),
        ("off_weight", ctypes.c_uint64),
        ("grad_dtype", ctypes.c_uint32),
        ("weight_dtype", ctypes.c_uint32),
        ("opt", ctypes.c_uint32),
        ("layout", ctypes.c_uint32),
        ("t", ctypes.c_uint64),
        ("lr", ctypes.c_double),
        ("beta1", ctypes.c_double),
        ("beta2", ctypes.c_double),
        ("eps", ctypes.c_double),
    ]


class LsoHostLayer(ctypes.Structure):
    _fields_ = [
        ("host_base", ctypes.c_void_p),
        ("bytes", ctypes.c_uint64),
        ("n", ctypes.c_uint64),
        ("off_master", ctypes.c_uint64),
        ("off_m", ctypes.c_uint64),
        ("off_v", ctypes.c_uint64),
        ("dev_weight", ctypes.c_void_p),
        ("opt", ctypes.c_uint32),
        ("layout", ctypes.c_uint32),
        ("t", ctypes.c_uint64),
        ("lr", ctypes.c_double),
        ("beta1", ctypes.c_double),
        ("beta2", ctypes.c_double),
        ("eps", ctypes.c_double),
        ("sq_norm", ctypes.c_void_p),
        ("grad_dtype", ctypes.c_uint32),
        ("reserved", ctypes.c_uint32),
    ]


class LsoFileLayer(ctypes.Structure):
    _fields_ = [
        ("fd", ctypes.c_int),
        ("flags", ctypes.c_uint32),
        ("file_offset", ctypes.c_uint64),
        ("bytes", ctypes.c_uint64),
        ("n", ctypes.c_uint64),
        ("off_master", ctypes.c_uint64),
        ("off_m", ctypes.c_uint64),
        ("off_v", ctypes.c_uint64),
        ("dev_weight", ctypes.c_void_p),
        ("opt", ctypes.c_uint32),
        ("layout", ctypes.c_uint32),
        ("t", ctypes.c_uint64),
        ("lr", ctypes.c_double),
        ("beta1", ctypes.c_double),
        ("beta2", ctypes.c_double),
        ("eps", ctypes.c_double),
        ("sq_norm", ctypes.c_void_p),
        ("grad_dtype", ctypes.c_uint32),
        ("reserved", ctypes.c_uint32),
    ]


GRAD_FN = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                           ctypes.c_uint64, ctypes.c_void_p)

# every symbol include/lso.h declares
EXPORTS = ("lso_adam_step", "lso_adam_step_noalloc", "lso_norm_workspace_bytes", "lso_adam_step_norms", "lso_validate_blocks",
           "lso_block_constants", "lso_kernel_launches", "lso_tiled_state_bytes",
           "lso_tiled_pack", "lso_tiled_unpack", "lso_stream_create", "lso_stream_layers",
           "lso_stream_files", "lso_shadow_format", "lso_shadow_state", "lso_shadow_commit",
           "lso_stream_copy_mode", "lso_stream_stats", "lso_stream_slot_weight", "lso_stream_destroy", "lso_host_alloc",
           "lso_host_free", "lso_status_string", "lso_last_error")

_lib = None
_probes = None


class LsoError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {detail}")


def lib():
    """The loaded liblso.so (raises if it was never built)."""
    global _lib
    if _lib is None:
        path = _build.lib_path("liblso.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                               "(no CPU fallback exists)")
        L = ctypes.CDLL(path)
        vp, sz, u64, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint64, ctypes.c_int
        L.lso_adam_step.argtypes = [vp, sz, vp]
        L.lso_adam_step_noalloc.argtypes = [vp, sz, vp]
        L.lso_norm_workspace_bytes.argtypes = [vp, sz]
        L.lso_norm_workspace_bytes.restype = u64
        L.lso_adam_step_norms.argtypes = [vp, sz, vp, vp, u64, vp]
        L.lso_validate_blocks.argtypes = [vp, sz]
        L.lso_block_constants.argtypes = [vp, ctypes.POINTER(ctypes.c_float)]
        L.lso_kernel_launches.argtypes = []
        L.lso_kernel_launches.restype = u64
        L.lso_tiled_state_bytes.argtypes = [u64]
        L.lso_tiled_state_bytes.restype = u64
        L.lso_tiled_pack.argtypes = [vp, vp, vp, vp, u64, vp]
        L.lso_tiled_unpack.argtypes = [vp, vp, vp, vp, u64, vp]
        L.lso_stream_create.argtypes = [u64, u64, vp, vp, i32, ctypes.POINTER(vp)]
        L.lso_stream_layers.argtypes = [vp, vp, sz]
        L.lso_stream_files.argtypes = [vp, vp, sz]
        L.lso_shadow_format.argtypes = [i32, u64, u64, u64]
        L.lso_shadow_state.argtypes = [i32, u64, u64, ctypes.POINTER(u64), ctypes.POINTER(u64),
                                       ctypes.POINTER(u64)]
        L.lso_shadow_commit.argtypes = [i32, u64, u64, u64, u64]
        L.lso_stream_copy_mode.argtypes = [vp, ctypes.POINTER(ctypes.c_uint32), ctypes.POINTER(ctypes.c_uint32)]
        L.lso_stream_copy_mode.restype = i32
        L.lso_stream_stats.argtypes = [vp, ctypes.POINTER(u64)]
        L.lso_stream_stats.restype = i32
        L.lso_stream_slot_weight.argtypes = [vp, i32]
        L.lso_stream_slot_weight.restype = vp
        L.lso_stream_destroy.argtypes = [vp]
        L.lso_host_alloc.argtypes = [u64, ctypes.POINTER(vp)]
        L.lso_host_free.argtypes = [vp]
        L.lso_status_string.argtypes = [i32]
        L.lso_status_string.restype = ctypes.c_char_p
        L.lso_last_error.argtypes = []
        L.lso_last_error.restype = ctypes.c_char_p
        for name in ("lso_adam_step", "lso_adam_step_noalloc", "lso_adam_step_norms", "lso_validate_blocks", "lso_block_constants",
                     "lso_tiled_pack", "lso_tiled_unpack", "lso_stream_create",
                     "lso_stream_layers", "lso_stream_files", "lso_shadow_format", "lso_shadow_state",
                     "lso_shadow_commit", "lso_stream_destroy", "lso_host_alloc", "lso_host_free"):
            getattr(L, name).restype = i32
        _lib = L
    return _lib


def probes():
    global _probes
    if _probes is None:
        path = _build.lib_path("liblso_probes.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build()")
        P = ctypes.CDLL(path)
        vp, u64, u32 = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32
        P.lso_probe_copy.argtypes = [vp, vp, u64, ctypes.c_uint, vp]
        P.lso_probe_copy.restype = ctypes.c_int
        P.lso_probe_copy_variant.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, u64, vp]
        P.lso_probe_copy_variant.restype = ctypes.c_int
        P.lso_probe_copy_shaped_cpol.argtypes = [vp, vp, vp, u64, ctypes.c_int, vp]
        P.lso_probe_copy_shaped_cpol.restype = ctypes.c_int
        P.lso_probe_copy_shaped.argtypes = [vp, vp, vp, u64, ctypes.c_int, vp]
        P.lso_probe_copy_shaped.restype = ctypes.c_int
        P.lso_probe_link_sdma.argtypes = [u64, ctypes.c_int, ctypes.POINTER(ctypes.c_uint32),
                                          ctypes.POINTER(ctypes.c_double)]
        P.lso_probe_link_sdma.restype = ctypes.c_int
        P.lso_probe_bf16_rne.argtypes = [u32, u64, vp, vp]
        P.lso_probe_bf16_rne.restype = ctypes.c_int
        P.lso_probe_sqrt.argtypes = [u32, u64, vp, vp]
        P.lso_probe_sqrt.restype = ctypes.c_int
        P.lso_probe_link.argtypes = [u64, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
        P.lso_probe_link.restype = ctypes.c_int
        P.lso_probe_link_mode.argtypes = [u64, ctypes.c_int, ctypes.c_int, ctypes.c_uint,
                                          ctypes.POINTER(ctypes.c_double)]
        P.lso_probe_link_mode.restype = ctypes.c_int
        P.lso_probe_file.argtypes = [ctypes.c_int, u64, u64, u64, ctypes.c_int,
                                     ctypes.POINTER(ctypes.c_double)]
        P.lso_probe_file.restype = ctypes.c_int
        _probes = P
    return _probes


def check(status: int, where: str) -> None:
    if status != LSO_OK:
        detail = lib().lso_last_error().decode(errors="replace")
        raise LsoError(status, where, detail)
