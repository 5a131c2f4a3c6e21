"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This package holds none of the optimizer's arithmetic.  It maps
(seed, stream, block, purpose, step, element index) to numbers with the
counter-based generator Philox4x32-10 (Salmon et al., SC'11), so any
element of any step can be regenerated on its own -- which is what lets a
sampled check of a 100 GB state rebuild just the elements it looks at.

Two implementations of the same published generator exist: ``synth_host.c``
(host, feeds the oracle) and ``csrc/synth_fill.hip`` (device, fills GPU
buffers, and stands in for the backward pass that would produce the
gradients).  A GPU test checks them against each other bit for bit.

Recipe (all configs): key = (seed, stream) with seed 1234 and stream the
workload number; counter = (index lo, index hi, block, purpose<<24 | step).
Purposes: 0 FP32 master init, 1 LoRA-A init, 2 BF16 gradients (redrawn per
step), 3 edge-case values (the raw Philox words mapped to subnormals, the
smallest normals, signed zeros and ordinary values; host side only).  A normal deviate is the centred Irwin-Hall sum of the eight 16-bit
halves of one Philox output times one FP32 scale; BF16 values are the
truncated upper half of that FP32 pattern.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
import threading

import numpy as np

SEED = 1234
PURPOSE_MASTER = 0
PURPOSE_LORA_A = 1
PURPOSE_GRAD = 2
PURPOSE_EDGE = 3   # values at the low end of the binary32 range (edge-case tests)

# standard deviation of the sum of eight independent uniform 16-bit integers
_IH8_SD = math.sqrt(8.0 * (65536.0 ** 2 - 1.0) / 12.0)

_HERE = os.path.dirname(os.path.abspath(__file__))
_HOST_SRC = os.path.join(_HERE, "synth_host.c")
_HOST_LIB = os.path.join(_HERE, "libsynth_host.so")
_DEV_SRC = os.path.join(_HERE, "csrc", "synth_fill.hip")
_DEV_LIB = os.path.join(_HERE, "libsynth_fill.so")
_lock = threading.Lock()
_host = None
_dev = None


def scale_for(sigma: float) -> float:
    """FP32 multiplier that turns the centred integer sum into N(0, sigma)."""
    return float(np.float32(sigma / _IH8_SD))


# ---------------------------------------------------------------- building

HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
               "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build_host() -> str:
    tmp = _HOST_LIB + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-shared", "-fPIC",
                           _HOST_SRC, "-o", tmp])
    os.replace(tmp, _HOST_LIB)
    return _HOST_LIB


def build_device() -> str:
    tmp = _DEV_LIB + ".tmp"
    subprocess.check_call(["/opt/rocm/bin/hipcc", *HIPCC_FLAGS, _DEV_SRC, "-o", tmp])
    os.replace(tmp, _DEV_LIB)
    return _DEV_LIB


def build() -> None:
    build_host()
    build_device()


# ----------------------------------------------------------------- host side

def _host_lib():
    global _host
    with _lock:
        if _host is None:
            if not os.path.exists(_HOST_LIB):
                build_host()
            lib = ctypes.CDLL(_HOST_LIB)
            vp, u64, u32, f32 = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_float
            lib.synth_philox4x32_10.argtypes = [vp, vp, vp]
            lib.synth_philox4x32_10.restype = None
            for name in ("synth_normal_f32", "synth_normal_bf16"):
                f = getattr(lib, name)
                f.argtypes = [vp, u64, u64, u32, u32, u32, u32, u32, f32]
                f.restype = None
            for name in ("synth_normal_f32_at", "synth_normal_bf16_at"):
                f = getattr(lib, name)
                f.argtypes = [vp, vp, u64, u32, u32, u32, u32, u32, f32]
                f.restype = None
            lib.synth_philox_words.argtypes = [vp, u64, u64, u32, u32, u32, u32, u32]
            lib.synth_philox_words.restype = None
            _host = lib
        return _host


def philox4x32_10(counter, key) -> list[int]:
    c = (ctypes.c_uint32 * 4)(*[int(x) & 0xFFFFFFFF for x in counter])
    k = (ctypes.c_uint32 * 2)(*[int(x) & 0xFFFFFFFF for x in key])
    o = (ctypes.c_uint32 * 4)()
    _host_lib().synth_philox4x32_10(c, k, o)
    return list(o)


def normal_f32(n: int, *, stream: int, block: int, purpose: int, step: int, sigma: float,
               start: int = 0, seed: int = SEED) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    _host_lib().synth_normal_f32(out.ctypes.data, start, n, seed, stream, block, purpose, step,
                                 scale_for(sigma))
    return out


def normal_bf16(n: int, *, stream: int, block: int, purpose: int, step: int, sigma: float,
                start: int = 0, seed: int = SEED) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    _host_lib().synth_normal_bf16(out.ctypes.data, start, n, seed, stream, block, purpose, step,
                                  scale_for(sigma))
    return out


def normal_f32_at(idx: np.ndarray, *, stream: int, block: int, purpose: int, step: int,
                  sigma: float, seed: int = SEED) -> np.ndarray:
    idx = np.ascontiguousarray(idx, dtype=np.uint64)
    out = np.empty(idx.size, dtype=np.float32)
    _host_lib().synth_normal_f32_at(out.ctypes.data, idx.ctypes.data, idx.size, seed, stream,
                                    block, purpose, step, scale_for(sigma))
    return out


def normal_bf16_at(idx: np.ndarray, *, stream: int, block: int, purpose: int, step: int,
                   sigma: float, seed: int = SEED) -> np.ndarray:
    idx = np.ascontiguousarray(idx, dtype=np.uint64)
    out = np.empty(idx.size, dtype=np.uint16)
    _host_lib().synth_normal_bf16_at(out.ctypes.data, idx.ctypes.data, idx.size, seed, stream,
                                     block, purpose, step, scale_for(sigma))
    return out


def philox_words(n: int, *, stream: int, block: int, purpose: int, step: int, start: int = 0,
                 seed: int = SEED) -> np.ndarray:
    """The raw Philox output of indices start .. start + n - 1: shape (n, 4)."""
    out = np.empty((n, 4), dtype=np.uint32)
    _host_lib().synth_philox_words(out.ctypes.data, start, n, seed, stream, block, purpose, step)
    return out


def edge_f32(n: int, *, stream: int, block: int, step: int, positive: bool = False,
             seed: int = SEED) -> np.ndarray:
    """FP32 values at the low end of the binary32 range.  By the first
    Philox word of each element, mod 4: a subnormal (exponent field 0,
    non-zero fraction), a value in one of the eight smallest normal binades
    (exponent field 1..8), zero, or an ordinary value in [2^-8, 2^-5).  The
    fraction comes from the second word, the sign from the third (none when
    positive)."""
    w = philox_words(n, stream=stream, block=block, purpose=PURPOSE_EDGE, step=step, seed=seed)
    cls = w[:, 0] & 3
    frac = w[:, 1] & 0x7FFFFF
    frac = np.where(cls == 0, np.maximum(frac, 1), np.where(cls == 2, 0, frac))
    w3 = w[:, 3].astype(np.int64)
    exp = np.select([cls == 0, cls == 1, cls == 2], [0, 1 + (w3 & 7), 0], 119 + w3 % 3)
    sign = np.zeros(n, np.uint32) if positive else w[:, 2] >> 31
    bits = (sign << 31) | (exp.astype(np.uint32) << 23) | frac.astype(np.uint32)
    return bits.astype(np.uint32).view(np.float32)


def edge_bf16(n: int, *, stream: int, block: int, step: int, seed: int = SEED) -> np.ndarray:
    """BF16 gradient patterns at the low end of the range.  By the first
    Philox word, mod 4: a BF16 subnormal (exponent field 0, non-zero
    fraction), a normal whose square lies below the FP32 normal range
    (exponent field 47..62: 2^-80 .. 2^-65), zero, or an ordinary gradient
    (exponent field 115..118: 2^-12 .. 2^-9).  Fraction from the second
    word, sign from the third."""
    w = philox_words(n, stream=stream, block=block, purpose=PURPOSE_EDGE, step=step, seed=seed)
    cls = w[:, 0] & 3
    frac = w[:, 1] & 0x7F
    frac = np.where(cls == 0, np.maximum(frac, 1), np.where(cls == 2, 0, frac))
    w3 = w[:, 3].astype(np.int64)
    exp = np.select([cls == 0, cls == 1, cls == 2], [0, 47 + (w3 & 15), 0], 115 + (w3 & 3))
    bits = ((w[:, 2] >> 31) << 15) | (exp.astype(np.uint32) << 7) | frac.astype(np.uint32)
    return bits.astype(np.uint16)


# --------------------------------------------------------------- device side

class _FillParams(ctypes.Structure):
    """Mirror of synth_fill_params in csrc/synth_fill.hip."""
    _fields_ = [("seed", ctypes.c_uint32), ("stream", ctypes.c_uint32),
                ("purpose", ctypes.c_uint32), ("step", ctypes.c_uint32),
                ("scale", ctypes.c_float), ("block_base", ctypes.c_uint32)]


def _dev_lib():
    global _dev
    with _lock:
        if _dev is None:
            if not os.path.exists(_DEV_LIB):
                raise RuntimeError(f"device input generator not built: {_DEV_LIB} "
                                   "(run __graft_entry__.build())")
            lib = ctypes.CDLL(_DEV_LIB)
            vp, u64, u32, f32, i32 = (ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32,
                                      ctypes.c_float, ctypes.c_int)
            for name in ("synth_fill_normal_f32", "synth_fill_normal_bf16"):
                f = getattr(lib, name)
                f.argtypes = [vp, u64, u64, u32, u32, u32, u32, u32, f32, vp]
                f.restype = i32
            lib.synth_fill_zero.argtypes = [vp, u64, vp]
            lib.synth_fill_zero.restype = i32
            _dev = lib
        return _dev


def device_fill_normal_f32(ptr: int, n: int, *, stream: int, block: int, purpose: int,
                           step: int, sigma: float, start: int = 0, seed: int = SEED,
                           hip_stream: int = 0) -> None:
    rc = _dev_lib().synth_fill_normal_f32(ptr, n, start, seed, stream, block, purpose, step,
                                          scale_for(sigma), hip_stream)
    if rc != 0:
        raise RuntimeError(f"synth_fill_normal_f32 failed ({rc})")


def device_fill_normal_bf16(ptr: int, n: int, *, stream: int, block: int, purpose: int,
                            step: int, sigma: float, start: int = 0, seed: int = SEED,
                            hip_stream: int = 0) -> None:
    rc = _dev_lib().synth_fill_normal_bf16(ptr, n, start, seed, stream, block, purpose, step,
                                           scale_for(sigma), hip_stream)
    if rc != 0:
        raise RuntimeError(f"synth_fill_normal_bf16 failed ({rc})")


def device_fill_zero(ptr: int, nbytes: int, hip_stream: int = 0) -> None:
    rc = _dev_lib().synth_fill_zero(ptr, nbytes, hip_stream)
    if rc != 0:
        raise RuntimeError(f"synth_fill_zero failed ({rc})")


def grad_callback(f32: bool = False):
    """(C function pointer, params struct) for the device gradient producer
    that a layer stream calls once per layer: it fills that layer's BF16
    gradient buffer (FP32 with ``f32``) with purpose-2 deviates for block =
    block_base + layer.  Set ``params.step`` before each streamed step."""
    lib = _dev_lib()
    fn = ctypes.cast(lib.synth_grad_fn_f32 if f32 else lib.synth_grad_fn, ctypes.c_void_p).value
    return fn, _FillParams


def library_path() -> str:
    return _DEV_LIB
