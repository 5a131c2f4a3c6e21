"""Reference oracle for the per-layer mixed-precision Adam update.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  It wraps the plain C
definition in ``adam_oracle.c`` (FP64 arithmetic, FP32 state, BF16 round to
nearest even), which shares nothing with the HIP library.  The product path
never calls it and has no CPU fallback.

Pins that tie it to the pages and to mathematics live in
``tests/test_oracle_pins.py``; every function here is pinned there.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "adam_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liblso_oracle.so")
# A test of the pins themselves points this at a deliberately broken build.
_OVERRIDE = os.environ.get("LSO_ORACLE_LIB")
_lib = None
_lock = threading.Lock()

# Contraction off: each C operator is one rounding.  No fast-math, so no
# flush-to-zero and no reassociation.
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC", "-pthread"]


def build() -> str:
    """Compile the oracle library with gcc (always recompiles)."""
    tmp = _LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = _OVERRIDE or _LIB_PATH
        if not _OVERRIDE and not os.path.exists(path):
            build()
        lib = ctypes.CDLL(path)
        u64, f32p, u16p, dbl, i32 = (ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_double, ctypes.c_int)
        lib.lso_oracle_adam.argtypes = [u64, f32p, f32p, f32p, u16p, u16p, u64,
                                        dbl, dbl, dbl, dbl, i32]
        lib.lso_oracle_adam.restype = i32
        lib.lso_oracle_adam_g32.argtypes = lib.lso_oracle_adam.argtypes
        lib.lso_oracle_adam_g32.restype = i32
        lib.lso_oracle_sgd.argtypes = [u64, f32p, u16p, u16p, dbl, i32]
        lib.lso_oracle_sgd.restype = i32
        lib.lso_oracle_sgd_g32.argtypes = lib.lso_oracle_sgd.argtypes
        lib.lso_oracle_sgd_g32.restype = i32
        lib.lso_oracle_accumulate_f32.argtypes = [u64, f32p, f32p]
        lib.lso_oracle_accumulate_f32.restype = i32
        lib.lso_oracle_sq_norm.argtypes = [u64, u16p, f32p]
        lib.lso_oracle_sq_norm.restype = dbl
        lib.lso_oracle_bf16_rne.argtypes = [ctypes.c_float]
        lib.lso_oracle_bf16_rne.restype = ctypes.c_uint16
        lib.lso_oracle_bf16_rne_array.argtypes = [f32p, u16p, u64]
        lib.lso_oracle_bf16_rne_array.restype = None
        _lib = lib
        return lib


def _ptr(a: np.ndarray | None):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _check(a: np.ndarray, dtype, n: int, name: str):
    if a.dtype != dtype or not a.flags.c_contiguous or a.size != n:
        raise ValueError(f"{name}: need contiguous {dtype} of {n} elements, got {a.dtype} {a.shape}")


def adam_step(master: np.ndarray, m: np.ndarray, v: np.ndarray, g_bits: np.ndarray,
              w_bits: np.ndarray | None, t: int, lr: float, beta1: float, beta2: float,
              eps: float, threads: int = 0) -> int:
    """One Adam step in place (frozen-incremental page, section "The Math").

    master, m, v: float32 state, updated in place.  g_bits: uint16 BF16
    gradient patterns, or float32 gradients (the LoRA article's FP32 adapter
    gradients).  w_bits: uint16 output for the BF16 re-cast of the new
    master, or None.  Returns the number of host threads used.
    """
    n = master.size
    _check(master, np.float32, n, "master")
    _check(m, np.float32, n, "m")
    _check(v, np.float32, n, "v")
    g32 = g_bits.dtype == np.float32
    _check(g_bits, np.float32 if g32 else np.uint16, n, "g")
    if w_bits is not None:
        _check(w_bits, np.uint16, n, "w")
    lib = _load()
    fn = lib.lso_oracle_adam_g32 if g32 else lib.lso_oracle_adam
    rc = fn(n, _ptr(master), _ptr(m), _ptr(v), _ptr(g_bits), _ptr(w_bits),
            int(t), float(lr), float(beta1), float(beta2), float(eps), int(threads))
    if rc < 0:
        raise ValueError("oracle rejected the arguments (t must be >= 1)")
    return rc


def sgd_step(master: np.ndarray, g_bits: np.ndarray, w_bits: np.ndarray | None, lr: float,
             subtractive: bool = False) -> None:
    """One plain gradient-descent step in FP32, additive (default) or
    subtractive spelling (frozen-incremental page, "The Assumption Everyone
    Makes").  g_bits: uint16 BF16 patterns or float32 gradients."""
    n = master.size
    _check(master, np.float32, n, "master")
    g32 = g_bits.dtype == np.float32
    _check(g_bits, np.float32 if g32 else np.uint16, n, "g")
    if w_bits is not None:
        _check(w_bits, np.uint16, n, "w")
    lib = _load()
    fn = lib.lso_oracle_sgd_g32 if g32 else lib.lso_oracle_sgd
    fn(n, _ptr(master), _ptr(g_bits), _ptr(w_bits), float(lr), 1 if subtractive else 0)


def accumulate_f32(w: np.ndarray, delta: np.ndarray) -> None:
    """w += delta in FP32 (the page's frozen-storage write-back on its own)."""
    n = w.size
    _check(w, np.float32, n, "w")
    _check(delta, np.float32, n, "delta")
    _load().lso_oracle_accumulate_f32(n, _ptr(w), _ptr(delta))


def sq_norm(g: np.ndarray) -> float:
    """Squared L2 norm of a gradient (uint16 BF16 patterns or float32), FP64
    in index order: the magnitude that progressive layer locking compares
    with its threshold (frozen-incremental page, "Progressive Layer
    Locking")."""
    g = np.ascontiguousarray(g)
    if g.dtype == np.uint16:
        return float(_load().lso_oracle_sq_norm(g.size, _ptr(g), None))
    if g.dtype == np.float32:
        return float(_load().lso_oracle_sq_norm(g.size, None, _ptr(g)))
    raise ValueError(f"gradient must be uint16 (BF16) or float32, got {g.dtype}")


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """BF16 round-to-nearest-even bit patterns (uint16) of float32 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().lso_oracle_bf16_rne_array(_ptr(x), _ptr(out), x.size)
    return out


def bf16_rne_scalar(x: float) -> int:
    return int(_load().lso_oracle_bf16_rne(ctypes.c_float(x)))
