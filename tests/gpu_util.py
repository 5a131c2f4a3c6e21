"""Helpers for the GPU tests: device arenas with canary bands, transfers,
and the parity measures.  Test infrastructure only."""
from __future__ import annotations

import contextlib
import ctypes
import os
import sys

import numpy as np

import layer_streamed_optimizer_amd as lso
import synth
from layer_streamed_optimizer_amd import configs

CANARY = 0xA5
GUARD = 256


def log(*a):
    """Name the case before each GPU step (flushed, so a crash still shows it)."""
    print("[gpu-test]", *a, file=sys.stderr, flush=True)


def torch():
    import torch as _t
    return _t


def to_dev(a: np.ndarray):
    t = torch()
    a = np.ascontiguousarray(a)
    return t.from_numpy(a.view(np.uint8).copy()).to("cuda")


TILE = configs.TILE   # elements per tile of the tiled state layout


def tile_state(master, m, v):
    """Host reference of the tiled layout: [master | m | v] per TILE
    elements, zero padding after the last element."""
    n = master.size
    nt = (n + TILE - 1) // TILE
    reg = np.zeros((nt, 3, TILE), np.float32)
    for k, a in enumerate((master, m, v)):
        pad = np.zeros(nt * TILE, np.float32)
        pad[:n] = a
        reg[:, k, :] = pad.reshape(nt, TILE)
    return reg.ravel()


def detile_state(region, n):
    """(master, m, v) of the first n elements of a tiled region."""
    nt = (n + TILE - 1) // TILE
    reg = np.asarray(region, np.float32)[: nt * 3 * TILE].reshape(nt, 3, TILE)
    return tuple(reg[:, k, :].ravel()[:n].copy() for k in range(3))


class Arena:
    """Blocks' arrays in one device buffer, each array surrounded by canary
    bytes (every byte of the buffer outside an array is CANARY).  With
    tiled=True a block's master, m and v live in one tiled region; with
    grad_f32=True the gradients are FP32 instead of BF16."""

    def __init__(self, sizes, adam=True, weight=True, extra_align=0, tiled=False, grad_f32=False):
        t = torch()
        self.sizes = list(sizes)
        self.adam, self.weight, self.tiled, self.grad_f32 = adam, weight, tiled, grad_f32
        self.off, self.nbytes = [], []
        pos = GUARD
        if tiled:
            names = ["state", "grad"] + (["weight"] if weight else [])
        else:
            names = ["master", "grad"] + (["m", "v"] if adam else []) + (["weight"] if weight else [])
        self.names = names
        for n in self.sizes:
            d, nb = {}, {}
            for name in names:
                if name == "state":
                    size = 12 * TILE * ((n + TILE - 1) // TILE)
                else:
                    size = self.esize(name) * n
                d[name] = pos + extra_align
                nb[name] = size
                pos += extra_align + size
                pos = (pos + GUARD - 1) // GUARD * GUARD + GUARD
            self.off.append(d)
            self.nbytes.append(nb)
        self.total = pos
        self.buf = t.full((self.total,), CANARY, dtype=t.uint8, device="cuda")
        self.base = int(self.buf.data_ptr())

    def esize(self, name):
        if name == "grad":
            return 4 if self.grad_f32 else 2
        return 2 if name == "weight" else 4

    def _put_raw(self, i, name, raw_u8):
        t = torch()
        o = self.off[i][name]
        assert raw_u8.nbytes == self.nbytes[i][name]
        self.buf[o:o + raw_u8.nbytes].copy_(t.from_numpy(raw_u8.copy()))

    def put(self, i, name, arr):
        n = self.sizes[i]
        if self.tiled and name in ("master", "m", "v"):
            cur = list(self.get_state(i))
            cur[("master", "m", "v").index(name)] = np.ascontiguousarray(arr, np.float32)
            self._put_raw(i, "state", tile_state(*cur).view(np.uint8))
            return
        dt = np.uint16 if self.esize(name) == 2 else np.float32
        a = np.ascontiguousarray(arr, dtype=dt)
        assert a.size == n
        self._put_raw(i, name, a.view(np.uint8))

    def get_state(self, i):
        o = self.off[i]["state"]
        raw = self.buf[o:o + self.nbytes[i]["state"]].cpu().numpy().view(np.float32)
        return detile_state(raw, self.sizes[i])

    def get(self, i, name):
        if self.tiled and name in ("master", "m", "v"):
            return self.get_state(i)[("master", "m", "v").index(name)]
        n = self.sizes[i]
        o = self.off[i][name]
        es = self.esize(name)
        raw = self.buf[o:o + es * n].cpu().numpy()
        return raw.view(np.uint16 if es == 2 else np.float32).copy()

    def addr(self, i, name):
        return self.base + self.off[i][name]

    def rows(self, t=1, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, opt=lso.LSO_OPT_ADAM):
        out = []
        gd = lso.LSO_DT_F32 if self.grad_f32 else lso.LSO_DT_BF16
        for i, n in enumerate(self.sizes):
            if self.tiled:
                out.append(dict(n=n, master=self.addr(i, "state"), grad=self.addr(i, "grad"),
                                weight=self.addr(i, "weight") if self.weight else None,
                                t=t, lr=lr, beta1=beta1, beta2=beta2, eps=eps, opt=opt,
                                layout=lso.LSO_LAYOUT_TILED, grad_dtype=gd))
                continue
            out.append(dict(n=n, master=self.addr(i, "master"), grad=self.addr(i, "grad"),
                            m=self.addr(i, "m") if self.adam else None,
                            v=self.addr(i, "v") if self.adam else None,
                            weight=self.addr(i, "weight") if self.weight else None,
                            t=t, lr=lr, beta1=beta1, beta2=beta2, eps=eps, opt=opt, grad_dtype=gd))
        return out

    def table(self, **kw):
        return lso.BlockTable.from_rows(self.rows(**kw))

    def canaries_intact(self) -> bool:
        host = self.buf.cpu().numpy()
        mask = np.ones(self.total, bool)
        for i in range(len(self.sizes)):
            for name, o in self.off[i].items():
                mask[o:o + self.nbytes[i][name]] = False
        return bool(np.all(host[mask] == CANARY))


# ----------------------------------------------------------- parity measures

def rms(x) -> float:
    x = np.asarray(x, np.float64)
    return float(np.sqrt(np.mean(x * x))) if x.size else 0.0


def rel_err_rms_floor(got, ref, floor=None) -> float:
    """max_i |got - ref| / max(|ref_i|, floor), floor = rms(ref) unless
    given: relative error with an RMS floor, so a moment that cancels to ~0
    (m is an exponential average of signed gradients) is judged at the scale
    of its quantity rather than at its own vanishing magnitude.  Callers with
    tiny blocks pass the RMS of the quantity over the whole call."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    if floor is None:
        floor = rms(ref)
    den = np.maximum(np.abs(ref), floor)
    den[den == 0] = 1.0
    return float(np.max(np.abs(got - ref) / den))


def bf16_value(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32)


def bf16_ulp(ref_bits):
    """Spacing of BF16 numbers at each reference value."""
    v = np.abs(bf16_value(ref_bits)).astype(np.float64)
    e = np.floor(np.log2(np.maximum(v, 2.0 ** -133)))
    return 2.0 ** (np.maximum(e, -126) - 7)


def call_scale(refs: list) -> dict:
    """RMS of each FP32 quantity over every block of a call (the floor of
    blocks too small to have a meaningful RMS of their own)."""
    out = {}
    for q in ("master", "m", "v"):
        parts = [np.asarray(r[q], np.float64) for r in refs if q in r]
        if parts:
            out[q] = rms(np.concatenate(parts))
    return out


# A block's own RMS is its floor.  Only blocks of fewer elements than this
# take the RMS of the whole call instead: the RMS of one to a few dozen
# elements is itself one of the values being judged (a one-element m block
# that cancels to ~0 would have a floor of ~0).
SMALL_BLOCK = 64


def block_floor(ref_q, pooled: float | None) -> float:
    """The RMS floor of one block's quantity: its own RMS, or for blocks of
    fewer than SMALL_BLOCK elements the larger of that and the call's."""
    own = rms(ref_q)
    if pooled is None or np.asarray(ref_q).size >= SMALL_BLOCK:
        return own
    return max(own, pooled)


def assert_parity(got: dict, ref: dict, tol: float, what: str = "", scale: dict | None = None) -> dict:
    """FP32 state within tol (relative, floored at the block's own RMS;
    scale gives the call's RMS per quantity, used only for blocks of fewer
    than SMALL_BLOCK elements); BF16 weight within one BF16 ulp (or tol at
    the master's RMS) and equal to the RNE of the GPU's own master bit for
    bit.  Returns the block's errors (as max_errors)."""
    import oracle
    errs = max_errors(got, ref, scale, tol)
    for q in ("master", "m", "v"):
        if q in errs:
            assert errs[q] <= tol, f"{what}: {q} relative error {errs[q]:.3g} > {tol:g}"
    if "weight" in got and "weight" in ref:
        gw = got["weight"]
        assert np.array_equal(gw, oracle.bf16_rne(got["master"])), f"{what}: w != bf16_rne(master)"
        assert errs["weight_over_bound"] <= 1.0, \
            f"{what}: BF16 weights beyond one ulp (worst {errs['weight_over_bound']:.3g} of the bound)"
    return errs


def max_errors(got: dict, ref: dict, scale: dict | None = None, tol: float = 1e-6) -> dict:
    """Largest FP32 errors (as in assert_parity), and for the BF16 weight
    the largest |w - w_ref| over its bound max(1 ulp, tol * rms(master))
    (<= 1 passes) plus how many weights differ at all."""
    out = {q: rel_err_rms_floor(got[q], ref[q],
                                block_floor(ref[q], None if scale is None else scale.get(q)))
           for q in ("master", "m", "v") if q in got and q in ref}
    if "weight" in got and "weight" in ref:
        d = np.abs(bf16_value(got["weight"]).astype(np.float64) - bf16_value(ref["weight"]))
        bound = np.maximum(bf16_ulp(ref["weight"]), tol * rms(ref["master"]))
        out["weight_over_bound"] = float(np.max(d / bound)) if d.size else 0.0
        out["weight_differing"] = int(np.count_nonzero(d))
    return out


class Worst:
    """The worst error per quantity over the blocks of a call, and which
    block (by label) it came from, for the log."""

    def __init__(self):
        self.val, self.where = {}, {}

    def add(self, label, errs: dict):
        for k, v in errs.items():
            if v >= self.val.get(k, -1.0):
                self.val[k], self.where[k] = v, label
        return errs

    def __repr__(self):
        return ", ".join(f"{k} {self.val[k]:.3g} ({self.where[k]})" for k in sorted(self.val))


# ----------------------------------------------------------------- raw HIP

_hip = None


def hip():
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                        ctypes.c_int, ctypes.c_void_p]
        _hip.hipMemcpyAsync.restype = ctypes.c_int
    return _hip


HIP_D2D = 3


# ------------------------------------------------------------ layer stream

LR, B1, B2, EPS = configs.LR, configs.BETA1, configs.BETA2, configs.EPS


class _Pageable:
    """Ordinary (pageable) host memory with the HostBuffer interface."""

    def __init__(self, nbytes):
        self.arr = np.empty(nbytes + 64, np.uint8)
        shift = (-self.arr.ctypes.data) % 64
        self.ptr = self.arr.ctypes.data + shift
        self.nbytes = nbytes
        self._shift = shift

    def view(self, dtype=np.uint8, offset=0, count=None):
        dt = np.dtype(dtype)
        if count is None:
            count = (self.nbytes - offset) // dt.itemsize
        return self.arr[self._shift + offset:self._shift + offset + count * dt.itemsize].view(dt)


class HostLayers:
    """Authoritative host blocks, one per layer: [master | m | v] planar or
    one tiled region; pinned (lso_host_alloc) or pageable, per layer."""

    def __init__(self, sizes, sid, pageable=False, tiled=False):
        self.sizes = sizes
        self.tiled = tiled
        self.bufs, self.lay = [], []
        for b, n in enumerate(sizes):
            om, omm, ov, nbytes = configs.host_layer_layout(n, tiled=tiled)
            pg = pageable(b) if callable(pageable) else pageable
            hb = _Pageable(nbytes) if pg else lso.host_alloc(nbytes)
            hb.view(np.uint8)[:] = 0
            master = synth.normal_f32(n, stream=sid, block=b, purpose=0, step=0, sigma=0.02)
            if tiled:
                z = np.zeros(n, np.float32)
                reg = tile_state(master, z, z)
                hb.view(np.float32, om, reg.size)[:] = reg
            else:
                hb.view(np.float32, om, n)[:] = master
            self.bufs.append(hb)
            self.lay.append((om, omm, ov, nbytes))

    def raw(self, b):
        """The whole block's bytes (a copy)."""
        return self.bufs[b].view(np.uint8, 0, self.lay[b][3]).copy()

    def get(self, b, q):
        om, omm, ov, nbytes = self.lay[b]
        n = self.sizes[b]
        if self.tiled:
            reg = self.bufs[b].view(np.float32, om, (nbytes - om) // 4)
            return detile_state(reg, n)[("master", "m", "v").index(q)]
        off = {"master": om, "m": omm, "v": ov}[q]
        return self.bufs[b].view(np.float32, off, self.sizes[b]).copy()

    def table(self, t, opt=lso.LSO_OPT_ADAM, lr=LR, dev_weight=None, grad_dtype=0):
        L = lso.LayerStream.layers(len(self.sizes))
        for b, n in enumerate(self.sizes):
            om, omm, ov, nbytes = self.lay[b]
            L[b]["host_base"] = self.bufs[b].ptr
            L[b]["bytes"] = nbytes
            L[b]["n"] = n
            L[b]["off_master"], L[b]["off_m"], L[b]["off_v"] = om, omm, ov
            L[b]["dev_weight"] = dev_weight[b] if dev_weight else 0
            L[b]["opt"] = opt
            L[b]["layout"] = lso.LSO_LAYOUT_TILED if self.tiled else lso.LSO_LAYOUT_PLANAR
            L[b]["t"] = t
            L[b]["lr"], L[b]["beta1"], L[b]["beta2"], L[b]["eps"] = lr, B1, B2, EPS
            L[b]["grad_dtype"] = grad_dtype
        return L


def synth_stream(sizes, sid, max_bytes=None, f32=False):
    fn, Params = synth.grad_callback(f32)
    params = Params(seed=synth.SEED, stream=sid, purpose=synth.PURPOSE_GRAD, step=1,
                    scale=synth.scale_for(1e-3), block_base=0)
    mb = max_bytes or max(configs.host_layer_layout(n)[3] for n in sizes)
    ls = lso.LayerStream(mb, max(sizes), fn, ctypes.addressof(params))
    return ls, params


@contextlib.contextmanager
def stream_pieces(tiles: int):
    """Layer streams created inside move tiled layers in pieces of `tiles`
    state tiles (LSO_STREAM_PIECE_BYTES, read at context creation)."""
    old = os.environ.get("LSO_STREAM_PIECE_BYTES")
    os.environ["LSO_STREAM_PIECE_BYTES"] = str(tiles * 12 * TILE)
    try:
        yield
    finally:
        if old is None:
            del os.environ["LSO_STREAM_PIECE_BYTES"]
        else:
            os.environ["LSO_STREAM_PIECE_BYTES"] = old


@contextlib.contextmanager
def stream_env(**env):
    """Layer streams created inside see these LSO_STREAM_* variables (read at
    context creation), e.g. stream_env(COPY="kernel")."""
    old = {k: os.environ.get("LSO_STREAM_" + k) for k in env}
    for k, v in env.items():
        os.environ["LSO_STREAM_" + k] = str(v)
    try:
        yield
    finally:
        for k, v in old.items():
            if v is None:
                del os.environ["LSO_STREAM_" + k]
            else:
                os.environ["LSO_STREAM_" + k] = v
