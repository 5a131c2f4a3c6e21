"""The disk tier's files: one preallocated file per layer plus a manifest.

The frozen-incremental page ("Training 70B Models on Consumer Hardware",
sections "Storage" and "Training Loop") keeps each layer's W, M and V in
files on an SSD and updates them one layer at a time; its "Limitations"
section asks for files preallocated contiguously (fragmented files slow
the reads to a crawl), and its section "The Math" keeps the global step t
beside the model state so a resumed run continues from it.

Here each layer's file holds the same block a host layer would: FP32
[master | m | v] with 4 KB-aligned sub-arrays, or one tiled region.  The
manifest (JSON, replaced atomically) records the geometry and the last
completed step t.  With shadow=True each file is a crash-consistent shadow
region instead (two data slots and two checksummed header copies, see
LSO_FILE_SHADOW in include/lso.h): the page's safety note asks for shadow
copies so that a crash mid-update leaves every layer wholly old or wholly
new, and each layer's header also records the t of its committed state.
This module only creates, opens and describes the files; every update
runs in liblso.so (lso_stream_files).
"""
from __future__ import annotations

import json
import mmap
import os

import numpy as np

from . import (FILE_LAYER_DTYPE, LSO_FILE_SHADOW, LSO_FILE_SYNC, LSO_LAYOUT_PLANAR, LSO_LAYOUT_TILED,
               LSO_OPT_ADAM, LSO_SHADOW_HEADER_BYTES, configs, shadow_format, shadow_state)

MANIFEST = "manifest.json"


def _fsync_dir(path: str) -> None:
    fd = os.open(path, os.O_RDONLY)
    try:
        os.fsync(fd)
    finally:
        os.close(fd)


class LayerFiles:
    """Per-layer state files in one directory.

    create() preallocates the files (posix_fallocate) and writes the
    manifest with t = 0; open() reopens them and reads t back.  direct=True
    opens the files with O_DIRECT, so reads and writes bypass the page cache
    and measure the storage itself.
    """

    def __init__(self, directory: str, sizes: list[int], tiled: bool, t: int, direct: bool,
                 shadow: bool = False):
        self.dir = directory
        self.sizes = list(sizes)
        self.tiled = tiled
        self.t = t
        self.direct = direct
        self.shadow = shadow
        self.geom = [configs.host_layer_layout(n, tiled=tiled) for n in self.sizes]
        self.fds: list[int] = []
        flags = os.O_RDWR | (os.O_DIRECT if direct else 0)
        for i in range(len(self.sizes)):
            self.fds.append(os.open(self.path(i), flags))

    # ------------------------------------------------------------ lifecycle

    def path(self, i: int) -> str:
        return os.path.join(self.dir, f"layer{i:04d}.state")

    @classmethod
    def create(cls, directory: str, sizes: list[int], tiled: bool = False, direct: bool = False,
               shadow: bool = False) -> "LayerFiles":
        os.makedirs(directory, exist_ok=True)
        for i, n in enumerate(sizes):
            nbytes = configs.host_layer_layout(n, tiled=tiled)[3]
            span = LSO_SHADOW_HEADER_BYTES + 2 * nbytes if shadow else nbytes
            fd = os.open(os.path.join(directory, f"layer{i:04d}.state"),
                         os.O_RDWR | os.O_CREAT | os.O_TRUNC, 0o644)
            try:
                os.posix_fallocate(fd, 0, span)   # zero-filled, allocated up front
                if shadow:
                    shadow_format(fd, 0, nbytes, 0)
            finally:
                os.close(fd)
        obj = cls(directory, sizes, tiled, 0, direct, shadow)
        obj.commit(0)
        return obj

    @classmethod
    def open(cls, directory: str, direct: bool = False) -> "LayerFiles":
        with open(os.path.join(directory, MANIFEST)) as f:
            man = json.load(f)
        return cls(directory, man["sizes"], man["layout"] == "tiled", int(man["t"]), direct,
                   bool(man.get("shadow", False)))

    def commit(self, t: int) -> None:
        """Record t as the last completed step: write a new manifest, flush
        it, rename it over the old one, flush the directory."""
        man = dict(version=1, t=int(t), sizes=self.sizes, shadow=self.shadow,
                   layout="tiled" if self.tiled else "planar",
                   files=[os.path.basename(self.path(i)) for i in range(len(self.sizes))],
                   bytes=[g[3] for g in self.geom])
        tmp = os.path.join(self.dir, MANIFEST + ".tmp")
        with open(tmp, "w") as f:
            json.dump(man, f)
            f.flush()
            os.fsync(f.fileno())
        os.replace(tmp, os.path.join(self.dir, MANIFEST))
        _fsync_dir(self.dir)
        self.t = int(t)

    def close(self) -> None:
        for fd in self.fds:
            os.close(fd)
        self.fds = []

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    # -------------------------------------------------------------- layers

    def bytes(self, i: int) -> int:
        return self.geom[i][3]

    def state(self, i: int) -> tuple[int, int, int]:
        """Shadow files: (epoch, t, data offset) of layer i's committed state;
        plain files: (0, manifest t, 0)."""
        if not self.shadow:
            return 0, self.t, 0
        return shadow_state(self.fds[i], 0, self.bytes(i))

    def _data_offset(self, i: int) -> int:
        return self.state(i)[2]

    def table(self, t: int, lr: float, beta1: float, beta2: float, eps: float,
              sync: bool = False, opt: int = LSO_OPT_ADAM, grad_dtype: int = 0) -> np.ndarray:
        """lso_file_layer rows for step t (grad_dtype: what the producer
        writes, LSO_DT_BF16 (0) or LSO_DT_F32)."""
        L = np.zeros(len(self.sizes), FILE_LAYER_DTYPE)
        for i, n in enumerate(self.sizes):
            om, omm, ov, nb = self.geom[i]
            L[i]["fd"] = self.fds[i]
            L[i]["flags"] = (LSO_FILE_SYNC if sync else 0) | (LSO_FILE_SHADOW if self.shadow else 0)
            L[i]["file_offset"], L[i]["bytes"], L[i]["n"] = 0, nb, n
            L[i]["off_master"], L[i]["off_m"], L[i]["off_v"] = om, omm, ov
            L[i]["opt"] = opt
            L[i]["layout"] = LSO_LAYOUT_TILED if self.tiled else LSO_LAYOUT_PLANAR
            L[i]["t"] = t
            L[i]["lr"], L[i]["beta1"], L[i]["beta2"], L[i]["eps"] = lr, beta1, beta2, eps
            L[i]["grad_dtype"] = grad_dtype
        return L

    def write_block(self, i: int, data) -> None:
        """Write a whole block (bytes-like of bytes(i) bytes) over the
        current state (shadow files: into the committed slot, for the
        initial state), through a page-aligned buffer (O_DIRECT needs one),
        and flush it."""
        nb = self.bytes(i)
        base = self._data_offset(i)
        buf = mmap.mmap(-1, nb)
        try:
            buf[:] = memoryview(data).cast("B")
            done = 0
            while done < nb:
                done += os.pwritev(self.fds[i], [memoryview(buf)[done:]], base + done)
            os.fdatasync(self.fds[i])
        finally:
            buf.close()

    def read_block(self, i: int) -> np.ndarray:
        """The whole block as uint8 (a copy); shadow files: the committed slot."""
        nb = self.bytes(i)
        base = self._data_offset(i)
        buf = mmap.mmap(-1, nb)
        try:
            done = 0
            while done < nb:
                k = os.preadv(self.fds[i], [memoryview(buf)[done:]], base + done)
                if k == 0:
                    raise EOFError(f"{self.path(i)} is shorter than its block")
                done += k
            return np.frombuffer(buf, dtype=np.uint8).copy()
        finally:
            buf.close()
