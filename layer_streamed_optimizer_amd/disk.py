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
completed step t.  This module only creates, opens and describes the
files; every update runs in liblso.so (lso_stream_files).
"""
from __future__ import annotations

import json
import mmap
import os

import numpy as np

from . import FILE_LAYER_DTYPE, LSO_FILE_SYNC, LSO_LAYOUT_PLANAR, LSO_LAYOUT_TILED, LSO_OPT_ADAM
from . import configs

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

    def __init__(self, directory: str, sizes: list[int], tiled: bool, t: int, direct: bool):
        self.dir = directory
        self.sizes = list(sizes)
        self.tiled = tiled
        self.t = t
        self.direct = direct
        self.geom = [configs.host_layer_layout(n, tiled=tiled) for n in self.sizes]
        self.fds: list[int] = []
        flags = os.O_RDWR | (os.O_DIRECT if direct else 0)
        for i in range(len(self.sizes)):
            self.fds.append(os.open(self.path(i), flags))

    # ------------------------------------------------------------ lifecycle

    def path(self, i: int) -> str:
        return os.path.join(self.dir, f"layer{i:04d}.state")

    @classmethod
    def create(cls, directory: str, sizes: list[int], tiled: bool = False,
               direct: bool = False) -> "LayerFiles":
        os.makedirs(directory, exist_ok=True)
        for i, n in enumerate(sizes):
            nbytes = configs.host_layer_layout(n, tiled=tiled)[3]
            fd = os.open(os.path.join(directory, f"layer{i:04d}.state"),
                         os.O_RDWR | os.O_CREAT | os.O_TRUNC, 0o644)
            try:
                os.posix_fallocate(fd, 0, nbytes)   # zero-filled, allocated up front
            finally:
                os.close(fd)
        obj = cls(directory, sizes, tiled, 0, direct)
        obj.commit(0)
        return obj

    @classmethod
    def open(cls, directory: str, direct: bool = False) -> "LayerFiles":
        with open(os.path.join(directory, MANIFEST)) as f:
            man = json.load(f)
        return cls(directory, man["sizes"], man["layout"] == "tiled", int(man["t"]), direct)

    def commit(self, t: int) -> None:
        """Record t as the last completed step: write a new manifest, flush
        it, rename it over the old one, flush the directory."""
        man = dict(version=1, t=int(t), sizes=self.sizes,
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

    def table(self, t: int, lr: float, beta1: float, beta2: float, eps: float,
              sync: bool = False, opt: int = LSO_OPT_ADAM) -> np.ndarray:
        """lso_file_layer rows for step t."""
        L = np.zeros(len(self.sizes), FILE_LAYER_DTYPE)
        for i, n in enumerate(self.sizes):
            om, omm, ov, nb = self.geom[i]
            L[i]["fd"], L[i]["flags"] = self.fds[i], LSO_FILE_SYNC if sync else 0
            L[i]["file_offset"], L[i]["bytes"], L[i]["n"] = 0, nb, n
            L[i]["off_master"], L[i]["off_m"], L[i]["off_v"] = om, omm, ov
            L[i]["opt"] = opt
            L[i]["layout"] = LSO_LAYOUT_TILED if self.tiled else LSO_LAYOUT_PLANAR
            L[i]["t"] = t
            L[i]["lr"], L[i]["beta1"], L[i]["beta2"], L[i]["eps"] = lr, beta1, beta2, eps
        return L

    def write_block(self, i: int, data) -> None:
        """Write a whole block (bytes-like of bytes(i) bytes) at offset 0,
        through a page-aligned buffer (O_DIRECT needs one)."""
        nb = self.bytes(i)
        buf = mmap.mmap(-1, nb)
        try:
            buf[:] = memoryview(data).cast("B")
            done = 0
            while done < nb:
                done += os.pwritev(self.fds[i], [memoryview(buf)[done:]], done)
        finally:
            buf.close()

    def read_block(self, i: int) -> np.ndarray:
        """The whole block as uint8 (a copy)."""
        nb = self.bytes(i)
        buf = mmap.mmap(-1, nb)
        try:
            done = 0
            while done < nb:
                k = os.preadv(self.fds[i], [memoryview(buf)[done:]], done)
                if k == 0:
                    raise EOFError(f"{self.path(i)} is shorter than its block")
                done += k
            return np.frombuffer(buf, dtype=np.uint8).copy()
        finally:
            buf.close()
