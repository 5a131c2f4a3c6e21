"""Progressive layer locking on top of the layer stream and the resident
update.

The frozen-incremental page (section "Progressive Layer Locking") locks a
layer once its gradient magnitude falls below a threshold; a locked layer
gets no gradient computation, no update and no I/O, and compute moves to
the layers still learning.  Its section "The Math" adds that per-layer
steps keep Adam's bias correction exact for a layer that is locked and
later resumed.

This class is the policy only (host bookkeeping, a few comparisons per
step).  The library does the work: a layer passed with n = 0 is skipped
entirely by lso_stream_layers / lso_stream_files (no transfer, no producer
call, no update, no write-back) and is a no-op block for lso_adam_step; the
gradient norms come from the update's own pass over the gradients
(sq_norm fields, lso_adam_step_norms).

Readings: the magnitude is the Euclidean norm of the layer's whole
gradient; a layer is locked after the step whose gradient norm is below the
threshold (that step's update is applied); each layer's t counts the
updates applied to it, so a resumed layer continues its own bias
correction.
"""
from __future__ import annotations

import numpy as np


class ProgressiveLocking:
    def __init__(self, n_layers: int, threshold: float):
        if threshold < 0:
            raise ValueError("threshold must be >= 0")
        self.threshold = float(threshold)
        self.t = np.zeros(n_layers, np.uint64)        # updates applied per layer
        self.locked = np.zeros(n_layers, bool)
        self.norm = np.full(n_layers, np.nan)         # last gradient norm seen per layer
        self._sq = np.full(n_layers, np.nan)          # filled by the library
        self._active = None

    # ------------------------------------------------------------ tables

    def prepare(self, layers: np.ndarray) -> np.ndarray:
        """The step's lso_host_layer / lso_file_layer table: a copy of
        `layers` (every layer, in order) with locked layers at n = 0, each
        active layer at its own next t, and its sq_norm pointed at this
        object's buffer."""
        if len(layers) != self.t.size:
            raise ValueError(f"expected {self.t.size} layers, got {len(layers)}")
        out = layers.copy()
        self._active = ~self.locked
        self._sq[:] = np.nan
        out["n"][self.locked] = 0
        out["t"] = np.where(self._active, self.t + 1, out["t"])
        base = self._sq.ctypes.data
        out["sq_norm"] = [base + 8 * i if a else 0 for i, a in enumerate(self._active)]
        return out

    def prepare_blocks(self, arr: np.ndarray) -> np.ndarray:
        """The same for an lso_block array (one block per layer) passed to
        lso_adam_step_norms; the norms then come back through commit(sq)."""
        if len(arr) != self.t.size:
            raise ValueError(f"expected {self.t.size} blocks, got {len(arr)}")
        out = arr.copy()
        self._active = ~self.locked
        out["n"][self.locked] = 0
        out["t"] = np.where(self._active, self.t + 1, out["t"])
        return out

    # ------------------------------------------------------------ results

    def commit(self, sq: np.ndarray | None = None) -> list[int]:
        """After a successful call: advance t of the layers that were
        updated, record their gradient norms and lock those below the
        threshold.  sq: the sums of g^2 per layer (resident path); the
        streamed path fills them itself.  Returns the layers locked now."""
        if self._active is None:
            raise RuntimeError("commit() without prepare()")
        a = self._active
        sq = self._sq if sq is None else np.asarray(sq, np.float64)
        if np.any(np.isnan(sq[a])):
            raise RuntimeError("a layer that was updated returned no gradient norm")
        self.t[a] += 1
        self.norm[a] = np.sqrt(sq[a])
        newly = a & (self.norm < self.threshold)
        self.locked |= newly
        self._active = None
        return [int(i) for i in np.flatnonzero(newly)]

    def unlock(self, layer: int) -> None:
        """Resume a locked layer; it continues from its own t."""
        self.locked[layer] = False

    def lock(self, layer: int) -> None:
        self.locked[layer] = True

    @property
    def active(self) -> list[int]:
        return [int(i) for i in np.flatnonzero(~self.locked)]

    def state(self) -> dict:
        """What a checkpoint keeps beside the state: per-layer t and locks."""
        return dict(t=[int(x) for x in self.t], locked=[bool(x) for x in self.locked],
                    threshold=self.threshold)

    @classmethod
    def from_state(cls, st: dict) -> "ProgressiveLocking":
        obj = cls(len(st["t"]), st["threshold"])
        obj.t[:] = st["t"]
        obj.locked[:] = st["locked"]
        return obj
