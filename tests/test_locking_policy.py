"""The progressive-locking policy on the CPU (no device work): tables it
prepares, per-layer t, locks and resumes."""
import numpy as np
import pytest

import layer_streamed_optimizer_amd as lso
from layer_streamed_optimizer_amd.locking import ProgressiveLocking


def test_prepare_and_commit_lock_below_threshold():
    L = lso.LayerStream.layers(3)
    L["n"] = [10, 20, 30]
    p = ProgressiveLocking(3, threshold=0.5)
    tab = p.prepare(L)
    assert tab["n"].tolist() == [10, 20, 30] and tab["t"].tolist() == [1, 1, 1]
    assert all(tab["sq_norm"] != 0)
    p._sq[:] = [1.0, 0.01, 0.25]          # what the library writes: sums of g^2
    assert p.commit() == [1]               # norm 0.1 < 0.5; 0.5 is not below
    assert p.t.tolist() == [1, 1, 1] and p.locked.tolist() == [False, True, False]
    tab = p.prepare(L)
    assert tab["n"].tolist() == [10, 0, 30] and tab["t"].tolist() == [2, 0, 2]
    assert tab["sq_norm"][1] == 0
    p._sq[[0, 2]] = [4.0, 9.0]
    assert p.commit() == []
    assert p.t.tolist() == [2, 1, 2]
    p.unlock(1)
    tab = p.prepare(L)
    assert tab["t"].tolist() == [3, 2, 3]  # layer 1 resumes at its own step


def test_commit_needs_a_norm_for_every_updated_layer():
    p = ProgressiveLocking(2, 1.0)
    p.prepare(lso.LayerStream.file_layers(2))
    with pytest.raises(RuntimeError):
        p.commit()
    with pytest.raises(RuntimeError):
        ProgressiveLocking(2, 1.0).commit()


def test_block_tables_and_state_round_trip():
    arr = np.zeros(2, lso.BLOCK_DTYPE)
    arr["n"] = [5, 6]
    p = ProgressiveLocking(2, 1e-3)
    p.lock(0)
    out = p.prepare_blocks(arr)
    assert out["n"].tolist() == [0, 6] and out["t"].tolist() == [0, 1]
    assert p.commit(np.array([np.nan, 1e-8])) == [1]
    q = ProgressiveLocking.from_state(p.state())
    assert q.t.tolist() == [0, 1] and q.locked.tolist() == [True, True] and q.threshold == 1e-3
