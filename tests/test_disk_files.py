"""The disk tier's file helper on the CPU: preallocation, the manifest that
carries t, the lso_file_layer rows, block read/write round trips."""
import json
import os
import tempfile

import numpy as np

import layer_streamed_optimizer_amd as lso
from layer_streamed_optimizer_amd import configs
from layer_streamed_optimizer_amd.disk import MANIFEST, LayerFiles


def test_create_preallocates_and_records_t0():
    sizes = [1000, 8192 * 2 + 3, 1]
    with tempfile.TemporaryDirectory() as d:
        with LayerFiles.create(d, sizes, tiled=False) as f:
            for i, n in enumerate(sizes):
                st = os.stat(f.path(i))
                assert st.st_size == configs.host_layer_layout(n)[3] == f.bytes(i)
                assert st.st_blocks * 512 >= st.st_size     # blocks allocated up front
            assert not np.any(f.read_block(1))               # zero-filled
        man = json.load(open(os.path.join(d, MANIFEST)))
        assert man["t"] == 0 and man["sizes"] == sizes and man["layout"] == "planar"
        assert not os.path.exists(os.path.join(d, MANIFEST + ".tmp"))


def test_commit_and_reopen_carry_t_and_geometry():
    with tempfile.TemporaryDirectory() as d:
        f = LayerFiles.create(d, [5000, 7], tiled=True)
        f.commit(41)
        f.close()
        g = LayerFiles.open(d)
        assert g.t == 41 and g.sizes == [5000, 7] and g.tiled
        assert g.bytes(0) == configs.host_layer_layout(5000, tiled=True)[3]
        g.close()


def test_block_round_trip():
    with tempfile.TemporaryDirectory() as d:
        with LayerFiles.create(d, [30000]) as f:
            data = np.random.default_rng(0).integers(0, 256, f.bytes(0), dtype=np.uint8)
            f.write_block(0, data)
            assert np.array_equal(f.read_block(0), data)


def test_table_rows():
    sizes = [4097, 100]
    with tempfile.TemporaryDirectory() as d:
        with LayerFiles.create(d, sizes) as f:
            L = f.table(7, 1e-3, 0.9, 0.999, 1e-8, sync=True)
            assert L.dtype == lso.FILE_LAYER_DTYPE
            for i, n in enumerate(sizes):
                om, omm, ov, nb = configs.host_layer_layout(n)
                assert L[i]["fd"] == f.fds[i] and L[i]["flags"] == lso.LSO_FILE_SYNC
                assert (L[i]["file_offset"], L[i]["bytes"], L[i]["n"]) == (0, nb, n)
                assert (L[i]["off_master"], L[i]["off_m"], L[i]["off_v"]) == (om, omm, ov)
                assert L[i]["t"] == 7 and L[i]["layout"] == lso.LSO_LAYOUT_PLANAR
                assert nb % 4096 == 0
