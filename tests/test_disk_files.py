"""The disk tier's file helper on the CPU: preallocation, the manifest that
carries t, the lso_file_layer rows, block read/write round trips."""
import json
import os
import tempfile

import numpy as np
import pytest

import layer_streamed_optimizer_amd as lso
from layer_streamed_optimizer_amd import _native
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


# ------------------------------------------------ crash-consistent shadow files

def _flip(path, offset):
    with open(path, "r+b") as f:
        f.seek(offset)
        b = f.read(1)
        f.seek(offset)
        f.write(bytes([b[0] ^ 0x40]))


def test_shadow_headers_pick_the_newest_valid_copy():
    """Header copy k holds the epochs with e % 2 == k; the committed state is
    the valid copy with the highest epoch; a damaged (torn) copy or a copy
    for the wrong size is not believed."""
    with tempfile.TemporaryDirectory() as d:
        with LayerFiles.create(d, [5000], shadow=True) as f:
            nb = f.bytes(0)
            H = lso.LSO_SHADOW_HEADER_BYTES
            assert f.state(0) == (0, 0, H)
            lso.shadow_commit(f.fds[0], 0, nb, 1, 7)
            assert f.state(0) == (1, 7, H + nb)
            lso.shadow_commit(f.fds[0], 0, nb, 2, 9)
            assert f.state(0) == (2, 9, H)
            _flip(f.path(0), 9)                  # epoch field of copy 0: checksum fails
            assert f.state(0) == (1, 7, H + nb)
            _flip(f.path(0), 4096 + 33)          # checksum of copy 1
            with pytest.raises(lso.LsoError) as e:
                f.state(0)
            assert e.value.status == _native.LSO_E_IO
            lso.shadow_commit(f.fds[0], 0, nb, 3, 11)
            assert f.state(0) == (3, 11, H + nb)
            # a header written for another block size is not this region's
            with pytest.raises(lso.LsoError):
                lso.shadow_state(f.fds[0], 0, nb - 4096)


def test_shadow_copy_position_is_checked():
    """A valid header for an odd epoch written where copy 0 lives (a stale or
    misplaced copy) is ignored."""
    with tempfile.TemporaryDirectory() as d:
        with LayerFiles.create(d, [5000], shadow=True) as f:
            nb = f.bytes(0)
            lso.shadow_commit(f.fds[0], 0, nb, 5, 1)     # goes to copy 1
            raw = os.pread(f.fds[0], 4096, 4096)
            os.pwrite(f.fds[0], raw, 0)                 # the same bytes into copy 0
            os.pwrite(f.fds[0], bytes(4096), 4096)      # copy 1 cleared
            with pytest.raises(lso.LsoError):
                f.state(0)


def test_shadow_validation_and_round_trip():
    with tempfile.TemporaryDirectory() as d:
        with LayerFiles.create(d, [3000, 7], shadow=True) as f:
            data = np.random.default_rng(1).integers(0, 256, f.bytes(0), dtype=np.uint8)
            f.write_block(0, data)
            assert np.array_equal(f.read_block(0), data)
            L = f.table(1, 1e-3, 0.9, 0.999, 1e-8)
            assert all(L["flags"] == lso.LSO_FILE_SHADOW)
            st = os.stat(f.path(0)).st_size
            assert st == lso.LSO_SHADOW_HEADER_BYTES + 2 * f.bytes(0)
        with pytest.raises(lso.LsoError) as e:
            lso.shadow_format(10 ** 6, 0, 4096)
        assert e.value.status == _native.LSO_E_INVALID
        fd = os.open(os.path.join(d, "x"), os.O_RDWR | os.O_CREAT, 0o644)
        with pytest.raises(lso.LsoError) as e:
            lso.shadow_format(fd, 0, 4096)          # the file is empty
        assert e.value.status == _native.LSO_E_INVALID
        with pytest.raises(lso.LsoError) as e:
            lso.shadow_format(fd, 100, 4096)
        assert e.value.status == _native.LSO_E_ALIGN
        os.close(fd)
        assert LayerFiles.open(d).shadow
