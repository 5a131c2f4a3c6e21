"""GPU tests of crash-consistent write-back (LSO_FILE_SHADOW): shadow files
give the bits of plain files, a process killed mid-step leaves every layer
wholly old or wholly new and resumes to the uninterrupted result, and a
failed write leaves its layer wholly old."""
import os
import resource
import signal
import subprocess
import sys
import tempfile

import numpy as np
import pytest

import layer_streamed_optimizer_amd as lso
from layer_streamed_optimizer_amd import configs
from layer_streamed_optimizer_amd.disk import LayerFiles

from gpu_util import B1, B2, EPS, LR, HostLayers, log, stream_pieces, synth_stream, torch

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def shadow_like(host, directory, direct=False):
    f = LayerFiles.create(directory, host.sizes, tiled=host.tiled, direct=direct, shadow=True)
    for b in range(len(host.sizes)):
        f.write_block(b, host.raw(b))
    return f


@pytest.mark.parametrize("tiled,pieces", [(False, 0), (True, 0), (True, 3)],
                         ids=["planar", "tiled", "tiled_in_pieces"])
def test_shadow_files_equal_plain_files_bitwise(tiled, pieces):
    T = torch()
    sizes = [100003, 4096 * 3 + 7, 65536, 1]
    sid = 90
    host = HostLayers(sizes, sid, tiled=tiled)
    mb = max(configs.host_layer_layout(n, tiled=tiled)[3] for n in sizes)
    with tempfile.TemporaryDirectory() as d:
        plain = LayerFiles.create(os.path.join(d, "p"), sizes, tiled=tiled)
        for b in range(len(sizes)):
            plain.write_block(b, host.raw(b))
        shadow = shadow_like(host, os.path.join(d, "s"), direct=True)
        if pieces:
            with stream_pieces(pieces):
                ls, params = synth_stream(sizes, sid, max_bytes=mb)
        else:
            ls, params = synth_stream(sizes, sid, max_bytes=mb)
        for t in (1, 2, 3):
            params.step = t
            ls.stream_files(plain.table(t, LR, B1, B2, EPS))
            ls.stream_files(shadow.table(t, LR, B1, B2, EPS))
            for b in range(len(sizes)):
                epoch, tt, off = shadow.state(b)
                assert (epoch, tt) == (t, t)
                assert off == lso.LSO_SHADOW_HEADER_BYTES + (t % 2) * shadow.bytes(b)
        T.cuda.synchronize()
        for b in range(len(sizes)):
            assert np.array_equal(shadow.read_block(b), plain.read_block(b)), b
        plain.close()
        shadow.close()
        ls.close()


def test_killed_mid_step_every_layer_wholly_old_or_new_and_resume_is_exact():
    T = torch()
    sid = 91
    n = 1 << 22                       # 48 MB blocks, so write-backs take a while
    sizes = [n] * 6
    kill_at = 4
    host = HostLayers(sizes, sid)
    init = [host.raw(b) for b in range(6)]
    with tempfile.TemporaryDirectory() as d:
        crash_dir, ref_dir = os.path.join(d, "crash"), os.path.join(d, "ref")
        for dd in (crash_dir, ref_dir):
            shadow_like(host, dd).close()
        log("crash test: child killed at layer", kill_at)
        r = subprocess.run([sys.executable, os.path.join(HERE, "shadow_crash_child.py"), crash_dir,
                            str(kill_at), str(sid)], capture_output=True, text=True, timeout=180)
        assert r.returncode == -signal.SIGKILL, (r.returncode, r.stdout[-2000:], r.stderr[-2000:])
        assert "killing the process" in r.stdout
        # the uninterrupted step, for the expected new state
        ref = LayerFiles.open(ref_dir)
        ls, params = synth_stream(sizes, sid, max_bytes=ref.bytes(0))
        params.step = 1
        ls.stream_files(ref.table(1, LR, B1, B2, EPS))
        crash = LayerFiles.open(crash_dir)
        epochs = []
        for b in range(6):
            epoch, t, _ = crash.state(b)
            data = crash.read_block(b)
            if epoch == 0:
                assert t == 0 and np.array_equal(data, init[b]), f"layer {b}: epoch 0 but not the old state"
            else:
                assert (epoch, t) == (1, 1), (b, epoch, t)
                assert np.array_equal(data, ref.read_block(b)), f"layer {b}: epoch 1 but not the new state"
            epochs.append(epoch)
        log("epochs after the kill", epochs)
        # layers written back before the producer of layer kill_at ran are
        # committed; layers from kill_at on never started
        assert all(e == 1 for e in epochs[:kill_at - 2]), epochs
        assert all(e == 0 for e in epochs[kill_at:]), epochs
        # resume: the layers still at epoch 0 take the step now
        L = crash.table(1, LR, B1, B2, EPS)
        L["n"][[e == 1 for e in epochs]] = 0
        ls.stream_files(L)
        T.cuda.synchronize()
        for b in range(6):
            assert crash.state(b)[:2] == (1, 1)
            assert np.array_equal(crash.read_block(b), ref.read_block(b)), b
        crash.close()
        ref.close()
        ls.close()


def test_failed_write_leaves_its_layer_wholly_old():
    """Six shadow regions in one file; a file-size limit on the process cuts
    layer 3's new data slot in the middle (EFBIG, forced from the host).
    Layers 0-2 commit, layer 3 stays wholly at its old epoch although half of
    its new slot was written, layers 4-5 are untouched."""
    T = torch()
    sid = 92
    n = 1 << 20
    om, omm, ov, nb = configs.host_layer_layout(n)
    span = lso.LSO_SHADOW_HEADER_BYTES + 2 * nb
    host = HostLayers([n] * 6, sid)
    before = [host.raw(b) for b in range(6)]
    ls, params = synth_stream([n] * 6, sid, max_bytes=nb)
    with tempfile.TemporaryDirectory() as d:
        fd = os.open(os.path.join(d, "all.state"), os.O_RDWR | os.O_CREAT, 0o644)
        os.posix_fallocate(fd, 0, 6 * span)
        for b in range(6):
            lso.shadow_format(fd, b * span, nb)
            os.pwrite(fd, before[b].tobytes(), b * span + lso.LSO_SHADOW_HEADER_BYTES)
        L = lso.LayerStream.file_layers(6)
        for b in range(6):
            L[b]["fd"], L[b]["flags"] = fd, lso.LSO_FILE_SHADOW
            L[b]["file_offset"], L[b]["bytes"], L[b]["n"] = b * span, nb, n
            L[b]["off_master"], L[b]["off_m"], L[b]["off_v"] = om, omm, ov
            L[b]["t"] = 1
            L[b]["lr"], L[b]["beta1"], L[b]["beta2"], L[b]["eps"] = LR, B1, B2, EPS
        limit = 3 * span + lso.LSO_SHADOW_HEADER_BYTES + nb + (nb // 2 // 4096) * 4096
        old_sig = signal.signal(signal.SIGXFSZ, signal.SIG_IGN)
        old_lim = resource.getrlimit(resource.RLIMIT_FSIZE)
        resource.setrlimit(resource.RLIMIT_FSIZE, (limit, old_lim[1]))
        try:
            params.step = 1
            st = ls.stream_files_status(L)
        finally:
            resource.setrlimit(resource.RLIMIT_FSIZE, old_lim)
            signal.signal(signal.SIGXFSZ, old_sig)
        assert st == lso._native.LSO_E_IO, lso.last_error()
        assert "layer 3" in lso.last_error()
        ls.stream_layers(host.table(1)[:3].copy())       # the expected new states
        T.cuda.synchronize()
        for b in range(6):
            epoch, t, off = lso.shadow_state(fd, b * span, nb)
            data = os.pread(fd, nb, off)
            if b < 3:
                assert (epoch, t) == (1, 1) and data == host.raw(b).tobytes(), b
            else:
                assert (epoch, t) == (0, 0) and data == before[b].tobytes(), b
        # half of layer 3's new slot did reach the file
        slot1 = os.pread(fd, nb // 2, 3 * span + lso.LSO_SHADOW_HEADER_BYTES + nb)
        assert slot1 != bytes(nb // 2)
        os.close(fd)
    ls.close()
