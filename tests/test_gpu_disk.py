"""GPU tests of the disk tier (lso_stream_files): file blocks give the same
bits as host blocks, match the oracle, resume from the manifest, and fail
cleanly on host-forced I/O errors (every kernel still completes)."""
import os
import resource
import signal
import tempfile

import numpy as np
import pytest

import layer_streamed_optimizer_amd as lso
import oracle
import synth
from layer_streamed_optimizer_amd import configs
from layer_streamed_optimizer_amd.disk import LayerFiles

from gpu_util import (B1, B2, EPS, LR, HostLayers, assert_parity, call_scale, detile_state, log,
                      synth_stream, torch)

pytestmark = pytest.mark.gpu

SIZES = [100003, 4096 * 3 + 7, 65536, 1, 8192 * 2 + 5]


def files_like(host: HostLayers, directory: str, direct: bool) -> LayerFiles:
    """Files holding the same initial blocks as the host layers."""
    f = LayerFiles.create(directory, host.sizes, tiled=host.tiled, direct=direct)
    for b in range(len(host.sizes)):
        f.write_block(b, host.raw(b))
    return f


def file_state(f: LayerFiles, b: int, q: str) -> np.ndarray:
    om, omm, ov, nb = f.geom[b]
    n = f.sizes[b]
    raw = f.read_block(b)
    if f.tiled:
        return detile_state(raw[om:].view(np.float32), n)[("master", "m", "v").index(q)]
    off = {"master": om, "m": omm, "v": ov}[q]
    return raw[off:off + 4 * n].view(np.float32).copy()


@pytest.mark.parametrize("tiled", [False, True], ids=["planar", "tiled"])
@pytest.mark.parametrize("direct", [False, True], ids=["buffered", "o_direct"])
def test_files_equal_host_blocks_bitwise_and_match_oracle(tiled, direct):
    T = torch()
    sid = 60
    log("disk tier", f"tiled={tiled} direct={direct}")
    host = HostLayers(SIZES, sid, tiled=tiled)
    ref = [dict(master=host.get(b, "master"), m=np.zeros(n, np.float32), v=np.zeros(n, np.float32))
           for b, n in enumerate(SIZES)]
    mb = max(configs.host_layer_layout(n, tiled=tiled)[3] for n in SIZES)
    with tempfile.TemporaryDirectory() as d:
        files = files_like(host, d, direct)
        ls, params = synth_stream(SIZES, sid, max_bytes=mb)
        for t in range(1, 4):
            params.step = t
            ls.stream_layers(host.table(t))
            ls.stream_files(files.table(t, LR, B1, B2, EPS))
            for b, n in enumerate(SIZES):
                g = synth.normal_bf16(n, stream=sid, block=b, purpose=2, step=t, sigma=1e-3)
                oracle.adam_step(ref[b]["master"], ref[b]["m"], ref[b]["v"], g, None, t, LR, B1, B2,
                                 EPS)
        T.cuda.synchronize()
        scale = call_scale(ref)
        for b in range(len(SIZES)):
            assert np.array_equal(files.read_block(b), host.raw(b)), b
            got = {q: file_state(files, b, q) for q in ("master", "m", "v")}
            assert_parity(got, ref[b], 1e-6, f"file layer {b}", scale)
        files.close()
        ls.close()


def test_files_with_fp32_gradients_equal_host_blocks_bitwise():
    """FP32-gradient layers (grad_dtype LSO_DT_F32) in O_DIRECT files, tiled:
    the same bits as the same layers streamed from host blocks, three steps."""
    T = torch()
    sid = 66
    host = HostLayers(SIZES, sid, tiled=True)
    mb = max(configs.host_layer_layout(n, tiled=True)[3] for n in SIZES)
    with tempfile.TemporaryDirectory() as d:
        files = files_like(host, d, direct=True)
        ls, params = synth_stream(SIZES, sid, max_bytes=mb, f32=True)
        for t in range(1, 4):
            params.step = t
            log("fp32-gradient files step", t)
            ls.stream_layers(host.table(t, grad_dtype=lso.LSO_DT_F32))
            ls.stream_files(files.table(t, LR, B1, B2, EPS, grad_dtype=lso.LSO_DT_F32))
        T.cuda.synchronize()
        for b in range(len(SIZES)):
            assert np.array_equal(files.read_block(b), host.raw(b)), b
        files.close()
        ls.close()


def test_resume_from_manifest_equals_uninterrupted_run():
    """Steps 1-2, close, reopen from the manifest (t comes back as 2), step 3:
    the same bits as three steps in one go.  LSO_FILE_SYNC on."""
    T = torch()
    sid = 61
    host = HostLayers(SIZES, sid)
    mb = max(configs.host_layer_layout(n)[3] for n in SIZES)
    with tempfile.TemporaryDirectory() as d:
        a = files_like(host, os.path.join(d, "a"), direct=True)
        b = files_like(host, os.path.join(d, "b"), direct=True)
        ls, params = synth_stream(SIZES, sid, max_bytes=mb)
        for t in range(1, 4):
            params.step = t
            ls.stream_files(a.table(t, LR, B1, B2, EPS, sync=True))
            a.commit(t)
        for t in (1, 2):
            params.step = t
            ls.stream_files(b.table(t, LR, B1, B2, EPS, sync=True))
            b.commit(t)
        b.close()
        b = LayerFiles.open(os.path.join(d, "b"), direct=True)
        assert b.t == 2 and b.sizes == SIZES
        params.step = b.t + 1
        ls.stream_files(b.table(b.t + 1, LR, B1, B2, EPS, sync=True))
        b.commit(b.t + 1)
        T.cuda.synchronize()
        for i in range(len(SIZES)):
            assert np.array_equal(a.read_block(i), b.read_block(i)), i
        assert LayerFiles.open(os.path.join(d, "b")).t == 3
        a.close()
        b.close()
        ls.close()


def test_layers_sharing_one_file_and_validation_errors():
    T = torch()
    sid = 62
    n = 50000
    om, omm, ov, nb = configs.host_layer_layout(n)
    host = HostLayers([n] * 3, sid)
    ls, params = synth_stream([n] * 3, sid, max_bytes=nb)
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "all.state")
        fd = os.open(path, os.O_RDWR | os.O_CREAT, 0o644)
        os.posix_fallocate(fd, 0, 3 * nb)
        for b in range(3):
            os.pwrite(fd, host.raw(b).tobytes(), b * nb)

        def table():
            L = lso.LayerStream.file_layers(3)
            for b in range(3):
                L[b]["fd"], L[b]["file_offset"], L[b]["bytes"], L[b]["n"] = fd, b * nb, nb, n
                L[b]["off_master"], L[b]["off_m"], L[b]["off_v"] = om, omm, ov
                L[b]["t"] = 1
                L[b]["lr"], L[b]["beta1"], L[b]["beta2"], L[b]["eps"] = LR, B1, B2, EPS
            return L

        E = lso._native
        L = table()
        L[1]["file_offset"] = nb + 4096            # overlaps layer 2's region
        assert ls.stream_files_status(L) == E.LSO_E_OVERLAP
        L = table()
        L[2]["file_offset"] = 2 * nb + 16          # not a 4 KB multiple
        assert ls.stream_files_status(L) == E.LSO_E_ALIGN
        L = table()
        L[2]["file_offset"] = 3 * nb               # past the end of the file
        assert ls.stream_files_status(L) == E.LSO_E_INVALID
        L = table()
        L[0]["flags"] = 8
        assert ls.stream_files_status(L) == E.LSO_E_INVALID
        ro = os.open(path, os.O_RDONLY)
        L = table()
        L[1]["fd"] = ro
        assert ls.stream_files_status(L) == E.LSO_E_INVALID
        assert "reading and writing" in lso.last_error()
        os.close(ro)
        L = table()
        L[0]["fd"] = 1 << 20
        assert ls.stream_files_status(L) == E.LSO_E_INVALID
        # nothing above touched the file; now the valid call
        for b in range(3):
            assert os.pread(fd, nb, b * nb) == host.raw(b).tobytes()
        params.step = 1
        ls.stream_files(table())
        ls.stream_layers(host.table(1))
        T.cuda.synchronize()
        for b in range(3):
            assert os.pread(fd, nb, b * nb) == host.raw(b).tobytes(), b
        os.close(fd)
    ls.close()


def test_read_failure_leaves_later_layers_untouched():
    """Layer 4's file is cut short by the gradient producer of layer 0 (a
    host-forced failure: its stage-in starts only after layer 1 is written
    back).  Layers 0-3 are written back, layers 4 and 5 keep their bytes, and
    the call reports LSO_E_IO naming layer 4."""
    T = torch()
    sid = 63
    sizes = [40000] * 6
    host = HostLayers(sizes, sid)
    fill = synth._dev_lib().synth_fill_normal_bf16
    with tempfile.TemporaryDirectory() as d:
        files = files_like(host, d, direct=False)
        before = [files.read_block(b) for b in range(6)]

        def producer(layer, dev_grad, n, stream):
            if layer == 0:
                os.ftruncate(files.fds[4], 4096)
            return fill(dev_grad, n, 0, synth.SEED, sid, layer, 2, 1, synth.scale_for(1e-3), stream)

        ls = lso.LayerStream(files.bytes(0), 40000, producer)
        st = ls.stream_files_status(files.table(1, LR, B1, B2, EPS))
        assert st == lso._native.LSO_E_IO, lso.last_error()
        assert "layer 4" in lso.last_error()
        T.cuda.synchronize()
        for b in range(6):
            if b < 4:
                assert not np.array_equal(files.read_block(b), before[b]), b
            elif b == 5:
                assert np.array_equal(files.read_block(b), before[b])
        assert os.pread(files.fds[4], 4096, 0) == before[4][:4096].tobytes()
        files.close()
        ls.close()


def test_write_failure_stops_the_write_back():
    """All six layers in one file; a file-size limit on the process makes
    every write at or beyond layer 3's region fail (EFBIG, forced from the
    host).  Layers 0-2 are new, layers 3-5 keep their bytes, and the call
    reports LSO_E_IO naming layer 3."""
    T = torch()
    sid = 64
    n = 1 << 20                       # 12 MB blocks: the limit sits far above any log file
    om, omm, ov, nb = configs.host_layer_layout(n)
    host = HostLayers([n] * 6, sid)
    ls, params = synth_stream([n] * 6, sid, max_bytes=nb)
    with tempfile.TemporaryDirectory() as d:
        fd = os.open(os.path.join(d, "all.state"), os.O_RDWR | os.O_CREAT, 0o644)
        os.posix_fallocate(fd, 0, 6 * nb)
        before = [host.raw(b).tobytes() for b in range(6)]
        for b in range(6):
            os.pwrite(fd, before[b], b * nb)
        L = lso.LayerStream.file_layers(6)
        for b in range(6):
            L[b]["fd"], L[b]["file_offset"], L[b]["bytes"], L[b]["n"] = fd, b * nb, nb, n
            L[b]["off_master"], L[b]["off_m"], L[b]["off_v"] = om, omm, ov
            L[b]["t"] = 1
            L[b]["lr"], L[b]["beta1"], L[b]["beta2"], L[b]["eps"] = LR, B1, B2, EPS
        old_sig = signal.signal(signal.SIGXFSZ, signal.SIG_IGN)
        old_lim = resource.getrlimit(resource.RLIMIT_FSIZE)
        resource.setrlimit(resource.RLIMIT_FSIZE, (3 * nb, old_lim[1]))
        try:
            params.step = 1
            st = ls.stream_files_status(L)
        finally:
            resource.setrlimit(resource.RLIMIT_FSIZE, old_lim)
            signal.signal(signal.SIGXFSZ, old_sig)
        assert st == lso._native.LSO_E_IO, lso.last_error()
        assert "layer 3" in lso.last_error()
        # the same three layers through host memory give the bytes to expect
        ls.stream_layers(host.table(1)[:3].copy())
        T.cuda.synchronize()
        for b in range(6):
            got = os.pread(fd, nb, b * nb)
            if b < 3:
                assert got == host.raw(b).tobytes(), b
                assert got != before[b], b
            else:
                assert got == before[b], b
        os.close(fd)
    ls.close()
