"""GPU tests of the fused gradient norms and of progressive layer locking
(frozen-incremental page, "Progressive Layer Locking"): norms against the
oracle, the update unchanged by the norm variant, locked layers skipped
entirely, per-layer t exact on resume."""
import ctypes
import os
import tempfile

import numpy as np
import pytest

import layer_streamed_optimizer_amd as lso
import oracle
import synth
from layer_streamed_optimizer_amd import configs
from layer_streamed_optimizer_amd.disk import LayerFiles
from layer_streamed_optimizer_amd.locking import ProgressiveLocking

from gpu_util import (B1, B2, EPS, LR, Arena, HostLayers, assert_parity, call_scale, log, torch)

pytestmark = pytest.mark.gpu

NORM_TOL = 2e-6   # stated bound: FP32 sums of <= 32 squares per lane, FP64 above


def grads(sizes, sid, step, f32=False, sigma=1e-3):
    fn = synth.normal_f32 if f32 else synth.normal_bf16
    return [fn(n, stream=sid, block=b, purpose=synth.PURPOSE_GRAD, step=step, sigma=sigma)
            for b, n in enumerate(sizes)]


def init_arena(arena, sizes, sid):
    for b, n in enumerate(sizes):
        arena.put(b, "master", synth.normal_f32(n, stream=sid, block=b, purpose=0, step=0, sigma=0.02))
        arena.put(b, "m", np.zeros(n, np.float32))
        arena.put(b, "v", np.zeros(n, np.float32))


def assert_norms(got, gs, what):
    for i, g in enumerate(gs):
        ref = oracle.sq_norm(g)
        if ref == 0.0:
            assert got[i] == 0.0, (what, i)
        else:
            assert abs(got[i] - ref) <= NORM_TOL * ref, (what, i, got[i], ref)


@pytest.mark.parametrize("f32", [False, True], ids=["bf16_grads", "f32_grads"])
@pytest.mark.parametrize("tiled", [False, True], ids=["planar", "tiled"])
@pytest.mark.parametrize("sizes", [[3 * 8192 + 17],
                                   [1, 7, 8193, 3 * 8192 + 17],
                                   [1, 2, 3, 5, 1023, 1024, 1025, 4097, 12345, 100003],
                                   [(32 << 20) + 4101]],   # a big call: four quads per lane when planar
                         ids=["one_block", "by_value", "table", "big_call"])
def test_norms_match_oracle_and_leave_the_update_unchanged(sizes, tiled, f32):
    T = torch()
    sid = 80
    log("norms", f"blocks={len(sizes)} tiled={tiled} f32={f32}")
    a, b, c = (Arena(sizes, tiled=tiled, grad_f32=f32) for _ in range(3))
    for ar in (a, b, c):
        init_arena(ar, sizes, sid)
    ta, tb, tc = a.table(), b.table(), c.table()
    ws_bytes = lso.norm_workspace_bytes(ta)
    ws = T.empty(max(ws_bytes, 8), dtype=T.uint8, device="cuda")
    sq_a = T.full((len(sizes),), -1.0, dtype=T.float64, device="cuda")
    sq_c = T.full((len(sizes),), -1.0, dtype=T.float64, device="cuda")
    for t in (1, 2):
        gs = grads(sizes, sid, t, f32)
        for ar in (a, b, c):
            for i, g in enumerate(gs):
                ar.put(i, "grad", g)
        for tab in (ta, tb, tc):
            tab.set_step(t)
        lso.adam_step_norms(ta, sq_a, ws, ws_bytes)
        lso.adam_step(tb)
        lso.adam_step_norms(tc, sq_c, ws, ws_bytes)
        T.cuda.synchronize()
        got = sq_a.cpu().numpy()
        assert_norms(got, gs, f"step {t}")
        assert np.array_equal(got.view(np.uint64), sq_c.cpu().numpy().view(np.uint64))
    for i in range(len(sizes)):
        for q in ("master", "m", "v", "weight"):
            assert np.array_equal(a.get(i, q).view(np.uint8), b.get(i, q).view(np.uint8)), (i, q)
    assert a.canaries_intact()


def test_zero_gradients_and_skipped_blocks():
    T = torch()
    sizes = [5000, 3, 70000]
    a = Arena(sizes)
    init_arena(a, sizes, 81)
    for i, n in enumerate(sizes):
        a.put(i, "grad", np.zeros(n, np.uint16))
    tab = a.table()
    tab.arr["n"][1] = 0                      # a skipped block
    sq = T.full((3,), 7.5, dtype=T.float64, device="cuda")
    ws_bytes = lso.norm_workspace_bytes(tab)
    ws = T.empty(ws_bytes, dtype=T.uint8, device="cuda")
    lso.adam_step_norms(tab, sq, ws, ws_bytes)
    T.cuda.synchronize()
    assert sq.cpu().numpy().tolist() == [0.0, 7.5, 0.0]


def test_streamed_layer_norms_match_oracle():
    T = torch()
    sizes = [100003, 4096 * 3 + 7, 65536, 1]
    sid = 82
    host = HostLayers(sizes, sid)
    fn, Params = synth.grad_callback()
    params = Params(seed=synth.SEED, stream=sid, purpose=synth.PURPOSE_GRAD, step=1,
                    scale=synth.scale_for(1e-3), block_base=0)
    ls = lso.LayerStream(max(configs.host_layer_layout(n)[3] for n in sizes), max(sizes), fn,
                         ctypes.addressof(params))
    out = np.full(len(sizes), np.nan)
    for t in (1, 2):
        params.step = t
        L = host.table(t)
        L["sq_norm"] = [out.ctypes.data + 8 * i for i in range(len(sizes))]
        ls.stream_layers(L)
        assert_norms(out, grads(sizes, sid, t), f"streamed step {t}")
    ls.close()


class Producer:
    """Python gradient producer: BF16 normals per (layer, step), sigma per
    layer; counts its calls per layer."""

    def __init__(self, sid, sigmas):
        self.sid, self.sigmas, self.step = sid, sigmas, 1
        self.calls = [0] * len(sigmas)
        self.fill = synth._dev_lib().synth_fill_normal_bf16

    def __call__(self, layer, dev_grad, n, stream):
        self.calls[layer] += 1
        return self.fill(dev_grad, n, 0, synth.SEED, self.sid, layer, synth.PURPOSE_GRAD, self.step,
                         synth.scale_for(self.sigmas[layer]), stream)

    def grad(self, layer, n, step):
        return synth.normal_bf16(n, stream=self.sid, block=layer, purpose=synth.PURPOSE_GRAD, step=step,
                                 sigma=self.sigmas[layer])


def locking_run(kind):
    """Four layers; layer 1's gradients are tiny and lock it after step 1.
    Steps 2-3 skip it; it is unlocked for step 4 and continues at its own
    t = 2.  Checked against the oracle with the same per-layer t."""
    T = torch()
    sizes = [50000] * 4
    sid = 83 if kind == "host" else 84
    prod = Producer(sid, [1e-3, 1e-7, 1e-3, 1e-3])
    host = HostLayers(sizes, sid, pageable=kind == "host")
    ref = [dict(master=host.get(b, "master"), m=np.zeros(n, np.float32), v=np.zeros(n, np.float32))
           for b, n in enumerate(sizes)]
    ls = lso.LayerStream(configs.host_layer_layout(sizes[0])[3], sizes[0], prod)
    lock = ProgressiveLocking(4, threshold=1e-3)
    d = tempfile.mkdtemp() if kind == "file" else None
    files = None
    if kind == "file":
        files = LayerFiles.create(d, sizes)
        for b in range(4):
            files.write_block(b, host.raw(b))
    snapshots = {}
    for step in (1, 2, 3, 4):
        if step == 4:
            lock.unlock(1)
        prod.step = step
        full = files.table(0, LR, B1, B2, EPS) if files else host.table(0)
        tab = lock.prepare(full)
        active = list(lock.active)
        log("locking", kind, "step", step, "active", active)
        (ls.stream_files if files else ls.stream_layers)(tab)
        newly = lock.commit()
        for b in active:
            oracle.adam_step(ref[b]["master"], ref[b]["m"], ref[b]["v"], prod.grad(b, sizes[b], step),
                             None, int(lock.t[b]), LR, B1, B2, EPS)
        if step == 1:
            assert newly == [1]
        if step == 4:
            assert newly == [1] and lock.t.tolist() == [4, 2, 4, 4]
        snapshots[step] = files.read_block(1) if files else host.raw(1)
    T.cuda.synchronize()
    # layer 1 was skipped entirely in steps 2 and 3
    assert prod.calls == [4, 2, 4, 4]
    assert np.array_equal(snapshots[1], snapshots[2]) and np.array_equal(snapshots[2], snapshots[3])
    assert not np.array_equal(snapshots[3], snapshots[4])
    scale = call_scale(ref)
    for b, n in enumerate(sizes):
        if files:
            raw = files.read_block(b)
            om, omm, ov, _ = files.geom[b]
            got = {q: raw[o:o + 4 * n].view(np.float32).copy()
                   for q, o in (("master", om), ("m", omm), ("v", ov))}
        else:
            got = {q: host.get(b, q) for q in ("master", "m", "v")}
        assert_parity(got, ref[b], 1e-6, f"{kind} layer {b}", scale)
    assert np.isclose(lock.norm[1], np.sqrt(oracle.sq_norm(prod.grad(1, sizes[1], 4))), rtol=NORM_TOL)
    ls.close()
    if files:
        files.close()
        for f in os.listdir(d):
            os.remove(os.path.join(d, f))
        os.rmdir(d)


@pytest.mark.parametrize("kind", ["host", "file"])
def test_progressive_locking_skips_locked_layers_and_resumes_exactly(kind):
    locking_run(kind)


def test_progressive_locking_resident_blocks():
    """The resident path: locked blocks go as n = 0 (a no-op block); norms
    from lso_adam_step_norms drive the policy."""
    T = torch()
    sizes = [20000, 20000, 20000]
    sid = 85
    sig = [1e-3, 1e-3, 1e-8]
    a = Arena(sizes)
    init_arena(a, sizes, sid)
    ref = [dict(master=a.get(b, "master"), m=np.zeros(n, np.float32), v=np.zeros(n, np.float32))
           for b, n in enumerate(sizes)]
    lock = ProgressiveLocking(3, threshold=1e-4)
    base = a.table()
    sq = T.zeros(3, dtype=T.float64, device="cuda")
    ws_bytes = lso.norm_workspace_bytes(base)
    ws = T.empty(ws_bytes, dtype=T.uint8, device="cuda")
    for step in (1, 2, 3):
        gs = [synth.normal_bf16(n, stream=sid, block=b, purpose=2, step=step, sigma=sig[b])
              for b, n in enumerate(sizes)]
        for b, g in enumerate(gs):
            a.put(b, "grad", g)
        tab = lso.BlockTable.from_array(lock.prepare_blocks(base.arr))
        active = list(lock.active)
        lso.adam_step_norms(tab, sq, ws, ws_bytes)
        T.cuda.synchronize()
        newly = lock.commit(sq.cpu().numpy())
        for b in active:
            oracle.adam_step(ref[b]["master"], ref[b]["m"], ref[b]["v"], gs[b], None, int(lock.t[b]),
                             LR, B1, B2, EPS)
        if step == 1:
            assert newly == [2]
    assert lock.t.tolist() == [3, 3, 1]
    scale = call_scale(ref)
    for b in range(3):
        got = {q: a.get(b, q) for q in ("master", "m", "v")}
        assert_parity(got, ref[b], 1e-6, f"resident locked block {b}", scale)
