"""GPU tests of layer streaming (lso_stream_layers): parity with the oracle,
bitwise agreement with the resident path, failure handling and the
persistence example, through the C ABI."""
import ctypes

import numpy as np
import pytest

import layer_streamed_optimizer_amd as lso
import oracle
import synth
from layer_streamed_optimizer_amd import _native, configs

from gpu_util import (HIP_D2D, HostLayers, assert_parity, call_scale, hip, log, stream_env,
                      stream_pieces, synth_stream, torch)

pytestmark = pytest.mark.gpu

LR, B1, B2, EPS = configs.LR, configs.BETA1, configs.BETA2, configs.EPS


def test_stream_layers_matches_oracle():
    T = torch()
    sizes = [100003, 4096 * 3 + 7, 65536, 1]
    sid = 40
    log("stream parity", sizes)
    host = HostLayers(sizes, sid)
    ref = [dict(master=host.get(b, "master"), m=np.zeros(n, np.float32), v=np.zeros(n, np.float32),
                weight=np.zeros(n, np.uint16)) for b, n in enumerate(sizes)]
    dev_w = [T.zeros(n, dtype=T.int16, device="cuda") for n in sizes]
    ls, params = synth_stream(sizes, sid)
    for t in range(1, 4):
        params.step = t
        ls.stream_layers(host.table(t, dev_weight=[int(w.data_ptr()) for w in dev_w]))
        for b, n in enumerate(sizes):
            g = synth.normal_bf16(n, stream=sid, block=b, purpose=2, step=t, sigma=1e-3)
            oracle.adam_step(ref[b]["master"], ref[b]["m"], ref[b]["v"], g, ref[b]["weight"], t,
                             LR, B1, B2, EPS)
    T.cuda.synchronize()
    scale = call_scale(ref)
    for b in range(len(sizes)):
        got = dict(master=host.get(b, "master"), m=host.get(b, "m"), v=host.get(b, "v"),
                   weight=dev_w[b].cpu().numpy().view(np.uint16))
        assert_parity(got, ref[b], 1e-6, f"streamed layer {b}", scale)
    ls.close()


def test_streamed_equals_resident_bitwise():
    """The same layers through lso_stream_layers and through lso_adam_step on
    HBM-resident copies, with the same device-generated gradients: bit for
    bit (the slot reuse must never let a copy overtake the update)."""
    T = torch()
    sizes = [300007, 262144, 5, 131072 + 3, 77777]
    sid = 41
    host = HostLayers(sizes, sid)
    res = []
    for b, n in enumerate(sizes):
        res.append(dict(master=T.from_numpy(host.get(b, "master")).cuda(),
                        m=T.zeros(n, dtype=T.float32, device="cuda"),
                        v=T.zeros(n, dtype=T.float32, device="cuda"),
                        g=T.empty(n, dtype=T.int16, device="cuda"),
                        w=T.empty(n, dtype=T.int16, device="cuda")))
    ls, params = synth_stream(sizes, sid)
    for t in range(1, 4):
        params.step = t
        log("streamed vs resident step", t)
        ls.stream_layers(host.table(t))
        rows = []
        for b, n in enumerate(sizes):
            synth.device_fill_normal_bf16(res[b]["g"].data_ptr(), n, stream=sid, block=b,
                                          purpose=2, step=t, sigma=1e-3,
                                          hip_stream=T.cuda.current_stream().cuda_stream)
            rows.append(dict(n=n, master=res[b]["master"], m=res[b]["m"], v=res[b]["v"],
                             grad=res[b]["g"], weight=res[b]["w"], t=t))
        lso.adam_step(lso.BlockTable.from_rows(rows))
    T.cuda.synchronize()
    for b in range(len(sizes)):
        for q in ("master", "m", "v"):
            assert np.array_equal(host.get(b, q).view(np.uint32),
                                  res[b][q].cpu().numpy().view(np.uint32)), (b, q)
    # the last layer's BF16 weight is still in its slot
    last = len(sizes) - 1
    n = sizes[last]
    slot = T.empty(n, dtype=T.int16, device="cuda")
    assert hip().hipMemcpyAsync(slot.data_ptr(), ls.slot_weight(last % 2), 2 * n, HIP_D2D,
                                T.cuda.current_stream().cuda_stream) == 0
    T.cuda.synchronize()
    assert np.array_equal(slot.cpu().numpy(), res[last]["w"].cpu().numpy())
    ls.close()


def test_grad_producer_failure_leaves_later_layers_untouched():
    """The producer fails at layer 2: layers 0 and 1 are fully written back,
    layers 2 and 3 keep their old host state, and the call reports
    LSO_E_CALLBACK (failure forced from the host; every kernel completes)."""
    T = torch()
    sizes = [50000, 50000, 50000, 50000]
    sid = 42
    host = HostLayers(sizes, sid)
    before = [host.get(b, "master") for b in range(4)]
    fill = synth._dev_lib().synth_fill_normal_bf16

    def producer(layer, dev_grad, n, stream):
        if layer == 2:
            return 5
        return fill(dev_grad, n, 0, synth.SEED, sid, layer, 2, 1, synth.scale_for(1e-3), stream)

    ls = lso.LayerStream(max(configs.host_layer_layout(n)[3] for n in sizes), max(sizes), producer)
    st = ls.stream_layers_status(host.table(1))
    assert st == lso._native.LSO_E_CALLBACK
    assert "layer 2" in lso.last_error()
    for b in range(4):
        now = host.get(b, "master")
        if b < 2:
            assert not np.array_equal(now, before[b]), b
            assert np.any(host.get(b, "v") != 0), b
        else:
            assert np.array_equal(now.view(np.uint32), before[b].view(np.uint32)), b
            assert not np.any(host.get(b, "m")), b
    ls.close()


def test_persistence_sgd_accumulates_in_host_block():
    """The page's persistence check on the streamed path: two streamed SGD
    steps whose deltas are BF16-exact add up in the authoritative host block
    bit for bit: [1, 2] -> [1.5, 2.25] -> [2.0, 2.5]."""
    T = torch()
    host = HostLayers([2], 43)
    host.bufs[0].view(np.float32, 0, 2)[:] = [1.0, 2.0]
    gbits = (np.array([0.5, 0.25], np.float32).view(np.uint32) >> 16).astype(np.uint16)
    gsrc = T.from_numpy(gbits.view(np.int16)).cuda()

    def producer(layer, dev_grad, n, stream):
        return hip().hipMemcpyAsync(dev_grad, gsrc.data_ptr(), 2 * n, HIP_D2D, stream)

    T.cuda.synchronize()
    ls = lso.LayerStream(configs.host_layer_layout(2)[3], 2, producer)
    # SGD: master + (-(lr * g)) with lr = -1 adds g
    ls.stream_layers(host.table(1, opt=lso.LSO_OPT_SGD, lr=-1.0))
    assert host.get(0, "master").tolist() == [1.5, 2.25]
    ls.stream_layers(host.table(2, opt=lso.LSO_OPT_SGD, lr=-1.0))
    assert host.get(0, "master").tolist() == [2.0, 2.5]
    ls.close()


def test_device_generator_matches_host_generator():
    """The two implementations of the input generator agree bit for bit."""
    T = torch()
    n = 1 << 20
    buf = T.empty(n, dtype=T.float32, device="cuda")
    synth.device_fill_normal_f32(buf.data_ptr(), n, stream=7, block=3, purpose=0, step=0,
                                 sigma=0.02, start=12345)
    g = T.empty(n, dtype=T.int16, device="cuda")
    synth.device_fill_normal_bf16(g.data_ptr(), n, stream=7, block=3, purpose=2, step=9, sigma=1e-3)
    T.cuda.synchronize()
    assert np.array_equal(buf.cpu().numpy(),
                          synth.normal_f32(n, stream=7, block=3, purpose=0, step=0, sigma=0.02,
                                           start=12345))
    assert np.array_equal(g.cpu().numpy().view(np.uint16),
                          synth.normal_bf16(n, stream=7, block=3, purpose=2, step=9, sigma=1e-3))


def test_pageable_and_mixed_host_blocks_equal_pinned_bitwise():
    """Pageable authoritative blocks go through the pinned staging buffers;
    the result is bit-identical to pinned blocks (all pageable, and
    alternating pinned / pageable layers)."""
    T = torch()
    sizes = [300007, 262144, 5, 131072 + 3, 77777]
    sid = 44
    ref = HostLayers(sizes, sid)
    pag = HostLayers(sizes, sid, pageable=True)
    mix = HostLayers(sizes, sid, pageable=lambda b: b % 2 == 1)
    ls, params = synth_stream(sizes, sid)
    for t in range(1, 4):
        params.step = t
        log("pinned / pageable / mixed step", t)
        for h in (ref, pag, mix):
            ls.stream_layers(h.table(t))
    T.cuda.synchronize()
    for b in range(len(sizes)):
        for q in ("master", "m", "v"):
            x = ref.get(b, q).view(np.uint32)
            assert np.array_equal(x, pag.get(b, q).view(np.uint32)), ("pageable", b, q)
            assert np.array_equal(x, mix.get(b, q).view(np.uint32)), ("mixed", b, q)
    ls.close()


def test_pageable_producer_failure_leaves_later_layers_untouched():
    T = torch()
    sizes = [40000] * 5
    sid = 45
    host = HostLayers(sizes, sid, pageable=True)
    before = [host.get(b, "master") for b in range(5)]
    fill = synth._dev_lib().synth_fill_normal_bf16

    def producer(layer, dev_grad, n, stream):
        if layer == 3:
            return 9
        return fill(dev_grad, n, 0, synth.SEED, sid, layer, 2, 1, synth.scale_for(1e-3), stream)

    ls = lso.LayerStream(configs.host_layer_layout(40000)[3], 40000, producer)
    assert ls.stream_layers_status(host.table(1)) == lso._native.LSO_E_CALLBACK
    for b in range(5):
        now = host.get(b, "master")
        if b < 3:
            assert not np.array_equal(now, before[b]), b
            assert np.any(host.get(b, "v") != 0), b
        else:
            assert np.array_equal(now.view(np.uint32), before[b].view(np.uint32)), b
            assert not np.any(host.get(b, "m")), b
    ls.close()


def test_stream_tiled_layers_match_planar_bitwise_and_oracle():
    """Tiled host blocks (one [master | m | v]-per-tile region per layer),
    pinned and pageable, give the planar results bit for bit; both match the
    oracle."""
    T = torch()
    sizes = [100003, 8192 * 3, 5, 65536 + 8191]
    sid = 46
    plan = HostLayers(sizes, sid)
    til = HostLayers(sizes, sid, tiled=True)
    tpg = HostLayers(sizes, sid, tiled=True, pageable=True)
    ref = [dict(master=plan.get(b, "master"), m=np.zeros(n, np.float32), v=np.zeros(n, np.float32))
           for b, n in enumerate(sizes)]
    ls, params = synth_stream(sizes, sid, max_bytes=max(
        max(configs.host_layer_layout(n, tiled=tl)[3] for n in sizes) for tl in (False, True)))
    for t in range(1, 4):
        params.step = t
        for h in (plan, til, tpg):
            ls.stream_layers(h.table(t))
        for b, n in enumerate(sizes):
            g = synth.normal_bf16(n, stream=sid, block=b, purpose=2, step=t, sigma=1e-3)
            oracle.adam_step(ref[b]["master"], ref[b]["m"], ref[b]["v"], g, None, t, LR, B1, B2, EPS)
    T.cuda.synchronize()
    scale = call_scale(ref)
    for b in range(len(sizes)):
        got = {q: til.get(b, q) for q in ("master", "m", "v")}
        for q in ("master", "m", "v"):
            assert np.array_equal(got[q].view(np.uint32), plan.get(b, q).view(np.uint32)), (b, q)
            assert np.array_equal(got[q].view(np.uint32), tpg.get(b, q).view(np.uint32)), (b, q)
        assert_parity(got, ref[b], 1e-6, f"tiled streamed layer {b}", scale)
    ls.close()


@pytest.mark.parametrize("pageable", [False, True], ids=["pinned", "pageable"])
def test_layers_moved_in_pieces_equal_whole_layers_bitwise(pageable):
    """Tiled layers cut into pieces of two tiles (ragged last pieces, a layer
    smaller than a piece) give the bits of whole-layer moves: state, BF16
    weights, and gradient norms within 1e-12."""
    T = torch()
    sizes = [100003, 8192 * 7 + 1, 5, 65536 + 8191]
    sid = 47
    whole = HostLayers(sizes, sid, tiled=True)
    piece = HostLayers(sizes, sid, tiled=True, pageable=pageable)
    mb = max(configs.host_layer_layout(n, tiled=True)[3] for n in sizes)
    ls_a, pa = synth_stream(sizes, sid, max_bytes=mb)
    with stream_pieces(2):
        ls_b, pb = synth_stream(sizes, sid, max_bytes=mb)
    wa = [T.zeros(n, dtype=T.int16, device="cuda") for n in sizes]
    wb = [T.zeros(n, dtype=T.int16, device="cuda") for n in sizes]
    na, nb = np.zeros(len(sizes)), np.zeros(len(sizes))
    for t in range(1, 4):
        pa.step = pb.step = t
        log("pieces step", t)
        La = whole.table(t, dev_weight=[int(w.data_ptr()) for w in wa])
        Lb = piece.table(t, dev_weight=[int(w.data_ptr()) for w in wb])
        La["sq_norm"] = [na.ctypes.data + 8 * i for i in range(len(sizes))]
        Lb["sq_norm"] = [nb.ctypes.data + 8 * i for i in range(len(sizes))]
        ls_a.stream_layers(La)
        ls_b.stream_layers(Lb)
        np.testing.assert_allclose(nb, na, rtol=1e-12)
    T.cuda.synchronize()
    for b in range(len(sizes)):
        assert np.array_equal(whole.raw(b), piece.raw(b)), b
        assert np.array_equal(wa[b].cpu().numpy(), wb[b].cpu().numpy()), b
    ls_a.close()
    ls_b.close()


@pytest.mark.parametrize("pageable", [False, True], ids=["pinned", "pageable"])
def test_every_copy_mode_gives_the_same_bits(pageable):
    """The four ways of moving blocks over the link (named SDMA engines, the
    default; runtime-chosen DMA engine for H2D with a D2H copy kernel; copy
    kernels; runtime-chosen DMA engines) give the same state, weights and
    norms bit for bit, on tiled layers in pieces and planar layers in one
    call, and each context reports the mode it was asked for."""
    T = torch()
    sizes_t = [100003, 8192 * 5 + 1]
    sizes_p = [7, 65536 + 8191]
    sizes = sizes_t + sizes_p
    sid = 48
    mb = max([configs.host_layer_layout(n, tiled=True)[3] for n in sizes_t] +
             [configs.host_layer_layout(n)[3] for n in sizes_p])
    runs = {}
    # the last run names the other engine pair itself (LSO_STREAM_SDMA)
    for name, mode, env in (("sdma-pair", "sdma-pair", {}), ("dma-in", "dma-in", {}),
                            ("kernel", "kernel", {}), ("dma", "dma", {}),
                            ("sdma 2,3", "sdma-pair", {"SDMA": "2,3"})):
        log("copy mode", name, "pageable" if pageable else "pinned")
        ht = HostLayers(sizes_t, sid, tiled=True, pageable=pageable)
        hp = HostLayers(sizes_p, sid + 1, pageable=pageable)
        with stream_pieces(2), stream_env(COPY=mode, **env):
            ls, prm = synth_stream(sizes, sid, max_bytes=mb)
        cm = ls.copy_mode()
        assert cm["mode"] == mode, cm
        if name == "sdma-pair":
            assert cm["h2d_engine"] and cm["d2h_engine"] and cm["h2d_engine"] != cm["d2h_engine"], cm
        if name == "sdma 2,3":
            assert (cm["h2d_engine"], cm["d2h_engine"]) == (4, 8), cm
        w = [T.zeros(n, dtype=T.int16, device="cuda") for n in sizes]
        norms = np.zeros(len(sizes))
        for t in range(1, 4):
            prm.step = t
            L = np.concatenate([ht.table(t), hp.table(t)])
            L["dev_weight"] = [int(x.data_ptr()) for x in w]
            L["sq_norm"] = [norms.ctypes.data + 8 * i for i in range(len(sizes))]
            ls.stream_layers(L)
        T.cuda.synchronize()
        raw = [ht.raw(b) for b in range(len(sizes_t))] + [hp.raw(b) for b in range(len(sizes_p))]
        runs[name] = (raw, [x.cpu().numpy() for x in w], norms.copy())
        ls.close()
    ref = runs["sdma-pair"]
    for mode, (raw, w, norms) in runs.items():
        for b in range(len(sizes)):
            assert np.array_equal(raw[b], ref[0][b]), (mode, b)
            assert np.array_equal(w[b], ref[1][b]), (mode, b)
        assert np.array_equal(norms, ref[2]), mode


@pytest.mark.parametrize("slots", [2, 3, 4])
def test_named_engines_many_small_pieces_any_slot_count(slots):
    """Forty layers, tiled ones cut into one-tile pieces and small planar
    ones, pinned and pageable mixed: the named-engine pipeline, with 2, 3 or
    4 device slots (each H2D chained on the engine to the slot's previous
    D2H, whose completion signals rotate over slots + staging buffers; a
    layer's producer is queued ahead at its first H2D), gives the bits of
    copy kernels with two slots -- state, weights and norms.  An H2D that
    overtook the slot's D2H, or an update that ran before its H2D had
    landed, would mix two pieces' data.  The unchained named-engine run and
    the dma-in run also fill every slot with NaN once its piece is copied
    back (LSO_STREAM_POISON).  Each context reports its pieces and whether it
    chained."""
    T = torch()
    rng = np.random.default_rng(7)
    sizes_t = [int(x) for x in rng.integers(1, 3 * 8192 + 5, 24)]
    sizes_p = [int(x) for x in rng.integers(1, 20000, 16)]
    sizes = sizes_t + sizes_p
    sid = 49
    mb = max([configs.host_layer_layout(n, tiled=True)[3] for n in sizes_t] +
             [configs.host_layer_layout(n)[3] for n in sizes_p])
    runs = {}
    # the named engines with each H2D chained on the engine to the slot's
    # previous D2H (the default), and unchained with slot poisoning
    for name, mode, k, poison in (("chained", "sdma-pair", slots, 0), ("sdma-pair", "sdma-pair", slots, 1),
                                  ("dma-in", "dma-in", slots, 1), ("kernel", "kernel", 2, 0)):
        log("many pieces", name, "slots", k, "poison", poison)
        ht = HostLayers(sizes_t, sid, tiled=True, pageable=lambda b: b % 3 == 1)
        hp = HostLayers(sizes_p, sid + 1, pageable=lambda b: b % 2 == 0)
        with stream_pieces(1), stream_env(COPY=mode, SLOTS=k, POISON=poison):
            ls, prm = synth_stream(sizes, sid, max_bytes=mb)
        assert ls.copy_mode()["mode"] == mode
        w = [T.zeros(n, dtype=T.int16, device="cuda") for n in sizes]
        norms = np.zeros(len(sizes))
        for t in range(1, 3):
            prm.step = t
            L = np.concatenate([ht.table(t), hp.table(t)])
            L["dev_weight"] = [int(x.data_ptr()) for x in w]
            L["sq_norm"] = [norms.ctypes.data + 8 * i for i in range(len(sizes))]
            ls.stream_layers(L)
        T.cuda.synchronize()
        st = ls.stats()
        pieces = sum((n + 8191) // 8192 for n in sizes_t) + len(sizes_p)
        assert st["pieces"] == pieces and st["chained"] == (name == "chained"), st
        log("many pieces", name, st)
        raw = [ht.raw(b) for b in range(len(sizes_t))] + [hp.raw(b) for b in range(len(sizes_p))]
        runs[name] = (raw, [x.cpu().numpy() for x in w], norms.copy())
        ls.close()
    b = runs["kernel"]
    for mode in ("chained", "sdma-pair", "dma-in"):
        a = runs[mode]
        for i in range(len(sizes)):
            assert np.array_equal(a[0][i], b[0][i]), (mode, i)
            assert np.array_equal(a[1][i], b[1][i]), (mode, i)
        assert np.array_equal(a[2], b[2]), mode


@pytest.mark.parametrize("pageable", [False, True], ids=["pinned", "pageable"])
def test_stream_fp32_gradients_match_oracle(pageable):
    """Layers whose producer writes FP32 gradients (grad_dtype LSO_DT_F32):
    tiled layers in two-tile pieces and planar layers, three steps, against
    the oracle's FP32-gradient step (state within 1e-6, weights the RNE of
    the streamed master) and its sum of g^2 (within 2e-6)."""
    T = torch()
    sizes_t = [100003, 8192 * 3 + 1]
    sizes_p = [7, 50000]
    sizes = sizes_t + sizes_p
    sid = 50
    ht = HostLayers(sizes_t, sid, tiled=True, pageable=pageable)
    hp = HostLayers(sizes_p, sid + 1, pageable=pageable)
    ref = [dict(master=ht.get(b, "master"), m=np.zeros(n, np.float32), v=np.zeros(n, np.float32),
                weight=np.zeros(n, np.uint16)) for b, n in enumerate(sizes_t)]
    ref += [dict(master=hp.get(b, "master"), m=np.zeros(n, np.float32), v=np.zeros(n, np.float32),
                 weight=np.zeros(n, np.uint16)) for b, n in enumerate(sizes_p)]
    mb = max([configs.host_layer_layout(n, tiled=True)[3] for n in sizes_t] +
             [configs.host_layer_layout(n)[3] for n in sizes_p])
    with stream_pieces(2):
        ls, prm = synth_stream(sizes, sid, max_bytes=mb, f32=True)
    w = [T.zeros(n, dtype=T.int16, device="cuda") for n in sizes]
    norms = np.zeros(len(sizes))
    for t in range(1, 4):
        prm.step = t
        log("fp32-gradient stream step", t)
        L = np.concatenate([ht.table(t, grad_dtype=lso.LSO_DT_F32), hp.table(t, grad_dtype=lso.LSO_DT_F32)])
        L["dev_weight"] = [int(x.data_ptr()) for x in w]
        L["sq_norm"] = [norms.ctypes.data + 8 * i for i in range(len(sizes))]
        ls.stream_layers(L)
        for b, n in enumerate(sizes):
            g = synth.normal_f32(n, stream=sid, block=b, purpose=2, step=t, sigma=1e-3)
            oracle.adam_step(ref[b]["master"], ref[b]["m"], ref[b]["v"], g, ref[b]["weight"], t,
                             LR, B1, B2, EPS)
            want = oracle.sq_norm(g)
            assert abs(norms[b] - want) <= 2e-6 * want, (t, b, norms[b], want)
    T.cuda.synchronize()
    ls.close()
    scale = call_scale(ref)
    for b in range(len(sizes)):
        h, k = (ht, b) if b < len(sizes_t) else (hp, b - len(sizes_t))
        got = dict(master=h.get(k, "master"), m=h.get(k, "m"), v=h.get(k, "v"),
                   weight=w[b].cpu().numpy().view(np.uint16))
        assert_parity(got, ref[b], 1e-6, f"fp32-gradient streamed layer {b}", scale)


def test_stream_gradient_buffers_grow_for_fp32_and_bf16_still_works():
    """One context: a BF16 call, then an FP32-gradient call (its gradient
    buffers grow to 4 bytes per parameter), then BF16 again -- the BF16
    layers match a fresh context's bit for bit and the FP32 layers match
    the resident FP32-gradient update bit for bit."""
    T = torch()
    sizes = [70001, 12345]
    sid = 51
    a = HostLayers(sizes, sid)          # BF16 layers, streamed by one context throughout
    a_ref = HostLayers(sizes, sid)      # the same through a fresh BF16-only context
    f = HostLayers(sizes, sid + 1)      # FP32-gradient layers
    fn16, P = synth.grad_callback()
    fn32, _ = synth.grad_callback(f32=True)
    mode = {"f32": False}
    p16 = P(seed=synth.SEED, stream=sid, purpose=synth.PURPOSE_GRAD, step=1,
            scale=synth.scale_for(1e-3), block_base=0)
    p32 = P(seed=synth.SEED, stream=sid + 1, purpose=synth.PURPOSE_GRAD, step=1,
            scale=synth.scale_for(1e-3), block_base=0)
    c16 = ctypes.cast(fn16, ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t,
                                             ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p))
    c32 = ctypes.cast(fn32, ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t,
                                             ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p))

    def producer(layer, g, n, s):
        if mode["f32"]:
            return c32(ctypes.addressof(p32), layer, g, n, s)
        return c16(ctypes.addressof(p16), layer, g, n, s)

    mb = max(configs.host_layer_layout(n)[3] for n in sizes)
    ls = lso.LayerStream(mb, max(sizes), producer)
    ls_ref, pr = synth_stream(sizes, sid)
    for t, f32 in ((1, False), (1, True), (2, False), (2, True), (3, False)):
        log("grow step", t, "f32" if f32 else "bf16")
        mode["f32"] = f32
        p16.step = p32.step = pr.step = t
        if f32:
            ls.stream_layers(f.table(t, grad_dtype=lso.LSO_DT_F32))
        else:
            ls.stream_layers(a.table(t))
            ls_ref.stream_layers(a_ref.table(t))
    ls.close()
    ls_ref.close()
    for b in range(len(sizes)):
        assert np.array_equal(a.raw(b), a_ref.raw(b)), b
    # the FP32-gradient layers against lso_adam_step with FP32 gradients
    res = []
    for b, n in enumerate(sizes):
        res.append(dict(master=T.from_numpy(synth.normal_f32(n, stream=sid + 1, block=b, purpose=0,
                                                             step=0, sigma=0.02)).cuda(),
                        m=T.zeros(n, dtype=T.float32, device="cuda"),
                        v=T.zeros(n, dtype=T.float32, device="cuda"),
                        g=T.empty(n, dtype=T.float32, device="cuda"),
                        w=T.empty(n, dtype=T.int16, device="cuda")))
    for t in (1, 2):
        rows = []
        for b, n in enumerate(sizes):
            synth.device_fill_normal_f32(res[b]["g"].data_ptr(), n, stream=sid + 1, block=b, purpose=2,
                                         step=t, sigma=1e-3,
                                         hip_stream=T.cuda.current_stream().cuda_stream)
            rows.append(dict(n=n, master=res[b]["master"], m=res[b]["m"], v=res[b]["v"],
                             grad=res[b]["g"], weight=res[b]["w"], t=t, grad_dtype=lso.LSO_DT_F32))
        lso.adam_step(lso.BlockTable.from_rows(rows))
    T.cuda.synchronize()
    for b in range(len(sizes)):
        for q in ("master", "m", "v"):
            assert np.array_equal(f.get(b, q).view(np.uint32), res[b][q].cpu().numpy().view(np.uint32)), (b, q)


def test_stream_rejects_unknown_gradient_dtype_and_reserved_bits():
    """grad_dtype outside {0, BF16, FP32} is LSO_E_DTYPE and a nonzero
    reserved field LSO_E_INVALID, both before anything moves: the host
    blocks keep their bytes."""
    sizes = [5000, 300]
    host = HostLayers(sizes, 52)
    before = [host.raw(b) for b in range(len(sizes))]
    ls, prm = synth_stream(sizes, 52)
    L = host.table(1)
    L[1]["grad_dtype"] = 7
    assert ls.stream_layers_status(L) == _native.LSO_E_DTYPE
    L = host.table(1)
    L[0]["reserved"] = 1
    assert ls.stream_layers_status(L) == _native.LSO_E_INVALID
    ls.close()
    for b in range(len(sizes)):
        assert np.array_equal(host.raw(b), before[b]), b
