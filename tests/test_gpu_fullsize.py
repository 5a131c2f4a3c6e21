"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times, on sampled outputs.

The state of the 1.1B / 6.7B-parameter workloads is initialised and its
gradients drawn on the device (device input generator); the oracle rebuilds
just the sampled elements from the host input generator (same counter-based
generator, bit-identical -- checked by test_gpu_stream) and runs the same
steps on them.  Samples per block: 65,536 elements at offset 0, the last
65,536 (ragged end), and six seeded 16-aligned offsets.  Every sample is
judged twice: against the FP64 oracle within the parity bound, and bit for
bit against the binary32 emulation of the kernel's own arithmetic
(tests/fp32_exact.py).
"""
import numpy as np
import pytest

import layer_streamed_optimizer_amd as lso
import oracle
import synth
import fp32_exact as fx
from layer_streamed_optimizer_amd import configs

from gpu_util import TILE, Worst, assert_parity, log, torch

pytestmark = pytest.mark.gpu

SAMPLE = 65536


def sample_offsets(n, seed):
    if n <= SAMPLE:
        return [(0, n)]
    rng = np.random.default_rng(seed)
    offs = {0, n - SAMPLE}
    while len(offs) < 8:
        offs.add(int(rng.integers(0, (n - SAMPLE) // 16)) * 16)
    return [(o, SAMPLE) for o in sorted(offs)]


def read_tiled(state, region_off, start, count):
    """master, m, v of elements [start, start + count) of a tiled region,
    de-tiled on the host from the covering tiles."""
    t0, t1 = start // TILE, (start + count - 1) // TILE + 1
    raw = state[region_off + 12 * TILE * t0: region_off + 12 * TILE * t1].cpu().numpy()
    reg = raw.view(np.float32).reshape(t1 - t0, 3, TILE)
    lo = start - t0 * TILE
    return {q: reg[:, k, :].ravel()[lo: lo + count].copy() for k, q in enumerate(("master", "m", "v"))}


def init_kind(spec):
    if spec.init == "zero":
        return None
    if spec.init == "lora_a":
        return synth.PURPOSE_LORA_A, configs.LORA_A_SIGMA
    return synth.PURPOSE_MASTER, configs.MASTER_SIGMA


def assert_bits(got, want, what):
    """Every array of got (read back) equals want's (the binary32 emulation)
    bit for bit."""
    for q, arr in want.items():
        if q not in got:
            continue
        g = np.ascontiguousarray(got[q])
        dt = np.uint16 if arr.dtype == np.uint16 else np.uint32
        bad = np.nonzero(g.view(dt) != np.ascontiguousarray(arr).view(dt))[0]
        assert bad.size == 0, (f"{what}: {q} differs from the binary32 emulation at {bad.size} "
                               f"elements, first at element {int(bad[0])} of the sample")


def emulate(master, grads, steps, weights=True):
    """The kernel's binary32 sequence over `steps` steps (vectorised; m = v =
    0 at the start); grads(t) gives step t's BF16 gradients."""
    p = np.asarray(master, np.float32).copy()
    m = np.zeros(p.size, np.float32)
    v = np.zeros(p.size, np.float32)
    w = None
    for t in range(1, steps + 1):
        c = fx.adam_constants(t, configs.LR, configs.BETA1, configs.BETA2, configs.EPS)
        p, m, v, w = fx.adam_binary32_v(p, m, v, grads(t), c)
    out = dict(master=p, m=m, v=v)
    if weights:
        out["weight"] = w
    return out


def run_resident_sampled(key, steps, tiled=True, grad_f32=False):
    """The benchmark's configuration: tiled state for the large workloads
    (grad_f32: FP32 gradients instead of BF16)."""
    T = torch()
    w = configs.get(key)
    sid = configs.STREAM_ID[key]
    sizes = [b.n for b in w.blocks]
    lay = configs.BlockArena(sizes, tiled=tiled, grad_f32=grad_f32)   # the bench's arrangement
    log(f"{key}: {w.params:,} params, {len(sizes)} blocks, {steps} steps, tiled={tiled}, f32 grads={grad_f32}")
    hs = T.cuda.current_stream().cuda_stream
    arena = T.empty(lay.total_bytes, dtype=T.uint8, device="cuda")
    state = grad = weight = arena
    sb = gb = wb = int(arena.data_ptr())
    scratch = T.empty(max(sizes), dtype=T.float32, device="cuda")
    for b, spec in enumerate(w.blocks):
        kind = init_kind(spec)
        dst = int(scratch.data_ptr()) if tiled else sb + lay.off_master[b]
        if kind is None:
            synth.device_fill_zero(dst, 4 * spec.n, hs)
        else:
            synth.device_fill_normal_f32(dst, spec.n, stream=sid, block=b,
                                         purpose=kind[0], step=0, sigma=kind[1], hip_stream=hs)
        if tiled:
            lso.tiled_pack(sb + lay.off_master[b], dst, None, None, n=spec.n, stream=hs)
        else:
            synth.device_fill_zero(sb + lay.off_m[b], 4 * spec.n, hs)
            synth.device_fill_zero(sb + lay.off_v[b], 4 * spec.n, hs)
    T.cuda.synchronize()
    del scratch
    layout = lso.LSO_LAYOUT_TILED if tiled else lso.LSO_LAYOUT_PLANAR
    gdt = lso.LSO_DT_F32 if grad_f32 else lso.LSO_DT_BF16
    rows = [dict(n=n, master=sb + lay.off_master[b], m=sb + lay.off_m[b], v=sb + lay.off_v[b],
                 grad=gb + lay.off_grad[0][b], weight=wb + lay.off_weight[b], layout=layout, grad_dtype=gdt)
            for b, n in enumerate(sizes)]
    fill_grad = synth.device_fill_normal_f32 if grad_f32 else synth.device_fill_normal_bf16
    host_grad = synth.normal_f32 if grad_f32 else synth.normal_bf16
    table = lso.BlockTable.from_rows(rows)
    for t in range(1, steps + 1):
        for b, n in enumerate(sizes):
            fill_grad(gb + lay.off_grad[0][b], n, stream=sid, block=b, purpose=synth.PURPOSE_GRAD,
                      step=t, sigma=configs.GRAD_SIGMA, hip_stream=hs)
        table.set_step(t)
        lso.adam_step(table, hs)
    T.cuda.synchronize()
    # oracle on the samples
    refs, gots, where, exact = [], [], [], []
    for b, spec in enumerate(w.blocks):
        for off, ln in sample_offsets(spec.n, 1000 + b):
            kind = init_kind(spec)
            if kind is None:
                master = np.zeros(ln, np.float32)
            else:
                master = synth.normal_f32(ln, stream=sid, block=b, purpose=kind[0], step=0,
                                          sigma=kind[1], start=off)
            ref = dict(master=master.copy(), m=np.zeros(ln, np.float32), v=np.zeros(ln, np.float32),
                       weight=np.zeros(ln, np.uint16))
            gs = [host_grad(ln, stream=sid, block=b, purpose=synth.PURPOSE_GRAD, step=t,
                            sigma=configs.GRAD_SIGMA, start=off) for t in range(1, steps + 1)]
            for t in range(1, steps + 1):
                oracle.adam_step(ref["master"], ref["m"], ref["v"], gs[t - 1], ref["weight"], t,
                                 configs.LR, configs.BETA1, configs.BETA2, configs.EPS)
            exact.append(emulate(master, lambda t, gs=gs: gs[t - 1], steps))

            def rd(buf, byte_off, es, dt):
                return buf[byte_off: byte_off + es * ln].cpu().numpy().view(dt)

            if tiled:
                got = read_tiled(state, lay.off_master[b], off, ln)
            else:
                got = dict(master=rd(state, lay.off_master[b] + 4 * off, 4, np.float32),
                           m=rd(state, lay.off_m[b] + 4 * off, 4, np.float32),
                           v=rd(state, lay.off_v[b] + 4 * off, 4, np.float32))
            got["weight"] = rd(weight, lay.off_weight[b] + 2 * off, 2, np.uint16)
            refs.append(ref)
            gots.append(got)
            where.append((b, off))
    worst = Worst()
    for ref, got, (b, off), ex in zip(refs, gots, where, exact):
        worst.add(f"block {b} offset {off}", assert_parity(got, ref, 1e-6, f"{key} block {b} offset {off}"))
        assert_bits(got, ex, f"{key} block {b} offset {off}")
    log(f"{key} sampled worst errors after {steps} steps: {worst}")
    log(f"{key}: every sample equals the binary32 emulation bit for bit")
    del state, grad, weight, arena
    T.cuda.empty_cache()


def test_c1_tinyllama_full_size_sampled():
    run_resident_sampled("c1", 10)


def test_c1_tinyllama_full_size_sampled_planar():
    run_resident_sampled("c1", 10, tiled=False)


def test_c1_tinyllama_full_size_sampled_f32_grads():
    run_resident_sampled("c1", 10, grad_f32=True)


def test_c3_llama7b_full_size_sampled():
    T = torch()
    free, _ = T.cuda.mem_get_info()
    if free < 130e9:
        pytest.skip("needs ~125 GB of free device memory")
    run_resident_sampled("c3", 5)


PIECE_BYTES = 512 << 20   # the stream's default largest piece of a tiled layer


def piece_starts(n, piece_bytes=PIECE_BYTES):
    """First element of every piece after the first of a tiled layer block:
    the layer's tiles spread evenly over as many pieces as pieces of at most
    piece_bytes take, the first (tiles % pieces) of them one tile longer
    (the rule of the stream's piece plan, restated)."""
    per = max(1, piece_bytes // (12 * TILE))
    tiles = (n + TILE - 1) // TILE
    if tiles <= per:
        return []
    k_n = (tiles + per - 1) // per
    q, r = divmod(tiles, k_n)
    return [(k * q + min(k, r)) * TILE for k in range(1, k_n)]


def make_host_layers(n_layers, n, tiled, pinned, sid):
    """Authoritative host blocks of n_layers 70B-shaped layers: master drawn
    on the device (the device generator equals the host one bit for bit),
    m = v = 0, copied down; page-locked (lso_host_alloc) or pageable."""
    import ctypes
    T = torch()
    om, omm, ov, nbytes = configs.host_layer_layout(n, tiled=tiled)
    hs = T.cuda.current_stream().cuda_stream
    stage = T.empty(nbytes, dtype=T.uint8, device="cuda")
    scratch = T.empty(n, dtype=T.float32, device="cuda") if tiled else None
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    hosts, ptrs = [], []
    for b in range(n_layers):
        if pinned:
            hb = lso.host_alloc(nbytes)
            ptr = hb.ptr
        else:
            hb = np.empty(nbytes, dtype=np.uint8)
            ptr = hb.ctypes.data
        synth.device_fill_zero(int(stage.data_ptr()), nbytes, hs)
        dst = int(scratch.data_ptr()) if tiled else int(stage.data_ptr()) + om
        synth.device_fill_normal_f32(dst, n, stream=sid, block=b, purpose=synth.PURPOSE_MASTER, step=0,
                                     sigma=configs.MASTER_SIGMA, hip_stream=hs)
        if tiled:
            lso.tiled_pack(int(stage.data_ptr()) + om, dst, None, None, n=n, stream=hs)
        T.cuda.synchronize()
        assert hip.hipMemcpy(ptr, int(stage.data_ptr()), nbytes, 2) == 0
        hosts.append(hb)
        ptrs.append(ptr)
        if b % 4 == 3 or b == n_layers - 1:
            log(f"host layers ready: {b + 1} of {n_layers}")
    del stage, scratch
    return hosts, ptrs, (om, omm, ov, nbytes)


def host_view(hb, pinned):
    """(float32 view of a host block, by byte offset and count)."""
    if pinned:
        return lambda off, cnt: hb.view(np.float32, off, cnt)
    return lambda off, cnt: hb[off: off + 4 * cnt].view(np.float32)


def oracle_samples(sid, layer, spans, steps, weights=False):
    """The oracle's state after `steps` steps for each (offset, length)
    span of a 70B-shaped layer, rebuilt from the host generator, and the
    binary32 emulation's (what the kernel must hold bit for bit)."""
    out, exact = [], []
    for off, ln in spans:
        master = synth.normal_f32(ln, stream=sid, block=layer, purpose=synth.PURPOSE_MASTER,
                                  step=0, sigma=configs.MASTER_SIGMA, start=off)
        ref = dict(master=master.copy(), m=np.zeros(ln, np.float32), v=np.zeros(ln, np.float32))
        if weights:
            ref["weight"] = np.zeros(ln, np.uint16)
        gs = [synth.normal_bf16(ln, stream=sid, block=layer, purpose=synth.PURPOSE_GRAD, step=t,
                                sigma=configs.GRAD_SIGMA, start=off) for t in range(1, steps + 1)]
        for t in range(1, steps + 1):
            oracle.adam_step(ref["master"], ref["m"], ref["v"], gs[t - 1], ref.get("weight"), t, configs.LR,
                             configs.BETA1, configs.BETA2, configs.EPS)
        out.append(ref)
        exact.append(emulate(master, lambda t, gs=gs: gs[t - 1], steps, weights))
    return out, exact


def read_host_sample(view, tiled, lay, off, ln):
    om, omm, ov, _ = lay
    if tiled:
        t0, t1 = off // TILE, (off + ln - 1) // TILE + 1
        reg = view(om + 12 * TILE * t0, 3 * TILE * (t1 - t0)).reshape(t1 - t0, 3, TILE)
        lo = off - t0 * TILE
        return {q: reg[:, k, :].ravel()[lo: lo + ln].copy() for k, q in enumerate(("master", "m", "v"))}
    return {q: view(o + 4 * off, ln).copy() for q, o in (("master", om), ("m", omm), ("v", ov))}


def run_streamed_sampled(n_layers, tiled, pinned, steps=3, check_weights=False):
    """n_layers full 70B-shaped layers streamed for `steps` steps through
    the stream's default pipeline; sampled parity of the authoritative host
    state of every layer (start, ragged end, six seeded offsets, and for a
    tiled layer the last and first elements around every piece boundary)
    and, with check_weights, of the BF16 re-cast the last two layers leave
    in the device slots."""
    import ctypes
    T = torch()
    sid = configs.STREAM_ID["c4"]
    n = configs.layer_params(**configs.LLAMA70B)
    log(f"c4 layer shape: {n_layers} x {n:,} params, tiled={tiled}, pinned={pinned}, {steps} steps")
    hosts, ptrs, lay = make_host_layers(n_layers, n, tiled, pinned, sid)
    om, omm, ov, nbytes = lay
    fn, Params = synth.grad_callback()
    prm = Params(seed=synth.SEED, stream=sid, purpose=synth.PURPOSE_GRAD, step=1,
                 scale=synth.scale_for(configs.GRAD_SIGMA), block_base=0)
    ls = lso.LayerStream(nbytes, n, fn, ctypes.addressof(prm))
    mode = ls.copy_mode()
    log(f"copy mode {mode}")
    L = lso.LayerStream.layers(n_layers)
    for b in range(n_layers):
        L[b]["host_base"], L[b]["bytes"], L[b]["n"] = ptrs[b], nbytes, n
        L[b]["off_master"], L[b]["off_m"], L[b]["off_v"] = om, omm, ov
        L[b]["layout"] = lso.LSO_LAYOUT_TILED if tiled else lso.LSO_LAYOUT_PLANAR
        L[b]["lr"], L[b]["beta1"], L[b]["beta2"], L[b]["eps"] = (configs.LR, configs.BETA1,
                                                                 configs.BETA2, configs.EPS)
    for t in range(1, steps + 1):
        prm.step = t
        L["t"] = t
        log(f"c4 streamed step {t}")
        ls.stream_layers(L)
    # the BF16 re-cast of the last two layers, still in the slots (slot = layer % 2)
    slot_w = {b: ls.slot_weight(b % 2) for b in range(max(0, n_layers - 2), n_layers)} if check_weights else {}
    worst = Worst()
    bounds = piece_starts(n) if tiled else []
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    wdev = T.empty(SAMPLE, dtype=T.int16, device="cuda") if slot_w else None
    for b in range(n_layers):
        spans = sample_offsets(n, 2000 + b)
        # just before and just after every piece boundary
        spans += [(p - SAMPLE // 2, SAMPLE) for p in bounds]
        refs, exact = oracle_samples(sid, b, spans, steps, weights=b in slot_w)
        view = host_view(hosts[b], pinned)
        for (off, ln), ref, ex in zip(spans, refs, exact):
            got = read_host_sample(view, tiled, lay, off, ln)
            if b in slot_w:
                assert hip.hipMemcpy(int(wdev.data_ptr()), slot_w[b] + 2 * off, 2 * ln, 3) == 0
                got["weight"] = wdev[:ln].cpu().numpy().view(np.uint16).copy()
            worst.add(f"layer {b} offset {off}",
                      assert_parity(got, ref, 1e-6, f"c4 layer {b} offset {off} (n={ln})"))
            assert_bits(got, ex, f"c4 layer {b} offset {off}")
        log(f"layer {b}: {len(spans)} samples checked, each bit for bit")
    log(f"c4 {n_layers} layers, {steps} steps, worst errors: {worst}")
    ls.close()
    if pinned:
        for hb in hosts:
            hb.close()
    hosts.clear()


@pytest.mark.parametrize("tiled", [True, False], ids=["tiled_in_pieces", "planar"])
def test_c4_layer_shape_streamed_sampled(tiled):
    """Three full 70B-shaped layers (855,654,400 params each, 10.27 GB
    page-locked host blocks) streamed for three steps; sampled parity of
    the authoritative host state, the piece boundaries of a tiled layer
    included."""
    run_streamed_sampled(3, tiled, pinned=True)


def test_c4_benchmark_configuration_16_pageable_layers():
    """The streamed configuration the benchmark times: all 16 layers of the
    70B-shaped slice, tiled state in pageable host memory (164 GB) staged
    through pinned buffers, moved in 512 MiB pieces on the default copy
    engines, three steps.  Every layer is sampled (its piece boundaries
    too), and the BF16 weights the last two layers leave in the device slots
    are checked against the oracle's re-cast."""
    mem = {}
    with open("/proc/meminfo") as f:
        for line in f:
            k, v = line.split(":", 1)
            mem[k] = int(v.split()[0]) * 1024
    need = 16 * configs.host_layer_layout(configs.layer_params(**configs.LLAMA70B), tiled=True)[3]
    if mem.get("MemAvailable", 0) < need + (24 << 30):
        pytest.skip(f"needs {need / 1e9:.0f} GB of host memory plus headroom")
    run_streamed_sampled(16, True, pinned=False, check_weights=True)


@pytest.mark.parametrize("tiled", [False, True], ids=["planar", "tiled"])
def test_block_of_more_than_2_32_elements_sampled(tiled):
    """One block of 2^32 + 2^17 + 4097 elements (64-bit element offsets, a
    ragged end; 69 GB of state, gradients and weights): sampled parity after
    two steps, including the elements around 2^31 and 2^32."""
    T = torch()
    free, _ = T.cuda.mem_get_info()
    if free < 80e9:
        pytest.skip("needs ~70 GB of free device memory")
    n = (1 << 32) + (1 << 17) + 4097
    sid = 77
    log(f"one block of {n:,} elements, tiled={tiled}")
    hs = T.cuda.current_stream().cuda_stream
    a = (4 * n + 4095) // 4096 * 4096          # planar arrays on 4 KB boundaries
    sbytes = lso.tiled_state_bytes(n) if tiled else 3 * a
    state = T.empty(sbytes, dtype=T.uint8, device="cuda")
    grad = T.empty(2 * n, dtype=T.uint8, device="cuda")
    weight = T.empty(2 * n, dtype=T.uint8, device="cuda")
    sb = int(state.data_ptr())
    if tiled:
        # master drawn planar, then packed with m = v = 0 into the tiled region
        master_tmp = T.empty(n, dtype=T.float32, device="cuda")
        synth.device_fill_normal_f32(int(master_tmp.data_ptr()), n, stream=sid, block=0, purpose=0,
                                     step=0, sigma=0.02, hip_stream=hs)
        lso.tiled_pack(sb, int(master_tmp.data_ptr()), None, None, n=n, stream=hs)
        T.cuda.synchronize()
        del master_tmp
        row = dict(n=n, master=sb, grad=grad, weight=weight, layout=lso.LSO_LAYOUT_TILED)
    else:
        synth.device_fill_normal_f32(sb, n, stream=sid, block=0, purpose=0, step=0, sigma=0.02,
                                     hip_stream=hs)
        synth.device_fill_zero(sb + a, 2 * a, hs)
        row = dict(n=n, master=sb, m=sb + a, v=sb + 2 * a, grad=grad, weight=weight)
    table = lso.BlockTable.from_rows([row])
    for t in (1, 2):
        synth.device_fill_normal_bf16(int(grad.data_ptr()), n, stream=sid, block=0, purpose=2, step=t,
                                      sigma=1e-3, hip_stream=hs)
        table.set_step(t)
        lso.adam_step(table, hs)
    T.cuda.synchronize()
    offs = [0, (1 << 31) - SAMPLE // 2, (1 << 32) - SAMPLE // 2, n - SAMPLE]
    refs, gots, exact = [], [], []
    for off in offs:
        master = synth.normal_f32(SAMPLE, stream=sid, block=0, purpose=0, step=0, sigma=0.02, start=off)
        ref = dict(master=master.copy(), m=np.zeros(SAMPLE, np.float32), v=np.zeros(SAMPLE, np.float32),
                   weight=np.zeros(SAMPLE, np.uint16))
        gs = [synth.normal_bf16(SAMPLE, stream=sid, block=0, purpose=2, step=t, sigma=1e-3, start=off)
              for t in (1, 2)]
        for t in (1, 2):
            oracle.adam_step(ref["master"], ref["m"], ref["v"], gs[t - 1], ref["weight"], t, configs.LR,
                             configs.BETA1, configs.BETA2, configs.EPS)
        exact.append(emulate(master, lambda t, gs=gs: gs[t - 1], 2))
        if tiled:
            got = read_tiled(state, 0, off, SAMPLE)
        else:
            got = {q: state[k * a + 4 * off: k * a + 4 * (off + SAMPLE)].cpu().numpy()
                   .view(np.float32).copy() for k, q in enumerate(("master", "m", "v"))}
        got["weight"] = weight[2 * off: 2 * (off + SAMPLE)].cpu().numpy().view(np.uint16).copy()
        refs.append(ref)
        gots.append(got)
    for off, ref, got, ex in zip(offs, refs, gots, exact):
        assert_parity(got, ref, 1e-6, f"element offset {off}")
        assert_bits(got, ex, f"element offset {off}")
    del state, grad, weight
    T.cuda.empty_cache()
