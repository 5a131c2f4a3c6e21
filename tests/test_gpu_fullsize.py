"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times, on sampled outputs.

The state of the 1.1B / 6.7B-parameter workloads is initialised and its
gradients drawn on the device (device input generator); the oracle rebuilds
just the sampled elements from the host input generator (same counter-based
generator, bit-identical -- checked by test_gpu_stream) and runs the same
steps on them.  Samples per block: 65,536 elements at offset 0, the last
65,536 (ragged end), and six seeded 16-aligned offsets.
"""
import numpy as np
import pytest

import layer_streamed_optimizer_amd as lso
import oracle
import synth
from layer_streamed_optimizer_amd import configs

from gpu_util import TILE, assert_parity, call_scale, log, max_errors, torch

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


def run_resident_sampled(key, steps, tiled=True):
    """The benchmark's configuration: tiled state for the large workloads."""
    T = torch()
    w = configs.get(key)
    sid = configs.STREAM_ID[key]
    sizes = [b.n for b in w.blocks]
    lay = configs.ResidentLayout(sizes, tiled=tiled)
    log(f"{key}: {w.params:,} params, {len(sizes)} blocks, {steps} steps, tiled={tiled}")
    hs = T.cuda.current_stream().cuda_stream
    state = T.empty(lay.state_bytes, dtype=T.uint8, device="cuda")
    grad = T.empty(lay.grad_bytes, dtype=T.uint8, device="cuda")
    weight = T.empty(lay.weight_bytes, dtype=T.uint8, device="cuda")
    sb, gb, wb = int(state.data_ptr()), int(grad.data_ptr()), int(weight.data_ptr())
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
    rows = [dict(n=n, master=sb + lay.off_master[b], m=sb + lay.off_m[b], v=sb + lay.off_v[b],
                 grad=gb + lay.off_grad[b], weight=wb + lay.off_weight[b], layout=layout)
            for b, n in enumerate(sizes)]
    table = lso.BlockTable.from_rows(rows)
    for t in range(1, steps + 1):
        for b, n in enumerate(sizes):
            synth.device_fill_normal_bf16(gb + lay.off_grad[b], n, stream=sid, block=b,
                                          purpose=synth.PURPOSE_GRAD, step=t,
                                          sigma=configs.GRAD_SIGMA, hip_stream=hs)
        table.set_step(t)
        lso.adam_step(table, hs)
    T.cuda.synchronize()
    # oracle on the samples
    refs, gots, where = [], [], []
    for b, spec in enumerate(w.blocks):
        for off, ln in sample_offsets(spec.n, 1000 + b):
            kind = init_kind(spec)
            if kind is None:
                master = np.zeros(ln, np.float32)
            else:
                master = synth.normal_f32(ln, stream=sid, block=b, purpose=kind[0], step=0,
                                          sigma=kind[1], start=off)
            ref = dict(master=master, m=np.zeros(ln, np.float32), v=np.zeros(ln, np.float32),
                       weight=np.zeros(ln, np.uint16))
            for t in range(1, steps + 1):
                g = synth.normal_bf16(ln, stream=sid, block=b, purpose=synth.PURPOSE_GRAD, step=t,
                                      sigma=configs.GRAD_SIGMA, start=off)
                oracle.adam_step(ref["master"], ref["m"], ref["v"], g, ref["weight"], t,
                                 configs.LR, configs.BETA1, configs.BETA2, configs.EPS)

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
    scale = call_scale(refs)
    worst = {}
    for ref, got, (b, off) in zip(refs, gots, where):
        assert_parity(got, ref, 1e-6, f"{key} block {b} offset {off}", scale)
        for k, v in max_errors(got, ref, scale).items():
            worst[k] = max(worst.get(k, 0.0), v)
    log(f"{key} sampled max errors after {steps} steps", worst)
    del state, grad, weight
    T.cuda.empty_cache()


def test_c1_tinyllama_full_size_sampled():
    run_resident_sampled("c1", 10)


def test_c1_tinyllama_full_size_sampled_planar():
    run_resident_sampled("c1", 10, tiled=False)


def test_c3_llama7b_full_size_sampled():
    T = torch()
    free, _ = T.cuda.mem_get_info()
    if free < 130e9:
        pytest.skip("needs ~125 GB of free device memory")
    run_resident_sampled("c3", 5)


@pytest.mark.parametrize("tiled", [True, False], ids=["tiled_in_pieces", "planar"])
def test_c4_layer_shape_streamed_sampled(tiled):
    """Three full 70B-shaped layers (855,654,400 params each, 10.27 GB host
    blocks) streamed for three steps through the same pipeline the benchmark
    times (tiled state moves in ~1 GiB pieces); sampled parity of the
    authoritative host state."""
    import ctypes
    T = torch()
    sid = configs.STREAM_ID["c4"]
    n = configs.layer_params(**configs.LLAMA70B)
    om, omm, ov, nbytes = configs.host_layer_layout(n, tiled=tiled)
    n_layers, steps = 3, 3
    log(f"c4 layer shape: {n_layers} x {n:,} params, {nbytes / 1e9:.2f} GB host blocks, tiled={tiled}")
    hs = T.cuda.current_stream().cuda_stream
    hosts = []
    stage = T.empty(nbytes, dtype=T.uint8, device="cuda")
    scratch = T.empty(n, dtype=T.float32, device="cuda") if tiled else None
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    for b in range(n_layers):
        hb = lso.host_alloc(nbytes)
        synth.device_fill_zero(int(stage.data_ptr()), nbytes, hs)
        dst = int(scratch.data_ptr()) if tiled else int(stage.data_ptr()) + om
        synth.device_fill_normal_f32(dst, n, stream=sid, block=b, purpose=synth.PURPOSE_MASTER, step=0,
                                     sigma=configs.MASTER_SIGMA, hip_stream=hs)
        if tiled:
            lso.tiled_pack(int(stage.data_ptr()) + om, dst, None, None, n=n, stream=hs)
        T.cuda.synchronize()
        assert hip.hipMemcpy(hb.ptr, int(stage.data_ptr()), nbytes, 2) == 0
        hosts.append(hb)
    del stage, scratch
    fn, Params = synth.grad_callback()
    prm = Params(seed=synth.SEED, stream=sid, purpose=synth.PURPOSE_GRAD, step=1,
                 scale=synth.scale_for(configs.GRAD_SIGMA), block_base=0)
    ls = lso.LayerStream(nbytes, n, fn, ctypes.addressof(prm))
    L = lso.LayerStream.layers(n_layers)
    for b in range(n_layers):
        L[b]["host_base"], L[b]["bytes"], L[b]["n"] = hosts[b].ptr, nbytes, n
        L[b]["off_master"], L[b]["off_m"], L[b]["off_v"] = om, omm, ov
        L[b]["layout"] = lso.LSO_LAYOUT_TILED if tiled else lso.LSO_LAYOUT_PLANAR
        L[b]["lr"], L[b]["beta1"], L[b]["beta2"], L[b]["eps"] = (configs.LR, configs.BETA1,
                                                                 configs.BETA2, configs.EPS)
    for t in range(1, steps + 1):
        prm.step = t
        L["t"] = t
        log(f"c4 streamed step {t}")
        ls.stream_layers(L)
    ls.close()
    refs, gots = [], []
    for b in range(n_layers):
        # the piece boundaries of a tiled layer fall on multiples of 10,922 tiles
        extra = [10922 * TILE - SAMPLE // 2] if tiled else []
        for off, ln in sample_offsets(n, 2000 + b) + [(o, SAMPLE) for o in extra]:
            ref = dict(master=synth.normal_f32(ln, stream=sid, block=b, purpose=synth.PURPOSE_MASTER,
                                               step=0, sigma=configs.MASTER_SIGMA, start=off),
                       m=np.zeros(ln, np.float32), v=np.zeros(ln, np.float32))
            for t in range(1, steps + 1):
                g = synth.normal_bf16(ln, stream=sid, block=b, purpose=synth.PURPOSE_GRAD, step=t,
                                      sigma=configs.GRAD_SIGMA, start=off)
                oracle.adam_step(ref["master"], ref["m"], ref["v"], g, None, t, configs.LR,
                                 configs.BETA1, configs.BETA2, configs.EPS)
            if tiled:
                t0, t1 = off // TILE, (off + ln - 1) // TILE + 1
                reg = hosts[b].view(np.float32, om + 12 * TILE * t0, 3 * TILE * (t1 - t0))
                reg = reg.reshape(t1 - t0, 3, TILE)
                lo = off - t0 * TILE
                got = {q: reg[:, k, :].ravel()[lo: lo + ln].copy()
                       for k, q in enumerate(("master", "m", "v"))}
            else:
                got = {q: hosts[b].view(np.float32, o + 4 * off, ln).copy()
                       for q, o in (("master", om), ("m", omm), ("v", ov))}
            refs.append(ref)
            gots.append(got)
    scale = call_scale(refs)
    for i, (ref, got) in enumerate(zip(refs, gots)):
        assert_parity(got, ref, 1e-6, f"c4 sample {i}", scale)
    for hb in hosts:
        hb.close()


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
    refs, gots = [], []
    for off in offs:
        ref = dict(master=synth.normal_f32(SAMPLE, stream=sid, block=0, purpose=0, step=0, sigma=0.02,
                                           start=off),
                   m=np.zeros(SAMPLE, np.float32), v=np.zeros(SAMPLE, np.float32),
                   weight=np.zeros(SAMPLE, np.uint16))
        for t in (1, 2):
            g = synth.normal_bf16(SAMPLE, stream=sid, block=0, purpose=2, step=t, sigma=1e-3, start=off)
            oracle.adam_step(ref["master"], ref["m"], ref["v"], g, ref["weight"], t, configs.LR,
                             configs.BETA1, configs.BETA2, configs.EPS)
        if tiled:
            got = read_tiled(state, 0, off, SAMPLE)
        else:
            got = {q: state[k * a + 4 * off: k * a + 4 * (off + SAMPLE)].cpu().numpy()
                   .view(np.float32).copy() for k, q in enumerate(("master", "m", "v"))}
        got["weight"] = weight[2 * off: 2 * (off + SAMPLE)].cpu().numpy().view(np.uint16).copy()
        refs.append(ref)
        gots.append(got)
    scale = call_scale(refs)
    for off, ref, got in zip(offs, refs, gots):
        assert_parity(got, ref, 1e-6, f"element offset {off}", scale)
    del state, grad, weight
    T.cuda.empty_cache()
