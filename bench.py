"""Benchmark of the per-layer mixed-precision Adam update on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config c3|c0|c1|c2|c4] [--gpus 1]

A step is one pass of the whole update over every block of the workload
(host constants, one ragged multi-tensor launch, the fused kernel) with
that step's gradients (BF16; FP32 with --grad-dtype f32) already resident
in HBM.  W untimed steps, then
K timed steps between two device synchronisations; one JSON line on stdout.

The default run is the LLaMA-7B-shaped resident update (c3, the HBM
headline), and nested in the same line under "streamed" the 70B-shaped
slice streamed from host memory (c4, the host-link headline: all 16
layers in pageable memory, 1 untimed and 3 timed steps of its own;
--no-streamed leaves it out).

Workloads (shapes from the pages, values synthetic, see
layer_streamed_optimizer_amd/configs.py):
  c0  one 1024x1024 block                                  (resident)
  c1  TinyLlama-1.1B shape, 25 blocks, 1,100,048,384 params (resident)
  c2  LoRA r=8 on TinyLlama, 308 ragged tensors, 6,307,840  (resident)
  c3  LLaMA-7B shape, 35 blocks, 6,738,415,616 params       (resident, ~108 GB, default)
  c4  70B-shaped slice, 16 layers of 855,654,400 params, streamed from
      ~164 GB of host memory                                 (streamed)
      --host-memory pageable (default) | pinned | file (the disk tier:
      one O_DIRECT file per layer, 6 layers by default)

Roofline: the fused kernel moves 28 algorithmic bytes per parameter (reads
2 g + 4 master + 4 m + 4 v, writes 4 + 4 + 4 + 2 w; 30 with FP32
gradients); its average launch
duration is measured with HIP events on the launch stream.  The CPU
baseline is the oracle (plain scalar FP64 C, all host cores) timed on a
bounded sample of the same workload: one full decoder-layer block for
the model-shaped workloads.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import mmap
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Gparams/s Adam step; % HBM peak (resident) / % host-link peak (streamed)"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
BYTES_PER_PARAM = {"bf16": 28, "f32": 30}   # algorithmic, resident kernel, by gradient dtype
REPEATS = 20                    # timed-region repeats for the launch-bound workloads
LINK_BYTES_PER_PARAM = 12       # streamed: [master | m | v] each way


def progress(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def environment() -> dict:
    """What the numbers were measured on."""
    import platform

    import torch

    env = dict(torch=torch.__version__, hip=getattr(torch.version, "hip", None),
               host_threads=os.cpu_count(), python=platform.python_version())
    try:
        p = torch.cuda.get_device_properties(0)
        env.update(gpu=p.name, gcn_arch=getattr(p, "gcnArchName", None),
                   gpu_memory_GB=round(p.total_memory / 1e9, 1), compute_units=p.multi_processor_count)
    except Exception as e:   # the record is informative only
        env["gpu"] = f"unavailable ({e})"
    try:
        with open("/proc/cpuinfo") as f:
            env["cpu"] = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
        with open("/proc/meminfo") as f:
            mem = {l.split(":")[0]: l.split(":")[1].strip() for l in f}
        env["host_memory_total"], env["host_memory_available"] = mem.get("MemTotal"), mem.get("MemAvailable")
        rocm = "/opt/rocm/.info/version"
        if os.path.exists(rocm):
            env["rocm"] = open(rocm).read().strip()
    except Exception:
        pass
    # kernel driver and board, where the system exposes them
    import glob
    for key, pattern in (("amdgpu_driver", "/sys/module/amdgpu/version"),
                         ("gpu_product", "/sys/class/drm/card*/device/product_name"),
                         ("gpu_vbios", "/sys/class/drm/card*/device/vbios_version")):
        for path in sorted(glob.glob(pattern)):
            try:
                value = open(path).read().strip()
            except OSError:
                continue
            if value:
                env[key] = value
                break
    return env


def kernel_hash() -> str:
    from layer_streamed_optimizer_amd.rocprof_summary import kernel_hash as kh
    return kh()


def measured_traffic(workload: str, grad_dtype: str = "bf16", norms: bool = False):
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source; else None."""
    tag = workload + ("" if grad_dtype == "bf16" else "_g32") + ("_norms" if norms else "")
    path = os.path.join(ROOT, "profiles", f"fused_adam_{tag}_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path, encoding="utf-8").read()
    m_hash = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_hash():
        return None
    return float(m_bytes.group(1))


# ------------------------------------------------------------ resident path

class HipEvents:
    """Timing events recorded with hipEventRecord on a raw stream handle:
    the launch stream's own events, with less host cost per record than a
    framework wrapper (which matters for steps of a few microseconds)."""

    def __init__(self, count: int):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(count):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(e.value)
        self.record = self.hip.hipEventRecord

    def ms(self, a: int, b: int) -> float:
        out = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(out), self.ev[a], self.ev[b]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return out.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)
        self.ev = []


def resident(args, w):
    import torch

    import layer_streamed_optimizer_amd as lso
    import synth
    from layer_streamed_optimizer_amd import configs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sid = configs.STREAM_ID[w.key]
    sizes = [b.n for b in w.blocks]
    tiled = args.layout == "tiled"
    g32 = args.grad_dtype == "f32"
    bpp = BYTES_PER_PARAM[args.grad_dtype]
    one = configs.ResidentLayout(sizes, tiled=tiled, grad_f32=g32)
    params = w.params
    total_steps = args.warmup + args.steps
    free, _total = torch.cuda.mem_get_info()
    scratch_bytes = 4 * max(sizes) if tiled else 0
    budget = free - one.state_bytes - one.weight_bytes - scratch_bytes - (8 << 30)
    n_sets = max(1, min(total_steps, budget // max(one.grad_bytes, 1)))
    if args.grad_sets:
        n_sets = max(1, min(n_sets, args.grad_sets))
    stream = torch.cuda.current_stream()
    hs = int(stream.cuda_stream)
    # A step that streams HBM (more than 1 GiB of traffic) gets one arena,
    # block after block [state | weights | gradient sets]: the arrays a
    # block's update streams together sit next to each other, which makes
    # its rate independent of where the arena lands.  A cache-sized step
    # (c0, c2) keeps three compact regions (states, weights, gradient sets):
    # spread over per-block groups its few hundred MB touch ten times the
    # pages, and c2 measured 34.0 us instead of 30.1.
    use_arena = bpp * params > (1 << 30)
    if args.arrangement != "auto":
        use_arena = args.arrangement == "arena"
    if use_arena:
        lay = configs.BlockArena(sizes, tiled=tiled, grad_f32=g32, grad_sets=n_sets)
        keep = [torch.empty(lay.total_bytes, dtype=torch.uint8, device=dev)]
        sb = wb = int(keep[0].data_ptr())
        grad_at = [[sb + o for o in lay.off_grad[r]] for r in range(n_sets)]
        arrangement = "one device arena, block after block [state | BF16 weights | gradient sets]"
    else:
        lay = one
        keep = [torch.empty(lay.state_bytes, dtype=torch.uint8, device=dev),
                torch.empty(lay.weight_bytes, dtype=torch.uint8, device=dev)]
        keep += [torch.empty(lay.grad_bytes, dtype=torch.uint8, device=dev) for _ in range(n_sets)]
        sb, wb = int(keep[0].data_ptr()), int(keep[1].data_ptr())
        grad_at = [[int(keep[2 + r].data_ptr()) + o for o in lay.off_grad] for r in range(n_sets)]
        arrangement = "three regions: all states, all BF16 weights, each gradient set"
    progress(f"{w.key}: {len(sizes)} blocks, {params:,} params, {args.layout} state "
             f"{lay.state_bytes / 1e9:.1f} GB, {n_sets} {args.grad_dtype} gradient sets of "
             f"{lay.grad_bytes / 1e9:.2f} GB; {arrangement}")
    scratch = torch.empty(max(sizes), dtype=torch.float32, device=dev) if tiled else None

    def fill_master(dst, b, spec):
        n = spec.n
        if spec.init == "zero":
            synth.device_fill_zero(dst, 4 * n, hs)
        else:
            lora = spec.init == "lora_a"
            synth.device_fill_normal_f32(
                dst, n, stream=sid, block=b,
                purpose=synth.PURPOSE_LORA_A if lora else synth.PURPOSE_MASTER, step=0,
                sigma=configs.LORA_A_SIGMA if lora else configs.MASTER_SIGMA, hip_stream=hs)

    def init_state():
        for b, spec in enumerate(w.blocks):
            if tiled:
                # master drawn planar, packed with m = v = 0 into the tiled region
                fill_master(int(scratch.data_ptr()), b, spec)
                lso.tiled_pack(sb + lay.off_master[b], int(scratch.data_ptr()), None, None,
                               n=spec.n, stream=hs)
            else:
                fill_master(sb + lay.off_master[b], b, spec)
                synth.device_fill_zero(sb + lay.off_m[b], 4 * spec.n, hs)
                synth.device_fill_zero(sb + lay.off_v[b], 4 * spec.n, hs)

    init_state()
    for r in range(n_sets):
        fill = synth.device_fill_normal_f32 if g32 else synth.device_fill_normal_bf16
        for b, n in enumerate(sizes):
            fill(grad_at[r][b], n, stream=sid, block=b, purpose=synth.PURPOSE_GRAD, step=r + 1,
                 sigma=configs.GRAD_SIGMA, hip_stream=hs)
    tables = []
    for r in range(n_sets):
        rows = [dict(n=n, master=sb + lay.off_master[b], m=sb + lay.off_m[b], v=sb + lay.off_v[b],
                     grad=grad_at[r][b], weight=wb + lay.off_weight[b], t=1,
                     lr=configs.LR, beta1=configs.BETA1, beta2=configs.BETA2, eps=configs.EPS,
                     layout=lso.LSO_LAYOUT_TILED if tiled else lso.LSO_LAYOUT_PLANAR,
                     grad_dtype=lso.LSO_DT_F32 if g32 else lso.LSO_DT_BF16)
                for b, n in enumerate(sizes)]
        tables.append(lso.BlockTable.from_rows(rows))
    # Upload every table once outside the timed region: an lr = 0 step
    # leaves the weights bit-exact; the moments are re-zeroed afterwards.
    for tab in tables:
        tab.arr["lr"] = 0.0
        lso.adam_step(tab, hs)
        tab.arr["lr"] = configs.LR
    init_state()
    torch.cuda.synchronize()
    progress("inputs resident; warming up")

    if args.norms:
        # the norm variant (progressive layer locking): per-block sums of g^2
        sq = torch.empty(len(sizes), dtype=torch.float64, device=dev)
        ws_bytes = lso.norm_workspace_bytes(tables[0])
        ws = torch.empty(max(ws_bytes, 8), dtype=torch.uint8, device=dev)

    def step(j):          # j = 1-based global step; grads of set (j-1) % n_sets
        tab = tables[(j - 1) % n_sets]
        tab.set_step(j)
        if args.norms:
            lso.adam_step_norms(tab, sq, ws, ws_bytes, hs)
        else:
            lso.adam_step(tab, hs)

    K = args.steps
    ev = HipEvents(max(2 * K, 2 * REPEATS))   # start of step k: 2k, end: 2k + 1
    rec = ev.record
    cold = None
    for j in range(1, args.warmup + 1):
        if j == 1:   # the first update of the run, timed on its own
            rec(ev.ev[0], hs)
            step(j)
            rec(ev.ev[1], hs)
            torch.cuda.synchronize()
            cold = ev.ms(0, 1)
        else:
            step(j)
    torch.cuda.synchronize()
    # The timed region: K steps back to back, one event at each end on the
    # launch stream (an event per step costs microseconds of host time,
    # which would dominate a small step).  Its GPU time over K is the
    # average launch duration when the launches run back to back, and an
    # upper bound of it otherwise.
    t0 = time.perf_counter()
    rec(ev.ev[0], hs)
    for k in range(K):
        step(args.warmup + 1 + k)
    rec(ev.ev[1], hs)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_ms = ev.ms(0, 1) / K
    achieved = bpp * params / (avg_ms * 1e-3) / 1e9
    # each launch on its own (a second pass, events around every step)
    for k in range(K):
        rec(ev.ev[2 * k], hs)
        step(args.warmup + K + 1 + k)
        rec(ev.ev[2 * k + 1], hs)
    torch.cuda.synchronize()
    kernel_ms = [ev.ms(2 * k, 2 * k + 1) for k in range(K)]
    j_next = args.warmup + 2 * K + 1
    repeats = None
    if w.key in ("c0", "c2"):
        # launch-latency-bound steps: the timed region again, REPEATS times,
        # and the median of its per-step time
        for r in range(REPEATS):
            rec(ev.ev[2 * r], hs)
            for k in range(K):
                step(j_next)
                j_next += 1
            rec(ev.ev[2 * r + 1], hs)
        torch.cuda.synchronize()
        per = sorted(ev.ms(2 * r, 2 * r + 1) / K for r in range(REPEATS))
        repeats = dict(regions=REPEATS, steps_each=K, median_us_per_step=per[REPEATS // 2] * 1e3,
                       min_us_per_step=per[0] * 1e3, max_us_per_step=per[-1] * 1e3)
    graph_rec = None
    if w.key in ("c0", "c2") and not args.norms:
        # the same steps captured into one HIP graph and replayed: the GPU's
        # own back-to-back time per step, without the host's submission
        # cost.  lso_adam_step is capturable here because every table is
        # already in the device-table cache (nothing is allocated or
        # uploaded); lso_adam_step_noalloc is capturable always (it writes
        # the table into its fixed array with a small kernel per 56 blocks).
        lso.adam_step_noalloc(tables[0], hs)   # (untimed) the scratch address is looked up once
        torch.cuda.synchronize()
        graph_rec = {}
        for name, fn in (("adam_step", lso.adam_step), ("adam_step_noalloc", lso.adam_step_noalloc)):
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
                cs = torch.cuda.current_stream().cuda_stream
                for k in range(K):
                    tab = tables[(j_next + k - 1) % n_sets]
                    tab.set_step(j_next + k)
                    fn(tab, cs)
            j_next += K
            graph.replay()
            torch.cuda.synchronize()
            gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(REPEATS)]
            for s_, e_ in gev:
                s_.record()
                graph.replay()
                e_.record()
            torch.cuda.synchronize()
            per = sorted(s_.elapsed_time(e_) / K for s_, e_ in gev)
            graph_rec[name] = dict(steps_per_replay=K, replays=REPEATS, median_us_per_step=per[REPEATS // 2] * 1e3,
                                   min_us_per_step=per[0] * 1e3,
                                   achieved_GBps=bpp * params / (per[REPEATS // 2] * 1e-3) / 1e9)
            del graph
        graph_rec["note"] = "K steps captured into one HIP graph per entry point, replayed; events around each replay"
        progress(f"graph replay: {graph_rec['adam_step']['median_us_per_step']:.1f} us per step "
                 f"({graph_rec['adam_step_noalloc']['median_us_per_step']:.1f} us through the no-alloc entry)")
    flushed = None
    if w.key in ("c0", "c2"):
        # these fit the 256 MB last-level cache: time the same steps again
        # with 512 MB written between them, so no state is cache-resident
        scratch_mall = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        for k in range(K):
            synth.device_fill_zero(int(scratch_mall.data_ptr()), 512 << 20, hs)
            rec(ev.ev[2 * k], hs)
            step(j_next)
            j_next += 1
            rec(ev.ev[2 * k + 1], hs)
        torch.cuda.synchronize()
        fl_ms = sorted(ev.ms(2 * k, 2 * k + 1) for k in range(K))
        f_avg = sum(fl_ms) / len(fl_ms)
        flushed = dict(kernel_avg_us=f_avg * 1e3, kernel_median_us=fl_ms[len(fl_ms) // 2] * 1e3,
                       achieved_GBps=bpp * params / (f_avg * 1e-3) / 1e9,
                       note="512 MB written between steps; the main figures are cache-resident")
        del scratch_mall
    ev.close()
    # the copy ceiling needs 16 GB: the inputs go first
    keep.clear()
    torch.cuda.empty_cache()
    ceiling = copy_ceiling(torch, dev)
    shaped = shaped_ceiling(torch, dev, tiled)
    progress(f"steps: wall {wall * 1e3:.3f} ms for {args.steps}; kernel avg {avg_ms * 1e3:.1f} us; "
             f"{achieved:.0f} GB/s; copy ceiling {ceiling:.0f} GB/s; update-shaped copy {shaped:.0f} GB/s")
    traffic = measured_traffic(w.key, args.grad_dtype, args.norms)
    result = dict(
        metric=METRIC, value=params * args.steps / wall / 1e9, unit="Gparams/s",
        ms_per_step=wall * 1e3 / args.steps,
        roofline=dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBPS, unit="GB/s",
                      frac=achieved / HBM_PEAK_GBPS, traffic=traffic),
        region_avg_us=avg_ms * 1e3,
        kernel_avg_us=sum(kernel_ms) / K * 1e3, kernel_min_us=min(kernel_ms) * 1e3,
        kernel_median_us=sorted(kernel_ms)[len(kernel_ms) // 2] * 1e3,
        kernel_first_step_us=cold * 1e3 if cold is not None else None,
        hbm_copy_ceiling_GBps=ceiling,
        frac_of_copy_ceiling=achieved / ceiling,
        hbm_update_shaped_copy_GBps=shaped,
        config=dict(workload=f"{w.key}: {w.title}", blocks=len(sizes), params=params,
                    state_layout=args.layout, grad_dtype=args.grad_dtype, bytes_per_param=bpp,
                    gradient_norms=bool(args.norms),
                    gradient_sets=n_sets,
                    arrays=arrangement,
                    hyper=dict(lr=configs.LR, beta1=configs.BETA1, beta2=configs.BETA2,
                               eps=configs.EPS)),
    )
    if repeats:
        result["region_repeats"] = repeats
    if flushed:
        result["cache_flushed"] = flushed
    if graph_rec:
        result["graph_replay"] = graph_rec
    del scratch
    return result


def copy_ceiling(torch, dev, nbytes=8 << 30) -> float:
    """GB/s (read + write) of a plain device copy: the measured HBM ceiling
    for a 1:1 read/write stream."""
    from layer_streamed_optimizer_amd import _native
    P = _native.probes()
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    hs = torch.cuda.current_stream().cuda_stream
    for _ in range(2):
        assert P.lso_probe_copy(a.data_ptr(), b.data_ptr(), nbytes, 0, hs) == 0
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    reps = 5
    for _ in range(reps):
        assert P.lso_probe_copy(a.data_ptr(), b.data_ptr(), nbytes, 0, hs) == 0
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    del a, b
    return 2 * nbytes / (ms * 1e-3) / 1e9


def shaped_ceiling(torch, dev, tiled: bool, n: int = 134_283 * 8192) -> float:
    """GB/s of the update's own traffic shape with no arithmetic: 14 bytes
    read and 14 written per element, in the same state layout and one
    1,024-element chunk per workgroup.  1.1 G elements (31 GB a pass), not a
    power of two, so the planar arrays do not sit a power of two apart."""
    from layer_streamed_optimizer_amd import _native
    P = _native.probes()
    state = torch.zeros(12 * n, dtype=torch.uint8, device=dev)
    grad = torch.zeros(2 * n, dtype=torch.uint8, device=dev)
    weight = torch.empty(2 * n, dtype=torch.uint8, device=dev)
    hs = torch.cuda.current_stream().cuda_stream
    args = (state.data_ptr(), grad.data_ptr(), weight.data_ptr(), n, int(tiled), hs)
    for _ in range(2):
        assert P.lso_probe_copy_shaped(*args) == 0
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    reps = 5
    for _ in range(reps):
        assert P.lso_probe_copy_shaped(*args) == 0
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    del state, grad, weight
    return 28 * n / (ms * 1e-3) / 1e9


def hbm_probe(nbytes: int = 8 << 30, reps: int = 6) -> dict:
    """The HBM ceiling for the update's 1:1 read/write traffic: every shape
    of lso_probe_copy_variant over nbytes, best-of-`reps` GB/s counting the
    bytes read plus the bytes written, each copy checked bit for bit."""
    import torch

    from layer_streamed_optimizer_amd import _native
    P = _native.probes()
    dev = torch.device("cuda:0")
    hs = torch.cuda.current_stream().cuda_stream
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    keep = src.clone()
    cases = [("base: 1 vector per lane, nt", 0, 0)]
    cases += [(f"direct-to-LDS read phase then write phase, {kb} KB per workgroup", 1, kb)
              for kb in (4, 8, 16, 32, 64)]
    cases += [(f"{p} vectors per lane in registers", 2, p) for p in (1, 2, 4, 8)]
    names = ["none", "nt", "sc1", "nt sc1", "sc0 sc1", "sc0 sc1 nt"]
    cases += [(f"cache policy: load {names[l]}, store {names[st]}", 3, l + 8 * st)
              for l in range(6) for st in range(6)]
    cases += [("in place (read and write the same addresses)", 4, 0), ("read only", 5, 0),
              ("write only", 6, 0)]
    cases += [(f"in place, load nt, store {names[st]}", 7, st) for st in range(6)]
    cases += [(f"{w}-byte vector per lane, load nt, store nt sc1", 8, w) for w in (4, 8, 16)]
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    rows = []
    for name, var, param in cases:
        dst.zero_()
        times = []
        for r in range(reps + 2):   # an even count: in place ends where it began
            s.record()
            rc = P.lso_probe_copy_variant(var, param, src.data_ptr(), dst.data_ptr(), nbytes, hs)
            e.record()
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(f"lso_probe_copy_variant({var}, {param}) failed ({rc})")
            if r >= 2:
                times.append(s.elapsed_time(e))
        moved = nbytes if var in (5, 6) else 2 * nbytes
        ok = None
        if var in (0, 1, 2, 3, 8):
            ok = bool(torch.equal(src, dst))
        elif var in (4, 7):
            ok = bool(torch.equal(src, keep))
        gbps = moved / (min(times) * 1e-3) / 1e9
        rows.append(dict(shape=name, variant=var, param=param, GBps=gbps, exact=ok))
        progress(f"hbm probe: {name}: {gbps:.0f} GB/s{'' if ok is not False else ' WRONG'}")
    del src, dst, keep
    # the update's own tiled traffic shape (14 B read, 14 B written per
    # element, in place) with each store policy
    n = 134_283 * 8192
    state = torch.zeros(12 * n, dtype=torch.uint8, device=dev)
    grad = torch.zeros(2 * n, dtype=torch.uint8, device=dev)
    weight = torch.empty(2 * n, dtype=torch.uint8, device=dev)
    for st_pol in range(6):
        times = []
        for r in range(reps + 2):
            s.record()
            rc = P.lso_probe_copy_shaped_cpol(state.data_ptr(), grad.data_ptr(), weight.data_ptr(), n, st_pol, hs)
            e.record()
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(f"lso_probe_copy_shaped_cpol({st_pol}) failed ({rc})")
            if r >= 2:
                times.append(s.elapsed_time(e))
        gbps = 28 * n / (min(times) * 1e-3) / 1e9
        name = f"update-shaped (tiled, in place), stores {names[st_pol]}"
        rows.append(dict(shape=name, variant="shaped", param=st_pol, GBps=gbps, exact=None))
        progress(f"hbm probe: {name}: {gbps:.0f} GB/s")
    del state, grad, weight
    return dict(hbm_probe=rows, bytes=nbytes, best_of=reps, unit="GB/s (read + write)")


def launch_floor() -> dict:
    """The floors of the launch-bound workloads (c0, c2): an empty
    one-workgroup launch, and at each workload's size the update's traffic
    shape with no arithmetic (lso_probe_copy_shaped, planar, the same
    1,024-element chunks) and a plain copy of the same bytes -- each warm
    (median of isolated launches), with 512 MB written before every launch,
    and back to back (100-200 launches between two events)."""
    import torch

    import synth
    from layer_streamed_optimizer_amd import _native
    P = _native.probes()
    dev = torch.device("cuda:0")
    hs = torch.cuda.current_stream().cuda_stream

    def isolated(fn, reps, flush=None):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for s, e in ev:
            if flush is not None:
                synth.device_fill_zero(flush.data_ptr(), flush.numel(), hs)
            s.record()
            if fn() != 0:
                raise RuntimeError("probe launch failed")
            e.record()
        torch.cuda.synchronize()
        d = sorted(s.elapsed_time(e) * 1e3 for s, e in ev)
        return dict(median_us=d[len(d) // 2], min_us=d[0])

    def back_to_back(fn, k):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        torch.cuda.synchronize()
        s.record()
        for _ in range(k):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) * 1e3 / k

    a = torch.zeros(1 << 20, dtype=torch.uint8, device=dev)
    b = torch.zeros(1 << 20, dtype=torch.uint8, device=dev)
    empty = lambda: P.lso_probe_copy(a.data_ptr(), b.data_ptr(), 16, 0, hs)
    out = dict(one_workgroup_launch=dict(isolated=isolated(empty, 200), back_to_back_us=back_to_back(empty, 2000)))
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    for name, n in (("c0", 1 << 20), ("c2", 6307840)):
        state = torch.zeros(12 * n, dtype=torch.uint8, device=dev)
        grad = torch.zeros(2 * n, dtype=torch.uint8, device=dev)
        w = torch.empty(2 * n, dtype=torch.uint8, device=dev)
        shaped = lambda: P.lso_probe_copy_shaped(state.data_ptr(), grad.data_ptr(), w.data_ptr(), n, 0, hs)
        out[f"shaped_{name}"] = dict(params=n, workgroups=n // 1024, warm=isolated(shaped, 100),
                                     flushed=isolated(shaped, 50, flush), back_to_back_us=back_to_back(shaped, 200))
        src = torch.zeros(14 * n, dtype=torch.uint8, device=dev)
        dst = torch.zeros(14 * n, dtype=torch.uint8, device=dev)
        copy = lambda: P.lso_probe_copy(src.data_ptr(), dst.data_ptr(), 14 * n, 0, hs)
        out[f"copy_{name}"] = dict(bytes_each_way=14 * n, warm=isolated(copy, 100),
                                   flushed=isolated(copy, 50, flush), back_to_back_us=back_to_back(copy, 200))
        progress(f"launch floor {name}: shaped {out[f'shaped_{name}']}, copy {out[f'copy_{name}']}")
        del state, grad, w, src, dst
    return dict(launch_floor=out, unit="us")


# ------------------------------------------------------------ streamed path

def link_peak(nbytes=4 << 30):
    """Host-link GB/s with page-locked buffers, measured by the probe
    library: each direction alone, and each direction while both run at
    once -- on the two SDMA engines the layer stream names (its default),
    with runtime-chosen DMA engines, with copy kernels, and with a DMA engine
    for H2D beside a copy kernel for D2H.  The streamed roofline takes the
    best concurrent figure of the slower direction over them."""
    from layer_streamed_optimizer_amd import _native
    P = _native.probes()
    res = {}
    # Now and then a D2H copy between one particular device buffer and one
    # particular page-locked host buffer runs at about half speed (~30 GB/s
    # even with nothing else running) for as long as both exist, while the
    # same buffers paired with others are fast: the probe allocates anew and
    # retries while D2H alone is far below H2D alone.
    for attempt in range(1, 4):
        eng = (ctypes.c_uint32 * 2)()
        out = (ctypes.c_double * 4)()
        # a different size each time, so the new buffers do not come back at
        # the addresses of the ones just freed
        rc = P.lso_probe_link_sdma(nbytes + (attempt - 1) * (192 << 20), 3, eng, out)
        if rc != 0:
            break
        r = dict(h2d=out[0], d2h=out[1], bidir_h2d=out[2], bidir_d2h=out[3],
                 engines=[int(eng[0]), int(eng[1])], attempts=attempt)
        if "sdma_pair" not in res or min(r["bidir_h2d"], r["bidir_d2h"]) > \
                min(res["sdma_pair"]["bidir_h2d"], res["sdma_pair"]["bidir_d2h"]):
            res["sdma_pair"] = r
        if out[1] >= 0.8 * out[0]:
            break
    # mode bit 0: H2D by a copy kernel; bit 1: D2H by a copy kernel
    for name, mode in (("dma", 0), ("kernel", 3), ("dma_h2d_kernel_d2h", 2)):
        out = (ctypes.c_double * 4)()
        rc = P.lso_probe_link_mode(nbytes, 3, mode, 128, out)
        if rc != 0:
            raise RuntimeError(f"lso_probe_link_mode failed ({rc})")
        res[name] = dict(h2d=out[0], d2h=out[1], bidir_h2d=out[2], bidir_d2h=out[3])
    res["bidir_per_direction"] = max(min(r["bidir_h2d"], r["bidir_d2h"]) for r in res.values())
    return res


def link_probe_sweep(sizes=(256 << 20, 1 << 30, 4 << 30, 10 << 30), reps: int = 10) -> list:
    """The host-link microbenchmark on its own: page-locked buffers of each
    size, H2D alone, D2H alone and both at once on two streams or engines,
    best of `reps`, for every engine choice the stream knows: the named SDMA
    pair, hipMemcpyAsync both ways (the runtime picks the engines), copy
    kernels both ways (128 workgroups), and hipMemcpyAsync H2D beside a D2H
    copy kernel."""
    from layer_streamed_optimizer_amd import _native
    P = _native.probes()
    rows = []
    for nbytes in sizes:
        eng = (ctypes.c_uint32 * 2)()
        out = (ctypes.c_double * 4)()
        rc = P.lso_probe_link_sdma(nbytes, reps, eng, out)
        results = {"sdma_pair": (rc, list(out))}
        for name, mode in (("dma", 0), ("kernel", 3), ("dma_h2d_kernel_d2h", 2)):
            out = (ctypes.c_double * 4)()
            rc = P.lso_probe_link_mode(nbytes, reps, mode, 128, out)
            results[name] = (rc, list(out))
        for name, (rc, o) in results.items():
            row = dict(bytes=nbytes, engines=name, status=rc)
            if rc == 0:
                row.update(h2d=o[0], d2h=o[1], both_h2d=o[2], both_d2h=o[3])
            rows.append(row)
        progress(f"link probe {nbytes >> 20} MiB: " +
                 ", ".join(f"{r['engines']} {r.get('both_h2d', 0):.1f}/{r.get('both_d2h', 0):.1f}"
                           for r in rows[-4:]))
    return rows


def best_link_peak(a: dict, b: dict) -> dict:
    """Per engine choice, the better of two link_peak measurements (by the
    slower direction while both run), and the streamed roofline peak over
    them: one probe can catch the link while the machine is still busy
    with something else (a previous process's pinned memory going away)."""
    worst = lambda r: min(r["bidir_h2d"], r["bidir_d2h"])
    res = {}
    for k in a:
        if k == "bidir_per_direction":
            continue
        res[k] = a[k] if k not in b or worst(a[k]) >= worst(b[k]) else b[k]
    res["bidir_per_direction"] = max(worst(r) for r in res.values())
    res["measured"] = "before and after the timed steps; the better of the two per engine choice"
    return res


def streamed(args, w):
    import numpy as np
    import torch

    import layer_streamed_optimizer_amd as lso
    import synth
    from layer_streamed_optimizer_amd import configs

    torch.cuda.set_device(0)
    sid = configs.STREAM_ID[w.key]
    n_layers = args.layers or len(w.blocks)
    n = w.blocks[0].n
    tiled = args.layout == "tiled"
    om, omm, ov, nbytes = configs.host_layer_layout(n, tiled=tiled)
    peak = link_peak()
    progress(f"link: {peak}")
    pinned = args.host_memory == "pinned"
    progress(f"{w.key}: {n_layers} x {nbytes / 1e9:.2f} GB host blocks, "
             f"{'pinned' if pinned else 'pageable (staged through pinned buffers)'}")
    hosts, ptrs = [], []
    hs = torch.cuda.current_stream().cuda_stream
    stage = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    scratch = torch.empty(n, dtype=torch.float32, device="cuda") if tiled else None
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    for b in range(n_layers):
        if pinned:
            hb = lso.host_alloc(nbytes)
            ptr = hb.ptr
        else:
            hb = np.empty(nbytes, dtype=np.uint8)
            ptr = hb.ctypes.data
        # initial state made on the device and copied down (untimed)
        synth.device_fill_zero(int(stage.data_ptr()), nbytes, hs)
        if tiled:
            synth.device_fill_normal_f32(int(scratch.data_ptr()), n, stream=sid, block=b,
                                         purpose=synth.PURPOSE_MASTER, step=0,
                                         sigma=configs.MASTER_SIGMA, hip_stream=hs)
            lso.tiled_pack(int(stage.data_ptr()) + om, int(scratch.data_ptr()), None, None, n=n,
                           stream=hs)
        else:
            synth.device_fill_normal_f32(int(stage.data_ptr()) + om, n, stream=sid, block=b,
                                         purpose=synth.PURPOSE_MASTER, step=0,
                                         sigma=configs.MASTER_SIGMA, hip_stream=hs)
        torch.cuda.synchronize()
        assert hip.hipMemcpy(ptr, int(stage.data_ptr()), nbytes, 2) == 0
        hosts.append(hb)
        ptrs.append(ptr)
        progress(f"layer {b} ready")
    del stage, scratch
    g32 = args.grad_dtype == "f32"
    fn, Params = synth.grad_callback(g32)
    prm = Params(seed=synth.SEED, stream=sid, purpose=synth.PURPOSE_GRAD, step=1,
                 scale=synth.scale_for(configs.GRAD_SIGMA), block_base=0)
    ls = lso.LayerStream(nbytes, n, fn, ctypes.addressof(prm))
    L = lso.LayerStream.layers(n_layers)
    L["grad_dtype"] = lso.LSO_DT_F32 if g32 else lso.LSO_DT_BF16
    for b in range(n_layers):
        L[b]["host_base"], L[b]["bytes"], L[b]["n"] = ptrs[b], nbytes, n
        L[b]["off_master"], L[b]["off_m"], L[b]["off_v"] = om, omm, ov
        L[b]["opt"] = lso.LSO_OPT_ADAM
        L[b]["layout"] = lso.LSO_LAYOUT_TILED if tiled else lso.LSO_LAYOUT_PLANAR
        L[b]["lr"], L[b]["beta1"], L[b]["beta2"], L[b]["eps"] = (configs.LR, configs.BETA1,
                                                                 configs.BETA2, configs.EPS)
    step_s, stats = [], []
    for j in range(1, args.warmup + args.steps + 1):
        prm.step = j
        L["t"] = j
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ls.stream_layers(L)
        dt = time.perf_counter() - t0
        progress(f"step {j}: {dt:.3f} s")
        if j > args.warmup:
            step_s.append(dt)
            stats.append(ls.stats())
    copy_mode = ls.copy_mode()
    ls.close()
    j_next = args.warmup + args.steps + 1
    compared = {}
    for label, env in getattr(args, "compare_modes", ()):
        # the same layers (their state carries on, t continues) through a
        # context made with other LSO_STREAM_* settings: 1 untimed step, then
        # the timed ones
        old = {k: os.environ.get(k) for k in env}
        os.environ.update(env)
        try:
            other = lso.LayerStream(nbytes, n, fn, ctypes.addressof(prm))
        finally:
            for k, v in old.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v
        times, st = [], None
        for k in range(1 + args.compare_steps):
            prm.step = j_next
            L["t"] = j_next
            j_next += 1
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            other.stream_layers(L)
            dt = time.perf_counter() - t0
            if k > 0:
                times.append(dt)
                st = other.stats()
        compared[label] = dict(env=env, copy_mode=other.copy_mode(), ms_per_step=1e3 * sum(times) / len(times),
                               steps=len(times), host_waits_per_piece=st["host_waits"] / max(1, st["pieces"]),
                               chained=st["chained"])
        other.close()
        progress(f"{label}: {compared[label]['ms_per_step']:.0f} ms per step, "
                 f"{compared[label]['host_waits_per_piece']:.1f} host wake-ups per piece")
    for hb in hosts:
        if pinned:
            hb.close()
    hosts.clear()
    peak = best_link_peak(peak, link_peak())
    progress(f"link after the steps, best of both: {peak['bidir_per_direction']:.1f} GB/s per direction")
    wall = sum(step_s)
    params = n * n_layers
    per_dir = LINK_BYTES_PER_PARAM * params / (wall / len(step_s)) / 1e9
    bidir_peak = peak["bidir_per_direction"]
    result = dict(
        metric=METRIC, value=params * len(step_s) / wall / 1e9, unit="Gparams/s",
        ms_per_step=wall * 1e3 / len(step_s),
        roofline=dict(bound="host-link", achieved=per_dir, peak=bidir_peak,
                      unit="GB/s per direction", frac=per_dir / bidir_peak, traffic=None),
        link_peak_GBps=peak,
        # against a one-way hipMemcpyAsync of page-locked memory (nothing in
        # the other direction): a looser reference than the duplex peak
        frac_of_hipmemcpy_one_way=per_dir / min(peak["dma"]["h2d"], peak["dma"]["d2h"]),
        pieces_per_step=stats[-1]["pieces"],
        host_waits_per_piece=sum(x["host_waits"] for x in stats) / max(1, sum(x["pieces"] for x in stats)),
        h2d_chained_on_engine=stats[-1]["chained"],
        other_modes=compared or None,
        config=dict(workload=f"{w.key}: {w.title}", layers=n_layers, layers_in_config=len(w.blocks),
                    params=params, host_memory="pinned" if pinned else "pageable+staged",
                    state_layout=args.layout,
                    host_bytes=nbytes * n_layers,
                    link_bytes_per_param_each_way=LINK_BYTES_PER_PARAM, copy_mode=copy_mode,
                    grad_dtype=args.grad_dtype),
    )
    return result


def storage_peak(directory: str, nbytes: int = 4 << 30, threads: int = 8) -> dict:
    """Sequential O_DIRECT pread / pwrite rates of the file system that holds
    the layer files, alone and both at once (lso_probe_file)."""
    import layer_streamed_optimizer_amd as lso

    path = os.path.join(directory, "storage_probe.bin")
    fd = os.open(path, os.O_RDWR | os.O_CREAT | os.O_DIRECT, 0o644)
    try:
        os.posix_fallocate(fd, 0, 2 * nbytes)
        out = (ctypes.c_double * 4)()
        rc = lso._native.probes().lso_probe_file(fd, 0, nbytes, nbytes, threads, out)
        if rc != 0:
            raise RuntimeError(f"lso_probe_file failed: {os.strerror(rc)}")
    finally:
        os.close(fd)
        os.remove(path)
    r = dict(read=out[0], write=out[1], duplex_read=out[2], duplex_write=out[3])
    r["duplex_per_direction"] = min(out[2], out[3])
    return r


def streamed_files(args, w):
    """c4's layers with their authoritative blocks in files (the disk tier):
    one preallocated file per layer, opened O_DIRECT."""
    import shutil
    import tempfile

    import torch

    import layer_streamed_optimizer_amd as lso
    import synth
    from layer_streamed_optimizer_amd import configs
    from layer_streamed_optimizer_amd.disk import LayerFiles

    torch.cuda.set_device(0)
    sid = configs.STREAM_ID[w.key]
    n = w.blocks[0].n
    tiled = args.layout == "tiled"
    om, _omm, _ov, nbytes = configs.host_layer_layout(n, tiled=tiled)
    base = args.file_dir or os.environ.get("LSO_FILE_DIR", "/var/tmp")
    free = shutil.disk_usage(base).free
    copies = 2 if args.shadow else 1          # shadow regions hold two data slots
    n_layers = args.layers or (3 if args.shadow else 6)
    if copies * n_layers * nbytes + (10 << 30) > free:
        sys.exit(f"{base} has {free / 1e9:.0f} GB free; {n_layers} layers need "
                 f"{copies * n_layers * nbytes / 1e9:.0f} GB plus 10 GB of headroom (use --layers)")
    d = tempfile.mkdtemp(prefix="lso_disk_", dir=base)
    try:
        peak = storage_peak(d)
        progress(f"storage: {peak}")
        files = LayerFiles.create(d, [n] * n_layers, tiled=tiled, direct=True, shadow=args.shadow)
        hs = torch.cuda.current_stream().cuda_stream
        stage = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        scratch = torch.empty(n, dtype=torch.float32, device="cuda") if tiled else None
        # page-aligned ordinary memory: O_DIRECT cannot transfer from
        # HIP-allocated pinned memory
        host = mmap.mmap(-1, nbytes)
        host_ptr = ctypes.addressof(ctypes.c_char.from_buffer(host))
        hip = ctypes.CDLL("libamdhip64.so")
        hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        view = memoryview(host)
        for b in range(n_layers):
            # initial state made on the device, written to the file (untimed)
            synth.device_fill_zero(int(stage.data_ptr()), nbytes, hs)
            dst = int(scratch.data_ptr()) if tiled else int(stage.data_ptr()) + om
            synth.device_fill_normal_f32(dst, n, stream=sid, block=b, purpose=synth.PURPOSE_MASTER,
                                         step=0, sigma=configs.MASTER_SIGMA, hip_stream=hs)
            if tiled:
                lso.tiled_pack(int(stage.data_ptr()) + om, dst, None, None, n=n, stream=hs)
            torch.cuda.synchronize()
            assert hip.hipMemcpy(host_ptr, int(stage.data_ptr()), nbytes, 2) == 0
            done, at = 0, files.state(b)[2]       # shadow files: the committed slot
            while done < nbytes:
                done += os.pwritev(files.fds[b], [view[done:]], at + done)
            progress(f"layer {b} written")
        del view
        del stage, scratch
        g32 = args.grad_dtype == "f32"
        fn, Params = synth.grad_callback(g32)
        prm = Params(seed=synth.SEED, stream=sid, purpose=synth.PURPOSE_GRAD, step=1,
                     scale=synth.scale_for(configs.GRAD_SIGMA), block_base=0)
        ls = lso.LayerStream(nbytes, n, fn, ctypes.addressof(prm))
        step_s = []
        for j in range(1, args.warmup + args.steps + 1):
            prm.step = j
            L = files.table(j, configs.LR, configs.BETA1, configs.BETA2, configs.EPS, sync=args.sync,
                            grad_dtype=lso.LSO_DT_F32 if g32 else 0)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            ls.stream_files(L)
            dt = time.perf_counter() - t0
            files.commit(j)
            progress(f"step {j}: {dt:.3f} s")
            if j > args.warmup:
                step_s.append(dt)
        copy_mode = ls.copy_mode()
        ls.close()
        files.close()
    finally:
        shutil.rmtree(d, ignore_errors=True)
    wall = sum(step_s)
    params = n * n_layers
    per_dir = LINK_BYTES_PER_PARAM * params / (wall / len(step_s)) / 1e9
    top = peak["duplex_per_direction"]
    return dict(
        metric=METRIC, value=params * len(step_s) / wall / 1e9, unit="Gparams/s",
        ms_per_step=wall * 1e3 / len(step_s),
        roofline=dict(bound="storage", achieved=per_dir, peak=top, unit="GB/s per direction",
                      frac=per_dir / top, traffic=None),
        storage_peak_GBps=peak,
        config=dict(workload=f"{w.key}: 70B-shaped slice, layer-streamed from files (disk tier"
                             + (", crash-consistent shadow regions)" if args.shadow else ")"),
                    layers=n_layers, layers_in_config=len(w.blocks), params=params,
                    host_memory="file (O_DIRECT, one preallocated file per layer"
                                + (", shadow region)" if args.shadow else ")"),
                    state_layout=args.layout, file_bytes=nbytes * n_layers,
                    storage_bytes_per_param_each_way=LINK_BYTES_PER_PARAM, copy_mode=copy_mode,
                    grad_dtype=args.grad_dtype,
                    flushed_per_layer=bool(args.sync or args.shadow)),
    )


# -------------------------------------------------------------- CPU baseline

def cpu_baseline(w, budget_s=12.0):
    """The oracle as it stands, on the host's cores, on a bounded sample:
    one full decoder-layer block of a model-shaped workload (its first
    layer), or the first blocks of the others (up to 64M params), repeated
    steps until budget_s of CPU time has passed.  Its inputs are drawn on
    the device and copied down (the device generator equals the host one
    bit for bit; the oracle's speed does not depend on the values)."""
    import numpy as np
    import torch

    import oracle
    import synth
    from layer_streamed_optimizer_amd import configs

    sid = configs.STREAM_ID[w.key]
    layer = next((b for b, spec in enumerate(w.blocks) if spec.name == "layer0"), None)
    if layer is not None:
        blocks = [(layer, w.blocks[layer].n)]
        what = f"one full decoder-layer block of {w.key} (block {layer}, {w.blocks[layer].n:,} params)"
    else:
        take, blocks = 0, []
        for b, spec in enumerate(w.blocks):
            if take >= (64 << 20):
                break
            n = min(spec.n, (64 << 20) - take)
            blocks.append((b, n))
            take += n
        what = f"first {take:,} params of {w.key} ({len(blocks)} block(s))"
    take = sum(n for _, n in blocks)
    hs = torch.cuda.current_stream().cuda_stream
    dev = torch.empty(4 * max(n for _, n in blocks), dtype=torch.uint8, device="cuda")

    def draw(n, b, purpose, step, sigma, bf16):
        fill = synth.device_fill_normal_bf16 if bf16 else synth.device_fill_normal_f32
        fill(int(dev.data_ptr()), n, stream=sid, block=b, purpose=purpose, step=step, sigma=sigma,
             hip_stream=hs)
        torch.cuda.synchronize()
        return dev[: (2 if bf16 else 4) * n].cpu().numpy().view(np.uint16 if bf16 else np.float32).copy()

    arrays = []
    for b, n in blocks:
        master = draw(n, b, synth.PURPOSE_MASTER, 0, configs.MASTER_SIGMA, False)
        g = draw(n, b, synth.PURPOSE_GRAD, 1, configs.GRAD_SIGMA, True)
        arrays.append((master, np.zeros(n, np.float32), np.zeros(n, np.float32), g,
                       np.zeros(n, np.uint16)))
    del dev
    steps, threads = 0, 0
    t0 = time.perf_counter()
    while True:
        steps += 1
        for master, m, v, g, wb in arrays:
            threads = oracle.adam_step(master, m, v, g, wb, steps, configs.LR, configs.BETA1, configs.BETA2,
                                       configs.EPS)
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    # one thread on the first block's first 8M params, for the per-core rate
    master, m, v, g, wb = arrays[0]
    k1 = min(master.size, 8 << 20)
    s1, t1 = 0, time.perf_counter()
    while True:
        s1 += 1
        oracle.adam_step(master[:k1], m[:k1], v[:k1], g[:k1], wb[:k1], steps + s1, configs.LR,
                         configs.BETA1, configs.BETA2, configs.EPS, threads=1)
        if time.perf_counter() - t1 >= budget_s / 4:
            break
    d1 = time.perf_counter() - t1
    return dict(value=take * steps / dt / 1e9, unit="Gparams/s", cores=threads, kind="oracle",
                sample=f"{what}, {steps} steps, {dt:.1f} s, inputs in host RAM",
                single_thread=dict(value=k1 * s1 / d1 / 1e9, unit="Gparams/s",
                                   sample=f"{k1:,} params, {s1} steps, {d1:.1f} s"))


# ---------------------------------------------------------------------- main

def placement_scan(positions: int = 12, reps: int = 4) -> dict:
    """The c3 update's rate against where its arrays sit in HBM: one pool of
    all free memory but 8 GiB, the whole working set (tiled state, weights,
    one gradient set: 107.8 GB) placed at `positions` offsets spread over it.
    At each offset, two arrangements of the same arrays: three regions (every
    block's state, then every block's weights, then every block's gradients)
    and one arena, block after block [state | weights | gradients] (the
    resident bench's BlockArena, so the arrays streamed together are
    adjacent); then the update's traffic shape with no arithmetic
    (lso_probe_copy_shaped_cpol, the update's stores) over the regions and a
    plain 8 GiB copy inside the state region.  Each figure is the average of
    `reps` launches after one."""
    import torch

    import layer_streamed_optimizer_amd as lso
    import synth
    from layer_streamed_optimizer_amd import _native, configs
    P = _native.probes()
    dev = torch.device("cuda:0")
    hs = torch.cuda.current_stream().cuda_stream
    w = configs.get("c3")
    sid = configs.STREAM_ID["c3"]
    sizes = [b.n for b in w.blocks]
    lay = configs.ResidentLayout(sizes, tiled=True, grad_f32=False)
    m2 = 2 << 20

    def up(x):
        return (x + m2 - 1) // m2 * m2

    # three regions
    off_w = up(lay.state_bytes)
    off_g = off_w + up(lay.weight_bytes)
    span_bytes = off_g + up(lay.grad_bytes)
    regions = [(lay.off_master[b], off_g + lay.off_grad[b], off_w + lay.off_weight[b]) for b in range(len(sizes))]
    # one arena, block after block (the resident bench's arrangement)
    one = configs.BlockArena(sizes, tiled=True)
    per_block = [(one.off_master[b], one.off_grad[0][b], one.off_weight[b]) for b in range(len(sizes))]
    assert one.total_bytes <= span_bytes
    n_shaped = w.params // 8192 * 8192
    copy_bytes = 8 << 30
    free, _ = torch.cuda.mem_get_info()
    total = (free - (8 << 30)) // m2 * m2
    if total < span_bytes + m2:
        raise RuntimeError("not enough device memory for the c3 working set")
    pool = torch.empty(total, dtype=torch.uint8, device=dev)
    base = int(pool.data_ptr())
    scratch = torch.empty(max(sizes), dtype=torch.float32, device=dev)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        fn()
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps

    def check(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed ({rc})")

    step = [0]

    def update_ms(origin, arrangement):
        for b, spec in enumerate(w.blocks):
            so, go, _ = arrangement[b]
            synth.device_fill_normal_f32(int(scratch.data_ptr()), spec.n, stream=sid, block=b,
                                         purpose=synth.PURPOSE_MASTER, step=0, sigma=configs.MASTER_SIGMA,
                                         hip_stream=hs)
            lso.tiled_pack(origin + so, int(scratch.data_ptr()), None, None, n=spec.n, stream=hs)
            synth.device_fill_normal_bf16(origin + go, spec.n, stream=sid, block=b, purpose=synth.PURPOSE_GRAD,
                                          step=1, sigma=configs.GRAD_SIGMA, hip_stream=hs)
        tab = lso.BlockTable.from_rows(
            dict(n=n, master=origin + arrangement[b][0], grad=origin + arrangement[b][1],
                 weight=origin + arrangement[b][2], t=1, lr=configs.LR, beta1=configs.BETA1,
                 beta2=configs.BETA2, eps=configs.EPS, layout=lso.LSO_LAYOUT_TILED, grad_dtype=lso.LSO_DT_BF16)
            for b, n in enumerate(sizes))

        def update():
            step[0] += 1
            tab.set_step(step[0])
            lso.adam_step(tab, hs)

        return timed(update)

    rows = []
    for k in range(positions):
        off = (total - span_bytes) * k // max(1, positions - 1) // m2 * m2
        origin = base + off
        t_regions = update_ms(origin, regions)
        t_arena = update_ms(origin, per_block)
        sb, wb, gb = origin, origin + off_w, origin + off_g
        t_copy = timed(lambda: check(P.lso_probe_copy(sb, sb + copy_bytes, copy_bytes, 0, hs), "copy"))
        t_shaped = timed(lambda: check(P.lso_probe_copy_shaped_cpol(sb, gb, wb, n_shaped, 3, hs), "shaped copy"))
        row = dict(offset_GB=off / 1e9, regions_ms=t_regions, regions_GBps=28 * w.params / (t_regions * 1e-3) / 1e9,
                   block_arena_ms=t_arena,
                   block_arena_GBps=28 * w.params / (t_arena * 1e-3) / 1e9,
                   shaped_GBps=28 * n_shaped / (t_shaped * 1e-3) / 1e9,
                   copy_GBps=2 * copy_bytes / (t_copy * 1e-3) / 1e9)
        rows.append(row)
        progress(f"placement +{row['offset_GB']:.1f} GB: three regions {t_regions:.3f} ms "
                 f"({row['regions_GBps']:.0f} GB/s), block arena {t_arena:.3f} ms, shaped copy {row['shaped_GBps']:.0f} GB/s, "
                 f"plain copy {row['copy_GBps']:.0f} GB/s")
    del pool, scratch
    return dict(placement_scan=rows, pool_GB=total / 1e9, working_set_GB=span_bytes / 1e9, reps=reps)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--config", default="c3", choices=["c0", "c1", "c2", "c3", "c4"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-streamed", action="store_true",
                    help="c3: leave out the nested streamed record (c4, 16 pageable layers)")
    ap.add_argument("--streamed-steps", type=int, default=3,
                    help="timed steps of the nested streamed record (after 1 untimed step)")
    ap.add_argument("--link-probe", action="store_true",
                    help="only the host-link microbenchmark: 256 MiB to 10 GiB page-locked "
                         "buffers, each direction alone and both at once, best of 10, for every "
                         "engine choice; one JSON line")
    ap.add_argument("--hbm-probe", action="store_true",
                    help="only the HBM ceiling sweep: every shape of the 1:1 read/write copy "
                         "probe over 8 GiB, best of 6; one JSON line")
    ap.add_argument("--launch-floor", action="store_true",
                    help="only the floors of the launch-bound workloads (c0, c2 sizes): an empty "
                         "launch, the update-shaped copy and a plain copy; one JSON line")
    ap.add_argument("--placement-scan", action="store_true",
                    help="only the placement scan: the c3 update, its traffic shape and a plain "
                         "copy with the working set at 12 offsets in one pool; one JSON line")
    ap.add_argument("--host-memory", choices=["pageable", "pinned", "file"], default="pageable",
                    help="c4: authoritative blocks in pageable memory (staged through pinned "
                         "buffers), page-locked (direct; limited by the host's page-locked "
                         "budget), or files (the disk tier, O_DIRECT)")
    ap.add_argument("--layers", type=int, default=0,
                    help="c4: layers to stream (0 = all 16; 6 for --host-memory file)")
    ap.add_argument("--shadow", action="store_true",
                    help="c4 with --host-memory file: crash-consistent shadow regions "
                         "(3 layers by default: two data slots per layer)")
    ap.add_argument("--sync", action="store_true",
                    help="c4 with --host-memory file: fdatasync each layer's file after its "
                         "write-back (LSO_FILE_SYNC; shadow regions always flush)")
    ap.add_argument("--file-dir", default=None,
                    help="c4 with --host-memory file: where the layer files go "
                         "(default $LSO_FILE_DIR or /var/tmp)")
    ap.add_argument("--arrangement", choices=["auto", "arena", "regions"], default="auto",
                    help="resident arrays: one block-by-block arena, three regions (states, weights, "
                         "gradient sets), or auto (the arena for steps of more than 1 GiB)")
    ap.add_argument("--layout", choices=["tiled", "planar"], default=None,
                    help="FP32 state layout (default: tiled for c1, c3, c4; planar for c0, c2)")
    ap.add_argument("--norms", action="store_true",
                    help="resident workloads: the update with per-block gradient norms "
                         "(progressive layer locking)")
    ap.add_argument("--grad-sets", type=int, default=0,
                    help="resident workloads: at most this many gradient sets rotate over the steps "
                         "(0: as many as fit, up to one per step)")
    ap.add_argument("--grad-dtype", choices=["bf16", "f32"], default="bf16",
                    help="gradient dtype (f32: the LoRA article's FP32 adapter gradients; for c4 "
                         "the device producer writes FP32)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the update is elementwise and would shard by "
              "contiguous 1/N ranges with no exchange inside the step; the library has no "
              "multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    if args.link_probe:
        import torch

        torch.cuda.set_device(0)
        print(json.dumps(dict(link_probe=link_probe_sweep(), unit="GB/s", best_of=10,
                              environment=environment())), flush=True)
        return
    if args.launch_floor:
        import torch

        torch.cuda.set_device(0)
        out = launch_floor()
        out["environment"] = environment()
        print(json.dumps(out), flush=True)
        return
    if args.placement_scan:
        import torch

        torch.cuda.set_device(0)
        out = placement_scan()
        out["environment"] = environment()
        print(json.dumps(out), flush=True)
        return
    if args.hbm_probe:
        import torch

        torch.cuda.set_device(0)
        out = hbm_probe()
        out["environment"] = environment()
        print(json.dumps(out), flush=True)
        return
    from layer_streamed_optimizer_amd import configs
    w = configs.get(args.config)
    defaults = {"c0": (10, 100), "c1": (2, 10), "c2": (5, 100), "c3": (2, 10), "c4": (1, 2)}
    dw, dk = defaults[args.config]
    if args.layout is None:
        args.layout = "planar" if args.config in ("c0", "c2") else "tiled"
    args.warmup = dw if args.warmup is None else args.warmup
    args.steps = dk if args.steps is None else args.steps
    if args.steps < 1:
        sys.exit("--steps must be >= 1")
    if w.streamed:
        res = streamed_files(args, w) if args.host_memory == "file" else streamed(args, w)
    else:
        res = resident(args, w)
    out = dict(metric=res.pop("metric"), value=res.pop("value"), unit=res.pop("unit"), n_gpus=1,
               steps=args.steps, warmup=args.warmup, ms_per_step=res.pop("ms_per_step"),
               higher_is_better=True, scaling="weak", vs_baseline=None, dtype="f32",
               data="synthetic", config=res.pop("config"), roofline=res.pop("roofline"))
    if not args.no_cpu_baseline:
        progress("timing the oracle on the host")
        out["cpu_baseline"] = cpu_baseline(w)
    out.update(res)
    if w.key == "c3" and not args.no_streamed:
        # the streamed headline in the same run: c4 as its benchmark
        # configuration (16 layers, pageable + staged, tiled, 512 MiB pieces)
        import torch
        torch.cuda.empty_cache()
        sa = argparse.Namespace(**vars(args))
        sa.layers, sa.host_memory, sa.layout, sa.grad_dtype = 0, "pageable", "tiled", "bf16"
        sa.warmup, sa.steps = 1, max(1, args.streamed_steps)
        # beside the default: the host carrying buffer-free, and the three
        # HIP streams tied by hipEvents (DMA H2D, copy-kernel D2H)
        sa.compare_modes = (("host-gated H2D (LSO_STREAM_CHAIN=0)", {"LSO_STREAM_CHAIN": "0"}),
                            ("three HIP streams tied by hipEvents (LSO_STREAM_COPY=dma-in)",
                             {"LSO_STREAM_COPY": "dma-in"}))
        sa.compare_steps = 1
        progress(f"streamed record: c4, {sa.warmup} untimed + {sa.steps} timed steps")
        r = streamed(sa, configs.get("c4"))
        out["streamed"] = dict(metric=r.pop("metric"), value=r.pop("value"), unit=r.pop("unit"),
                               steps=sa.steps, warmup=sa.warmup, ms_per_step=r.pop("ms_per_step"),
                               config=r.pop("config"), roofline=r.pop("roofline"), **r)
        if not args.no_cpu_baseline:
            progress("timing the oracle on one 70B-shaped layer")
            out["streamed"]["cpu_baseline"] = cpu_baseline(configs.get("c4"), budget_s=8.0)
    out["environment"] = environment()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
