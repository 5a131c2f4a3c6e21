"""lso_adam_step_noalloc (the entry point for callers that cannot allocate)
against lso_adam_step, through the C ABI: the same inputs in two arenas,
one updated by each entry point, must end bit for bit equal (both run the
same fused kernel with the same constants; only where the block table lives
differs), and both match the oracle.  Two calls in a row, the second with a
smaller table, so the second reads none of the first call's entries left in
the shared scratch array."""
import numpy as np
import pytest

import layer_streamed_optimizer_amd as lso
import oracle
import synth
from layer_streamed_optimizer_amd import configs

from gpu_util import Arena, Worst, assert_parity, log, torch

pytestmark = pytest.mark.gpu

LR, B1, B2, EPS = configs.LR, configs.BETA1, configs.BETA2, configs.EPS
QUANTITIES = ("master", "m", "v", "weight")


def fill(arenas, sizes, sid, init, t):
    """Initial state (t == 1) and step t's gradients, the same in every arena;
    returns the host copies for the oracle."""
    gs = []
    for i, n in enumerate(sizes):
        if t == 1:
            if init[i] == "zero":
                master = np.zeros(n, np.float32)
            else:
                sig = configs.LORA_A_SIGMA if init[i] == "lora_a" else configs.MASTER_SIGMA
                master = synth.normal_f32(n, stream=sid, block=i, purpose=synth.PURPOSE_MASTER, step=0,
                                          sigma=sig)
            for a in arenas:
                a.put(i, "master", master)
                a.put(i, "m", np.zeros(n, np.float32))
                a.put(i, "v", np.zeros(n, np.float32))
        g = synth.normal_bf16(n, stream=sid, block=i, purpose=synth.PURPOSE_GRAD, step=t, sigma=1e-3)
        for a in arenas:
            a.put(i, "grad", g)
        gs.append(g)
    return gs


def run_pair(sizes, init, sid, steps, what):
    """`steps` steps of the same blocks through both entry points; the
    no-alloc arena is also checked against the oracle."""
    T = torch()
    log(f"no-alloc {what}: {len(sizes)} blocks, {sum(sizes):,} params, {steps} steps")
    ref_a, na_a = Arena(sizes), Arena(sizes)
    ref_t, na_t = ref_a.table(), na_a.table()
    refs = [dict(master=None) for _ in sizes]
    for t in range(1, steps + 1):
        gs = fill([ref_a, na_a], sizes, sid, init, t)
        if t == 1:
            for i in range(len(sizes)):
                refs[i] = dict(master=ref_a.get(i, "master").copy(), m=np.zeros(sizes[i], np.float32),
                               v=np.zeros(sizes[i], np.float32), weight=np.zeros(sizes[i], np.uint16))
        ref_t.set_step(t)
        na_t.set_step(t)
        lso.adam_step(ref_t)
        lso.adam_step_noalloc(na_t)
        for i, g in enumerate(gs):
            r = refs[i]
            oracle.adam_step(r["master"], r["m"], r["v"], g, r["weight"], t, LR, B1, B2, EPS)
    T.cuda.synchronize()
    worst = Worst()
    for i in range(len(sizes)):
        for q in QUANTITIES:
            a, b = ref_a.get(i, q), na_a.get(i, q)
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"{what}: block {i} {q} differs"
        got = {q: na_a.get(i, q) for q in QUANTITIES}
        worst.add(f"block {i}", assert_parity(got, refs[i], 1e-6, f"{what} block {i}"))
    assert ref_a.canaries_intact() and na_a.canaries_intact()
    log(f"no-alloc {what}: equal to lso_adam_step bit for bit; oracle worst {worst}")


def test_noalloc_equals_adam_step_two_calls_second_smaller():
    w = configs.get("c2")
    sizes = [b.n for b in w.blocks]
    init = [b.init for b in w.blocks]
    # call 1: the 308 LoRA tensors (a 308-entry table in the scratch array)
    run_pair(sizes, init, configs.STREAM_ID["c2"], 3, "308 LoRA tensors")
    # call 2: a smaller ragged table; entries 17.. of the array still hold
    # call 1's blocks
    small = [1, 7, 8, 9, 4095, 4097, 8191, 12345, 100003, 2048, 16, 17, 45056, 3, 5, 16384, 999]
    run_pair(small, ["normal"] * len(small), 95, 3, "17 ragged blocks")


def test_noalloc_mixed_launches_and_split_sets():
    """Tiled and planar blocks, BF16 and FP32 gradients, and more than 16
    hyper-parameter sets in one call: several launches, each with its own
    part of the scratch array, against lso_adam_step bit for bit."""
    T = torch()
    kinds = [(False, False), (True, False), (False, True), (True, True)]
    sizes = [3000 + 131 * i for i in range(6)]
    arenas = {k: (Arena(sizes, tiled=k[0], grad_f32=k[1]), Arena(sizes, tiled=k[0], grad_f32=k[1]))
              for k in kinds}
    rows = {0: [], 1: []}
    for k, pair in arenas.items():
        for j, a in enumerate(pair):
            for i, n in enumerate(sizes):
                master = synth.normal_f32(n, stream=96, block=i, purpose=0, step=0, sigma=0.02)
                a.put(i, "master", master)
                a.put(i, "m", np.zeros(n, np.float32))
                a.put(i, "v", np.zeros(n, np.float32))
                g = (synth.normal_f32 if k[1] else synth.normal_bf16)(n, stream=96, block=i, purpose=2,
                                                                      step=1, sigma=1e-3)
                a.put(i, "grad", g)
            rows[j] += a.rows()
    for j in (0, 1):
        for i, r in enumerate(rows[j]):
            r["t"], r["lr"] = 1 + (i % 4), 1e-3 * (1 + (i % 18))   # 24 distinct sets
    tab_ref, tab_na = lso.BlockTable.from_rows(rows[0]), lso.BlockTable.from_rows(rows[1])
    before = lso.launch_count()
    lso.adam_step(tab_ref)
    mid = lso.launch_count()
    lso.adam_step_noalloc(tab_na)
    after = lso.launch_count()
    T.cuda.synchronize()
    # (kind, set group) pairs present: 5 launches, three of them with tables
    # of more than 4 blocks (in the scratch array) and two by value
    assert after - mid == mid - before == 5, (mid - before, after - mid)
    for k, (a, b) in arenas.items():
        for i in range(len(sizes)):
            for q in QUANTITIES:
                assert np.array_equal(a.get(i, q).view(np.uint8), b.get(i, q).view(np.uint8)), (k, i, q)
        assert a.canaries_intact() and b.canaries_intact()


def test_noalloc_too_many_entries_rejected_and_nothing_written():
    """More table entries than the scratch array holds: LSO_E_INVALID, and
    no array of the call is touched."""
    T = torch()
    n_blocks = lso._native.LSO_NOALLOC_MAX_BLOCKS + 1
    sizes = [16] * n_blocks
    a = Arena(sizes)
    before = a.buf.clone()
    tab = a.table()
    st = lso._native.lib().lso_adam_step_noalloc(tab.ptr, len(tab), lso.stream_handle(None))
    assert st == lso._native.LSO_E_INVALID
    assert "exceed" in lso.last_error()
    T.cuda.synchronize()
    assert T.equal(before, a.buf)


def test_noalloc_steps_captured_in_a_hip_graph_replay_like_eager():
    """The callers this entry point is for: three steps of the 308 LoRA
    tensors captured into one HIP graph (the table writes and the updates,
    no allocation inside the capture), replayed four times with new
    gradients copied in eagerly and a synchronisation between replays; after
    every replay the state equals three eager lso_adam_step calls, bit for
    bit."""
    T = torch()
    w = configs.get("c2")
    sizes = [b.n for b in w.blocks]
    init = [b.init for b in w.blocks]
    sid = configs.STREAM_ID["c2"]
    ga, ea, warm = Arena(sizes), Arena(sizes), Arena(sizes)
    fill([ga, ea, warm], sizes, sid, init, 1)
    # one call outside the capture: the scratch array's address is looked up
    lso.adam_step_noalloc(warm.table())
    T.cuda.synchronize()
    tg, te = ga.table(), ea.table()
    graph = T.cuda.CUDAGraph()
    cap = T.cuda.Stream()
    log("no-alloc: capturing three steps of 308 tensors")
    with T.cuda.graph(graph, stream=cap):
        for t in range(1, 4):
            tg.set_step(t)
            lso.adam_step_noalloc(tg, T.cuda.current_stream())
    T.cuda.synchronize()
    for r in range(4):
        fill([ga, ea], sizes, sid, init, 10 + r)   # new gradients, eagerly
        T.cuda.synchronize()
        graph.replay()
        for t in range(1, 4):
            te.set_step(t)
            lso.adam_step(te)
        T.cuda.synchronize()
        for i in range(len(sizes)):
            for q in QUANTITIES:
                assert np.array_equal(ga.get(i, q).view(np.uint8), ea.get(i, q).view(np.uint8)), (r, i, q)
        log(f"no-alloc graph replay {r}: equal to the eager steps")
    assert ga.canaries_intact() and ea.canaries_intact()


def test_noalloc_first_call_under_capture_is_refused_in_a_fresh_process():
    """The array's address is looked up once per device, outside any capture:
    in a fresh process the first call made under capture returns
    LSO_E_INVALID and writes nothing; after one call outside, captured calls
    replay like eager ones (tests/noalloc_capture_child.py)."""
    import os
    import subprocess
    import sys
    here = os.path.dirname(os.path.abspath(__file__))
    log("no-alloc: capture rule in a child process")
    r = subprocess.run([sys.executable, os.path.join(here, "noalloc_capture_child.py")],
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "capture rule ok" in r.stdout
