"""The kernel's FP32 arithmetic, bit for bit.

Per element the update is a fixed sequence of binary32 operations: two
explicit FMAs for the moments, a correctly rounded square root, an FMA for
sqrt(v) * r + eps, one product, a correctly rounded division, one addition
to the master, and the BF16 round-to-nearest-even of the result, with the
constants computed in FP64 and rounded once to FP32 (the library's
lso_block_constants).  tests/fp32_exact.py carries out the same sequence in
exact rational arithmetic rounded once per operation, so every output bit
is fixed: this test compares master, m, v and the BF16 weight exactly,
three steps in a row, for planar and tiled state, blocks passed by value
(one block, and a few) and through a device table, with BF16 and with FP32
gradients.  Half of the masters
start at 0, so the first step writes each element's step itself (any
rounding difference in the root or the division shows in those bits).

The FP64 oracle defines the update and is compared with a tolerance
elsewhere; this is the check of the FP32 contract the kernel states.
"""
import numpy as np
import pytest

import fp32_exact as fx
import layer_streamed_optimizer_amd as lso
import synth

from gpu_util import Arena, log, torch

pytestmark = pytest.mark.gpu

STREAM = 95
STEPS = 3

CASES = [
    # sizes, tiled, FP32 gradients, (lr, beta1, beta2, eps)
    ([3001], False, False, (1e-3, 0.9, 0.999, 1e-8)),                       # one block by value
    ([5, 1029, 2000], False, False, (1e-3, 0.9, 0.999, 1e-8)),              # a few by value
    ([1, 7, 1024, 1500, 33, 2049], False, False, (2e-3, 0.8, 0.99, 1e-3)),  # device table, large eps
    ([8195], True, False, (1e-3, 0.9, 0.999, 1e-8)),                        # tiled, one block
    ([5, 1030, 8192, 300, 17], True, False, (1e-3, 0.9, 0.95, 1e-6)),       # tiled, device table
    ([2500, 9, 700], False, True, (1e-3, 0.9, 0.999, 1e-8)),                # FP32 gradients, by value
    ([8200, 5, 1030, 64, 300], True, True, (1e-3, 0.9, 0.999, 1e-8)),       # FP32 gradients, tiled table
]


def constants(t, lr, b1, b2, eps):
    """The emulation's constants, checked equal to the library's."""
    c = fx.adam_constants(t, lr, b1, b2, eps)
    lib = lso.block_constants(t=t, lr=lr, beta1=b1, beta2=b2, eps=eps)
    assert np.array_equal(c.view(np.uint32), lib.view(np.uint32)), (c, lib)
    return c


def first_diff(got, want):
    gb, wb = np.asarray(got).view(np.uint32 if got.dtype == np.float32 else np.uint16), \
        np.asarray(want).view(np.uint32 if want.dtype == np.float32 else np.uint16)
    idx = np.nonzero(gb != wb)[0]
    return idx.size, (int(idx[0]), hex(int(gb[idx[0]])), hex(int(wb[idx[0]]))) if idx.size else None


@pytest.mark.parametrize("sizes,tiled,f32,hyper", CASES,
                         ids=["one_block", "by_value", "table", "tiled_one_block", "tiled_table",
                              "f32_grads_by_value", "f32_grads_tiled_table"])
def test_update_bit_exact_against_binary32_emulation(sizes, tiled, f32, hyper):
    lr, b1, b2, eps = hyper
    log("fp32 exact", f"sizes={sizes} tiled={tiled} f32_grads={f32} hyper={hyper}")
    T = torch()
    arena = Arena(sizes, tiled=tiled, grad_f32=f32)
    state = []
    for i, n in enumerate(sizes):
        master = synth.normal_f32(n, stream=STREAM, block=i, purpose=synth.PURPOSE_MASTER, step=0, sigma=0.02)
        master[::2] = 0.0
        m = synth.normal_f32(n, stream=STREAM, block=i, purpose=synth.PURPOSE_MASTER, step=101, sigma=1e-4)
        v = np.abs(synth.normal_f32(n, stream=STREAM, block=i, purpose=synth.PURPOSE_MASTER, step=102,
                                    sigma=1e-6)).astype(np.float32)
        state.append([master, m, v])
        arena.put(i, "master", master)
        arena.put(i, "m", m)
        arena.put(i, "v", v)
    table = arena.table(lr=lr, beta1=b1, beta2=b2, eps=eps)
    for t in range(1, STEPS + 1):
        c = constants(t, lr, b1, b2, eps)
        draw = synth.normal_f32 if f32 else synth.normal_bf16
        gs = [draw(n, stream=STREAM, block=i, purpose=synth.PURPOSE_GRAD, step=t, sigma=1e-3)
              for i, n in enumerate(sizes)]
        for i, g in enumerate(gs):
            arena.put(i, "grad", g)
        table.set_step(t)
        lso.adam_step(table, T.cuda.current_stream())
        T.cuda.synchronize()
        for i, n in enumerate(sizes):
            p, m, v, w = fx.adam_binary32(*state[i], gs[i], c)
            got = {"master": arena.get(i, "master"), "m": arena.get(i, "m"), "v": arena.get(i, "v"),
                   "weight": arena.get(i, "weight")}
            for name, want in (("master", p), ("m", m), ("v", v), ("weight", w)):
                count, where = first_diff(got[name], want)
                assert count == 0, (f"step {t} block {i} (n={n}) {name}: {count} elements differ; "
                                    f"first (index, got, emulated): {where}")
            state[i] = [p, m, v]
    assert arena.canaries_intact(), "a write landed outside its array"
    log("fp32 exact", f"{sum(sizes)} elements x {STEPS} steps identical")
