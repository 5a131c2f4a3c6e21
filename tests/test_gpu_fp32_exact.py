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

A second set of cases starts from values at the bottom of the binary32
range (subnormal and tiny masters, moments and gradients, signed zeros, a
subnormal eps, and SGD): the kernel keeps subnormals through every
operation, so its bits still equal the emulation's, with hundreds of
subnormal results per case.

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


# Inputs at the bottom of the binary32 range (synth.edge_f32 / edge_bf16: a
# quarter subnormal, a quarter in the smallest normal binades or with squares
# below them, a quarter signed zeros).  The kernel keeps subnormals (no flush
# to zero in any operation), so its bits still equal the emulation's; the
# vectorised emulation used here is pinned to the rational one on the same
# kind of inputs.
EDGE_STREAM = 94
EDGE_CASES = [
    # sizes, tiled, FP32 gradients, (lr, beta1, beta2, eps)
    ([2085], False, False, (1e-3, 0.9, 0.999, 1e-8)),                       # one block by value
    ([5, 1029, 600], False, False, (1e-3, 0.5, 0.75, 1.0)),                 # a few by value
    ([1, 7, 1024, 1500, 33, 2049], False, False, (1e-2, 0.9, 0.99, 1e-40)), # table, subnormal eps
    ([8195], True, False, (1e-3, 0.5, 0.75, 1.0)),                          # tiled, one block
    ([5, 1030, 8192, 17], True, False, (1e-3, 0.9, 0.999, 1e-30)),          # tiled, table
    ([2500, 9, 700], False, True, (1e-3, 0.9, 0.999, 1e-8)),                # FP32 gradients
    ([8200, 5, 1030], True, True, (1e-2, 0.9, 0.99, 1e-40)),                # FP32 gradients, tiled
]


def subnormals(x) -> int:
    u = np.asarray(x, np.float32).view(np.uint32)
    return int(np.count_nonzero((((u >> 23) & 0xFF) == 0) & ((u & 0x7FFFFF) != 0)))


@pytest.mark.parametrize("sizes,tiled,f32,hyper", EDGE_CASES,
                         ids=["one_block", "by_value", "table_subnormal_eps", "tiled_one_block",
                              "tiled_table", "f32_grads", "f32_grads_tiled_subnormal_eps"])
def test_subnormal_and_tiny_values_bit_exact(sizes, tiled, f32, hyper):
    lr, b1, b2, eps = hyper
    log("fp32 edge", f"sizes={sizes} tiled={tiled} f32_grads={f32} hyper={hyper}")
    T = torch()
    arena = Arena(sizes, tiled=tiled, grad_f32=f32)
    state = []
    for i, n in enumerate(sizes):
        st = [synth.edge_f32(n, stream=EDGE_STREAM, block=i, step=0),
              synth.edge_f32(n, stream=EDGE_STREAM, block=i, step=1),
              synth.edge_f32(n, stream=EDGE_STREAM, block=i, step=2, positive=True)]
        state.append(st)
        for name, x in zip(("master", "m", "v"), st):
            arena.put(i, name, x)
    table = arena.table(lr=lr, beta1=b1, beta2=b2, eps=eps)
    produced = [0, 0, 0]   # subnormal results: master, m, v
    for t in range(1, STEPS + 1):
        c = constants(t, lr, b1, b2, eps)
        draw = synth.edge_f32 if f32 else synth.edge_bf16
        gs = [draw(n, stream=EDGE_STREAM, block=i, step=10 + t) for i, n in enumerate(sizes)]
        for i, g in enumerate(gs):
            arena.put(i, "grad", g)
        table.set_step(t)
        lso.adam_step(table, T.cuda.current_stream())
        T.cuda.synchronize()
        for i, n in enumerate(sizes):
            p, m, v, w = fx.adam_binary32_v(*state[i], gs[i], c)
            for name, want in (("master", p), ("m", m), ("v", v), ("weight", w)):
                count, where = first_diff(arena.get(i, name), want)
                assert count == 0, (f"step {t} block {i} (n={n}) {name}: {count} elements differ; "
                                    f"first (index, got, emulated): {where}")
            produced = [k + subnormals(x) for k, x in zip(produced, (p, m, v))]
            state[i] = [p, m, v]
    assert min(produced) > 100, f"too few subnormal results to exercise the case: {produced}"
    assert arena.canaries_intact(), "a write landed outside its array"
    log("fp32 edge", f"{sum(sizes)} elements x {STEPS} steps identical; {produced} subnormal results")


def test_sgd_subnormal_and_tiny_values_bit_exact():
    """SGD (master + -(s g), no fused operation) on the same kind of inputs,
    BF16 and FP32 gradients: numpy's binary32 product and sum, which the
    emulation's rational SGD step equals on such inputs."""
    log("fp32 edge", "sgd")
    T = torch()
    sizes = [3001, 17, 1030]
    for f32 in (False, True):
        arena = Arena(sizes, adam=False, grad_f32=f32)
        masters = [synth.edge_f32(n, stream=EDGE_STREAM, block=10 + i, step=0) for i, n in enumerate(sizes)]
        for i, x in enumerate(masters):
            arena.put(i, "master", x)
        lib_s = lso.block_constants(t=1, lr=0.5, opt=lso.LSO_OPT_SGD)[4]
        assert lib_s == np.float32(0.5)
        table = arena.table(lr=0.5, opt=lso.LSO_OPT_SGD)
        for t in range(1, STEPS + 1):
            draw = synth.edge_f32 if f32 else synth.edge_bf16
            gs = [draw(n, stream=EDGE_STREAM, block=10 + i, step=10 + t) for i, n in enumerate(sizes)]
            for i, g in enumerate(gs):
                arena.put(i, "grad", g)
            table.set_step(t)
            lso.adam_step(table, T.cuda.current_stream())
            T.cuda.synchronize()
            for i, g in enumerate(gs):
                gf = g if f32 else (g.astype(np.uint32) << 16).view(np.float32)
                want = masters[i] + (-(np.float32(0.5) * gf))
                for name, ref in (("master", want), ("weight", fx.bf16_rne_bits_v(want))):
                    count, where = first_diff(arena.get(i, name), ref)
                    assert count == 0, f"f32={f32} step {t} block {i} {name}: {count} differ; first {where}"
                masters[i] = want
        assert sum(subnormals(x) for x in masters) > 0
        assert arena.canaries_intact()


WIDE_STREAM = 93


def wide_grads(n, block, step, f32):
    """Gradients over the upper exponent range, from the seeded Philox
    words: a quarter with |g| in [2^64, 2^128) (g*g overflows binary32), the
    rest with |g| in [1, 2^64); random signs and fractions.  Returns the
    gradients (BF16 patterns or FP32) and the mask of the large ones."""
    w = synth.philox_words(n, stream=WIDE_STREAM, block=block, purpose=synth.PURPOSE_EDGE, step=step)
    w = w.astype(np.uint64)
    big = (w[:, 0] & 3) == 0
    e = np.where(big, 64 + w[:, 3] % 64, w[:, 3] % 64) + 127   # biased exponent field, at most 254
    sign = w[:, 2] >> 31
    if f32:
        bits = (sign << 31) | (e << 23) | (w[:, 1] & 0x7FFFFF)
        return bits.astype(np.uint32).view(np.float32), big
    return ((sign << 15) | (e << 7) | (w[:, 1] & 0x7F)).astype(np.uint16), big


@pytest.mark.parametrize("tiled,f32", [(False, False), (True, False), (False, True), (True, True)],
                         ids=["planar", "tiled", "planar_f32_grads", "tiled_f32_grads"])
def test_large_gradients_and_the_overflow_of_their_square(tiled, f32):
    """Gradients from 1 to 2^128.  Below 2^64 every quantity stays finite:
    the kernel equals the binary32 emulation bit for bit, and its masters and
    weights are within the parity bound of the FP64 oracle.  From 2^64 up,
    g*g overflows binary32 (the kernel forms c2 * (g*g), one rounding for a
    BF16 g in range): v becomes +inf, the step -(s m')/inf is a zero, the
    master keeps its bits and nothing turns NaN -- IEEE arithmetic on the
    kernel's own operation order.  (The FP64 oracle keeps v finite until
    c2 g^2 itself leaves the binary32 range, so there the two differ.)"""
    import oracle
    from gpu_util import assert_parity
    sizes = [4101, 1030]
    lr, b1, b2, eps = 1e-3, 0.9, 0.999, 1e-8
    log("fp32 wide", f"sizes={sizes} tiled={tiled} f32_grads={f32}")
    T = torch()
    arena = Arena(sizes, tiled=tiled, grad_f32=f32)
    state, ref, never_big = [], [], []
    for i, n in enumerate(sizes):
        master = synth.normal_f32(n, stream=WIDE_STREAM, block=i, purpose=synth.PURPOSE_MASTER, step=0, sigma=0.02)
        st = [master, np.zeros(n, np.float32), np.zeros(n, np.float32)]
        state.append(st)
        ref.append([x.copy() for x in st] + [np.zeros(n, np.uint16)])
        never_big.append(np.ones(n, bool))
        for name, x in zip(("master", "m", "v"), st):
            arena.put(i, name, x)
    table = arena.table(lr=lr, beta1=b1, beta2=b2, eps=eps)
    overflowed = 0
    for t in range(1, STEPS + 1):
        c = constants(t, lr, b1, b2, eps)
        drawn = [wide_grads(n, i, t, f32) for i, n in enumerate(sizes)]
        for i, (g, _) in enumerate(drawn):
            arena.put(i, "grad", g)
        table.set_step(t)
        lso.adam_step(table, T.cuda.current_stream())
        T.cuda.synchronize()
        for i, n in enumerate(sizes):
            g, big = drawn[i]
            with np.errstate(all="ignore"):
                p, m, v, w = fx.adam_binary32_v(*state[i], g, c)
            got = {q: arena.get(i, q) for q in ("master", "m", "v", "weight")}
            for name, want in (("master", p), ("m", m), ("v", v), ("weight", w)):
                count, where = first_diff(got[name], want)
                assert count == 0, (f"step {t} block {i} {name}: {count} elements differ; "
                                    f"first (index, got, emulated): {where}")
            # the overflow regime, stated directly
            inf_v = np.isposinf(got["v"])
            assert np.all(inf_v[big]), "a square that overflows leaves v finite"
            assert np.array_equal(got["master"][inf_v].view(np.uint32), state[i][0][inf_v].view(np.uint32)), \
                "a step taken where v is +inf"
            assert not any(np.isnan(got[q]).any() for q in ("master", "m", "v")), "NaN appeared"
            overflowed += int(np.count_nonzero(big))
            # the FP64 oracle, where nothing has overflowed
            never_big[i] &= ~big
            ok = never_big[i]
            r = ref[i]
            oracle.adam_step(r[0], r[1], r[2], g, r[3], t, lr, b1, b2, eps)
            assert_parity({"master": got["master"][ok], "weight": got["weight"][ok]},
                          {"master": r[0][ok], "weight": r[3][ok]}, 1e-6, f"step {t} block {i} finite")
            state[i] = [p, m, v]
    assert overflowed > 1000
    assert arena.canaries_intact(), "a write landed outside its array"
    log("fp32 wide", f"identical; {overflowed} overflowing squares")


NOWEIGHT_STREAM = 92


@pytest.mark.parametrize("tiled,f32,n", [(True, False, 5 * 8192 + 3), (True, True, 5 * 8192 + 3),
                                         (False, False, (32 << 20) + 4096 + 5)],
                         ids=["tiled", "tiled_f32_grads", "planar_big_call"])
def test_without_weights_bit_exact(tiled, f32, n):
    """weight_dtype NONE on full chunks of every path that moves weights 16
    bytes per lane (tiled chunks with BF16 and FP32 gradients, planar chunks
    of a call above 32 M elements): master, m and v equal the emulation bit
    for bit over two steps, and no byte outside the arrays is touched."""
    log("fp32 no weights", f"n={n} tiled={tiled} f32_grads={f32}")
    T = torch()
    arena = Arena([n], tiled=tiled, grad_f32=f32, weight=False)
    master = synth.normal_f32(n, stream=NOWEIGHT_STREAM, block=0, purpose=synth.PURPOSE_MASTER, step=0, sigma=0.02)
    state = [master, np.zeros(n, np.float32), np.zeros(n, np.float32)]
    for name, x in zip(("master", "m", "v"), state):
        arena.put(0, name, x)
    table = arena.table()
    for t in (1, 2):
        c = constants(t, 1e-3, 0.9, 0.999, 1e-8)
        draw = synth.normal_f32 if f32 else synth.normal_bf16
        g = draw(n, stream=NOWEIGHT_STREAM, block=0, purpose=synth.PURPOSE_GRAD, step=t, sigma=1e-3)
        arena.put(0, "grad", g)
        table.set_step(t)
        lso.adam_step(table, T.cuda.current_stream())
        T.cuda.synchronize()
        p, m, v, _ = fx.adam_binary32_v(*state, g, c)
        for name, want in (("master", p), ("m", m), ("v", v)):
            count, where = first_diff(arena.get(0, name), want)
            assert count == 0, f"step {t} {name}: {count} elements differ; first {where}"
        state = [p, m, v]
    assert arena.canaries_intact(), "a write landed outside the arrays (a weight store with no weights?)"
