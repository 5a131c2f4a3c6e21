"""Pins of the exact binary32 emulator (tests/fp32_exact.py) against
independent IEEE implementations: numpy's float32 arithmetic and
float64-to-float32 conversion (round to nearest even in hardware), torch's
BF16 cast, and hand-worked ties, underflow and fused-versus-unfused cases."""
from fractions import Fraction

import numpy as np
import pytest

import fp32_exact as fx


def bits(x) -> int:
    return int(np.float32(x).view(np.uint32))


def same(a, b) -> bool:
    return bits(a) == bits(b)


def random_f32(rng, n, lo=-30, hi=30):
    """Finite float32 values over a wide exponent range, both signs."""
    mant = rng.uniform(1.0, 2.0, n)
    exp = rng.integers(lo, hi, n)
    sign = rng.choice([-1.0, 1.0], n)
    return (sign * np.ldexp(mant, exp)).astype(np.float32)


def test_round32_matches_hardware_conversion_from_float64():
    rng = np.random.default_rng(1)
    xs = np.concatenate([rng.normal(0, 1, 4000) * np.ldexp(1.0, rng.integers(-160, 120, 4000)),
                         rng.uniform(-1, 1, 1000) * 2.0 ** -140,        # subnormal range
                         rng.uniform(-1, 1, 200) * 2.0 ** 128])         # overflow range
    with np.errstate(over="ignore"):
        want = xs.astype(np.float32)
    for x, w in zip(xs, want):
        assert same(fx.round32(Fraction(float(x))), w), x


@pytest.mark.parametrize("q,want", [
    (Fraction(1) + Fraction(1, 2 ** 24), 1.0),                      # tie, even below
    (Fraction(1) + Fraction(3, 2 ** 24), 1.0 + 2.0 ** -22),         # tie, even above
    (-(Fraction(1) + Fraction(1, 2 ** 24)), -1.0),
    (Fraction(1, 2 ** 150), 0.0),                                   # half the least subnormal: to 0
    (Fraction(3, 2 ** 150), 2.0 ** -148),                           # tie between subnormals
    (-Fraction(1, 2 ** 151), -0.0),                                 # underflow keeps the sign
    (Fraction((1 << 24) - 1) * 2 ** 104 + Fraction(2 ** 103), float("inf")),   # max + half ulp
    (Fraction((1 << 24) - 1) * 2 ** 104 + Fraction(2 ** 102), float(np.finfo(np.float32).max)),
])
def test_round32_ties_underflow_overflow(q, want):
    assert same(fx.round32(q), np.float32(want))


def test_add_mul_div_match_numpy_float32():
    rng = np.random.default_rng(2)
    a = random_f32(rng, 3000)
    b = random_f32(rng, 3000)
    with np.errstate(all="ignore"):
        s, p, d = a + b, a * b, a / b
    for i in range(a.size):
        assert same(fx.add(a[i], b[i]), s[i])
        assert same(fx.mul(a[i], b[i]), p[i])
        assert same(fx.div(a[i], b[i]), d[i])
    # cancellation and zero signs
    assert same(fx.add(np.float32(1.5), np.float32(-1.5)), np.float32(0.0))
    assert same(fx.add(np.float32(-0.0), np.float32(-0.0)), np.float32(-0.0))
    assert same(fx.mul(np.float32(-0.0), np.float32(3.0)), np.float32(-0.0))


def test_sqrt_matches_numpy_float32():
    rng = np.random.default_rng(3)
    xs = np.abs(random_f32(rng, 4000, -149, 127))
    xs = np.concatenate([xs, np.array([0.0, 2.0 ** -149, 2.0 ** -126, 4.0, 2.0, 3.0,
                                       float(np.finfo(np.float32).max)], np.float32)])
    want = np.sqrt(xs)
    for x, w in zip(xs, want):
        assert same(fx.sqrt(x), w), x
    assert same(fx.sqrt(np.float32(-0.0)), np.float32(-0.0))


def test_fma_rounds_once():
    # (1 + 2^-12)^2 - 1 = 2^-11 + 2^-24 exactly (representable); a separate
    # product would first round 1 + 2^-11 + 2^-24 to 1 + 2^-11 (a tie to even)
    a = np.float32(1.0 + 2.0 ** -12)
    assert same(fx.fma(a, a, np.float32(-1.0)), np.float32(2.0 ** -11 + 2.0 ** -24))
    assert same(fx.add(fx.mul(a, a), np.float32(-1.0)), np.float32(2.0 ** -11))
    # reductions to the single operations
    rng = np.random.default_rng(4)
    x, y, z = random_f32(rng, 500), random_f32(rng, 500), random_f32(rng, 500)
    for i in range(500):
        assert same(fx.fma(x[i], y[i], np.float32(0.0)), fx.mul(x[i], y[i])) or fx.mul(x[i], y[i]) == 0
        assert same(fx.fma(x[i], np.float32(1.0), z[i]), fx.add(x[i], z[i]))
    # zero signs: (+0)(-1) + (-0) = -0; 1*1 + (-1) = +0
    assert same(fx.fma(np.float32(0.0), np.float32(-1.0), np.float32(-0.0)), np.float32(-0.0))
    assert same(fx.fma(np.float32(1.0), np.float32(1.0), np.float32(-1.0)), np.float32(0.0))


def test_bf16_rne_matches_torch_cast():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    xs = np.concatenate([random_f32(rng, 5000, -130, 127),
                         np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8),
                                   float(np.finfo(np.float32).max)], np.float32)])
    want = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    for x, w in zip(xs, want):
        assert fx.bf16_rne_bits(x) == int(w), x


@pytest.mark.parametrize("f32_grads", [False, True], ids=["bf16_grads", "f32_grads"])
def test_adam_binary32_agrees_with_the_fp64_oracle(f32_grads):
    """The binary32 sequence the kernel follows stays within the parity
    tolerance of the FP64 definition (1e-6 of each quantity's RMS, BF16
    weights within one spacing or that bound), three steps in a row: a
    dropped term, a wrong sign or a misplaced constant in the emulation
    would not."""
    oracle = pytest.importorskip("oracle")
    import synth
    n = 3000
    rng_master = synth.normal_f32(n, stream=96, block=0, purpose=synth.PURPOSE_MASTER, step=0, sigma=0.02)
    rng_master[::2] = 0.0
    emu = [rng_master.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)]
    ref = [rng_master.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)]
    w_ref = np.zeros(n, np.uint16)
    lr, b1, b2, eps = 1e-3, 0.9, 0.999, 1e-8
    for t in range(1, 4):
        draw = synth.normal_f32 if f32_grads else synth.normal_bf16
        g = draw(n, stream=96, block=0, purpose=synth.PURPOSE_GRAD, step=t, sigma=1e-3)
        p, m, v, w = fx.adam_binary32(*emu, g, fx.adam_constants(t, lr, b1, b2, eps))
        emu = [p, m, v]
        oracle.adam_step(ref[0], ref[1], ref[2], g, w_ref, t, lr, b1, b2, eps)
        for got, want in zip(emu, ref):
            floor = float(np.sqrt(np.mean(want.astype(np.float64) ** 2)))
            err = np.abs(got.astype(np.float64) - want) / np.maximum(np.abs(want.astype(np.float64)), floor)
            assert float(err.max()) <= 1e-6
        # weights: one BF16 spacing, or the FP32 bound where the master is
        # near 0 (as the GPU parity tests judge them)
        wv = fx_bf16(w).astype(np.float64)
        rv = fx_bf16(w_ref).astype(np.float64)
        spacing = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(rv), 2.0 ** -126))) - 7)
        bound = np.maximum(spacing, 1e-6 * float(np.sqrt(np.mean(ref[0].astype(np.float64) ** 2))))
        assert np.all(np.abs(wv - rv) <= bound)


def fx_bf16(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32)


def test_vectorised_fma_equals_the_rational_one():
    """fma_v against fma over random operands of every scale, and over
    constructed ties (a*b + c exactly half-way between two binary32 values,
    nudged both ways by a tiny c) where binary64 rounding alone goes wrong."""
    rng = np.random.default_rng(7)
    a = random_f32(rng, 4000, -40, 40)
    b = random_f32(rng, 4000, -40, 40)
    c = random_f32(rng, 4000, -80, 80)
    got = fx.fma_v(a, b, c)
    for i in range(a.size):
        assert same(got[i], fx.fma(a[i], b[i], c[i])), (a[i], b[i], c[i])
    # ties: a = A * 2^-23 with A odd and b = 1.5 make a*b = 3A * 2^-24, a
    # binary32 midpoint in [1.5, 2); c = +-2^-60 (lost in binary64) decides
    ta, tb, tc = [], [], []
    for A in range((1 << 23) + 1, (1 << 23) + 400, 2):
        for cc in (2.0 ** -60, -2.0 ** -60, 0.0):
            ta.append(A * 2.0 ** -23); tb.append(1.5); tc.append(cc)
    ta, tb, tc = (np.array(q, np.float32) for q in (ta, tb, tc))
    got = fx.fma_v(ta, tb, tc)
    naive = (ta.astype(np.float64) * tb.astype(np.float64) + tc.astype(np.float64)).astype(np.float32)
    assert np.count_nonzero(naive.view(np.uint32) != got.view(np.uint32)) > 100   # the case is live
    for i in range(ta.size):
        assert same(got[i], fx.fma(ta[i], tb[i], tc[i])), (ta[i], tb[i], tc[i])
    zs = fx.fma_v(np.array([0.0, 1.0], np.float32), np.array([-1.0, 1.0], np.float32),
                  np.array([-0.0, -1.0], np.float32))
    assert same(zs[0], np.float32(-0.0)) and same(zs[1], np.float32(0.0))


@pytest.mark.parametrize("f32_grads", [False, True], ids=["bf16_grads", "f32_grads"])
def test_vectorised_adam_step_equals_the_rational_one(f32_grads):
    import synth
    n = 4000
    master = synth.normal_f32(n, stream=97, block=0, purpose=synth.PURPOSE_MASTER, step=0, sigma=0.02)
    master[::3] = 0.0
    m = synth.normal_f32(n, stream=97, block=0, purpose=synth.PURPOSE_MASTER, step=1, sigma=1e-4)
    v = np.abs(synth.normal_f32(n, stream=97, block=0, purpose=synth.PURPOSE_MASTER, step=2, sigma=1e-6))
    a = [master, m, v]
    b = [master.copy(), m.copy(), v.copy()]
    for t in range(1, 4):
        draw = synth.normal_f32 if f32_grads else synth.normal_bf16
        g = draw(n, stream=97, block=0, purpose=synth.PURPOSE_GRAD, step=t, sigma=1e-3)
        c = fx.adam_constants(t, 1e-3, 0.9, 0.999, 1e-8)
        ra = fx.adam_binary32(*a, g, c)
        rb = fx.adam_binary32_v(*b, g, c)
        for x, y in zip(ra, rb):
            dt = np.uint16 if x.dtype == np.uint16 else np.uint32
            assert np.array_equal(np.asarray(x).view(dt), np.asarray(y).view(dt))
        a, b = list(ra[:3]), list(rb[:3])


# Hyper-parameter sets for inputs at the bottom of the range: the usual ones
# (a denominator of about eps); eps = 1 with dyadic betas (deltas of
# subnormal moments are subnormal themselves); eps = 1e-30 (the root of a
# subnormal v decides the denominator); a subnormal eps.
EDGE_HYPER = [(1e-3, 0.9, 0.999, 1e-8), (1e-3, 0.5, 0.75, 1.0), (1e-3, 0.9, 0.999, 1e-30),
              (1e-2, 0.9, 0.99, 1e-40)]
EDGE_IDS = ["eps_1e-8", "eps_1", "eps_1e-30", "eps_subnormal"]


def subnormal_count(x) -> int:
    u = np.asarray(x, np.float32).view(np.uint32)
    return int(np.count_nonzero(((u >> 23) & 0xFF) == 0) - np.count_nonzero((u & 0x7FFFFFFF) == 0))


def test_edge_inputs_reach_the_bottom_of_the_range():
    import synth
    f = synth.edge_f32(4000, stream=98, block=0, step=0)
    u = f.view(np.uint32)
    assert 800 < subnormal_count(f) < 1200                      # a quarter subnormal
    assert 800 < np.count_nonzero(((u >> 23) & 0xFF) - 1 < 8) < 1200   # smallest normal binades
    assert np.count_nonzero(u == 0x80000000) > 300              # signed zeros both ways
    assert np.all(synth.edge_f32(4000, stream=98, block=0, step=2, positive=True) >= 0)
    g = synth.edge_bf16(4000, stream=98, block=0, step=1).astype(np.uint32)
    gf = (g << 16).view(np.float32)
    assert subnormal_count(gf) > 800                            # BF16 subnormals
    sq = gf.astype(np.float64) ** 2
    assert np.count_nonzero((sq > 0) & (sq < 2.0 ** -126)) > 400   # squares below the normal range
    assert np.all(np.isfinite(gf))


@pytest.mark.parametrize("hyper", EDGE_HYPER, ids=EDGE_IDS)
@pytest.mark.parametrize("f32_grads", [False, True], ids=["bf16_grads", "f32_grads"])
def test_vectorised_adam_step_equals_the_rational_one_at_the_bottom_of_the_range(hyper, f32_grads):
    """Subnormal and tiny masters, moments and gradients (signed zeros
    among them), three steps: the vectorised emulation, which the GPU tests
    use, gives the rational one's bits, and subnormal results occur."""
    import synth
    n = 1500
    a = [synth.edge_f32(n, stream=98, block=0, step=0), synth.edge_f32(n, stream=98, block=0, step=1),
         synth.edge_f32(n, stream=98, block=0, step=2, positive=True)]
    b = [x.copy() for x in a]
    produced = 0
    for t in range(1, 4):
        g = (synth.edge_f32 if f32_grads else synth.edge_bf16)(n, stream=98, block=0, step=10 + t)
        c = fx.adam_constants(t, *hyper)
        ra = fx.adam_binary32(*a, g, c)
        rb = fx.adam_binary32_v(*b, g, c)
        for x, y in zip(ra, rb):
            dt = np.uint16 if x.dtype == np.uint16 else np.uint32
            assert np.array_equal(np.asarray(x).view(dt), np.asarray(y).view(dt))
        assert all(np.all(np.isfinite(x)) for x in ra[:3])
        produced += sum(subnormal_count(x) for x in ra[:3])
        a, b = list(ra[:3]), list(rb[:3])
    assert produced > 100, "no subnormal results: the inputs do not exercise the case"


def test_sgd_emulation_equals_numpy_float32_at_the_bottom_of_the_range():
    import synth
    n = 3000
    master = synth.edge_f32(n, stream=98, block=1, step=0)
    for g in (synth.edge_bf16(n, stream=98, block=1, step=1), synth.edge_f32(n, stream=98, block=1, step=2)):
        gf = g if g.dtype == np.float32 else (g.astype(np.uint32) << 16).view(np.float32)
        s = np.float32(0.5)
        p, w = fx.sgd_binary32(master, g, s)
        want = master + (-(s * gf))
        assert np.array_equal(p.view(np.uint32), want.view(np.uint32))
        assert np.array_equal(w, fx.bf16_rne_bits_v(want))
        assert subnormal_count(p) > 100
