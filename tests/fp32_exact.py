"""Exact IEEE binary32 arithmetic for tests: every operation is carried out
on rationals (fractions.Fraction) and rounded once, to nearest with ties to
even, with gradual underflow, overflow to infinity and IEEE signed zeros.
Finite inputs only.

The fused kernel's per-element arithmetic is a fixed sequence of such
operations (explicit FMAs, one square root and one division, each
correctly rounded; no contraction), so a step can be reproduced bit for bit
here and compared with the kernel's stored master, m, v and BF16 weight.
This is test infrastructure, separate from the FP64 oracle (which defines
the update itself and is compared with a tolerance).
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

_MIN_QUANTUM_EXP = -149          # spacing of subnormals
_MAX_FINITE = Fraction((1 << 24) - 1) * (Fraction(2) ** 104)


def _floor_log2(a: Fraction) -> int:
    """e with 2**e <= a < 2**(e+1), for a > 0."""
    n, d = a.numerator, a.denominator
    e = n.bit_length() - d.bit_length()
    if (n << -e if e < 0 else n) < (d << e if e > 0 else d):
        e -= 1
    return e


def round32(q: Fraction, zero_negative: bool = False) -> np.float32:
    """q rounded to the nearest binary32 (ties to even).  An exact zero
    takes the sign the operation's IEEE rule gives (zero_negative)."""
    if q == 0:
        return np.float32(-0.0) if zero_negative else np.float32(0.0)
    neg = q < 0
    a = -q if neg else q
    qexp = max(_floor_log2(a) - 23, _MIN_QUANTUM_EXP)
    scaled = a / (Fraction(2) ** qexp)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n & 1):
        n += 1
    mag = Fraction(n) * (Fraction(2) ** qexp)
    if mag > _MAX_FINITE:
        val = math.inf
    else:
        val = float(mag)           # exact: mag has at most 24 significant bits
    return np.float32(-val if neg else val)


def exact(x) -> Fraction:
    x = np.float32(x)
    if not np.isfinite(x):
        raise ValueError("finite inputs only")
    return Fraction(float(x))


def _neg(x) -> bool:
    return bool(np.signbit(np.float32(x)))


def add(a, b) -> np.float32:
    # an exact zero sum is +0 unless both operands are -0
    return round32(exact(a) + exact(b), zero_negative=_neg(a) and _neg(b))


def mul(a, b) -> np.float32:
    return round32(exact(a) * exact(b), zero_negative=_neg(a) != _neg(b))


def div(a, b) -> np.float32:
    qb = exact(b)
    if qb == 0:
        raise ZeroDivisionError("division by zero is outside these tests")
    return round32(exact(a) / qb, zero_negative=_neg(a) != _neg(b))


def fma(a, b, c) -> np.float32:
    """a*b + c with a single rounding."""
    p = exact(a) * exact(b)
    s = p + exact(c)
    if s == 0:
        p_neg = _neg(a) != _neg(b)
        # an exact zero: -0 only when the product and c are zeros of sign -
        zero_negative = p == 0 and exact(c) == 0 and p_neg and _neg(c)
        return round32(s, zero_negative)
    return round32(s)


def sqrt(a) -> np.float32:
    """Correctly rounded square root: the integer square root of the
    operand scaled to far more bits than binary32 keeps, with the remainder
    as the sticky bit."""
    q = exact(a)
    if q < 0:
        raise ValueError("negative operand")
    if q == 0:
        return np.float32(a)     # sqrt(+-0) = +-0
    # q = N / D; sqrt(q) = sqrt(N * D) / D.  Scale by 4**k so the integer
    # root carries at least 60 bits beyond binary32's 24.
    n, d = q.numerator, q.denominator
    k = max(0, 100 - (n * d).bit_length() // 2)
    x = n * d << (2 * k)
    r = math.isqrt(x)
    root = Fraction(r, d << k)
    if r * r != x:
        # sticky: the true root lies strictly between r and r + 1, far below
        # the rounding position, so nudge it off any tie
        root += Fraction(1, (d << k) * 2)
    return round32(root)


def neg(a) -> np.float32:
    return np.float32(-np.float32(a))


def bf16_rne_bits(x) -> int:
    """BF16 bits of a finite binary32 by round to nearest even (integer
    form: the upper 16 bits after adding 0x7FFF plus the lowest kept bit)."""
    u = int(np.float32(x).view(np.uint32))
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF


def bf16_to_f32(bits: int) -> np.float32:
    return np.uint32(int(bits) << 16).view(np.float32)


# ---------------------------------------------------------- the Adam step

def adam_constants(t: int, lr: float, beta1: float, beta2: float, eps: float) -> np.ndarray:
    """The step's constants as the library forms them: in FP64, each
    rounded once to FP32 (b1, 1 - b1, b2, 1 - b2, lr / (1 - b1^t),
    1 / sqrt(1 - b2^t), eps, 0)."""
    return np.array([beta1, 1.0 - beta1, beta2, 1.0 - beta2, lr / (1.0 - beta1 ** t),
                     1.0 / math.sqrt(1.0 - beta2 ** t), eps, 0.0], np.float64).astype(np.float32)


def adam_binary32(master, m, v, g_bits, c):
    """One Adam step of every element as the kernel orders it in binary32:
    m' = fma(b1, m, (1-b1) g); v' = fma(b2, v, (1-b2)(g g));
    den = fma(sqrt(v'), r, eps); master' = master + -((s m') / den); the
    BF16 weight is master' rounded to nearest even.  g_bits: BF16 patterns
    (uint16) or FP32 gradients (float32; then g*g rounds).  Returns new
    arrays."""
    b1, c1, b2, c2, s, r, e = (np.float32(x) for x in c[:7])
    out_p, out_m, out_v = master.copy(), m.copy(), v.copy()
    out_w = np.zeros(master.size, np.uint16)
    f32_grads = np.asarray(g_bits).dtype == np.float32
    for i in range(master.size):
        g = np.float32(g_bits[i]) if f32_grads else bf16_to_f32(g_bits[i])
        m1 = fma(b1, m[i], mul(c1, g))
        v1 = fma(b2, v[i], mul(c2, mul(g, g)))
        den = fma(sqrt(v1), r, e)
        delta = neg(div(mul(s, m1), den))
        p = add(master[i], delta)
        out_p[i], out_m[i], out_v[i] = p, m1, v1
        out_w[i] = bf16_rne_bits(p)
    return out_p, out_m, out_v, out_w


def sgd_binary32(master, g_bits, s):
    """One SGD step as the kernel orders it in binary32: master' = master +
    -(s g), a product and a sum each rounded once (nothing fused).  g_bits:
    BF16 patterns or FP32 gradients.  Returns (master', BF16 weight bits)."""
    s = np.float32(s)
    out_p = np.asarray(master, np.float32).copy()
    out_w = np.zeros(out_p.size, np.uint16)
    f32_grads = np.asarray(g_bits).dtype == np.float32
    for i in range(out_p.size):
        g = np.float32(g_bits[i]) if f32_grads else bf16_to_f32(g_bits[i])
        out_p[i] = add(out_p[i], neg(mul(s, g)))
        out_w[i] = bf16_rne_bits(out_p[i])
    return out_p, out_w


# ------------------------------------------------- vectorised, for large samples
#
# numpy's float32 add, multiply, divide and sqrt are the IEEE binary32
# operations (one rounding, to nearest even).  Only the FMA needs work: the
# product of two binary32 values is exact in binary64, and TwoSum gives the
# exact sum as s + e; s rounded to binary32 is the correct result except when
# s lies exactly half-way between two binary32 values and e != 0, where the
# sign of e decides.  Pinned against the rational functions above.

def _two_sum(a, b):
    s = a + b
    bb = s - a
    return s, (a - (s - bb)) + (b - bb)


def fma_v(a, b, c):
    """Correctly rounded a*b + c for binary32 arrays."""
    a64, b64, c64 = (np.asarray(x, np.float32).astype(np.float64) for x in (a, b, c))
    s, e = _two_sum(a64 * b64, c64)
    with np.errstate(over="ignore"):
        r = s.astype(np.float32)
        r64 = r.astype(np.float64)
        other = np.nextafter(r, np.where(s > r64, np.float32(np.inf), np.float32(-np.inf))).astype(np.float32)
        mid = (r64 + other.astype(np.float64)) * 0.5
    tie = (s != r64) & (s == mid) & (e != 0)
    # at a tie the exact value lies beyond the midpoint on e's side
    toward_other = tie & ((e > 0) == (other.astype(np.float64) > r64))
    out = np.where(toward_other, other, r)
    # an exact zero: -0 only when a*b and c are both zeros of sign -
    zero = (s == 0) & (e == 0)
    if np.any(zero):
        pz = (a64 * b64 == 0) & (np.signbit(a64) != np.signbit(b64))
        neg0 = zero & pz & (c64 == 0) & np.signbit(c64)
        out = np.where(zero, np.where(neg0, np.float32(-0.0), np.float32(0.0)), out)
    return out.astype(np.float32)


def bf16_rne_bits_v(x):
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return (((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF).astype(np.uint16)


def adam_binary32_v(master, m, v, g_bits, c):
    """adam_binary32 on whole arrays (the same sequence of binary32
    operations, vectorised)."""
    b1, c1, b2, c2, s, r, e = (np.float32(x) for x in c[:7])
    g = np.asarray(g_bits)
    g = g.astype(np.float32) if g.dtype == np.float32 else (g.astype(np.uint32) << 16).view(np.float32)
    f32 = lambda x: np.asarray(x, np.float32)
    m1 = fma_v(b1, f32(m), c1 * g)
    v1 = fma_v(b2, f32(v), c2 * (g * g))
    den = fma_v(np.sqrt(v1), r, e)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        delta = -((s * m1) / den)
    p = f32(master) + delta
    return p.astype(np.float32), m1, v1, bf16_rne_bits_v(p)
