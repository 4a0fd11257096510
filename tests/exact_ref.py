"""Exact checker for tiny inputs: the step evaluated with rational arithmetic.

Every binary32 operation of the numerics contract is modelled by its
definition: compute the exact rational result with ``fractions.Fraction``,
then round it to the nearest binary32 value (ties to even, with gradual
underflow).  Binary64 parts (the sums of squares and the square root of a
scale) use Python floats, which are IEEE binary64.  Nothing here calls the
C oracle or the GPU library; it is an independent model used to pin the
oracle's build (operation order, no fused multiply-add, no flush of
subnormals, the bit layout and the segment bookkeeping) on tiny inputs.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

_TWO = Fraction(2)


def f32(q) -> Fraction:
    """Round a rational to the nearest binary32 value (ties to even)."""
    q = Fraction(q)
    if q == 0:
        return Fraction(0)
    neg = q < 0
    a = -q if neg else q
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if _TWO ** e > a:
        e -= 1
    while _TWO ** (e + 1) <= a:
        e += 1
    quantum_exp = max(e, -126) - 23  # subnormals share the quantum 2^-149
    quantum = _TWO ** quantum_exp
    r = round(a / quantum)  # Fraction.__round__: half to even
    res = r * quantum
    if res >= _TWO ** 128:
        raise OverflowError("binary32 overflow")
    return -res if neg else res


def coef(beta):
    """(fl32(beta), fl32(1 - beta)) with 1 - beta formed in binary64."""
    return F(np.float32(beta)), F(np.float32(1.0 - float(beta)))


def F(x) -> Fraction:
    """Exact value of a binary32/binary16/binary64 number."""
    return Fraction(float(x))


def as_f32_array(vals) -> np.ndarray:
    return np.array([float(v) for v in vals], dtype=np.float32)


def sign(c: Fraction, negzero=False) -> int:
    """sign(0) = +1 (also for -0.0, which a Fraction cannot carry)."""
    return -1 if c < 0 else 1


def scale(cs) -> Fraction:
    """||c||_2 / sqrt(len): sum of exact squares in binary64, in index order,
    sqrt in binary64, rounded once to binary32."""
    s = 0.0
    for c in cs:
        s += float(c) * float(c)
    return f32(Fraction(math.sqrt(s / len(cs))))


def onebit(cs, seg):
    """Compress vector cs (Fractions) with segment offsets seg.
    Returns (bits list of 0/1, scales, residuals)."""
    bits = [1 if c < 0 else 0 for c in cs]
    scales, err = [], [None] * len(cs)
    for j in range(len(seg) - 1):
        lo, hi = int(seg[j]), int(seg[j + 1])
        s = scale(cs[lo:hi])
        scales.append(s)
        for k in range(lo, hi):
            err[k] = f32(cs[k] - s * sign(cs[k]))
    return bits, scales, err


def seg_of(seg, k):
    j = 0
    while int(seg[j + 1]) <= k:
        j += 1
    return j


def compress(g, m, delta, wseg, beta1):
    """g, delta: [n][d] numpy; m: [d].  Returns (bits[n][d], scales[n][..],
    new delta[n][d]) as Python lists of ints / Fractions."""
    b1, omb1 = coef(beta1)
    n, d = delta.shape
    out_bits, out_scales, out_delta = [], [], []
    for i in range(n):
        cs = []
        for k in range(d):
            p = f32(f32(b1 * F(m[k])) + f32(omb1 * F(g[i][k])))
            cs.append(f32(p + F(delta[i][k])))
        b, s, e = onebit(cs, wseg)
        out_bits.append(b)
        out_scales.append(s)
        out_delta.append(e)
    return out_bits, out_scales, out_delta


def server(bits, scales, wseg, sseg, eps):
    n = len(bits)
    d = len(eps)
    a = []
    for k in range(d):
        j = seg_of(wseg, k)
        t = Fraction(0)
        for i in range(n):
            t = f32(t + scales[i][j] * (-1 if bits[i][k] else 1))
        a.append(f32(f32(t / n) + F(eps[k])))
    return onebit(a, sseg)


def update(sbits, sscales, sseg, denom, x, lr):
    lr = F(np.float32(lr))
    d = len(x)
    m_new, x_new = [], []
    for k in range(d):
        mh = sscales[seg_of(sseg, k)] * (-1 if sbits[k] else 1)
        m_new.append(mh)
        x_new.append(f32(F(x[k]) - f32(f32(lr * mh) / F(denom[k]))))
    return m_new, x_new


def adam_warmup(g, x, m, v, lr, beta1, beta2, eta, bc1=1.0, bc2=1.0):
    """One warm-up step; returns new (x, m, v) as lists of Fractions.
    sqrt of a binary32 value: math.sqrt on its binary64 image is correctly
    rounded there, and rounding that once more to binary32 equals the
    correctly rounded binary32 square root (binary64 carries more than
    2*24+2 bits)."""
    n, d = g.shape
    b1, omb1 = coef(beta1)
    b2, omb2 = coef(beta2)
    lr, eta = F(np.float32(lr)), F(np.float32(eta))
    bc1, bc2 = F(np.float32(bc1)), F(np.float32(bc2))
    xs, ms, vs = [], [], []
    for k in range(d):
        t = Fraction(0)
        for i in range(n):
            t = f32(t + F(g[i][k]))
        gb = f32(t / n)
        mk = f32(f32(b1 * F(m[k])) + f32(omb1 * gb))
        vk = f32(f32(b2 * F(v[k])) + f32(omb2 * f32(gb * gb)))
        root = f32(Fraction(math.sqrt(float(f32(vk / bc2)))))
        xk = f32(F(x[k]) - f32(f32(lr * f32(mk / bc1)) / f32(root + eta)))
        xs.append(xk)
        ms.append(mk)
        vs.append(vk)
    return xs, ms, vs


def pack(bits_list, d):
    """0/1 list -> uint64 words, LSB = lowest coordinate."""
    W = (d + 63) // 64
    words = [0] * W
    for k, b in enumerate(bits_list):
        if b:
            words[k // 64] |= 1 << (k % 64)
    return np.array(words, dtype=np.uint64)
