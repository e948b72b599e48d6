"""A model of the order the vector-ALU decode kernels document (include/w4g.h,
qmm_gemv): per output row, K in chunks of 1024; lane l of a 32-lane half wave
owns elements [32 l, 32 l + 32) of each chunk, four code words of eight codes;
word i's codes pair as (128 + q[8i + j], 128 + q[8i + j + 4]) against
(x[8i + j], x[8i + j + 4]), j = 0..3, each pair added by one dot2 into D from
zero; X is the same pairs' x summed against (1, 1) by dot2 in the same order;
the lane then adds s D and (b - 128 s) X to its running sum with fused
multiply-adds (b - 128 s itself one), chunk after chunk; the 32 lane sums meet
in a fixed tree: lanes i and i + 16 add, then within each 16 lanes i and 15 - i,
within each 8 i and 7 - i, then i and i ^ 2, then i and i ^ 1.

Every step is exact rational arithmetic rounded once to fp32 (nearest even).
For the fused multiply-adds and the adds that is their definition; for the
dot2 it is a model, single rounding of the exact a0 b0 + a1 b1 + c, which the
instruction follows where its terms do not cancel (with activations and codes
of one sign every dot2 adds terms of one sign).  Test infrastructure: only
tests call it; it shares nothing with the library.
"""
from fractions import Fraction

import numpy as np

CHUNK = 1024


def _f32(fr):
    """Round a Fraction to the nearest fp32, ties to even (normal range or zero)."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    assert -126 <= e <= 127, "outside the fp32 normal range"
    q = a / Fraction(2) ** (e - 23)
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * Fraction(n) * Fraction(2) ** (e - 23)


def _bf16(bits):
    v = np.array([int(bits) << 16], dtype=np.uint32).view(np.float32)[0]
    return Fraction(float(v))


def _codes(wq_row, K):
    w = np.asarray(wq_row, dtype=np.uint32)
    return [(int(w[k // 8]) >> (4 * (k % 8))) & 15 for k in range(K)]


def row(wq_row, sc_row, bi_row, x_row):
    """The fp32 result of one output row (as a Fraction) for one row of x."""
    K = len(x_row)
    assert K % CHUNK == 0
    q = _codes(wq_row, K)
    x = [_bf16(v) for v in x_row]
    lanes = []
    for l in range(32):
        acc = Fraction(0)
        for c in range(K // CHUNK):
            base = c * CHUNK + 32 * l
            d = Fraction(0)
            h = Fraction(0)
            for i in range(4):
                for j in range(4):
                    k0, k1 = base + 8 * i + j, base + 8 * i + j + 4
                    d = _f32((128 + q[k0]) * x[k0] + (128 + q[k1]) * x[k1] + d)
                    h = _f32(x[k0] + x[k1] + h)
            g = base // 64
            s = _bf16(sc_row[g])
            cb = _f32(-128 * s + _bf16(bi_row[g]))
            acc = _f32(s * d + acc)
            acc = _f32(cb * h + acc)
        lanes.append(acc)
    v = [_f32(lanes[i % 16] + lanes[i % 16 + 16]) for i in range(32)]
    for partner in (lambda i: (i & ~15) | (15 - (i & 15)), lambda i: (i & ~7) | (7 - (i & 7)),
                    lambda i: i ^ 2, lambda i: i ^ 1):
        v = [_f32(v[i] + v[partner(i)]) for i in range(32)]
    assert all(t == v[0] for t in v)
    return v[0]


def f32_bits(fr):
    return int(np.array([float(fr)], dtype=np.float32).view(np.uint32)[0])
