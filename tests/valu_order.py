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

Other code widths (qmm_gemv_bits): 2-bit word t of a lane holds its elements
16t .. 16t + 15 and pairs fields (j, j + 8), j = 0..7; an 8-bit code is its two
nibbles l + 16 h, word t holds elements 4t .. 4t + 3, and each word adds
(l0, l2), (l1, l3) against (x0, x2), (x1, x3) into Dl and the high nibbles
likewise into Dh, D = fma(16, Dh, Dl) and the bias term's constant 2176 s; X
then sums the pairs (x0, x2), (x1, x3), (x4, x6), (x5, x7) of each
8-element block.
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


def _codes(wq_row, K, bits):
    w = np.asarray(wq_row, dtype=np.uint32)
    per = 32 // bits
    mask = (1 << bits) - 1
    return [(int(w[k // per]) >> (bits * (k % per))) & mask for k in range(K)]


def _segment(q, x, base, bits):
    """D and X of one lane's 32 elements starting at `base`."""
    d = Fraction(0)
    h = Fraction(0)
    if bits == 4:
        for i in range(4):
            for j in range(4):
                k0, k1 = base + 8 * i + j, base + 8 * i + j + 4
                d = _f32((128 + q[k0]) * x[k0] + (128 + q[k1]) * x[k1] + d)
                h = _f32(x[k0] + x[k1] + h)
    elif bits == 2:
        for t in range(2):
            for j in range(8):
                k0, k1 = base + 16 * t + j, base + 16 * t + j + 8
                d = _f32((128 + q[k0]) * x[k0] + (128 + q[k1]) * x[k1] + d)
        for i in range(4):  # X over each 8-element block's halves of the 16-element pairing
            t, half = divmod(i, 2)
            for j in range(4):
                k0 = base + 16 * t + 4 * half + j
                h = _f32(x[k0] + x[k0 + 8] + h)
    else:
        dl = Fraction(0)
        dh = Fraction(0)
        for t in range(8):
            k = base + 4 * t
            lo = [q[k + j] & 15 for j in range(4)]
            hi = [q[k + j] >> 4 for j in range(4)]
            dl = _f32((128 + lo[0]) * x[k] + (128 + lo[2]) * x[k + 2] + dl)
            dl = _f32((128 + lo[1]) * x[k + 1] + (128 + lo[3]) * x[k + 3] + dl)
            dh = _f32((128 + hi[0]) * x[k] + (128 + hi[2]) * x[k + 2] + dh)
            dh = _f32((128 + hi[1]) * x[k + 1] + (128 + hi[3]) * x[k + 3] + dh)
        d = _f32(16 * dh + dl)
        for i in range(4):
            k = base + 8 * i
            for a, b in ((0, 2), (1, 3), (4, 6), (5, 7)):
                h = _f32(x[k + a] + x[k + b] + h)
    return d, h


def row(wq_row, sc_row, bi_row, x_row, bits=4):
    """The fp32 result of one output row (as a Fraction) for one row of x."""
    K = len(x_row)
    assert K % CHUNK == 0
    q = _codes(wq_row, K, bits)
    x = [_bf16(v) for v in x_row]
    const = 2176 if bits == 8 else 128  # 128 per expanded field, 128 + 16 * 128 per 8-bit code
    lanes = []
    for l in range(32):
        acc = Fraction(0)
        for c in range(K // CHUNK):
            base = c * CHUNK + 32 * l
            d, h = _segment(q, x, base, bits)
            g = base // 64
            s = _bf16(sc_row[g])
            cb = _f32(-const * s + _bf16(bi_row[g]))
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
