"""Pins of the CPU oracle to things other than itself.

Each pin takes a loaded oracle library and raises AssertionError on a
mismatch.  ``test_oracle_pins.py`` runs them against the real oracle;
``test_oracle_planted.py`` runs them against oracle builds with one planted
mistake each and checks that some pin goes red.

What fixes the expected values (never the oracle itself, never the GPU):
  * hand-computed dequantization values (tests/golden/dequant_hand.json);
  * closed forms (constant codes, power-of-two scale and bias);
  * integer special case (s = 1, b = 0) against numpy's int64 matmul;
  * exact rational brute force (fractions.Fraction) on tiny shapes, rounded to
    fp32 by a correctly rounding helper written here;
  * numpy's float64 dot on the dequantized matrix (library routine);
  * invariants: row permutation, power-of-two scaling, negation;
  * argmax: hand-built rows for each rule and numpy's argmax (first
    occurrence) on finite rows;
  * bf16 store: hand-worked roundings and torch's CPU bfloat16 conversion;
  * 2- and 8-bit codes: tables packed with numpy's little-endian views and bit
    packing, read back one weight at a time, as an integer mat-vec and by exact
    rational brute force.
"""
import json
import os
from fractions import Fraction

import numpy as np

import oracle
from w4_gemv_greedy_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
SENTINEL = 0xFFFFFFFF


def _bf16(v):
    """bf16 bits of a value that bf16 holds exactly (checked)."""
    f = np.array([v], np.float32)
    u = int(f.view(np.uint32)[0])
    assert u & 0xFFFF == 0, f"{v} is not a bf16 value"
    return u >> 16


def _f32_of_bits(u):
    return float(np.array([u], np.uint32).view(np.float32)[0])


def frac_to_f32(fr):
    """Round a Fraction to the nearest fp32 (ties to even), normal range only."""
    if fr == 0:
        return 0.0
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    # a in [2^e, 2^(e+1)): 24 significant bits -> quantum 2^(e-23)
    q = a / Fraction(2) ** (e - 23)
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    assert -126 <= e <= 127
    return sign * float(Fraction(n) * Fraction(2) ** (e - 23))


def _codes_to_words(codes):
    """Pack [N][K] codes into [N][K/8] uint32, element 8i+j in bits [4j, 4j+4)."""
    codes = np.asarray(codes, dtype=np.uint32)
    N, K = codes.shape
    c = codes.reshape(N, K // 8, 8)
    words = np.zeros((N, K // 8), np.uint32)
    for j in range(8):
        words |= c[:, :, j] << np.uint32(4 * j)
    return words


# ---------------------------------------------------------------- products

def pin_hand_dequant(lib):
    """P1: hand-computed w values and one-hot products (layout, nibble order, formula)."""
    g = json.load(open(os.path.join(GOLDEN, "dequant_hand.json")))
    K = g["K"]
    wq = np.array([[int(w, 16) for w in row] for row in g["words"]], np.uint32)
    sc = np.array([[int(v, 16) for v in row] for row in g["scales"]], np.uint16)
    bi = np.array([[int(v, 16) for v in row] for row in g["biases"]], np.uint16)
    w = oracle.dequant(wq, sc, bi, lib=lib)
    for r, cols in g["expected_w"].items():
        for k, v in cols.items():
            assert w[int(r), int(k)] == v, (r, k, w[int(r), int(k)], v)
    # one-hot x = e_k reads column k exactly, across every nibble position and the group edge
    for k in list(range(16)) + [62, 63, 64, 65, 71, 72, 127]:
        x = np.zeros((1, K), np.uint16)
        x[0, k] = _bf16(1.0)
        y = oracle.qmm(wq, sc, bi, x, lib=lib)
        want = [float(g["expected_w"][str(r)].get(str(k), w[r, k])) for r in range(2)]
        for r in range(2):
            if str(k) in g["expected_w"][str(r)]:
                assert y[0, r] == want[r], (k, r, y[0, r], want[r])
    x = np.full((1, K), _bf16(1.0), np.uint16)
    y = oracle.qmm(wq, sc, bi, x, lib=lib)
    assert list(y[0]) == g["expected_row_sums"]["y"], y


def pin_closed_form(lib):
    """P2: x = 1, constant code c, s = 2^-a, b = -2^-e  ->  y = K (c 2^-a - 2^-e) exactly."""
    for K, c, a, e, N in [(64, 3, 6, 3, 2), (128, 15, 5, 1, 3), (1024, 0, 4, 7, 1),
                          (5120, 9, 8, 5, 2), (192, 8, 3, 0, 4)]:
        wq = np.full((N, K // 8), c * 0x11111111, np.uint32)
        sc = np.full((N, K // 64), _bf16(2.0 ** -a), np.uint16)
        bi = np.full((N, K // 64), _bf16(-(2.0 ** -e)), np.uint16)
        x = np.full((2, K), _bf16(1.0), np.uint16)
        y = oracle.qmm(wq, sc, bi, x, lib=lib)
        want = K * (c * 2.0 ** -a - 2.0 ** -e)
        assert np.all(y == np.float32(want)), (K, c, a, e, y, want)


def pin_integer_matvec(lib):
    """P3: s = 1, b = 0, small integer x -> integer mat-vec, compared with int64 numpy matmul."""
    r = np.random.default_rng(11)
    for M, N, K in [(2, 3, 192), (3, 5, 64), (1, 7, 320)]:
        codes = r.integers(0, 16, size=(N, K))
        xi = r.integers(-100, 101, size=(M, K))
        wq = _codes_to_words(codes)
        sc = np.full((N, K // 64), _bf16(1.0), np.uint16)
        bi = np.zeros((N, K // 64), np.uint16)
        x = synth.f32_to_bf16_bits(xi.astype(np.float32))
        y = oracle.qmm(wq, sc, bi, x, lib=lib)
        want = xi.astype(np.int64) @ codes.astype(np.int64).T
        assert np.array_equal(y, want.astype(np.float32)), (M, N, K)


def pin_scale_bias_layout(lib):
    """P3b: one distinct power-of-two scale and bias per (row, group); the [N][G] table order."""
    N, K = 3, 256
    G = K // 64
    codes = np.full((N, K), 1, np.int64)
    wq = _codes_to_words(codes)
    sc = np.zeros((N, G), np.uint16)
    bi = np.zeros((N, G), np.uint16)
    for n in range(N):
        for g in range(G):
            sc[n, g] = _bf16(2.0 ** -(n * G + g))
            bi[n, g] = _bf16(2.0 ** -(20 + n * G + g))
    for g in range(G):
        x = np.zeros((1, K), np.uint16)
        x[0, g * 64:(g + 1) * 64] = _bf16(1.0)
        y = oracle.qmm(wq, sc, bi, x, lib=lib)
        for n in range(N):
            want = 64 * (2.0 ** -(n * G + g) + 2.0 ** -(20 + n * G + g))
            assert y[0, n] == np.float32(want), (n, g, y[0, n], want)


def pin_bruteforce(lib):
    """P4: exact rational evaluation of tiny products, rounded once to fp32."""
    for seed, (M, N, K) in enumerate([(1, 2, 64), (2, 3, 128), (2, 4, 64), (1, 1, 128)]):
        wq, sc, bi = synth.weights(N, K, workload=100 + seed)
        x = synth.activations(M, K, workload=100 + seed)
        y = oracle.qmm(wq, sc, bi, x, lib=lib)
        for n in range(N):
            ws = []
            for k in range(K):
                q = (int(wq[n, k // 8]) >> (4 * (k % 8))) & 0xF
                s = Fraction(_f32_of_bits(int(sc[n, k // 64]) << 16))
                b = Fraction(_f32_of_bits(int(bi[n, k // 64]) << 16))
                ws.append(Fraction(frac_to_f32(q * s + b)))
            for m in range(M):
                acc = sum(Fraction(_f32_of_bits(int(x[m, k]) << 16)) * ws[k] for k in range(K))
                want = frac_to_f32(acc)
                assert y[m, n] == np.float32(want), (M, N, K, m, n, y[m, n], want)


def pin_numpy_dot(lib):
    """P5: numpy float64 dot on the dequantized matrix, config-1 shape, within 1 fp32 ulp."""
    N, K = 512, 5120
    wq, sc, bi = synth.weights(N, K, workload=1)
    x = synth.activations(2, K, workload=1)
    w = oracle.dequant(wq, sc, bi, lib=lib).astype(np.float64)
    ref = (synth.bf16_bits_to_f32(x).astype(np.float64) @ w.T).astype(np.float32)
    y = oracle.qmm(wq, sc, bi, x, lib=lib)
    ulp = np.spacing(np.abs(ref))
    assert np.all(np.abs(y.astype(np.float64) - ref) <= ulp), np.max(np.abs(y - ref) / ulp)


def pin_dequant_bits(lib):
    """P1b: dequant of random codes equals q*s+b computed from codes unpacked by integer ops."""
    N, K = 4, 256
    wq, sc, bi = synth.weights(N, K, workload=7)
    w = oracle.dequant(wq, sc, bi, lib=lib)
    s = synth.bf16_bits_to_f32(sc)
    b = synth.bf16_bits_to_f32(bi)
    for n in range(N):
        for k in range(0, K, 5):
            q = (int(wq[n, k // 8]) >> (4 * (k % 8))) & 0xF
            want = frac_to_f32(q * Fraction(float(s[n, k // 64])) + Fraction(float(b[n, k // 64])))
            assert w[n, k] == np.float32(want), (n, k)


def pin_invariants(lib):
    """P6: row permutation permutes y; x*2^j scales y by 2^j; -x gives -y (all exact)."""
    N, K, M = 64, 1024, 3
    wq, sc, bi = synth.weights(N, K, workload=8)
    x = synth.activations(M, K, workload=8)
    y = oracle.qmm(wq, sc, bi, x, lib=lib)
    p = np.random.default_rng(3).permutation(N)
    yp = oracle.qmm(wq[p], sc[p], bi[p], x, lib=lib)
    assert np.array_equal(yp, y[:, p])
    for j in (-3, 5):
        xs = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(x) * np.float32(2.0 ** j))
        assert np.array_equal(oracle.qmm(wq, sc, bi, xs, lib=lib), y * np.float32(2.0 ** j))
    xn = x ^ np.uint16(0x8000)
    assert np.array_equal(oracle.qmm(wq, sc, bi, xn, lib=lib), -y)


def pin_rows_subset(lib):
    """The sampled-rows entry equals the matching columns of the full product."""
    N, K, M = 40, 640, 2
    wq, sc, bi = synth.weights(N, K, workload=9)
    x = synth.activations(M, K, workload=9)
    y = oracle.qmm(wq, sc, bi, x, lib=lib)
    rows = [0, 39, 7, 7, 20]
    assert np.array_equal(oracle.qmm_rows(wq, sc, bi, x, rows, lib=lib), y[:, rows])


# ---------------------------------------------------------------- argmax

def _am(lib, row):
    return int(oracle.argmax(np.asarray(row, np.float32), lib=lib)[0])


def pin_argmax_rules(lib):
    """A1-A10: lowest id on ties, ends of the row, tail, all-equal, non-finite, signed zero, denormals."""
    V = 2048 + 512
    base = -np.abs(np.random.default_rng(5).standard_normal(V).astype(np.float32)) - 1.0
    r = base.copy(); r[[700, 1500]] = 5.0
    assert _am(lib, r) == 700, "A1 tie -> lower id"
    r = base.copy(); r[[1023, 1024]] = 5.0
    assert _am(lib, r) == 1023, "A1 tie across a 1024 boundary"
    r = base.copy(); r[0] = 5.0
    assert _am(lib, r) == 0, "A2 max at id 0"
    r = base.copy(); r[V - 1] = 5.0
    assert _am(lib, r) == V - 1, "A3 max at id V-1"
    r = base.copy(); r[2048 + 100] = 5.0
    assert _am(lib, r) == 2148, "A4 max in the tail block"
    assert _am(lib, np.full(V, 0.25, np.float32)) == 0, "A5 all equal -> 0"
    for bad, name in ((np.nan, "A6 NaN"), (np.inf, "A7 +Inf"), (-np.inf, "A8 -Inf")):
        for pos in (0, 1024, V - 1):
            r = base.copy(); r[pos] = bad
            assert _am(lib, r) == SENTINEL, (name, pos)
    r = base.copy(); r[5] = 1e30; r[6] = np.array([0x7FC12345], np.uint32).view(np.float32)[0]
    assert _am(lib, r) == SENTINEL, "A6 NaN with a payload after a huge value"
    r = base.copy(); r[300] = np.float32(-0.0); r[900] = np.float32(0.0)
    assert _am(lib, r) == 300, "A9 -0.0/+0.0 tie -> lower id"
    r = base.copy(); r[300] = np.float32(0.0); r[900] = np.float32(-0.0)
    assert _am(lib, r) == 300, "A9 +0.0/-0.0 tie -> lower id"
    r = base.copy(); d = np.array([1, 2, 3], np.uint32).view(np.float32)
    r[400], r[401], r[402] = d[0], d[2], d[1]
    assert _am(lib, r) == 401, "A10 largest denormal"
    r = base.copy(); r[400] = -d[1]; r[401] = -d[0]
    r[:] = np.where(np.arange(V) < 400, -5.0, r)
    assert _am(lib, r[:403]) == 401, "A10 negative denormals: -1ulp beats -2ulp"
    assert _am(lib, np.array([3.0], np.float32)) == 0, "single element"
    assert _am(lib, np.array([np.inf], np.float32)) == SENTINEL, "single +Inf"


def pin_argmax_numpy(lib):
    """A: 1000 seeded finite rows equal numpy's argmax (first occurrence), fp32 and bf16 input."""
    r = np.random.default_rng(17)
    x = (r.standard_normal((1000, 3000)) * 3).astype(np.float32)
    # coarse values make exact ties common
    x[500:] = np.round(x[500:] * 4) / 4
    ids = oracle.argmax(x, lib=lib)
    assert np.array_equal(ids, np.argmax(x, axis=1).astype(np.uint32))
    xb = synth.f32_to_bf16_bits(x)
    ids_b = oracle.argmax(xb, lib=lib)
    assert np.array_equal(ids_b, np.argmax(synth.bf16_bits_to_f32(xb), axis=1).astype(np.uint32))


def pin_argmax_bf16_nonfinite(lib):
    """bf16 rows: NaN, +Inf, -Inf bit patterns trip the sentinel; -0/+0 tie."""
    V = 1500
    row = synth.f32_to_bf16_bits(-np.abs(np.random.default_rng(2).standard_normal(V)).astype(np.float32))
    for bits in (0x7FC0, 0x7F81, 0xFFC0, 0x7F80, 0xFF80):
        r = row.copy(); r[777] = bits
        assert int(oracle.argmax(r, lib=lib)[0]) == SENTINEL, hex(bits)
    r = row.copy(); r[10] = 0x8000; r[20] = 0x0000
    assert int(oracle.argmax(r, lib=lib)[0]) == 10


def pin_top2_lexsort(lib):
    """Top two: the first two ids of numpy's stable sort by value descending (a
    lexsort on (id, -value)), on random rows and on coarse rows full of ties,
    fp32 and bf16; the gap is their fp32 difference with zeros counted as +0."""
    r = np.random.default_rng(23)
    x = (r.standard_normal((600, 2500)) * 3).astype(np.float32)
    x[300:] = np.round(x[300:] * 2) / 2            # many exact ties, at the top too
    x[550:, 100] = x[550:].max(axis=1)              # a tie for first place at id 100 or above
    x[580:] = np.where(x[580:] == 0, np.float32(-0.0), x[580:])  # -0.0 among the zeros
    for data, vals in ((x, x), (synth.f32_to_bf16_bits(x), None)):
        vals = synth.bf16_bits_to_f32(data) if vals is None else vals
        ids, gaps = oracle.argmax_top2(data, lib=lib)
        for i in range(vals.shape[0]):
            order = np.lexsort((np.arange(vals.shape[1]), -vals[i].astype(np.float64)))
            a, b = order[0], order[1]
            assert (ids[i, 0], ids[i, 1]) == (a, b), (i, ids[i], a, b)
            want = np.float32(vals[i, a] + np.float32(0)) - np.float32(vals[i, b] + np.float32(0))
            assert gaps[i].tobytes() == np.float32(want).tobytes(), (i, gaps[i], want)


def pin_top2_rules(lib):
    """Top two on hand-made rows: ties, +-0, denormals, the last id, non-finite rows."""
    def t2(row):
        ids, gaps = oracle.argmax_top2(np.asarray(row, np.float32), lib=lib)
        return int(ids[0, 0]), int(ids[0, 1]), float(gaps[0])
    assert t2([1, 2, 3]) == (2, 1, 1.0)
    assert t2([5, 5, 1]) == (0, 1, 0.0)               # tied winners: lower id first
    assert t2([3, 5, 5]) == (1, 2, 0.0)
    assert t2([7, 1, 7, 7]) == (0, 2, 0.0)
    assert t2([1, 4, 2, 4, 3]) == (1, 3, 0.0)
    assert t2([0.0, -0.0]) == (0, 1, 0.0)
    assert t2([-0.0, 0.0]) == (0, 1, 0.0)
    ids, gaps = oracle.argmax_top2(np.array([[-0.0, 0.0, -1.0]], np.float32), lib=lib)
    assert gaps[0].tobytes() == np.float32(0.0).tobytes()   # never -0.0
    d1, d2 = np.float32(2.0 ** -148), np.float32(2.0 ** -149)  # two and one times the least denormal
    assert t2([d2, d1, 0.0]) == (1, 0, float(d1 - d2))       # denormals compare exactly
    assert t2([-3, -2, -1]) == (2, 1, 1.0)                   # winner at the last id
    ids, gaps = oracle.argmax_top2(np.array([[1, np.nan, 2], [np.inf, 1, 2], [1, 2, -np.inf]],
                                            np.float32), lib=lib)
    assert np.all(ids == SENTINEL) and np.all(np.isnan(gaps))


def pin_bf16_store(lib):
    """bf16 store: hand-worked roundings (ties to even, overflow to infinity, signed
    zero, denormals, NaN kept) and torch's CPU fp32 -> bfloat16 conversion (a
    nearest-even library routine) on random values, exact midpoints and
    specials."""
    import torch

    def b(v):
        return int(oracle.to_bf16(np.array([v], np.float32), lib=lib)[0])
    assert b(1.0) == 0x3F80
    assert b(1.0 + 2.0 ** -8) == 0x3F80            # midpoint of 0x3F80 and 0x3F81: to even
    assert b(1.0 + 3 * 2.0 ** -8) == 0x3F82        # midpoint of 0x3F81 and 0x3F82: to even
    assert b(1.0 + 2.0 ** -8 + 2.0 ** -20) == 0x3F81  # just past the midpoint
    assert b(-(1.0 + 2.0 ** -8)) == 0xBF80
    assert b(-0.0) == 0x8000 and b(0.0) == 0x0000
    assert b((2 - 2.0 ** -8) * 2.0 ** 127) == 0x7F80   # midpoint of the largest bf16 and 2^128
    assert b((2 - 2.0 ** -7) * 2.0 ** 127) == 0x7F7F
    assert b(2.0 ** -149) == 0x0000                # below half the least bf16 denormal
    assert b(3 * 2.0 ** -134) == 0x0002            # 1.5 least denormals: tie to even (2)
    assert b(float("inf")) == 0x7F80 and b(float("-inf")) == 0xFF80
    nan = oracle.to_bf16(np.array([np.nan, -np.nan], np.float32), lib=lib)
    assert np.all((nan & 0x7F80) == 0x7F80) and np.all((nan & 0x7F) != 0)
    assert (int(nan[1]) >> 15) == (int(np.array([-np.nan], np.float32).view(np.uint32)[0]) >> 31)
    r = np.random.default_rng(31)
    v = (r.standard_normal(60000) * np.exp2(r.integers(-140, 120, 60000))).astype(np.float32)
    u = r.integers(0, 1 << 32, 20000, dtype=np.uint64).astype(np.uint32)
    mids = ((u & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)   # exact midpoints
    mids = mids[np.isfinite(mids)]
    special = np.array([0.0, -0.0, np.inf, -np.inf, 3.4028235e38, -3.4028235e38, 1e-45, -1e-45,
                        1.1754944e-38, 2.0 ** -133, 2.0 ** -134, 65504.0], np.float32)
    allv = np.concatenate([v, mids, special]).astype(np.float32)
    want = torch.from_numpy(allv).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.to_bf16(allv, lib=lib)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(allv[i], hex(got[i]), hex(want[i])) for i in bad[:5]]


def pack_codes(codes, bits):
    """[N][K] codes -> [N][K*bits/32] uint32 words, element (32/bits) i + j in bits
    [bits j, bits j + bits) of word i, built with numpy's little-endian views and
    bit packing rather than shifts: 8-bit codes are the bytes of little-endian
    words; 2- and 4-bit codes are a little-endian bit stream."""
    codes = np.ascontiguousarray(codes)
    N, K = codes.shape
    if bits == 8:
        return codes.astype(np.uint8).view("<u4").reshape(N, K // 4).astype(np.uint32)
    bitplanes = ((codes[..., None].astype(np.uint32) >> np.arange(bits, dtype=np.uint32)) & 1).astype(np.uint8)
    packed = np.packbits(bitplanes.reshape(N, K * bits), axis=1, bitorder="little")
    return packed.view("<u4").reshape(N, K * bits // 32).astype(np.uint32)


def pin_bits_hand_dequant(lib):
    """Other widths: s = 2^-6, b = -1/8, so w = q/64 - 1/8 exactly; one-hot x reads
    single weights (every field position of a word, both sides of a group boundary)
    and the dequantized table matches code by code."""
    for bits in (2, 8):
        r = np.random.default_rng(bits)
        N, K = 3, 128
        codes = r.integers(0, 1 << bits, size=(N, K), dtype=np.int64)
        codes[0, :4] = [0, (1 << bits) - 1, 1, (1 << bits) // 2]
        wq = pack_codes(codes, bits)
        sc = np.full((N, K // 64), _bf16(2.0 ** -6), np.uint16)
        bi = np.full((N, K // 64), _bf16(-0.125), np.uint16)
        want = codes.astype(np.float64) / 64.0 - 0.125
        w = oracle.dequant(wq, sc, bi, lib=lib, bits=bits)
        assert np.array_equal(w.astype(np.float64), want), bits
        for k in list(range(0, 32 // bits + 1)) + [63, 64, 65, K - 1]:
            x = np.zeros((1, K), np.uint16)
            x[0, k] = _bf16(1.0)
            y = oracle.qmm(wq, sc, bi, x, lib=lib, bits=bits)
            assert np.array_equal(y[0].astype(np.float64), want[:, k]), (bits, k)


def pin_bits_integer_matvec(lib):
    """Other widths with s = 1, b = 0 and small integer x: an integer mat-vec,
    compared with numpy's int64 matmul (exact in fp32 at these sizes)."""
    for bits in (2, 8):
        r = np.random.default_rng(100 + bits)
        N, K, M = 7, 256, 3
        codes = r.integers(0, 1 << bits, size=(N, K), dtype=np.int64)
        xi = r.integers(-8, 9, size=(M, K), dtype=np.int64)
        x = np.vectorize(lambda v: _bf16(float(v)))(xi).astype(np.uint16)
        sc = np.full((N, K // 64), _bf16(1.0), np.uint16)
        bi = np.zeros((N, K // 64), np.uint16)
        y = oracle.qmm(pack_codes(codes, bits), sc, bi, x, lib=lib, bits=bits)
        assert np.array_equal(y.astype(np.int64), xi @ codes.T), bits


def pin_bits_bruteforce(lib):
    """Other widths: exact rational evaluation of tiny products with random bf16
    scales, biases and activations, rounded once to fp32."""
    for bits in (2, 8):
        r = np.random.default_rng(200 + bits)
        N, K, M = 2, 128, 2
        codes = r.integers(0, 1 << bits, size=(N, K), dtype=np.int64)
        sc = synth.f32_to_bf16_bits(r.uniform(0.002, 0.02, (N, K // 64)).astype(np.float32))
        bi = synth.f32_to_bf16_bits(r.normal(0, 0.05, (N, K // 64)).astype(np.float32))
        x = synth.f32_to_bf16_bits(r.normal(0, 1, (M, K)).astype(np.float32))
        y = oracle.qmm(pack_codes(codes, bits), sc, bi, x, lib=lib, bits=bits)
        xf = synth.bf16_bits_to_f32(x).astype(np.float64)
        sf = synth.bf16_bits_to_f32(sc).astype(np.float64)
        bf = synth.bf16_bits_to_f32(bi).astype(np.float64)
        for m in range(M):
            for n in range(N):
                tot = Fraction(0)
                for k in range(K):
                    w = Fraction(np.float32(codes[n, k] * sf[n, k // 64] + bf[n, k // 64]).item())
                    tot += Fraction(xf[m, k].item()) * w
                assert y[m, n] == np.float32(frac_to_f32(tot)), (bits, m, n)


PRODUCT_PINS = [pin_hand_dequant, pin_closed_form, pin_integer_matvec, pin_scale_bias_layout,
                pin_bruteforce, pin_numpy_dot, pin_dequant_bits, pin_invariants, pin_rows_subset,
                pin_bf16_store, pin_bits_hand_dequant, pin_bits_integer_matvec, pin_bits_bruteforce]
ARGMAX_PINS = [pin_argmax_rules, pin_argmax_numpy, pin_argmax_bf16_nonfinite, pin_top2_rules,
               pin_top2_lexsort]
ALL_PINS = PRODUCT_PINS + ARGMAX_PINS
