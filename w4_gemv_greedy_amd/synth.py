"""Seeded synthetic inputs for the W4 g64 products and the greedy argmax.

This module only draws inputs; it holds none of the products' or the argmax's
arithmetic.  The same bytes feed the CPU oracle and the GPU library.  bf16
tensors are returned as numpy uint16 bit patterns.

Recipe (one stream per tensor: numpy PCG64 seeded with
SeedSequence([workload, matrix, tensor, layer])):
  * packed codes: uniform random uint32 words, so every 4-bit code is
    independently uniform on 0..15, eight codes per word along K;
  * scale: sign * U[0.002, 0.02] with the sign +-1 equiprobable, rounded to
    bf16 (round to nearest even);
  * bias: fp32 (-8 * scale + N(0, 1e-3)), rounded to bf16;
  * activations: N(0, 1) rounded to bf16;
  * logits: N(0, 3) fp32 (plus a bf16 copy), with planted rows (exact ties
    across block boundaries and in the tail, NaN, +Inf, -Inf, a -0/+0 tie,
    adjacent denormals).
"""
import numpy as np

# matrix ids used in seeds
O_PROJ, GATE_UP, DOWN, LM_HEAD, GENERIC = 0, 1, 2, 3, 9
# tensor ids used in seeds
T_CODES, T_SCALE_MAG, T_SCALE_SIGN, T_BIAS_EPS, T_ACT, T_LOGITS = 0, 1, 2, 3, 4, 5

# the model widths the workloads use
HIDDEN = 5120
INTERMEDIATE = 17408
VOCAB = 248320


def rng(workload, matrix, tensor, layer=0):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [int(workload), int(matrix), int(tensor), int(layer)])))


def f32_to_bf16_bits(a):
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    r = r.astype(np.uint16)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return r


def bf16_bits_to_f32(h):
    """Widen bf16 bits to fp32 (exact)."""
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def weights(N, K, workload=0, matrix=GENERIC, layer=0, bits=4):
    """(codes [N][K*bits/32] uint32, scales [N][K/64] bf16 bits, biases [N][K/64] bf16 bits).

    Other code widths (2 or 8 bits, 32/bits codes per word): the same recipe with
    the scale magnitude multiplied by 16 / 2^bits and the bias centred at
    -2^(bits-1) * scale, so the dequantized weights span the 4-bit workload's range.
    """
    if K % 64:
        raise ValueError("K must be a multiple of 64")
    if bits not in (2, 4, 8):
        raise ValueError("bits must be 2, 4 or 8")
    G = K // 64
    codes = rng(workload, matrix, T_CODES, layer).integers(
        0, 1 << 32, size=(N, K * bits // 32), dtype=np.uint32, endpoint=False)
    mag = rng(workload, matrix, T_SCALE_MAG, layer).random((N, G), dtype=np.float32)
    mag = np.float32(0.002) + np.float32(0.018) * mag
    if bits != 4:
        mag = (mag * np.float32(16.0 / (1 << bits))).astype(np.float32)
    sign = rng(workload, matrix, T_SCALE_SIGN, layer).integers(0, 2, size=(N, G), dtype=np.int8)
    s = np.where(sign == 1, mag, -mag).astype(np.float32)
    scales = f32_to_bf16_bits(s)
    eps = rng(workload, matrix, T_BIAS_EPS, layer).normal(0.0, 1e-3, size=(N, G)).astype(np.float32)
    b = (np.float32(-(1 << (bits - 1))) * bf16_bits_to_f32(scales) + eps).astype(np.float32)
    biases = f32_to_bf16_bits(b)
    return codes, scales, biases


def activations(M, K, workload=0, matrix=GENERIC, layer=0):
    """x [M][K] bf16 bits drawn N(0, 1)."""
    x = rng(workload, matrix, T_ACT, layer).standard_normal((M, K), dtype=np.float32)
    return f32_to_bf16_bits(x)


def logits(rows, V, workload=3, sigma=3.0):
    """[rows][V] fp32 logits drawn N(0, sigma)."""
    return (rng(workload, LM_HEAD, T_LOGITS).standard_normal((rows, V), dtype=np.float32)
            * np.float32(sigma)).astype(np.float32)


def planted_logits(V, workload=3, block=1024):
    """Eight fp32 rows of N(0, 3) logits with one planted case each.

    Returns (logits [8][V], notes) where notes[r] names the case; the expected
    id of each row is whatever the oracle says, the cases only make sure the
    edges are exercised.
    """
    if V < 2 * block + 8:
        raise ValueError("V too small for the planted cases")
    x = logits(8, V, workload)
    g = rng(workload, LM_HEAD, T_LOGITS, layer=1)
    notes = []
    # 0: plain row
    notes.append("plain")
    # 1: the maximum duplicated across a block boundary (ids block-1 and block)
    m = x[1].max() + 1.0
    x[1, block - 1] = m
    x[1, block] = m
    notes.append(f"tie across the block boundary at {block - 1}/{block}")
    # 2: a single NaN at a random id
    x[2, int(g.integers(0, V))] = np.nan
    notes.append("one NaN")
    # 3: +Inf
    x[3, int(g.integers(0, V))] = np.inf
    notes.append("+Inf")
    # 4: -Inf
    x[4, int(g.integers(0, V))] = -np.inf
    notes.append("-Inf")
    # 5: a three-way tie, the last copy in the tail block
    m = x[5].max() + 2.0
    tail0 = (V // block) * block if V % block else V - block
    for i in (int(g.integers(0, tail0)), int(g.integers(0, tail0)), V - 1):
        x[5, i] = m
    notes.append("three-way tie, one copy at V-1")
    # 6: every value negative except a -0.0 / +0.0 tie
    x[6] = -np.abs(x[6]) - 1.0
    i0, i1 = sorted(int(v) for v in g.choice(V, size=2, replace=False))
    x[6, i0] = np.float32(-0.0)
    x[6, i1] = np.float32(0.0)
    notes.append(f"-0.0 at {i0} ties +0.0 at {i1}")
    # 7: every value negative except two adjacent positive denormals
    x[7] = -np.abs(x[7]) - 1.0
    j = int(g.integers(0, V - 1))
    x[7, j] = np.array([1], np.uint32).view(np.float32)[0]
    x[7, j + 1] = np.array([2], np.uint32).view(np.float32)[0]
    notes.append(f"denormals 1 and 2 ulp at {j}/{j + 1}")
    return x, notes
