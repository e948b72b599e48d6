"""The vector-ALU decode order, checked bit for bit against a model of it
(valu_order.py: the documented chunks, lane segments, pair order, fused
multiply-adds and lane tree, every step rounded once to fp32) on inputs where
each dot2 adds terms of one sign (codes 0..15 expand to 128 + q > 0, and the
activations are taken non-negative), so that the model of the dot2's rounding
holds.  Rows come from the per-CU kernel (B = 1 and, with the transposed lane
tree, B = 8) and from the step-staged kernel (x spanning nine chunks), and are
compared at B = 1 and B = 8."""
import numpy as np
import pytest

import valu_order
from gpu_util import down, up_bf16, up_u32
from w4_gemv_greedy_amd import synth

pytestmark = pytest.mark.gpu
w4g = pytest.importorskip("w4_gemv_greedy_amd")


def _positive(x, narrow):
    x = np.asarray(x, dtype=np.uint16) & np.uint16(0x7FFF)  # |x|
    if narrow:  # every activation in [1, 2): products within one binade of each other
        x = (x & np.uint16(0x007F)) | np.uint16(0x3F80)
    return x


@pytest.mark.parametrize("N,K,rows,narrow", [
    (24, 1024, [0, 7, 23], True),
    (24, 1024, [0, 7, 23], False),
    (6400, 2048, [0, 1, 24, 3333, 6399], False),   # 25 rows per CU: the per-CU kernel at B = 8 too
    (12, 9216, [0, 11], False),                     # nine chunks: the step-staged kernel
])
def test_valu_order_bitwise(N, K, rows, narrow):
    wq, sc, bi = synth.weights(N, K, workload=91)
    x = _positive(synth.activations(8, K, workload=91), narrow)
    W = (up_u32(wq), up_bf16(sc), up_bf16(bi))
    y8 = down(w4g.qmm_gemv(*W, up_bf16(x), kernel=w4g.GEMV_VALU)).view(np.uint32)
    y1 = down(w4g.qmm_gemv(*W, up_bf16(x[:1]), kernel=w4g.GEMV_VALU)).view(np.uint32)
    bad = []
    for n in rows:
        for b in (0, 5):
            want = valu_order.f32_bits(valu_order.row(wq[n], sc[n], bi[n], x[b]))
            got = int(y8[b, n])
            if got != want:
                bad.append((n, b, hex(got), hex(want)))
        if int(y1[0, n]) != int(y8[0, n]):
            bad.append((n, "B=1 vs B=8", hex(int(y1[0, n])), hex(int(y8[0, n]))))
    assert not bad, bad


def test_valu_order_signed_activations():
    """With signed activations a dot2 can cancel, where the instruction rounds
    more coarsely than the model; most rows still equal the model bit for bit
    and the others stay within fp32 accuracy of it (seeded, so deterministic:
    500 of 512 rows equal here)."""
    N, K = 64, 1024
    wq, sc, bi = synth.weights(N, K, workload=92)
    x = synth.activations(8, K, workload=92)
    y = down(w4g.qmm_gemv(up_u32(wq), up_bf16(sc), up_bf16(bi), up_bf16(x)))
    want = np.array([[float(valu_order.row(wq[n], sc[n], bi[n], x[b])) for n in range(N)] for b in range(8)],
                    dtype=np.float32)
    equal = int(np.sum(y.view(np.uint32) == want.view(np.uint32)))
    print(f"signed activations: {equal} of {y.size} rows equal the model bit for bit")
    assert equal >= 0.9 * y.size
    err = np.max(np.abs(y.astype(np.float64) - want), axis=1) / np.max(np.abs(want.astype(np.float64)), axis=1)
    assert np.all(err <= 2e-6), err


@pytest.mark.parametrize("bits", [2, 8])
@pytest.mark.parametrize("N,K,rows", [(24, 1024, [0, 7, 23]), (6400, 2048, [0, 3333, 6399]), (12, 9216, [0, 11])])
def test_valu_order_other_widths_bitwise(bits, N, K, rows):
    """The 2- and 8-bit orders (the same kernels with the lane's segment held in
    BITS-bit fields) against the model bit for bit, non-negative activations,
    B = 1 and 8."""
    wq, sc, bi = synth.weights(N, K, workload=93, bits=bits)
    x = _positive(synth.activations(8, K, workload=93), False)
    W = (up_u32(wq), up_bf16(sc), up_bf16(bi))
    y8 = down(w4g.qmm_gemv(*W, up_bf16(x), bits=bits)).view(np.uint32)
    y1 = down(w4g.qmm_gemv(*W, up_bf16(x[:1]), bits=bits)).view(np.uint32)
    bad = []
    for n in rows:
        for b in (0, 5):
            want = valu_order.f32_bits(valu_order.row(wq[n], sc[n], bi[n], x[b], bits=bits))
            if int(y8[b, n]) != want:
                bad.append((n, b, hex(int(y8[b, n])), hex(want)))
        if int(y1[0, n]) != int(y8[0, n]):
            bad.append((n, "B=1 vs B=8"))
    assert not bad, bad
