"""Top two per logit row on the GPU (vocab_argmax_top2) against the oracle,
bit for bit (ids and gaps), on identical logits: the planted full-vocabulary
rows (ties across the block boundary, NaN, +-Inf, signed zeros, denormals),
tie-heavy random rows, bf16, small and ragged vocabularies and pitched rows."""
import numpy as np
import pytest

import oracle
from gpu_util import down, ids_down, up_bf16, up_f32
from w4_gemv_greedy_amd import synth

pytestmark = pytest.mark.gpu
w4g = pytest.importorskip("w4_gemv_greedy_amd")


def _top2_gpu(x, bf16=False, vocab=None):
    t = up_bf16(x) if bf16 else up_f32(x)
    ids2, gaps = w4g.vocab_argmax_top2(t, vocab=vocab)
    return ids_down(ids2), down(gaps)


def _same(got, want):
    (gi, gg), (wi, wg) = got, want
    assert np.array_equal(gi, wi), (gi, wi)
    assert np.array_equal(gg.view(np.uint32), wg.view(np.uint32)) or (
        np.array_equal(np.isnan(gg), np.isnan(wg)) and
        np.array_equal(gg[~np.isnan(gg)].view(np.uint32), wg[~np.isnan(wg)].view(np.uint32))), (gg, wg)


def test_top2_planted_full_vocab():
    x, notes = synth.planted_logits(synth.VOCAB)
    got, want = _top2_gpu(x), oracle.argmax_top2(x)
    _same(got, want)
    assert np.array_equal(got[0][:, 0], oracle.argmax(x))   # the winner is the argmax
    xb = synth.f32_to_bf16_bits(x)
    xb[7] = synth.f32_to_bf16_bits(-np.abs(x[7]) - 1.0)
    xb[7, 100], xb[7, 101] = 0x0001, 0x0002                  # bf16 denormals on top
    _same(_top2_gpu(xb, bf16=True), oracle.argmax_top2(xb))


@pytest.mark.parametrize("V", [2, 3, 5, 1023, 1024, 1025, 3000, 4096])
def test_top2_small_vocab(V):
    r = np.random.default_rng(V + 7)
    x = np.round(r.standard_normal((7, V)) * 2).astype(np.float32)  # many exact ties
    x[1, V // 2] = np.nan
    x[2, :] = 0.0
    x[2, V - 1] = -0.0
    x[3, :] = -1.0
    x[3, V - 1] = 5.0                                               # winner at the last id
    x[4, ::2] = 9.0                                                 # a tie for first place
    x[5, 0] = -np.inf
    _same(_top2_gpu(x), oracle.argmax_top2(x))


def test_top2_random_rows_bitexact():
    r = np.random.default_rng(321)
    x = (r.standard_normal((48, 70000)) * 3).astype(np.float32)
    x[24:] = np.round(x[24:] * 2) / 2
    _same(_top2_gpu(x), oracle.argmax_top2(x))


def test_top2_pitched_rows():
    r = np.random.default_rng(5)
    full = r.standard_normal((3, 2200)).astype(np.float32)
    V = 2049
    full[:, V:] = 1e30  # padding beyond vocab must be ignored
    _same(_top2_gpu(full, vocab=V), oracle.argmax_top2(np.ascontiguousarray(full[:, :V])))
