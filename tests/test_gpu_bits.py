"""GPU parity of the other code widths (2- and 8-bit affine group-64 codes,
qmm_gemv_bits) against the CPU oracle: small ragged shapes over every batch
size that fits, batch invariance and run-to-run bits, the one-workgroup-per-CU
layout, and the full-size 8-bit LM head with its greedy argmax."""
import numpy as np
import pytest

import oracle
from gpu_util import assert_close, down, ids_down, up_bf16, up_u32
from w4_gemv_greedy_amd import synth

pytestmark = pytest.mark.gpu
w4g = pytest.importorskip("w4_gemv_greedy_amd")


def _case(N, K, rows, bits, seed):
    wq, sc, bi = synth.weights(N, K, workload=70 + seed, bits=bits)
    x = synth.activations(rows, K, workload=70 + seed)
    return wq, sc, bi, x


SHAPES = [(37, 64), (70, 1088), (129, 2048), (300, 5120), (40, 17408), (9477, 1024)]


@pytest.mark.parametrize("bits", [2, 8])
@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("B", [1, 2, 3, 4, 5, 8])
def test_gemv_bits_matches_oracle(N, K, B, bits):
    # (at K = 17,408 from B = 5 the batch runs in two parts whose x fits in LDS)
    if N * K > 2_000_000 and B > 2:
        pytest.skip("large shape: B = 1 and 2 only")
    wq, sc, bi, x = _case(N, K, B, bits, N + K + B)
    y = down(w4g.qmm_gemv(up_u32(wq), up_bf16(sc), up_bf16(bi), up_bf16(x), bits=bits))
    e = assert_close(y, oracle.qmm(wq, sc, bi, x, bits=bits), f"gemv w{bits} N={N} K={K} B={B}")
    print(f"w{bits} N={N} K={K} B={B}: normwise {e:.2e}")


@pytest.mark.parametrize("K", [5120, 17408])
@pytest.mark.parametrize("bits", [2, 8])
def test_gemv_bits_batch_invariance_and_determinism(bits, K):
    wq, sc, bi, x = _case(300, K, 8, bits, 5)
    W = (up_u32(wq), up_bf16(sc), up_bf16(bi))
    y8 = down(w4g.qmm_gemv(*W, up_bf16(x), bits=bits))
    y8b = down(w4g.qmm_gemv(*W, up_bf16(x), bits=bits))
    assert np.array_equal(y8.view(np.uint32), y8b.view(np.uint32))
    for m in (0, 5):
        y1 = down(w4g.qmm_gemv(*W, up_bf16(x[m:m + 1]), bits=bits))
        assert np.array_equal(y1[0].view(np.uint32), y8[m].view(np.uint32)), f"w{bits} row {m}"


def test_gemv_bits4_is_qmm_gemv():
    wq, sc, bi, x = _case(200, 2048, 3, 4, 9)
    W = (up_u32(wq), up_bf16(sc), up_bf16(bi), up_bf16(x))
    a = down(w4g.qmm_gemv(*W))
    b = down(w4g.qmm_gemv(*W, bits=4))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_w8_lm_head_full_size():
    """The 8-bit LM head at full size, B = 1: sampled rows against the oracle and
    the greedy argmax bit-exact on the GPU's logits."""
    N, K = synth.VOCAB, synth.HIDDEN
    wq, sc, bi = synth.weights(N, K, workload=6, matrix=synth.LM_HEAD, bits=8)
    x = synth.activations(1, K, workload=6, matrix=synth.LM_HEAD)
    W = (up_u32(wq), up_bf16(sc), up_bf16(bi))
    logits_t = w4g.qmm_gemv(*W, up_bf16(x), bits=8)
    logits = down(logits_t)
    r = np.random.default_rng(8)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(N - 64, N), r.choice(N, 256, replace=False)]))
    ref = oracle.qmm_rows(wq, sc, bi, x, rows, bits=8)
    e = assert_close(logits[:, rows], ref, "w8 lm_head")
    ids = ids_down(w4g.vocab_argmax(logits_t))
    assert ids[0] == oracle.argmax(logits)[0]
    print(f"w8 lm_head: normwise {e:.2e} over {rows.size} rows, id {ids[0]}")
