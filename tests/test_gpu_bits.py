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


def _bits_head(wq, sc, bi, x, bits, want_logits=True):
    W = (up_u32(wq), up_bf16(sc), up_bf16(bi))
    X = up_bf16(x)
    ids, logits = w4g.qmm_gemv_argmax(*W, X, want_logits=want_logits, bits=bits)
    ref_logits = w4g.qmm_gemv(*W, X, bits=bits)
    two_pass = w4g.vocab_argmax(ref_logits)
    return (ids_down(ids), down(logits) if logits is not None else None, down(ref_logits),
            ids_down(two_pass))


# shapes over every layout the 2- and 8-bit products take: one workgroup per CU
# share (x whole in LDS), the step-staged kernel (at most 24 rows per CU from
# B = 3, and where x does not fit), the batch in parts (K = 40,960 holds one row
# of x in LDS over more than 24 rows per CU), and 32-row workgroups for the
# vocabulary-wide head at B = 1
@pytest.mark.parametrize("bits", [2, 8])
@pytest.mark.parametrize("N,K", [(37, 64), (1000, 1024), (5000, 5120), (3000, 17408), (6400, 40960),
                                 (140000, 1024)])
@pytest.mark.parametrize("B", [1, 3, 8])
def test_bits_fused_head_matches_two_pass(N, K, B, bits):
    """The fused head at 2 and 8 bits: logits bitwise those of qmm_gemv_bits,
    ids bitwise those of the two-pass argmax over them and of the oracle's
    argmax of them."""
    wq, sc, bi, x = _case(N, K, B, bits, N % 89 + B)
    ids, logits, ref_logits, two_pass = _bits_head(wq, sc, bi, x, bits)
    assert np.array_equal(logits.view(np.uint32), ref_logits.view(np.uint32)), "logits differ"
    assert np.array_equal(ids, two_pass), (ids, two_pass)
    assert np.array_equal(ids, oracle.argmax(ref_logits)), "ids differ from the oracle's argmax"
    if K <= 1024:
        assert_close(logits, oracle.qmm(wq, sc, bi, x, bits=bits), f"w{bits} head N={N} K={K} B={B}")


@pytest.mark.parametrize("bits", [2, 8])
def test_bits_fused_head_planted_rows(bits):
    """Non-finite and tied rows through the fused head: an activation row holding
    +Inf makes its logits non-finite and its id the sentinel; a row of x that is
    all zeros makes every logit of that row zero, a tie the lowest id wins."""
    N, K, B = 5000, 1024, 3
    wq, sc, bi, x = _case(N, K, B, bits, 17)
    x = x.copy()
    x[1, 100] = 0x7F80      # +Inf (bf16 bits)
    x[2, :] = 0              # all +0.0: every logit of row 2 is exactly zero
    ids, logits, ref_logits, two_pass = _bits_head(wq, sc, bi, x, bits)
    assert np.array_equal(logits.view(np.uint32), ref_logits.view(np.uint32))
    assert ids[1] == 0xFFFFFFFF and ids[2] == 0
    assert np.array_equal(ids, two_pass)
    assert np.array_equal(ids, oracle.argmax(ref_logits))


def test_w8_lm_head_fused_full_size():
    """The fused W8 LM head at full size, B = 1 and 8: logits bitwise those of
    qmm_gemv_bits, ids those of the two-pass argmax and the oracle's."""
    N, K = synth.VOCAB, synth.HIDDEN
    wq, sc, bi = synth.weights(N, K, workload=6, matrix=synth.LM_HEAD, bits=8)
    x = synth.activations(8, K, workload=6, matrix=synth.LM_HEAD)
    for B in (1, 8):
        ids, logits, ref_logits, two_pass = _bits_head(wq, sc, bi, x[:B], 8)
        assert np.array_equal(logits.view(np.uint32), ref_logits.view(np.uint32)), f"B={B}"
        assert np.array_equal(ids, two_pass), (B, ids, two_pass)
        assert np.array_equal(ids, oracle.argmax(ref_logits)), f"B={B}"
        ids_only, none, _, _ = _bits_head(wq, sc, bi, x[:B], 8, want_logits=False)
        assert none is None and np.array_equal(ids_only, ids)
        print(f"w8 fused head B={B}: ids {ids.tolist()}")
