"""The decode product with the argmax's first pass fused into its epilogue
(qmm_gemv_argmax): the logits are bitwise those of qmm_gemv (the same kernel
family, vector-ALU or matrix-core, chosen by shape the same way), the
ids are bitwise those of the two-pass argmax over those logits and of the
oracle's argmax, at small ragged shapes, at the full lm_head shape, and on
planted rows (ties across workgroups, a tie to a lower id, non-finite rows)."""
import numpy as np
import pytest

import oracle
from gpu_util import assert_close, down, ids_down, up_bf16, up_u32
from w4_gemv_greedy_amd import synth

pytestmark = pytest.mark.gpu
w4g = pytest.importorskip("w4_gemv_greedy_amd")

BF16_INF = 0x7F80


def _case(N, K, B, seed):
    wq, sc, bi = synth.weights(N, K, workload=70 + seed)
    x = synth.activations(B, K, workload=70 + seed)
    return wq, sc, bi, x


def _run(wq, sc, bi, x, want_logits=True):
    W = (up_u32(wq), up_bf16(sc), up_bf16(bi))
    X = up_bf16(x)
    ids, logits = w4g.qmm_gemv_argmax(*W, X, want_logits=want_logits)
    ref_logits = w4g.qmm_gemv(*W, X)
    two_pass = w4g.vocab_argmax(ref_logits)
    out = (ids_down(ids), down(logits) if logits is not None else None, down(ref_logits),
           ids_down(two_pass))
    return out


@pytest.mark.parametrize("N,K", [(37, 64), (1000, 1024), (4099, 2048), (20000, 5120), (3000, 17408),
                                 (6001, 12288), (40000, 8192)])
@pytest.mark.parametrize("B", [1, 2, 3, 8])
def test_fused_matches_two_pass(N, K, B):
    """Fused logits bitwise those of qmm_gemv and ids those of the two-pass
    argmax, over every family and layout qmm_gemv picks for these shapes (at
    B = 8 with K = 17408 and 12288 the matrix cores stage x per step with one
    and two 16-row tiles per CU, the latter with a ragged last workgroup; at
    40000 x 8192 they hold x whole and fold each batch of results into the
    record as it is reduced)."""
    wq, sc, bi, x = _case(N, K, B, N % 97 + B)
    ids, logits, ref_logits, two_pass = _run(wq, sc, bi, x)
    assert np.array_equal(logits.view(np.uint32), ref_logits.view(np.uint32)), "logits differ"
    assert np.array_equal(ids, two_pass), (ids, two_pass)
    assert np.array_equal(ids, oracle.argmax(ref_logits)), "ids differ from the oracle's argmax"
    if K <= 2048:
        assert_close(logits, oracle.qmm(wq, sc, bi, x), f"fused logits N={N} K={K} B={B}")


def test_fused_without_logits():
    wq, sc, bi, x = _case(5000, 1024, 4, 3)
    ids, logits, _, two_pass = _run(wq, sc, bi, x, want_logits=False)
    assert logits is None
    assert np.array_equal(ids, two_pass)


def _copy_row(wq, sc, bi, src, dst):
    wq[dst], sc[dst], bi[dst] = wq[src], sc[src], bi[src]


@pytest.mark.parametrize("B,K,N", [(1, 1024, 9000), (3, 1024, 9000), (8, 10240, 9000), (4, 1024, 12000)])
def test_fused_planted_rows(B, K, N):
    """Equal rows give equal logits bit for bit (each row's arithmetic is its own),
    so copying a batch row's winner to a lower id must move the answer there, a
    copy to a higher id must not, and an infinite scale makes the row fail.
    (B = 8 at K = 10240 runs the matrix-core family with the activations staged
    in stages, B = 4 over 12000 rows its one-workgroup-per-CU kernel.)"""
    wq, sc, bi, x = _case(N, K, B, 11)
    ids0, _, ref0, _ = _run(wq, sc, bi, x)
    win = int(ids0[0])
    assert win < N
    # a copy of batch row 0's winner far away (another workgroup) at a higher id: no change
    hi = (win + 4500) % N if (win + 4500) % N > win else N - 1
    _copy_row(wq, sc, bi, win, hi)
    ids1, _, ref1, two1 = _run(wq, sc, bi, x)
    assert ref1[0, hi] == ref1[0, win]
    assert ids1[0] == win and np.array_equal(ids1, two1)
    # and at a lower id: the lower id wins
    lo = 0 if win > 0 else None
    if lo is not None:
        _copy_row(wq, sc, bi, win, lo)
        ids2, _, ref2, two2 = _run(wq, sc, bi, x)
        assert ids2[0] == lo and np.array_equal(ids2, two2)
    # an infinite scale in one row: every batch row fails
    sc[N // 3, 0] = BF16_INF
    ids3, logits3, _, two3 = _run(wq, sc, bi, x)
    assert not np.all(np.isfinite(logits3[:, N // 3]))
    assert np.all(ids3 == 0xFFFFFFFF) and np.array_equal(ids3, two3)


@pytest.mark.parametrize("B", [1, 8])
def test_fused_full_lm_head(B):
    N, K = synth.VOCAB, 5120
    wq, sc, bi = synth.weights(N, K, workload=5, matrix=synth.LM_HEAD, layer=0)
    x = synth.activations(B, K, workload=6, matrix=synth.LM_HEAD, layer=B)
    ids, logits, ref_logits, two_pass = _run(wq, sc, bi, x)
    assert np.array_equal(logits.view(np.uint32), ref_logits.view(np.uint32))
    assert np.array_equal(ids, two_pass)
    assert np.array_equal(ids, oracle.argmax(ref_logits))
    # the oracle's own logits at the winning ids and a sample
    rows = np.unique(np.concatenate([ids.astype(np.int64), np.arange(64), np.arange(N - 64, N)]))
    assert_close(logits[:, rows], oracle.qmm_rows(wq, sc, bi, x, rows), f"lm_head B={B}")
