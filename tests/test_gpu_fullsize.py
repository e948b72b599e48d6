"""Parity at the full model shapes, in the configurations the benchmark runs.

The GPU computes every output; the oracle checks a sample of output rows it
can afford one by one (the first and last 64 rows and 256 seeded random ones),
against the same seeded inputs.  The argmax is bit-exact on the GPU's own
logits, and end to end the greedy id must match the oracle's unless the
oracle's top-two gap is within the products' error bound."""
import numpy as np
import pytest

import oracle
from gpu_util import assert_close, down, ids_down, up_bf16, up_u32
from w4_gemv_greedy_amd import synth

pytestmark = pytest.mark.gpu
w4g = pytest.importorskip("w4_gemv_greedy_amd")

SHAPES = {"o_proj": (5120, 5120, synth.O_PROJ), "gate_up": (34816, 5120, synth.GATE_UP),
          "down": (5120, 17408, synth.DOWN), "lm_head": (248320, 5120, synth.LM_HEAD)}
_cache = {}


def _weights(name):
    if name not in _cache:
        N, K, mid = SHAPES[name]
        wq, sc, bi = synth.weights(N, K, workload=5, matrix=mid, layer=0)
        _cache.clear()  # keep one full matrix on the host and the GPU at a time
        _cache[name] = (wq, sc, bi, (up_u32(wq), up_bf16(sc), up_bf16(bi)))
    return _cache[name]


def _sample_rows(N, seed):
    r = np.random.default_rng(seed)
    rows = np.concatenate([np.arange(64), np.arange(N - 64, N), r.choice(N, 256, replace=False)])
    return np.unique(rows)


@pytest.mark.parametrize("family", ["valu", "mfma", "auto"])
@pytest.mark.parametrize("B", [1, 4, 8])
@pytest.mark.parametrize("name", list(SHAPES))
def test_gemv_full_shape(name, B, family):
    wq, sc, bi, W = _weights(name)
    N, K, mid = SHAPES[name]
    x = synth.activations(B, K, workload=5, matrix=mid, layer=B)
    kernel = {"valu": 1, "mfma": 2, "auto": 0}[family]
    y = down(w4g.qmm_gemv(*W, up_bf16(x), kernel=kernel))
    rows = _sample_rows(N, B)
    ref = oracle.qmm_rows(wq, sc, bi, x, rows)
    e = assert_close(y[:, rows], ref, f"{name} B={B} {family}")
    print(f"{name} B={B} {family}: normwise {e:.2e} over {rows.size} sampled rows")


@pytest.mark.parametrize("name", ["o_proj", "gate_up", "down"])
def test_gemm_prompt_full_shape(name):
    """M = 512 against the oracle on sampled columns; then the shorter prompts the
    benchmark times (128, 64, 16 rows: other tile variants) must reproduce the
    first rows bit for bit, and the bf16 store at 128 rows must be the
    nearest-even rounding of the fp32 result."""
    import torch
    wq, sc, bi, W = _weights(name)
    N, K, mid = SHAPES[name]
    M = 512
    x = synth.activations(M, K, workload=4, matrix=mid, layer=0)
    X = up_bf16(x)
    y = down(w4g.qmm_gemm(*W, X))
    cols = np.unique(np.concatenate([np.arange(32), np.arange(N - 32, N),
                                     np.random.default_rng(1).choice(N, 64, replace=False)]))
    ref = oracle.qmm_rows(wq, sc, bi, x, cols)
    e = assert_close(y[:, cols], ref, f"prompt {name}")
    print(f"prompt {name} M=512: normwise {e:.2e} over {cols.size} sampled columns x 512 rows")
    for m in (128, 64, 16):
        ym = down(w4g.qmm_gemm(*W, X[:m].contiguous()))
        assert np.array_equal(ym.view(np.uint32), y[:m].view(np.uint32)), f"prompt {name} M={m}"
    yb = w4g.qmm_gemm(*W, X[:128].contiguous(), out_dtype=torch.bfloat16)
    want = torch.from_numpy(y[:128]).to(torch.bfloat16)
    assert torch.equal(yb.cpu().view(torch.int16), want.view(torch.int16)), f"prompt {name} bf16 store"


def test_lm_head_argmax_end_to_end():
    wq, sc, bi, W = _weights("lm_head")
    N, K, mid = SHAPES["lm_head"]
    B = 4
    x = synth.activations(B, K, workload=3, matrix=mid, layer=0)
    logits = w4g.qmm_gemv(*W, up_bf16(x))
    ids = ids_down(w4g.vocab_argmax(logits))
    lg = down(logits)
    # bit-exact on identical logits
    assert np.array_equal(ids, oracle.argmax(lg))
    # end to end against the oracle's own logits
    ref = oracle.qmm(wq, sc, bi, x)
    assert_close(lg, ref, "lm_head logits")
    want = oracle.argmax(ref)
    for m in range(B):
        if ids[m] != want[m]:
            top2 = np.sort(ref[m])[-2:]
            bound = 2e-5 * np.max(np.abs(ref[m]))
            assert top2[1] - top2[0] <= 2 * bound, f"row {m}: id {ids[m]} vs {want[m]} beyond a tie"


@pytest.mark.parametrize("name", list(SHAPES))
def test_default_gemv_batch_invariant(name):
    """The library's own choice of kernel (qmm_gemv, qmm_gemv_argmax) depends on
    K and the matrix alone, never on the batch: row m of an 8-row call is bit
    for bit the row computed in a 1-, 3- or 5-row call, and the fused head's
    logits and ids agree at every batch size (a request served beside others
    gets the bits it gets alone)."""
    wq, sc, bi, W = _weights(name)
    N, K, mid = SHAPES[name]
    x = synth.activations(8, K, workload=5, matrix=mid, layer=11)
    X = up_bf16(x)
    y8 = down(w4g.qmm_gemv(*W, X))
    for Bn in (1, 3, 5):
        yb = down(w4g.qmm_gemv(*W, X[:Bn].contiguous()))
        assert np.array_equal(yb.view(np.uint32), y8[:Bn].view(np.uint32)), f"{name}: B={Bn} differs from B=8"
    y1 = down(w4g.qmm_gemv(*W, X[7:8].contiguous()))
    assert np.array_equal(y1[0].view(np.uint32), y8[7].view(np.uint32)), f"{name}: row 7 alone differs"
    rows = _sample_rows(N, 11)[:96]
    assert_close(y8[:, rows], oracle.qmm_rows(wq, sc, bi, x, rows), f"{name} B=8 default")
    if name == "lm_head":
        ids8, lg8 = w4g.qmm_gemv_argmax(*W, X)
        assert np.array_equal(down(lg8).view(np.uint32), y8.view(np.uint32))
        ids8 = ids_down(ids8)
        assert np.array_equal(ids8, oracle.argmax(y8))
        for Bn in (1, 3):
            ids_b, lg_b = w4g.qmm_gemv_argmax(*W, X[:Bn].contiguous())
            assert np.array_equal(down(lg_b).view(np.uint32), y8[:Bn].view(np.uint32))
            assert np.array_equal(ids_down(ids_b), ids8[:Bn])


@pytest.mark.parametrize("B", [1, 3, 8])
def test_default_gemv_row_slice_with_whole(B):
    """A call over a row slice that names its whole matrix (whole = 248,320)
    gives the whole head's rows bit for bit: an 8-way shard of the vocabulary
    (31,040 rows: another layout and rows per CU) and an unaligned slice."""
    wq, sc, bi, W = _weights("lm_head")
    N, K, mid = SHAPES["lm_head"]
    x = synth.activations(B, K, workload=5, matrix=mid, layer=20 + B)
    X = up_bf16(x)
    y = down(w4g.qmm_gemv(*W, X))
    for lo, hi in ((3 * 31040, 4 * 31040), (100003, 105123)):
        ys = down(w4g.qmm_gemv(W[0][lo:hi], W[1][lo:hi], W[2][lo:hi], X, whole=N))
        assert np.array_equal(ys.view(np.uint32), y[:, lo:hi].view(np.uint32)), f"rows [{lo}, {hi}) at B={B}"
