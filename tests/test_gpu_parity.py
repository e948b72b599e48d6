"""GPU parity of the HIP library against the CPU oracle at sizes the oracle
finishes quickly, spanning several tiles and ragged tails.  Calls go through
the C ABI (ctypes) with device pointers and the current stream."""
import numpy as np
import pytest

import oracle
from gpu_util import (assert_close, down, ids_down, up_bf16, up_f32, up_u32)
from w4_gemv_greedy_amd import synth

pytestmark = pytest.mark.gpu

w4g = pytest.importorskip("w4_gemv_greedy_amd")


def _case(N, K, rows, seed):
    wq, sc, bi = synth.weights(N, K, workload=50 + seed)
    x = synth.activations(rows, K, workload=50 + seed)
    return wq, sc, bi, x


GEMV_SHAPES = [(37, 64), (64, 1088), (129, 2048), (200, 5120), (40, 17408), (9, 3072)]
FAMILIES = {"valu": 1, "mfma": 2, "auto": 0, "valu_regs": 3}


@pytest.mark.parametrize("family", ["valu", "mfma"])
@pytest.mark.parametrize("N,K", GEMV_SHAPES)
@pytest.mark.parametrize("B", [1, 2, 4, 8])
def test_gemv_matches_oracle(N, K, B, family):
    wq, sc, bi, x = _case(N, K, B, N + K)
    y = down(w4g.qmm_gemv(up_u32(wq), up_bf16(sc), up_bf16(bi), up_bf16(x), kernel=FAMILIES[family]))
    ref = oracle.qmm(wq, sc, bi, x)
    e = assert_close(y, ref, f"gemv[{family}] B={B} N={N} K={K}")
    print(f"gemv[{family}] B={B} N={N} K={K} normwise {e:.2e}")


@pytest.mark.parametrize("family", ["valu", "mfma", "auto"])
@pytest.mark.parametrize("B", [3, 5, 6, 7])
def test_gemv_odd_batches(B, family):
    wq, sc, bi, x = _case(70, 1024, B, 7)
    y = down(w4g.qmm_gemv(up_u32(wq), up_bf16(sc), up_bf16(bi), up_bf16(x), kernel=FAMILIES[family]))
    assert_close(y, oracle.qmm(wq, sc, bi, x), f"gemv[{family}] B={B}")


@pytest.mark.parametrize("K", [5120, 17408])
@pytest.mark.parametrize("family", ["valu", "mfma"])
def test_gemv_batch_invariance_and_determinism(family, K):
    # at K = 17408 the vector-ALU family stages x in registers for B >= 2 and in
    # LDS for B = 1: the two variants must give the same bits
    wq, sc, bi, x = _case(300, K, 8, 3)
    W = (up_u32(wq), up_bf16(sc), up_bf16(bi))
    k = FAMILIES[family]
    y8 = down(w4g.qmm_gemv(*W, up_bf16(x), kernel=k))
    y8b = down(w4g.qmm_gemv(*W, up_bf16(x), kernel=k))
    assert np.array_equal(y8.view(np.uint32), y8b.view(np.uint32)), "not run-to-run deterministic"
    for m in (0, 3, 7):
        y1 = down(w4g.qmm_gemv(*W, up_bf16(x[m:m + 1]), kernel=k))
        assert np.array_equal(y1[0].view(np.uint32), y8[m].view(np.uint32)), f"row {m} differs at B=1"
    for Bn in (2, 5):
        yb = down(w4g.qmm_gemv(*W, up_bf16(x[:Bn]), kernel=k))
        assert np.array_equal(yb.view(np.uint32), y8[:Bn].view(np.uint32)), f"B={Bn} differs"


@pytest.mark.parametrize("kernel", ["valu", "mfma", "mfma_step", "gemm"])
@pytest.mark.parametrize("B", [1, 5])
def test_power_of_two_scaling_bitwise(kernel, B):
    """Every step is linear in x and every rounding commutes with a power-of-two
    scale: x * 4 gives exactly 4 y in both decode families, the step-staged
    variant and the prompt product (a dropped term, a wrong scale factor or a
    non-linear shortcut shows here).  Negation is not checked: the hardware's
    fused bf16 dot products (v_dot2 and the matrix cores) measured not
    sign-symmetric bit for bit on some outputs."""
    import torch
    wq, sc, bi, x = _case(700, 3072, B, 41 + B)
    W = (up_u32(wq), up_bf16(sc), up_bf16(bi))
    X = up_bf16(x)
    if kernel == "gemm":
        run = lambda xx: down(w4g.qmm_gemm(*W, xx))  # noqa: E731
    else:
        k = {"valu": w4g.GEMV_VALU, "mfma": w4g.GEMV_MFMA, "mfma_step": w4g.GEMV_MFMA_STEP}[kernel]
        run = lambda xx: down(w4g.qmm_gemv(*W, xx, kernel=k))  # noqa: E731
    y = run(X)
    y4 = run((X.float() * 4).to(torch.bfloat16))
    assert np.array_equal(y4.view(np.uint32), (y * np.float32(4)).view(np.uint32))


_SLICE_CASES = {}


def _slice_case(N, K, rows):
    key = (N, K, rows)
    if key not in _SLICE_CASES:
        _SLICE_CASES.clear()
        wq, sc, bi, x = _case(N, K, rows, 61)
        _SLICE_CASES[key] = (wq, sc, bi, x, (up_u32(wq), up_bf16(sc), up_bf16(bi)))
    return _SLICE_CASES[key]


@pytest.mark.parametrize("family", ["valu", "mfma"])
@pytest.mark.parametrize("B", [1, 3, 8])
@pytest.mark.parametrize("N,K,lo,hi", [(248320, 5120, 100003, 105123),   # vocabulary head: layouts differ
                                       (34816, 5120, 17408, 34816),      # gate-up: the up half alone
                                       (5120, 17408, 1000, 1777),        # down: one tile per CU alone
                                       (40000, 8192, 777, 30777)])       # results not held in LDS
def test_gemv_row_slice_invariance(B, family, N, K, lo, hi):
    """A row's bits do not depend on N or on where the row sits: the rows
    [lo, hi) of a product equal, bit for bit, a product over those rows alone
    (a different grid, layout and tile position; the stacked gate-up's halves
    are the member matrices).  Within a family the K reduction is a function
    of K alone."""
    wq, sc, bi, x, W = _slice_case(N, K, 8)
    k = FAMILIES[family]
    X = up_bf16(x[:B])
    y = down(w4g.qmm_gemv(*W, X, kernel=k))
    ys = down(w4g.qmm_gemv(up_u32(wq[lo:hi]), up_bf16(sc[lo:hi]), up_bf16(bi[lo:hi]), X, kernel=k))
    assert np.array_equal(ys.view(np.uint32), y[:, lo:hi].view(np.uint32))
    rows = np.array([lo, (lo + hi) // 2, hi - 1])
    assert_close(y[:, rows], oracle.qmm_rows(wq, sc, bi, x[:B], rows), f"gemv[{family}] N={N} K={K} B={B}")


@pytest.mark.parametrize("M,N,K,lo,hi", [(200, 5120, 5120, 1000, 3000), (64, 34816, 5120, 17408, 34816),
                                         (33, 5120, 17408, 130, 4000)])
def test_gemm_column_slice_invariance(M, N, K, lo, hi):
    """The prompt product's columns [lo, hi) equal, bit for bit, a product over
    those weight rows alone (other tiles, grid and kernel choice)."""
    wq, sc, bi, x = _case(N, K, M, 5)
    X = up_bf16(x)
    y = down(w4g.qmm_gemm(up_u32(wq), up_bf16(sc), up_bf16(bi), X))
    ys = down(w4g.qmm_gemm(up_u32(wq[lo:hi]), up_bf16(sc[lo:hi]), up_bf16(bi[lo:hi]), X))
    assert np.array_equal(ys.view(np.uint32), y[:, lo:hi].view(np.uint32))


@pytest.mark.parametrize("family", ["valu", "mfma"])
def test_gemv_row_permutation_bitwise(family):
    wq, sc, bi, x = _case(96, 2048, 2, 4)
    p = np.random.default_rng(0).permutation(96)
    k = FAMILIES[family]
    y = down(w4g.qmm_gemv(up_u32(wq), up_bf16(sc), up_bf16(bi), up_bf16(x), kernel=k))
    yp = down(w4g.qmm_gemv(up_u32(wq[p]), up_bf16(sc[p]), up_bf16(bi[p]), up_bf16(x), kernel=k))
    assert np.array_equal(yp.view(np.uint32), y[:, p].view(np.uint32))


@pytest.mark.parametrize("B", [1, 2, 4])
@pytest.mark.parametrize("N,K", [(70, 1088), (300, 5120), (64, 17408)])
def test_gemv_valu_variants_bitwise(N, K, B):
    """The LDS-staged and register-staged vector-ALU variants give the same bits."""
    wq, sc, bi, x = _case(N, K, B, 31)
    W = (up_u32(wq), up_bf16(sc), up_bf16(bi), up_bf16(x))
    a = down(w4g.qmm_gemv(*W, kernel=1))
    b = down(w4g.qmm_gemv(*W, kernel=3))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("bits", [4, 2, 8])
@pytest.mark.parametrize("N,K", [(5120, 17408), (6001, 12352), (700, 9280)])
def test_gemv_valu_step_staged(N, K, bits):
    """Batches whose paired activations exceed LDS where a CU's share is at most
    24 rows (down_proj from B = 5) run the step-staged vector-ALU kernel, the
    activations staged a chunk at a time by waves of their own: every batch row
    bitwise equal to the same row alone (B = 1 keeps x whole in LDS), over full
    shares (20 and 24 rows per CU), a short share, a ragged last chunk (12352 =
    12 chunks + 64) and all three code widths; sampled rows close to the oracle;
    for 4-bit codes the fused argmax epilogue too (logits bitwise those of
    qmm_gemv, ids those of the two-pass argmax)."""
    wq, sc, bi = synth.weights(N, K, workload=90 + bits, bits=bits)
    x = synth.activations(8, K, workload=90 + bits)
    W = (up_u32(wq), up_bf16(sc), up_bf16(bi))
    y8 = down(w4g.qmm_gemv(*W, up_bf16(x), bits=bits))
    for B in (5, 6, 7):
        yb = down(w4g.qmm_gemv(*W, up_bf16(x[:B]), bits=bits))
        assert np.array_equal(yb.view(np.uint32), y8[:B].view(np.uint32)), f"B={B} differs from B=8"
    for m in range(8):
        y1 = down(w4g.qmm_gemv(*W, up_bf16(x[m:m + 1]), bits=bits))
        assert np.array_equal(y1[0].view(np.uint32), y8[m].view(np.uint32)), f"row {m} differs at B=1"
    rng = np.random.default_rng(N + K + bits)
    rows = np.unique(np.r_[0:24, N - 24:N, rng.choice(N, 40, replace=False)])
    ref = oracle.qmm(wq[rows], sc[rows], bi[rows], x, bits=bits)
    assert_close(y8[:, rows], ref, f"step-staged w{bits} N={N} K={K}")
    if bits == 4:
        ids, logits = w4g.qmm_gemv_argmax(*W, up_bf16(x))
        assert np.array_equal(down(logits).view(np.uint32), y8.view(np.uint32)), "fused logits differ"
        two_pass = ids_down(w4g.vocab_argmax(up_f32(y8)))
        assert np.array_equal(ids_down(ids), two_pass)
        assert np.array_equal(ids_down(ids), oracle.argmax(y8))


@pytest.mark.parametrize("B", [2, 5, 8])
def test_gemv_wide_share_layout(B):
    """More than 512 rows per CU (the vocabulary-wide head's layout at B >= 2:
    four rows per half wave) over a ragged share and a ragged last chunk: every
    batch row bitwise equal to the row alone, sampled rows against the oracle,
    and the fused argmax epilogue equal to the two-pass argmax."""
    N, K = 140001, 1088
    wq, sc, bi, x = _case(N, K, B, 60 + B)
    W = (up_u32(wq), up_bf16(sc), up_bf16(bi))
    y = down(w4g.qmm_gemv(*W, up_bf16(x)))
    for m in (0, B - 1):
        y1 = down(w4g.qmm_gemv(*W, up_bf16(x[m:m + 1])))
        assert np.array_equal(y1[0].view(np.uint32), y[m].view(np.uint32)), f"row {m} differs at B=1"
    rows = np.unique(np.r_[0:600, N - 600:N, np.random.default_rng(B).choice(N, 200, replace=False)])
    assert_close(y[:, rows], oracle.qmm(wq[rows], sc[rows], bi[rows], x), f"wide share B={B}")
    ids, logits = w4g.qmm_gemv_argmax(*W, up_bf16(x))
    assert np.array_equal(down(logits).view(np.uint32), y.view(np.uint32))
    assert np.array_equal(ids_down(ids), ids_down(w4g.vocab_argmax(up_f32(y))))
    assert np.array_equal(ids_down(ids), oracle.argmax(y))


@pytest.mark.parametrize("N,K", [(9477, 1024), (8193, 3072), (5120, 2048), (300, 17408)])
def test_gemv_per_cu_layout(N, K):
    """B = 1 with one workgroup per CU (an equal share of rows each, half waves
    striding through it; ragged shares and a last workgroup with an odd row
    count; at 300 x 17408 the step-staged kernel, x staged a chunk at a time)
    against the oracle, and bitwise equal to the same rows computed by the
    layout of B = 2 and by the register-staged variant."""
    wq, sc, bi, x = _case(N, K, 2, N % 97)
    W = (up_u32(wq), up_bf16(sc), up_bf16(bi))
    y1 = down(w4g.qmm_gemv(*W, up_bf16(x[:1]), kernel=1))
    y2 = down(w4g.qmm_gemv(*W, up_bf16(x), kernel=1))
    yr = down(w4g.qmm_gemv(*W, up_bf16(x[:1]), kernel=3))
    assert np.array_equal(y1[0].view(np.uint32), y2[0].view(np.uint32))
    assert np.array_equal(y1.view(np.uint32), yr.view(np.uint32))
    assert_close(y1, oracle.qmm(wq, sc, bi, x[:1]), f"gemv per-CU N={N} K={K}")


def test_gemv_short_layout_ragged():
    """B = 1 over more than 511 rows per CU takes the short workgroups (32 rows
    each, two groups of two rows per half wave): a row count that leaves the
    last workgroup ragged (29 rows) and a ragged last chunk of K, on sampled
    rows against the oracle, bitwise equal to the per-CU layout of B = 2 and
    to the fused head's logits, whose id matches the two-pass argmax."""
    N, K = 131101, 1088
    wq, sc, bi, x = _case(N, K, 2, 3)
    W = (up_u32(wq), up_bf16(sc), up_bf16(bi))
    y1 = down(w4g.qmm_gemv(*W, up_bf16(x[:1])))
    y2 = down(w4g.qmm_gemv(*W, up_bf16(x)))
    assert np.array_equal(y1[0].view(np.uint32), y2[0].view(np.uint32))
    ids, lg = w4g.qmm_gemv_argmax(*W, up_bf16(x[:1]))
    assert np.array_equal(down(lg).view(np.uint32), y1.view(np.uint32))
    assert ids_down(ids)[0] == oracle.argmax(y1)[0]
    rows = np.unique(np.concatenate([np.arange(40), np.arange(N - 70, N),
                                     np.random.default_rng(4).choice(N, 200, replace=False)]))
    assert_close(y1[:, rows], oracle.qmm_rows(wq, sc, bi, x[:1], rows), f"gemv short N={N} K={K}")


@pytest.mark.parametrize("N,K", [(300, 73728), (6999, 12288), (33, 9920), (9000, 10240)])
@pytest.mark.parametrize("B", [1, 3, 8])
def test_gemv_mfma_large_k(N, K, B):
    """K too large for eight rows of activations in the per-CU kernel's LDS: the
    step-staged kernel takes a CU's 16-row tiles one or two at a time (N = 300:
    one tile; 6999: two, the last workgroup ragged; K = 9920: an odd group
    count; N = 9000: three tiles, a pair and then a single); against the oracle.
    The fused head over the same shape is checked against the plain product of
    the family the automatic choice takes (the matrix cores or the vector
    path, depending on the shape)."""
    if N * K * B > 250_000_000 and B != 3:
        pytest.skip("large shape: B = 3 only")
    wq, sc, bi, x = _case(N, K, B, 21)
    W = (up_u32(wq), up_bf16(sc), up_bf16(bi))
    y = down(w4g.qmm_gemv(*W, up_bf16(x), kernel=2))
    y_ref = oracle.qmm(wq, sc, bi, x)
    assert_close(y, y_ref, f"gemv[mfma] N={N} K={K} B={B}")
    ya = down(w4g.qmm_gemv(*W, up_bf16(x)))
    assert_close(ya, y_ref, f"gemv[auto] N={N} K={K} B={B}")
    ids, lg = w4g.qmm_gemv_argmax(*W, up_bf16(x))
    assert np.array_equal(down(lg).view(np.uint32), ya.view(np.uint32))
    assert np.array_equal(ids_down(ids), oracle.argmax(ya))


@pytest.mark.parametrize("B,N,K", [(8, 5120, 5120), (3, 300, 1024), (1, 33, 128), (5, 1000, 8256),
                                   (8, 6001, 4096), (2, 70000, 2048), (4, 37, 8320), (8, 40000, 8192),
                                   (8, 40000, 8064)])
def test_gemv_mfma_step_variant_bitwise(B, N, K):
    """The step-staged per-CU matrix-core kernel, forced where the whole-x one
    runs, gives the same bits: one order whichever of the two K selects (an odd
    group count, a ragged last workgroup, several tile pairs per CU; at
    40000 x 8192 the whole-x kernel's results do not fit in its LDS beside the
    activations and are stored batch by batch; at 40000 x 8064 in batches of
    five tiles, so the whole-x kernel's two sets of waves, on alternate tiles,
    meet batches that start on either set)."""
    wq, sc, bi, x = _case(N, K, B, 31 + B)
    W = (up_u32(wq), up_bf16(sc), up_bf16(bi), up_bf16(x))
    a = down(w4g.qmm_gemv(*W, kernel=w4g.GEMV_MFMA))
    b = down(w4g.qmm_gemv(*W, kernel=w4g.GEMV_MFMA_STEP))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    rows = np.unique(np.concatenate([np.arange(min(N, 20)), np.arange(max(0, N - 20), N)]))
    assert_close(a[:, rows], oracle.qmm_rows(wq, sc, bi, x, rows), f"gemv[mfma] N={N} K={K} B={B}")


def test_gemv_families_agree():
    wq, sc, bi, x = _case(256, 5120, 4, 12)
    W = (up_u32(wq), up_bf16(sc), up_bf16(bi), up_bf16(x))
    a = down(w4g.qmm_gemv(*W, kernel=1))
    b = down(w4g.qmm_gemv(*W, kernel=2))
    assert_close(a, b, "valu vs mfma")


GEMM_SHAPES = [(1, 37, 64), (7, 130, 1088), (130, 256, 1024), (64, 128, 5120), (33, 70, 17408)]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_matches_oracle(M, N, K):
    wq, sc, bi, x = _case(N, K, M, M + N + K)
    y = down(w4g.qmm_gemm(up_u32(wq), up_bf16(sc), up_bf16(bi), up_bf16(x)))
    ref = oracle.qmm(wq, sc, bi, x)
    e = assert_close(y, ref, f"gemm M={M} N={N} K={K}")
    print(f"gemm M={M} N={N} K={K} normwise {e:.2e}")


def test_gemm_deterministic_and_row_independent():
    wq, sc, bi, x = _case(256, 2048, 160, 9)
    W = (up_u32(wq), up_bf16(sc), up_bf16(bi))
    y = down(w4g.qmm_gemm(*W, up_bf16(x)))
    y2 = down(w4g.qmm_gemm(*W, up_bf16(x)))
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
    ys = down(w4g.qmm_gemm(*W, up_bf16(x[:5])))
    assert np.array_equal(ys.view(np.uint32), y[:5].view(np.uint32)), "prompt rows depend on M"


def _offset_copy(t):
    """The same bf16 table starting 2 bytes past a 4-byte boundary."""
    import torch
    flat = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
    flat[1:] = t.reshape(-1)
    return flat[1:].view(t.shape)


@pytest.mark.parametrize("M,N,K", [(130, 256, 1024), (64, 200, 5120)])
def test_gemm_kernels_agree_bitwise(M, N, K):
    """Even G with 4-byte aligned scales takes the LDS-load kernel; a scale table
    2 bytes off alignment takes the register-staged one.  Same order, same bits."""
    wq, sc, bi, x = _case(N, K, M, 3 * M + N)
    X = up_bf16(x)
    W = up_u32(wq)
    S, Bi = up_bf16(sc), up_bf16(bi)
    y_lds = down(w4g.qmm_gemm(W, S, Bi, X))
    S2, B2 = _offset_copy(S), _offset_copy(Bi)
    assert S2.data_ptr() % 4 == 2
    y_reg = down(w4g.qmm_gemm(W, S2, B2, X))
    assert np.array_equal(y_lds.view(np.uint32), y_reg.view(np.uint32))
    assert_close(y_lds, oracle.qmm(wq, sc, bi, x), f"gemm M={M} N={N} K={K}")


def test_gemm_tile_variants_bitwise():
    """The main loops (register-staged 128 x 128 tiles from 512 tiles up,
    LDS-load 128 x 128 from 256, LDS-load 64 x 128 from 128, LDS-load 64 x 64
    below) follow one order: the rows they share are bitwise equal, and sampled
    columns match the oracle."""
    N, K = 8155, 256                      # 64 column tiles of 128, the last ragged
    wq, sc, bi, x = _case(N, K, 1000, 77)
    W = (up_u32(wq), up_bf16(sc), up_bf16(bi))
    X = up_bf16(x)
    y_reg = down(w4g.qmm_gemm(*W, X))                         # 8 x 64 = 512 tiles
    y_lds = down(w4g.qmm_gemm(*W, X[:500].contiguous()))      # 4 x 64 = 256 tiles
    y_half = down(w4g.qmm_gemm(*W, X[:300].contiguous()))     # 3 x 64 = 192: 64 x 128 tiles
    y_small = down(w4g.qmm_gemm(*W, X[:100].contiguous()))    # 64 x 64 tiles
    assert np.array_equal(y_lds.view(np.uint32), y_reg[:500].view(np.uint32))
    assert np.array_equal(y_half.view(np.uint32), y_reg[:300].view(np.uint32))
    assert np.array_equal(y_small.view(np.uint32), y_reg[:100].view(np.uint32))
    cols = np.unique(np.concatenate([np.arange(40), np.arange(N - 40, N),
                                     np.random.default_rng(5).choice(N, 60, replace=False)]))
    assert_close(y_reg[:, cols], oracle.qmm_rows(wq, sc, bi, x, cols), "gemm tile variants")


def test_gemm_small_grid_variants_bitwise():
    """Small grids over a wide matrix: past 32 rows, where 64 x 64 tiles would
    outnumber the CUs, 64 x 128 tiles run (100 rows: 2 x 129); at 20 rows the
    64 x 64 tiles stay (257 of them, a column tile too many for the short-prompt
    kernel).  Their rows are bitwise the rows of a 600-row prompt (register-
    staged 128 x 128 tiles) and sampled columns match the oracle."""
    N, K = 16390, 256                     # 129 column tiles of 128, the last ragged
    wq, sc, bi, x = _case(N, K, 600, 91)
    W = (up_u32(wq), up_bf16(sc), up_bf16(bi))
    X = up_bf16(x)
    y_reg = down(w4g.qmm_gemm(*W, X))                         # 5 x 129 = 645 tiles
    y_mid = down(w4g.qmm_gemm(*W, X[:100].contiguous()))      # 64 x 128 tiles
    y_few = down(w4g.qmm_gemm(*W, X[:20].contiguous()))       # 64 x 64 tiles
    assert np.array_equal(y_mid.view(np.uint32), y_reg[:100].view(np.uint32))
    assert np.array_equal(y_few.view(np.uint32), y_reg[:20].view(np.uint32))
    cols = np.unique(np.concatenate([np.arange(40), np.arange(N - 40, N),
                                     np.random.default_rng(6).choice(N, 60, replace=False)]))
    assert_close(y_mid[:, cols], oracle.qmm_rows(wq, sc, bi, x[:100], cols), "gemm small grid")


@pytest.mark.parametrize("N,K", [(70, 128), (1000, 384), (333, 1152), (5120, 5120)])
def test_gemm_short_prompt_kernel(N, K):
    """Prompts of at most 32 rows over a narrow matrix take the short-prompt
    kernel (groups dealt to eight waves; 16-row tiles up to 16 rows, 32-row
    tiles up to 32; G = 2, 6, 18, 80 cover one partial round, a ragged last
    round and whole rounds).  Their rows must be bitwise the rows of a 40-row
    prompt, which the tiled loops compute, and match the oracle."""
    wq, sc, bi, x = _case(N, K, 40, N + 7 * K)
    W = (up_u32(wq), up_bf16(sc), up_bf16(bi))
    X = up_bf16(x)
    y40 = down(w4g.qmm_gemm(*W, X))
    for m in (1, 5, 16, 17, 32):
        ym = down(w4g.qmm_gemm(*W, X[:m].contiguous()))
        assert np.array_equal(ym.view(np.uint32), y40[:m].view(np.uint32)), f"M={m} N={N} K={K}"
    cols = np.unique(np.concatenate([np.arange(min(N, 40)), np.arange(max(0, N - 40), N),
                                     np.random.default_rng(3).choice(N, min(N, 64), replace=False)]))
    assert_close(y40[:, cols], oracle.qmm_rows(wq, sc, bi, x, cols), f"short prompt N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [(1, 37, 64), (7, 130, 1088), (130, 256, 1024), (33, 70, 17408),
                                   (500, 1100, 512), (16, 1000, 384), (32, 70, 1152)])
def test_gemm_bf16_store(M, N, K):
    """bf16 output: the fp32 result (itself held to the 2e-3 bar elsewhere) rounded
    to nearest-even, bit for bit as torch's CPU conversion of the fp32 output
    rounds it, and within one bf16 step of the oracle's rounded result away
    from zero.  The
    normwise error then stays below bf16's own unit roundoff 2^-8 plus the fp32
    error; 2^-8 exceeds 2e-3, so the fp32 bar cannot apply to a bf16 store."""
    import torch
    wq, sc, bi, x = _case(N, K, M, 5 * M + N)
    W = (up_u32(wq), up_bf16(sc), up_bf16(bi))
    X = up_bf16(x)
    y32 = down(w4g.qmm_gemm(*W, X))
    yb_t = w4g.qmm_gemm(*W, X, out_dtype=torch.bfloat16)
    assert yb_t.dtype == torch.bfloat16
    yb = down(yb_t.view(torch.int16)).view(np.uint16)
    want = torch.from_numpy(y32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(yb, want), "bf16 store is not the rounding of the fp32 result"
    ref = oracle.qmm(wq, sc, bi, x)
    rb = oracle.to_bf16(ref)
    # one bf16 step apart at most, away from zero (near zero the fp32 error of
    # the sum, not the store, sets the distance, and signs may differ)
    step = np.abs(yb.astype(np.int32) - rb.astype(np.int32))
    away = np.abs(ref) > 1e-3 * np.max(np.abs(ref), axis=1, keepdims=True)
    assert np.all(step[away] <= 1), int(np.max(step[away]))
    yf = (yb.astype(np.uint32) << 16).view(np.float32)
    bound = 2.0 ** -8 + 2e-5
    assert_close(yf, ref, f"gemm bf16 M={M} N={N} K={K}", tol=bound, tight=bound)


def test_gemm_bf16_store_nan():
    """A NaN activation makes its whole output row NaN in both stores."""
    import torch
    wq, sc, bi, x = _case(96, 1024, 6, 4)
    x = x.copy()
    x[2, 700] = 0x7FC0
    W = (up_u32(wq), up_bf16(sc), up_bf16(bi))
    y32 = down(w4g.qmm_gemm(*W, up_bf16(x)))
    yb = down(w4g.qmm_gemm(*W, up_bf16(x), out_dtype=torch.bfloat16).float())
    assert np.all(np.isnan(y32[2])) and np.all(np.isnan(yb[2]))
    assert np.all(np.isfinite(np.delete(y32, 2, axis=0))) and np.all(np.isfinite(np.delete(yb, 2, axis=0)))


def _argmax_gpu(logits_np, bf16=False):
    t = up_bf16(logits_np) if bf16 else up_f32(logits_np)
    return ids_down(w4g.vocab_argmax(t))


def test_argmax_planted_full_vocab():
    x, notes = synth.planted_logits(synth.VOCAB)
    got = _argmax_gpu(x)
    want = oracle.argmax(x)
    assert np.array_equal(got, want), list(zip(notes, got, want))
    assert want[2] == want[3] == want[4] == 0xFFFFFFFF
    xb = synth.f32_to_bf16_bits(x)
    xb[7] = synth.f32_to_bf16_bits(-np.abs(x[7]) - 1.0)
    xb[7, 100], xb[7, 101] = 0x0001, 0x0002  # bf16 denormals
    gotb = _argmax_gpu(xb, bf16=True)
    assert np.array_equal(gotb, oracle.argmax(xb))


@pytest.mark.parametrize("V", [1, 5, 1023, 1024, 1025, 3000, 4096])
def test_argmax_small_vocab(V):
    r = np.random.default_rng(V)
    x = np.round(r.standard_normal((6, V)) * 2).astype(np.float32)  # many exact ties
    x[1, V // 2] = np.nan
    x[2, :] = 0.0
    x[2, V - 1] = -0.0
    assert np.array_equal(_argmax_gpu(x), oracle.argmax(x))


def test_argmax_pitched_rows():
    torch = pytest.importorskip("torch")
    r = np.random.default_rng(1)
    full = r.standard_normal((3, 2100)).astype(np.float32)
    V = 2049
    full[:, V:] = 1e30  # padding beyond vocab must be ignored
    t = up_f32(full)
    got = ids_down(w4g.vocab_argmax(t, vocab=V))
    assert np.array_equal(got, oracle.argmax(np.ascontiguousarray(full[:, :V])))
    del torch


def test_argmax_random_rows_bitexact():
    r = np.random.default_rng(123)
    x = (r.standard_normal((64, 50000)) * 3).astype(np.float32)
    x[32:] = np.round(x[32:] * 2) / 2
    assert np.array_equal(_argmax_gpu(x), oracle.argmax(x))
