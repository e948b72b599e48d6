"""HIP-graph capture of the library's calls: replays must equal eager results.

The calls allocate nothing and issue no memsets, so they can be captured.  The
graph is replayed several times with the program's own eager work and
synchronizations in between, and every replay is checked bitwise against the
eager result."""
import numpy as np
import pytest

from gpu_util import down, ids_down, up_bf16, up_u32
from w4_gemv_greedy_amd import synth

pytestmark = pytest.mark.gpu
w4g = pytest.importorskip("w4_gemv_greedy_amd")


def test_graph_replays_match_eager():
    torch = pytest.importorskip("torch")
    N, K, V = 2048, 5120, 70000
    wq, sc, bi = synth.weights(N, K, workload=70)
    hq, hs, hb = synth.weights(V, K, workload=71)
    W = (up_u32(wq), up_bf16(sc), up_bf16(bi))
    H = (up_u32(hq), up_bf16(hs), up_bf16(hb))
    x1 = up_bf16(synth.activations(1, K, workload=70))
    x8 = up_bf16(synth.activations(8, K, workload=72))
    xm = up_bf16(synth.activations(96, K, workload=73))
    dev = x1.device
    y1 = torch.empty((1, N), dtype=torch.float32, device=dev)
    y8 = torch.empty((8, N), dtype=torch.float32, device=dev)
    ym = torch.empty((96, N), dtype=torch.float32, device=dev)
    lg = torch.empty((1, V), dtype=torch.float32, device=dev)
    ids = torch.empty(1, dtype=torch.int32, device=dev)
    wsg = torch.empty(w4g.workspace_bytes(w4g.OP_GEMM, 96, N, K), dtype=torch.uint8, device=dev)
    wsa = torch.empty(w4g.workspace_bytes(w4g.OP_ARGMAX, 1, V, 0), dtype=torch.uint8, device=dev)

    def work():
        w4g.qmm_gemv(*W, x1, y1)
        w4g.qmm_gemv(*W, x8, y8)
        w4g.qmm_gemm(*W, xm, ym, wsg)
        w4g.qmm_gemv(*H, x1, lg)
        w4g.vocab_argmax(lg, ids, wsa)

    work()
    ref = [down(t).copy() for t in (y1, y8, ym, lg)] + [ids_down(ids).copy()]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for rep in range(4):
        for t in (y1, y8, ym, lg):
            t.fill_(float("nan"))
        ids.fill_(-2)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [down(t) for t in (y1, y8, ym, lg)] + [ids_down(ids)]
        for a, b, name in zip(got, ref, ("gemv b1", "gemv b8", "gemm", "lm_head", "ids")):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"replay {rep}: {name}"
        _ = torch.ones(1000, device=dev).sum().item()  # eager work between replays
