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
    Nd, Kd = 1000, 17408  # down-shaped: the step-staged kernels at B = 1 and 8
    wq, sc, bi = synth.weights(N, K, workload=70)
    hq, hs, hb = synth.weights(V, K, workload=71)
    dq, ds, db = synth.weights(Nd, Kd, workload=74)
    V8 = 20000  # the fused head at 8 bits (short workgroups, then the combine)
    eq, es, eb = synth.weights(V8, K, workload=78, bits=8)
    W = (up_u32(wq), up_bf16(sc), up_bf16(bi))
    H = (up_u32(hq), up_bf16(hs), up_bf16(hb))
    D = (up_u32(dq), up_bf16(ds), up_bf16(db))
    E = (up_u32(eq), up_bf16(es), up_bf16(eb))
    x1 = up_bf16(synth.activations(1, K, workload=70))
    x8 = up_bf16(synth.activations(8, K, workload=72))
    xm = up_bf16(synth.activations(96, K, workload=73))
    xs = up_bf16(synth.activations(16, K, workload=75))  # the short-prompt GEMM kernel
    xd1 = up_bf16(synth.activations(1, Kd, workload=76))
    xd8 = up_bf16(synth.activations(8, Kd, workload=77))
    dev = x1.device
    y1 = torch.empty((1, N), dtype=torch.float32, device=dev)
    y8 = torch.empty((8, N), dtype=torch.float32, device=dev)
    ym = torch.empty((96, N), dtype=torch.float32, device=dev)
    ys = torch.empty((16, N), dtype=torch.float32, device=dev)
    yd1 = torch.empty((1, Nd), dtype=torch.float32, device=dev)
    yd8 = torch.empty((8, Nd), dtype=torch.float32, device=dev)
    lg = torch.empty((1, V), dtype=torch.float32, device=dev)
    ids = torch.empty(1, dtype=torch.int32, device=dev)
    wsg = torch.empty(w4g.workspace_bytes(w4g.OP_GEMM, 96, N, K), dtype=torch.uint8, device=dev)
    wss = torch.empty(w4g.workspace_bytes(w4g.OP_GEMM, 16, N, K), dtype=torch.uint8, device=dev)
    wsa = torch.empty(w4g.workspace_bytes(w4g.OP_ARGMAX, 1, V, 0), dtype=torch.uint8, device=dev)
    # the fused heads: 4-bit over the V rows at B = 8, 8-bit over V8 rows at B = 1
    lgf = torch.empty((8, V), dtype=torch.float32, device=dev)
    idsf = torch.empty(8, dtype=torch.int32, device=dev)
    wsf = torch.empty(w4g.workspace_bytes(w4g.OP_GEMV_ARGMAX, 8, V, K), dtype=torch.uint8, device=dev)
    lg8 = torch.empty((1, V8), dtype=torch.float32, device=dev)
    ids8 = torch.empty(1, dtype=torch.int32, device=dev)
    ws8 = torch.empty(w4g.workspace_bytes(w4g.OP_GEMV_BITS_ARGMAX, 1, V8, K), dtype=torch.uint8, device=dev)
    outs = (y1, y8, ym, ys, yd1, yd8, lg, lgf, lg8)
    names = ("gemv b1", "gemv b8", "gemm", "gemm 16 rows", "down b1", "down b8", "lm_head", "fused head b8",
             "w8 fused head")

    def work():
        w4g.qmm_gemv(*W, x1, y1)
        w4g.qmm_gemv(*W, x8, y8)
        w4g.qmm_gemm(*W, xm, ym, wsg)
        w4g.qmm_gemm(*W, xs, ys, wss)
        w4g.qmm_gemv(*D, xd1, yd1)
        w4g.qmm_gemv(*D, xd8, yd8)
        w4g.qmm_gemv(*H, x1, lg)
        w4g.vocab_argmax(lg, ids, wsa)
        w4g.qmm_gemv_argmax(*H, x8, logits=lgf, ids=idsf, workspace=wsf)
        w4g.qmm_gemv_argmax(*E, x1, logits=lg8, ids=ids8, workspace=ws8, bits=8)

    work()
    id_outs = (ids, idsf, ids8)
    ref = [down(t).copy() for t in outs] + [ids_down(t).copy() for t in id_outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for rep in range(4):
        for t in outs:
            t.fill_(float("nan"))
        for t in id_outs:
            t.fill_(-2)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [down(t) for t in outs] + [ids_down(t) for t in id_outs]
        for a, b, name in zip(got, ref, names + ("ids", "fused ids b8", "w8 fused ids")):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"replay {rep}: {name}"
        _ = torch.ones(1000, device=dev).sum().item()  # eager work between replays
