"""Benchmark: the synthetic decode sweep of the W4 g64 hot path on one MI355X.

One step = 16 layer-equivalents of (o_proj 5120x5120, fused gate-up
5120 -> 34816, down_proj 17408 -> 5120) W4 g64 products back to back on one
stream, then the 248,320-row lm_head product (logits written) and the greedy
argmax over the full vocabulary (qmm_gemv_argmax: the argmax's first pass in
the product's epilogue).  Every product takes its own pre-generated bf16 input (no
norm or activation between them; the inputs are seeded synthetic data of the
model's shapes, the weights seeded synthetic codes, scales and biases).  The
step is captured once in a HIP graph and replayed.

Printed: one JSON line.  `value` is the algorithmic bytes of a step
(0.5625*N*K + 2*B*K + 4*B*N per product, 4*B*V for the argmax) over the
measured step time, in GB/s.  The line also carries the roofline of the
dominant kernel (the gate-up product), the oracle timed on the host cores, and
secondary figures: lm_head+argmax microseconds per token, the prompt products
at 512, 128, 64 and 16 rows (fp32 and, at 128, bf16 store), the batch-8 sweep,
the sweep as eager launches, per-call eager percentiles of the batch-1
products, and the measured ceilings the products are read against (a
read-only HBM stream of each product's bytes, a matrix-core loop with no
memory traffic, and torch's bf16 matmul on dequantized weights).

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 50] [--batch 1]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 matrix cores, vendor figure
METRIC = "W4 g64 GEMV GB/s (% HBM peak); lm_head+argmax µs/token; prompt GEMM TFLOPS"

HIDDEN, INTER, VOCAB, LAYERS = 5120, 17408, 248320, 16


def gemv_bytes(N, K, B):
    return int(0.5625 * N * K) + 2 * B * K + 4 * B * N


def step_bytes(B):
    per_layer = (gemv_bytes(HIDDEN, HIDDEN, B) + gemv_bytes(2 * INTER, HIDDEN, B)
                 + gemv_bytes(HIDDEN, INTER, B))
    return LAYERS * per_layer + gemv_bytes(VOCAB, HIDDEN, B) + 4 * B * VOCAB


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--batch", type=int, default=1)
    p.add_argument("--no-graph", action="store_true", help="time eager launches instead of a graph")
    p.add_argument("--skip-extras", action="store_true",
                   help="only the headline sweep (used for profiler runs)")
    p.add_argument("--skip-cpu", action="store_true", help="skip the oracle CPU baseline")
    p.add_argument("--probe", choices=PROBES,
                   help="run only one kernel a few times (for hardware-counter runs) and exit")
    return p.parse_args()


PROFILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                       "gemv_gate_up_b1_hbm_counters.txt")
GEMV_SRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "w4_gemv_greedy_amd", "csrc",
                        "gemv.hip")


def counted_traffic():
    """HBM bytes per gate-up launch from the committed counter summary, or None
    when the kernel source changed since the counters were taken."""
    import hashlib
    try:
        text = open(PROFILE).read()
    except OSError:
        return None
    fields = dict(line.split(":", 1) for line in text.splitlines() if ":" in line and not line.startswith(" "))
    want = fields.get("source_sha256", "").strip()
    have = hashlib.sha256(open(GEMV_SRC, "rb").read()).hexdigest()
    if not want or want != have:
        return None
    try:
        return int(fields["traffic_bytes_per_launch"].strip())
    except (KeyError, ValueError):
        return None


PROBES = ["copy"] + [f"{p}_b{b}_{f}" for p in ("o_proj", "gate_up", "down", "lm_head")
                      for b in (1, 8) for f in ("auto", "mfma")] + \
         ["lm_head_argmax_b1", "gemm_o_proj", "gemm_gate_up", "gemm_down"]


def probe(kind):
    """A short, fixed workload for hardware-counter collection: a plain 1 GiB
    device copy (the calibration), one decode product (`<product>_b<B>_<family>`,
    four launches over distinct copies of the matrix, three rounds), the fused
    lm_head + argmax at B=1, or a 512-row prompt product (`gemm_<product>`)."""
    import torch
    import w4_gemv_greedy_amd as w4g
    from w4_gemv_greedy_amd import synth
    dev = torch.device("cuda:0")
    if kind == "copy":
        # plain device copy of 1 GiB: reads 1 GiB and writes 1 GiB
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        return
    shapes = {"o_proj": (HIDDEN, HIDDEN, synth.O_PROJ), "gate_up": (2 * INTER, HIDDEN, synth.GATE_UP),
              "down": (HIDDEN, INTER, synth.DOWN), "lm_head": (VOCAB, HIDDEN, synth.LM_HEAD)}
    if kind.startswith("gemm_"):
        N, K, mid = shapes[kind[5:]]
        mats = [Mat(N, K, 4, mid, l, dev) for l in range(2)]
        x = make_x(512, K, 4, mid, 0, dev)
        y = torch.empty((512, N), dtype=torch.float32, device=dev)
        ws = torch.empty(w4g.workspace_bytes(w4g.OP_GEMM, 512, N, K), dtype=torch.uint8, device=dev)
        for _ in range(3):
            for m in mats:
                w4g.qmm_gemm(m.wq, m.sc, m.bi, x, y, ws)
        torch.cuda.synchronize()
        return
    if kind == "lm_head_argmax_b1":
        N, K, mid = shapes["lm_head"]
        m = Mat(N, K, 5, mid, 0, dev)
        x = make_x(1, K, 5, mid, 0, dev)
        ids = torch.empty(1, dtype=torch.int32, device=dev)
        ws = torch.empty(w4g.workspace_bytes(w4g.OP_GEMV_ARGMAX, 1, N, K), dtype=torch.uint8, device=dev)
        for _ in range(6):
            w4g.qmm_gemv_argmax(m.wq, m.sc, m.bi, x, None, ids, ws, want_logits=False)
        torch.cuda.synchronize()
        return
    name, b, fam = kind.rsplit("_", 2)
    N, K, mid = shapes[name]
    B = int(b[1:])
    kernel = w4g.GEMV_AUTO if fam == "auto" else w4g.GEMV_MFMA
    mats = [Mat(N, K, 5, mid, l, dev) for l in range(1 if name == "lm_head" else 4)]
    x = make_x(B, K, 5, mid, 0, dev)
    y = torch.empty((B, N), dtype=torch.float32, device=dev)
    for _ in range(3):
        for m in mats:
            w4g.qmm_gemv(m.wq, m.sc, m.bi, x, y, kernel=kernel)
    torch.cuda.synchronize()


class Mat:
    """One quantized matrix resident on the GPU."""

    def __init__(self, N, K, workload, matrix, layer, dev, bits=4):
        from w4_gemv_greedy_amd import synth
        import torch
        wq, sc, bi = synth.weights(N, K, workload=workload, matrix=matrix, layer=layer, bits=bits)
        self.N, self.K, self.bits = N, K, bits
        self.wq = torch.from_numpy(wq.view(np.int32)).to(dev)
        self.sc = torch.from_numpy(sc.view(np.int16)).to(dev).view(torch.bfloat16)
        self.bi = torch.from_numpy(bi.view(np.int16)).to(dev).view(torch.bfloat16)


def make_x(M, K, workload, matrix, layer, dev):
    from w4_gemv_greedy_amd import synth
    import torch
    x = synth.activations(M, K, workload=workload, matrix=matrix, layer=layer)
    return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def host_info():
    """nproc and the CPU model of the host the oracle runs on."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpu_model": model}


def cpu_baseline(budget_s=8.0):
    """The oracle (plain C, OpenMP over output elements, fp64 sums) on the host cores.

    All cores: whole batch-1 products of one layer (o_proj, gate-up, down) and
    the lm_head plus the argmax, repeated until `budget_s` is spent; the rate is
    their algorithmic bytes over the oracle's time, and the decode step of 16
    layers plus the head follows from the per-call times (ms per token at B=1).
    One core: a seeded sample of output rows of the same products (1/32 of each
    matrix), scaled to whole calls.  Per config: ms per call at B = 1, 4, 8 and
    for the 512-row prompt, from a row (or column) sample at all cores, scaled.
    Every product's work is proportional to its output count, so a row sample
    scales exactly up to the sample's own timing noise.
    """
    import oracle
    from w4_gemv_greedy_amd import synth
    oracle.load()
    threads = oracle.threads()
    mats = {}
    for name, N, K, mid in (("o_proj", HIDDEN, HIDDEN, synth.O_PROJ),
                            ("gate_up", 2 * INTER, HIDDEN, synth.GATE_UP),
                            ("down", HIDDEN, INTER, synth.DOWN),
                            ("lm_head", VOCAB, HIDDEN, synth.LM_HEAD)):
        wq, sc, bi = synth.weights(N, K, workload=5, matrix=mid, layer=0)
        x = synth.activations(8, K, workload=5, matrix=mid, layer=0)
        mats[name] = (N, K, wq, sc, bi, x)

    # all cores, whole batch-1 calls
    done_bytes, spent, counts, per_call = 0, 0.0, {}, {}
    while spent < budget_s:
        for name, (N, K, wq, sc, bi, x) in mats.items():
            t0 = time.perf_counter()
            y = oracle.qmm(wq, sc, bi, x[:1], threads=threads)
            if name == "lm_head":
                oracle.argmax(y)
                done_bytes += 4 * VOCAB
            dt = time.perf_counter() - t0
            spent += dt
            per_call.setdefault(name, []).append(dt)
            done_bytes += gemv_bytes(N, K, 1)
            counts[name] = counts.get(name, 0) + 1
    ms = {k: 1e3 * float(np.median(v)) for k, v in per_call.items()}
    step_ms = LAYERS * (ms["o_proj"] + ms["gate_up"] + ms["down"]) + ms["lm_head"]

    def sampled(name, B, frac, thr, reps=1):
        N, K, wq, sc, bi, x = mats[name]
        rows = np.unique(np.random.default_rng(B).choice(N, max(8, int(N * frac)), replace=False))
        best = None
        for _ in range(reps):
            t0 = time.perf_counter()
            oracle.qmm_rows(wq, sc, bi, x[:B], rows, threads=thr)
            dt = time.perf_counter() - t0
            best = dt if best is None else min(best, dt)
        return 1e3 * best * N / rows.size

    # one core, a 1/32 row sample of each batch-1 product
    one = {name: sampled(name, 1, 1 / 32, 1) for name in mats}
    one_step_ms = LAYERS * (one["o_proj"] + one["gate_up"] + one["down"]) + one["lm_head"]
    # per config, all cores (row samples; the 512-row prompt on 64 output columns)
    cfg = {"1_o_proj_b1": round(ms["o_proj"], 3)}
    for name in ("gate_up", "down"):
        cfg[f"2_{name}_b1"] = round(ms[name], 3)
        for B in (4, 8):
            cfg[f"2_{name}_b{B}"] = round(sampled(name, B, 1 / 16, threads), 3)
    cfg["3_lm_head_argmax_b1"] = round(ms["lm_head"], 3)
    for name in ("o_proj", "gate_up", "down"):
        N, K, wq, sc, bi, _ = mats[name]
        xp = synth.activations(512, K, workload=4, matrix=synth.O_PROJ, layer=0)
        cols = np.arange(0, N, N // 64)[:64]
        t0 = time.perf_counter()
        oracle.qmm_rows(wq, sc, bi, xp, cols, threads=threads)
        cfg[f"4_prompt_m512_{name}"] = round(1e3 * (time.perf_counter() - t0) * N / cols.size, 1)
    cfg["5_decode_step_b1_ms_per_token"] = round(step_ms, 2)
    sample = ", ".join(f"{v} x {k}" for k, v in counts.items())
    return {"value": round(step_bytes(1) / (step_ms * 1e-3) / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"whole batch-1 products of one layer plus lm_head+argmax ({sample}, "
                      f"{done_bytes / 1e9:.2f} GB in {spent:.1f} s), the decode step's rate from their "
                      f"median per-call times (16 layers plus the head)",
            "host": dict(host_info(), oracle_threads=threads),
            "one_core": {"value": round(step_bytes(1) / (one_step_ms * 1e-3) / 1e9, 4), "unit": "GB/s",
                         "cores": 1, "ms_per_token_b1": round(one_step_ms, 1),
                         "ms_per_call_b1": {k: round(v, 2) for k, v in one.items()},
                         "sample": "1/32 of the output rows of each batch-1 product, scaled to whole calls"},
            "ms_per_call": cfg}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    if args.probe:
        probe(args.probe)
        return
    import torch
    import w4_gemv_greedy_amd as w4g
    from w4_gemv_greedy_amd import synth
    from w4_gemv_greedy_amd import _lib

    _lib.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B = args.batch
    if not 1 <= B <= 8:
        sys.exit("--batch must be 1..8")

    t0 = time.perf_counter()
    layers = []
    for l in range(LAYERS):
        layers.append((Mat(HIDDEN, HIDDEN, 5, synth.O_PROJ, l, dev),
                       Mat(2 * INTER, HIDDEN, 5, synth.GATE_UP, l, dev),
                       Mat(HIDDEN, INTER, 5, synth.DOWN, l, dev)))
    head = Mat(VOCAB, HIDDEN, 5, synth.LM_HEAD, 0, dev)
    log(f"weights resident ({step_bytes(1) / 1e9:.2f} GB algorithmic per step), "
        f"{time.perf_counter() - t0:.1f} s")

    def inputs(Bn):
        xs = []
        for l in range(LAYERS):
            xs.append((make_x(Bn, HIDDEN, 5, synth.O_PROJ, l, dev), make_x(Bn, HIDDEN, 5, synth.GATE_UP, l, dev),
                       make_x(Bn, INTER, 5, synth.DOWN, l, dev)))
        return xs, make_x(Bn, HIDDEN, 5, synth.LM_HEAD, 0, dev)

    def outputs(Bn):
        return (torch.empty((Bn, HIDDEN), dtype=torch.float32, device=dev),
                torch.empty((Bn, 2 * INTER), dtype=torch.float32, device=dev),
                torch.empty((Bn, HIDDEN), dtype=torch.float32, device=dev),
                torch.empty((Bn, VOCAB), dtype=torch.float32, device=dev),
                torch.empty(Bn, dtype=torch.int32, device=dev),
                torch.empty(w4g.workspace_bytes(w4g.OP_GEMV_ARGMAX, Bn, VOCAB, HIDDEN), dtype=torch.uint8,
                            device=dev))

    def make_step(Bn):
        xs, xh = inputs(Bn)
        yo, yg, yd, logits, ids, ws = outputs(Bn)

        def step(skip_gate_up=False):
            for l in range(LAYERS):
                o, g, d = layers[l]
                xo, xg, xd = xs[l]
                w4g.qmm_gemv(o.wq, o.sc, o.bi, xo, yo)
                if not skip_gate_up:
                    w4g.qmm_gemv(g.wq, g.sc, g.bi, xg, yg)
                w4g.qmm_gemv(d.wq, d.sc, d.bi, xd, yd)
            # the lm_head product (its logits written) and the greedy argmax, the
            # argmax's first pass fused into the product
            w4g.qmm_gemv_argmax(head.wq, head.sc, head.bi, xh, logits, ids, ws)
        return step, ids, logits

    def timed(fn, steps, warmup, graph, reps=1):
        # graph mode captures `reps` back-to-back calls per replay, so the replay's own
        # launch cost is spread over them; the result is per call
        if graph:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                for _ in range(2):
                    fn()
            torch.cuda.current_stream().wait_stream(s)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(reps):
                    fn()
            run = g.replay
        else:
            run = fn
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t_wall = time.perf_counter()
        e0.record()
        for _ in range(steps):
            run()
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_wall
        return e0.elapsed_time(e1) / steps / (reps if graph else 1), wall

    graph = not args.no_graph
    step, ids, logits = make_step(B)
    ms, wall = timed(step, args.steps, args.warmup, graph)
    nbytes = step_bytes(B)
    value = nbytes / (ms * 1e-3) / 1e9
    log(f"sweep B={B}: {ms * 1e3:.1f} us/step, {value:.0f} GB/s ({graph=}), wall {wall:.2f} s")

    # dominant kernel: the gate-up product, timed inside the sweep.  HIP events
    # around graph replays time the step with and without its 16 gate-up
    # launches (alternating, three rounds each, medians); the difference over 16
    # is the average gate-up launch as it runs in the step, neighbours and the
    # gap to the next kernel included.  (The same 16 launches alone, back to
    # back, run slower; that figure is among the secondary ones.)
    gu_bytes = gemv_bytes(2 * INTER, HIDDEN, B)
    with_gu, without_gu = [], []
    for _ in range(3):
        with_gu.append(timed(step, args.steps, 2, graph)[0])
        without_gu.append(timed(lambda: step(skip_gate_up=True), args.steps, 2, graph)[0])
    with_gu.sort()
    without_gu.sort()
    gu_us = (with_gu[1] - without_gu[1]) * 1e3 / LAYERS
    gu_gbs = gu_bytes / (gu_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(gu_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gu_gbs / HBM_PEAK_GBS, 4), "traffic": counted_traffic() if B == 1 else None,
                "kernel": "gemv_valu_kernel (gate_up 5120 -> 34816)", "avg_launch_us": round(gu_us, 2),
                "bytes_per_launch": gu_bytes, "method": "graph-timed step with minus without its 16 launches"}
    log(f"gate_up launch avg {gu_us:.2f} us in the sweep ({with_gu[1] * 1e3:.1f} - {without_gu[1] * 1e3:.1f} "
        f"us per step over {LAYERS}) -> {gu_gbs:.0f} GB/s")

    extras = {}
    if not args.skip_extras:
        extras = secondary(torch, w4g, synth, layers, head, dev, timed, args, make_step)

    cpu = None
    if not args.skip_cpu:
        cpu = cpu_baseline()
        log(f"cpu baseline {cpu}")

    out = {"metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
           "data": "synthetic",
           "config": {"workload": "decode sweep: 16 x (o_proj 5120x5120, gate_up 5120->34816, "
                                  "down 17408->5120) + lm_head 5120->248320 + greedy argmax",
                      "batch": B, "bytes_per_step": nbytes, "hip_graph": graph,
                      "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2)},
           "roofline": roofline, "cpu_baseline": cpu, "secondary": extras}
    print(json.dumps(out), flush=True)


def ceilings(torch, layers, dev, timed):
    """Measured ceilings: a read-only HBM stream of each product's bytes, with plain
    and with non-temporal loads (a graph of launches cycling over enough copies to
    defeat the 256 MB cache; the best of three launch shapes), a matrix-core loop
    with no memory traffic, and torch's
    bf16 matmul (hipBLASLt) on weights dequantized to bf16 (2 bytes per weight
    against 0.5625), for the 512-row prompt shapes."""
    import ctypes
    from w4_gemv_greedy_amd import build as hip_build
    if not os.path.exists(hip_build.CEILING_LIB):
        log("ceilings skipped: libw4g_ceiling.so not built")
        return None
    lib = ctypes.CDLL(hip_build.CEILING_LIB)
    P, SZ, I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.w4g_ceiling_read.argtypes = [P, SZ, I, I, I, I, P, P]
    lib.w4g_ceiling_read.restype = I
    lib.w4g_ceiling_mfma.argtypes = [I, I, P, P]
    lib.w4g_ceiling_mfma.restype = I
    out = {"hbm_read": {}}
    sink = torch.zeros(1 << 20, dtype=torch.float32, device=dev)

    def stream():
        return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

    for name, nbytes, copies in (("o_proj", gemv_bytes(HIDDEN, HIDDEN, 1), 40),
                                 ("down", gemv_bytes(HIDDEN, INTER, 1), 12),
                                 ("gate_up", gemv_bytes(2 * INTER, HIDDEN, 1), 6),
                                 ("lm_head", gemv_bytes(VOCAB, HIDDEN, 1), 2)):
        nb = nbytes // 16 * 16
        bufs = [torch.full((nb,), c, dtype=torch.uint8, device=dev) for c in range(copies)]
        launches = max(16, copies)  # every copy once per replay
        entry = {"bytes": nb}
        for nt, key in ((0, "plain"), (1, "nontemporal")):
            best = None
            for blocks, threads, u in ((256, 1024, 4), (2048, 256, 4), (4096, 256, 2)):
                def run(blocks=blocks, threads=threads, u=u, nt=nt):
                    for i in range(launches):
                        st = lib.w4g_ceiling_read(bufs[i % copies].data_ptr(), nb, blocks, threads, u, nt,
                                                  sink.data_ptr(), stream())
                        if st != 0:
                            raise RuntimeError(f"w4g_ceiling_read: hip error {st}")
                ms, _ = timed(run, 10, 2, True)
                us = ms * 1e3 / launches
                if best is None or us < best[0]:
                    best = (us, f"{blocks}x{threads}, {u} loads in flight")
            entry[key] = {"us": round(best[0], 2), "GBps": round(nb / (best[0] * 1e-6) / 1e9, 1), "launch": best[1]}
        out["hbm_read"][name] = entry
        del bufs
    torch.cuda.empty_cache()

    # the codes of each layer matrix read in the shape of one wave load of a decode
    # kernel (non-temporal 16-byte loads): which load layouts can stream at HBM rate
    lib.w4g_ceiling_read_rows.argtypes = [P, ctypes.c_int64, ctypes.c_int64, I, I, I, I, P, P]
    lib.w4g_ceiling_read_rows.restype = I
    pats = ((0, "half_wave_512B_per_row", 2, 512), (1, "mfma16_in_place_64B_per_row", 16, 64),
            (2, "mfma16_adjacent_lanes_64B_per_row", 16, 64), (3, "mfma32_in_place_32B_per_row", 32, 32))
    out["code_load_layouts"] = {}
    for name, rows, K, copies in (("o_proj", HIDDEN, HIDDEN, 40), ("gate_up", 2 * INTER, HIDDEN, 6),
                                  ("down", HIDDEN, INTER, 12)):
        rb = K // 2
        bufs = [torch.full((rows * rb,), c, dtype=torch.uint8, device=dev) for c in range(copies)]
        launches = max(16, copies)
        entry = {"bytes": rows * rb}
        for pat, key, tr, per in pats:
            tiles = -(-rows // tr)
            # whole rows per unit where there are enough tiles, else the most slices
            # per row that keep the units at 4096 or fewer; one workgroup per CU,
            # one unit per wave up to 4096 units, else 8 waves striding through them
            cands = [k for k in range(1, rb // per + 1) if rb % (k * per) == 0 and tiles * k <= 4096]
            sl = cands[-1] if cands else 1
            units = tiles * sl
            blocks = 256
            threads = 64 * max(1, min(16, -(-units // blocks))) if units <= 4096 else 512

            def run(pat=pat, sl=sl, blocks=blocks, threads=threads):
                for i in range(launches):
                    st = lib.w4g_ceiling_read_rows(bufs[i % copies].data_ptr(), rows, rb, pat, sl, blocks, threads,
                                                   sink.data_ptr(), stream())
                    if st != 0:
                        raise RuntimeError(f"w4g_ceiling_read_rows: hip error {st}")
            ms, _ = timed(run, 10, 2, True)
            us = ms * 1e3 / launches
            entry[key] = {"us": round(us, 2), "GBps": round(rows * rb / (us * 1e-6) / 1e9, 1), "slices": sl,
                          "launch": f"{blocks}x{threads}"}
        out["code_load_layouts"][name] = entry
        del bufs
    torch.cuda.empty_cache()

    blocks, iters = 1024, 400
    flop = blocks * 4 * iters * 8 * 32768

    def mf():
        st = lib.w4g_ceiling_mfma(blocks, iters, sink.data_ptr(), stream())
        if st != 0:
            raise RuntimeError(f"w4g_ceiling_mfma: hip error {st}")
    ms, _ = timed(mf, 10, 2, True)
    out["mfma_bf16_loop_TFLOPS"] = round(flop / (ms * 1e-3) / 1e12, 1)

    # torch bf16 matmul on dequantized weights (w = q*s + b, rounded to bf16)
    shifts = torch.arange(0, 32, 4, dtype=torch.int32, device=dev)
    tm = {}
    for name, idx, N, K in (("o_proj", 0, HIDDEN, HIDDEN), ("gate_up", 1, 2 * INTER, HIDDEN),
                            ("down", 2, HIDDEN, INTER)):
        m = layers[0][idx]
        q = ((m.wq.unsqueeze(-1) >> shifts) & 15).reshape(N, K).float()
        w = (q.view(N, K // 64, 64) * m.sc.float().unsqueeze(-1) + m.bi.float().unsqueeze(-1))
        w = w.reshape(N, K).to(torch.bfloat16).contiguous()
        del q
        x = torch.randn((512, K), device=dev).to(torch.bfloat16)
        y = torch.empty((512, N), dtype=torch.bfloat16, device=dev)

        def mm(x=x, w=w, y=y):
            torch.mm(x, w.t(), out=y)
        ms, _ = timed(mm, 10, 3, True, reps=4)
        tm[name] = round(2.0 * 512 * N * K / (ms * 1e-3) / 1e12, 1)
        del w
    out["torch_bf16_matmul_m512_TFLOPS"] = tm
    torch.cuda.empty_cache()
    return out


def eager_percentiles(torch, w4g, copies, dev, calls=160):
    """Per-call times of the batch-1 products as eager launches (HIP events around
    each call, cycling over distinct copies of each matrix: 40 for o_proj, 16
    for gate-up and down): median, p10 and p90 in us."""
    res = {}
    from w4_gemv_greedy_amd import synth
    for name, idx, N, K in (("o_proj", 0, HIDDEN, HIDDEN), ("gate_up", 1, 2 * INTER, HIDDEN),
                            ("down", 2, HIDDEN, INTER)):
        x = make_x(1, K, 5, synth.GENERIC, 98, dev)
        y = torch.empty((1, N), dtype=torch.float32, device=dev)
        mats = copies[idx]
        for m in mats:
            w4g.qmm_gemv(m.wq, m.sc, m.bi, x, y)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
        torch.cuda.synchronize()
        for i in range(calls):
            m = mats[i % len(mats)]
            ev[i][0].record()
            w4g.qmm_gemv(m.wq, m.sc, m.bi, x, y)
            ev[i][1].record()
        torch.cuda.synchronize()
        t = np.sort(np.array([a.elapsed_time(b) * 1e3 for a, b in ev]))
        res[name] = {"median_us": round(float(np.median(t)), 2), "p10_us": round(float(np.percentile(t, 10)), 2),
                     "p90_us": round(float(np.percentile(t, 90)), 2), "calls": calls, "copies": len(mats)}
    return res


def secondary(torch, w4g, synth, layers, head, dev, timed, args, make_step):
    ex = {}
    # the sweep as eager launches (no graph)
    step_e, _, _ = make_step(1)
    ms_e, _ = timed(step_e, 10, 3, False)
    ex["sweep_b1_eager_us"] = round(ms_e * 1e3, 1)
    # distinct copies of each matrix for the per-product timings, so that no call
    # finds its matrix in the 256 MB cache: o_proj over 40 copies (590 MB: the
    # 16 layers' and 24 more), gate-up and down over the 16 layers' (1.6 GB and
    # 0.8 GB)
    extra_o = [Mat(HIDDEN, HIDDEN, 5, synth.O_PROJ, 100 + c, dev) for c in range(24)]
    copies = {0: [lay[0] for lay in layers] + extra_o, 1: [lay[1] for lay in layers],
              2: [lay[2] for lay in layers]}
    ex["b1_eager_per_call"] = eager_percentiles(torch, w4g, copies, dev)
    log(f"sweep B=1 eager {ex['sweep_b1_eager_us']} us/step; per call {ex['b1_eager_per_call']}")
    # the 16 gate-up launches of a step alone, back to back in a graph
    xg_in = [make_x(1, HIDDEN, 5, synth.GATE_UP, l, dev) for l in range(LAYERS)]
    yg_out = torch.empty((1, 2 * INTER), dtype=torch.float32, device=dev)

    def gate_up_only():
        for l in range(LAYERS):
            g = layers[l][1]
            w4g.qmm_gemv(g.wq, g.sc, g.bi, xg_in[l], yg_out)
    ms_g, _ = timed(gate_up_only, 10, 2, True)
    ex["gate_up_b1_graph16_us"] = round(ms_g * 1e3 / LAYERS, 2)

    # lm_head + argmax per token (batch 1)
    xh = make_x(1, HIDDEN, 5, synth.LM_HEAD, 1, dev)
    logits = torch.empty((1, VOCAB), dtype=torch.float32, device=dev)
    ids = torch.empty(1, dtype=torch.int32, device=dev)
    ws = torch.empty(w4g.workspace_bytes(w4g.OP_ARGMAX, 1, VOCAB, 0), dtype=torch.uint8, device=dev)

    def head_step():
        w4g.qmm_gemv(head.wq, head.sc, head.bi, xh, logits)
        w4g.vocab_argmax(logits, ids, ws)
    ms, _ = timed(head_step, 10, 2, True, reps=4)
    ex["lm_head_argmax_us_per_token"] = round(ms * 1e3, 2)
    ex["lm_head_argmax_GBps"] = round((gemv_bytes(VOCAB, HIDDEN, 1) + 4 * VOCAB) / (ms * 1e-3) / 1e9, 1)

    # the same with the argmax's first pass fused into the product (logits kept / not written)
    ws_f = torch.empty(w4g.workspace_bytes(w4g.OP_GEMV_ARGMAX, 1, VOCAB, HIDDEN), dtype=torch.uint8,
                       device=dev)

    def head_fused():
        w4g.qmm_gemv_argmax(head.wq, head.sc, head.bi, xh, logits, ids, ws_f)

    def head_fused_ids_only():
        w4g.qmm_gemv_argmax(head.wq, head.sc, head.bi, xh, None, ids, ws_f, want_logits=False)
    ms, _ = timed(head_fused, 10, 2, True, reps=4)
    ex["lm_head_argmax_fused_us_per_token"] = round(ms * 1e3, 2)
    ms, _ = timed(head_fused_ids_only, 10, 2, True, reps=4)
    ex["lm_head_argmax_fused_ids_only_us_per_token"] = round(ms * 1e3, 2)
    log(f"lm_head+argmax fused {ex['lm_head_argmax_fused_us_per_token']} us/token, ids only "
        f"{ex['lm_head_argmax_fused_ids_only_us_per_token']} us/token")

    def argmax_only():
        w4g.vocab_argmax(logits, ids, ws)
    ms, _ = timed(argmax_only, 20, 3, True, reps=20)
    ex["argmax_us"] = round(ms * 1e3, 2)
    ids2 = torch.empty((1, 2), dtype=torch.int32, device=dev)
    gaps = torch.empty(1, dtype=torch.float32, device=dev)
    ws2 = torch.empty(w4g.workspace_bytes(w4g.OP_ARGMAX_TOP2, 1, VOCAB, 0), dtype=torch.uint8,
                      device=dev)

    def top2_only():
        w4g.vocab_argmax_top2(logits, ids2, gaps, ws2)
    ms, _ = timed(top2_only, 20, 3, True, reps=20)
    ex["argmax_top2_us"] = round(ms * 1e3, 2)
    log(f"lm_head+argmax {ex['lm_head_argmax_us_per_token']} us/token, argmax alone {ex['argmax_us']} us, "
        f"top two {ex['argmax_top2_us']} us")

    # per-product averages at batch 1, 4, 8: the library's own choice and both
    # kernel families, each cycling through the distinct copies above
    for fam_name, fam in (("auto", w4g.GEMV_AUTO), ("valu", w4g.GEMV_VALU), ("mfma", w4g.GEMV_MFMA)):
        for Bn in (1, 4, 8):
            if fam_name == "valu" and Bn == 1:
                continue  # the automatic choice is the vector-ALU kernel at B = 1
            for name, idx, N, K, mid in (("o_proj", 0, HIDDEN, HIDDEN, synth.O_PROJ),
                                         ("gate_up", 1, 2 * INTER, HIDDEN, synth.GATE_UP),
                                         ("down", 2, HIDDEN, INTER, synth.DOWN)):
                x = make_x(Bn, K, 5, mid, 99, dev)
                y = torch.empty((Bn, N), dtype=torch.float32, device=dev)
                mats = copies[idx]

                def run(mats=mats, x=x, y=y, fam=fam):
                    for m in mats:
                        w4g.qmm_gemv(m.wq, m.sc, m.bi, x, y, kernel=fam)
                ms, _ = timed(run, 5, 2, True)
                us = ms * 1e3 / len(mats)
                gbs = gemv_bytes(N, K, Bn) / (us * 1e-6) / 1e9
                ex[f"gemv_{name}_b{Bn}_{fam_name}"] = {"us": round(us, 2), "GBps": round(gbs, 1),
                                                      "pct_peak": round(100 * gbs / HBM_PEAK_GBS, 1),
                                                      "copies": len(mats)}
    log("per-product: " + ", ".join(f"{k} {v['us']}us {v['GBps']}GB/s" for k, v in ex.items()
                                    if k.startswith("gemv_")))
    del extra_o, copies
    torch.cuda.empty_cache()

    # other code widths (B = 1): the 8-bit LM head with the greedy argmax, and the
    # gate-up product at 8 and 2 bits, cycling over enough copies that none is
    # served from the 256 MB cache
    head8 = Mat(VOCAB, HIDDEN, 5, synth.LM_HEAD, 0, dev, bits=8)

    def head8_step():
        w4g.qmm_gemv(head8.wq, head8.sc, head8.bi, xh, logits, bits=8)
        w4g.vocab_argmax(logits, ids, ws)
    ms, _ = timed(head8_step, 10, 2, True, reps=4)
    ex["w8_lm_head_argmax_us_per_token"] = round(ms * 1e3, 2)
    ex["w8_lm_head_argmax_GBps"] = round((1.0625 * VOCAB * HIDDEN + 2 * HIDDEN + 8 * VOCAB) / (ms * 1e-3) / 1e9, 1)
    # the same head with the argmax's first pass fused into the product (ids only)
    ws8 = torch.empty(w4g.workspace_bytes(w4g.OP_GEMV_BITS_ARGMAX, 1, VOCAB, HIDDEN), dtype=torch.uint8,
                      device=dev)

    def head8_fused():
        w4g.qmm_gemv_argmax(head8.wq, head8.sc, head8.bi, xh, ids=ids, workspace=ws8, want_logits=False, bits=8)
    ms, _ = timed(head8_fused, 10, 2, True, reps=4)
    ex["w8_lm_head_argmax_fused_ids_only_us_per_token"] = round(ms * 1e3, 2)
    del head8, ws8
    xg1 = make_x(1, HIDDEN, 5, synth.GATE_UP, 0, dev)
    yg1 = torch.empty((1, 2 * INTER), dtype=torch.float32, device=dev)
    for bits, copies in ((8, 4), (2, 6)):
        mats = [Mat(2 * INTER, HIDDEN, 5, synth.GATE_UP, l, dev, bits=bits) for l in range(copies)]

        def run_bits(mats=mats, bits=bits):
            for m in mats:
                w4g.qmm_gemv(m.wq, m.sc, m.bi, xg1, yg1, bits=bits)
        ms, _ = timed(run_bits, 10, 2, True)
        us = ms * 1e3 / copies
        nb = (bits / 8 + 0.0625) * 2 * INTER * HIDDEN + 2 * HIDDEN + 4 * 2 * INTER
        ex[f"w{bits}_gate_up_b1"] = {"us": round(us, 2), "GBps": round(nb / (us * 1e-6) / 1e9, 1)}
        del mats
    log(f"other widths: w8 lm_head+argmax {ex['w8_lm_head_argmax_us_per_token']} us/token "
        f"({ex['w8_lm_head_argmax_GBps']} GB/s; fused, ids only "
        f"{ex['w8_lm_head_argmax_fused_ids_only_us_per_token']}), w8 gate_up {ex['w8_gate_up_b1']}, w2 gate_up {ex['w2_gate_up_b1']}")
    torch.cuda.empty_cache()

    # prompt products: the 512-row pass, the 128-row round and short prompts of 64
    # and 16 rows (where the weight stream, not the matrix cores, sets the time).
    # Each timed call walks the 16 layers' weights, so no call finds its matrix in
    # the 256 MB cache; the 128-row round is also timed with the bf16 store.
    for M in (512, 128, 64, 16):
        pr = {}
        for name, idx, N, K, mid in (("o_proj", 0, HIDDEN, HIDDEN, synth.O_PROJ),
                                     ("gate_up", 1, 2 * INTER, HIDDEN, synth.GATE_UP),
                                     ("down", 2, HIDDEN, INTER, synth.DOWN)):
            x = make_x(M, K, 4, mid, 0, dev)
            ws = torch.empty(max(1, w4g.workspace_bytes(w4g.OP_GEMM, M, N, K)), dtype=torch.uint8, device=dev)
            for dt in ((torch.float32, torch.bfloat16) if M == 128 else (torch.float32,)):
                y = torch.empty((M, N), dtype=dt, device=dev)

                def run(idx=idx, x=x, y=y, ws=ws):
                    for lay in layers:
                        m = lay[idx]
                        w4g.qmm_gemm(m.wq, m.sc, m.bi, x, y, ws)
                ms, _ = timed(run, 3 if M == 512 else 10, 1, True)
                us = ms * 1e3 / len(layers)
                tf = 2.0 * M * N * K / (us * 1e-6) / 1e12
                gbs = (0.5625 * N * K + 2.0 * M * K + y.element_size() * M * N) / (us * 1e-6) / 1e9
                pr[name + ("" if dt == torch.float32 else "_bf16out")] = {
                    "us": round(us, 1), "TFLOPS": round(tf, 1),
                    "pct_mfma_peak": round(100 * tf / BF16_PEAK_TFLOPS, 1), "GBps": round(gbs, 1)}
        ex[f"prompt_gemm_m{M}"] = pr
        log(f"prompt M={M}: " + ", ".join(f"{k} {v['us']}us {v['TFLOPS']}TF {v['GBps']}GB/s"
                                          for k, v in pr.items()))

    # the batch-8 sweep
    if args.batch != 8:
        xs8 = [(make_x(8, HIDDEN, 6, synth.O_PROJ, l, dev), make_x(8, HIDDEN, 6, synth.GATE_UP, l, dev),
                make_x(8, INTER, 6, synth.DOWN, l, dev)) for l in range(LAYERS)]
        xh8 = make_x(8, HIDDEN, 6, synth.LM_HEAD, 0, dev)
        yo = torch.empty((8, HIDDEN), dtype=torch.float32, device=dev)
        yg = torch.empty((8, 2 * INTER), dtype=torch.float32, device=dev)
        lg = torch.empty((8, VOCAB), dtype=torch.float32, device=dev)
        ids8 = torch.empty(8, dtype=torch.int32, device=dev)
        ws8 = torch.empty(w4g.workspace_bytes(w4g.OP_ARGMAX, 8, VOCAB, 0), dtype=torch.uint8, device=dev)

        def step8(fam=w4g.GEMV_AUTO):
            for l in range(LAYERS):
                o, g, d = layers[l]
                w4g.qmm_gemv(o.wq, o.sc, o.bi, xs8[l][0], yo, kernel=fam)
                w4g.qmm_gemv(g.wq, g.sc, g.bi, xs8[l][1], yg, kernel=fam)
                w4g.qmm_gemv(d.wq, d.sc, d.bi, xs8[l][2], yo, kernel=fam)
            w4g.qmm_gemv(head.wq, head.sc, head.bi, xh8, lg, kernel=fam)
            w4g.vocab_argmax(lg, ids8, ws8)
        # the library's own choice (the vector-ALU family: a row's bits at B = 8
        # are its bits at B = 1), and the matrix-core family named explicitly
        for key, fam in (("sweep_b8", w4g.GEMV_AUTO), ("sweep_b8_mfma", w4g.GEMV_MFMA)):
            ms, _ = timed(lambda fam=fam: step8(fam), 10, 2, True)
            ex[key] = {"us_per_step": round(ms * 1e3, 1), "us_per_token": round(ms * 1e3 / 8, 2),
                       "GBps": round(step_bytes(8) / (ms * 1e-3) / 1e9, 1)}
            log(f"{key}: {ex[key]}")

        # the head alone at B = 8: product + two-pass argmax, and fused
        ws8f = torch.empty(w4g.workspace_bytes(w4g.OP_GEMV_ARGMAX, 8, VOCAB, HIDDEN), dtype=torch.uint8,
                           device=dev)

        def head8(fam=w4g.GEMV_AUTO):
            w4g.qmm_gemv(head.wq, head.sc, head.bi, xh8, lg, kernel=fam)
            w4g.vocab_argmax(lg, ids8, ws8)

        def head8_fused():
            w4g.qmm_gemv_argmax(head.wq, head.sc, head.bi, xh8, None, ids8, ws8f, want_logits=False)
        ms, _ = timed(head8, 10, 2, True, reps=2)
        ms_m, _ = timed(lambda: head8(w4g.GEMV_MFMA), 10, 2, True, reps=2)
        ms_f, _ = timed(head8_fused, 10, 2, True, reps=2)
        ex["lm_head_argmax_b8"] = {"us_per_call": round(ms * 1e3, 1), "mfma_us_per_call": round(ms_m * 1e3, 1),
                                   "fused_ids_only_us_per_call": round(ms_f * 1e3, 1)}
        log(f"lm_head+argmax B=8: {ex['lm_head_argmax_b8']}")

    ex["ceilings"] = ceilings(torch, layers, dev, timed)
    log(f"ceilings: {ex['ceilings']}")
    return ex


if __name__ == "__main__":
    main()
