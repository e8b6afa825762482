#!/usr/bin/env python3
"""Benchmark of the SAGE batch-one decode path on one MI355X.

Default workload: one Qwen3-4B-shaped decoder layer at batch one (q 4096x2560, k/v 1024x2560,
o 2560x4096, gate/up 9728x2560, down 2560x9728), split (K, V) = (64, 4), codes drawn directly
(synthetic, seeded). A step is one pass over the layer's seven projections in dependency order:
q|k|v in one launch (they read the same input), o, gate|up in one launch, down. Every step uses a
different copy of the layer's packed weights, and the copies together exceed 512 MB, twice the
MI355X's 256 MB last-level cache, so weights stream from HBM as they would in a model.

The timed region replays a HIP graph of the steps (launching from Python per kernel would measure
the host, not the GPU). It prints one JSON line: whole-step packed-weight GB/s (the metric), the
per-step time, tokens/s of the layer, the roofline of the dominant launch (gate|up) from HIP
events around a graph of such launches on their stream, the HBM traffic measured with counters
(profiles/), a plain streaming read of the same bytes as the reference floor, and
the CPU oracle's rate on a bounded sample of the same workload.

  python bench.py [--steps K] [--warmup W] [--mode compiled|eager]
                  [--workload layer|sweep|gemm|prefill|moe|encode|single|all]

The secondary workloads print one JSON line per case (not the headline line); `encode` times the
fixed-codebook GPU encoder (sage_encode_fields) on 9728x2560 for three splits.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # dense fp16, published
FP64_PEAK_TFLOPS = 78.6        # fp64, published
MALL_BYTES = 256 << 20


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="layer",
                    choices=["layer", "sweep", "gemm", "prefill", "moe", "encode", "decode",
                             "single", "all"])
    ap.add_argument("--copies", type=int, default=0, help="weight copies to rotate (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", default="compiled", choices=["compiled", "eager"],
                    help="compiled: inputs arrive permuted, matrices run with pi = NULL (the "
                         "paper's compiled decoding); eager: each launch gathers through pi")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--eager", action="store_true", help="launch from Python (no graph)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 256 MiB device copy (a kernel of known traffic, used to "
                         "scale rocprofv3 FETCH_SIZE / WRITE_SIZE readings)")
    return ap.parse_args()


# ------------------------------------------------------------------------------------------------
# inputs on the device (seeded synthetic fields, packed by libsage)
# ------------------------------------------------------------------------------------------------

def upload_pack(c):
    import numpy as np
    import torch
    import bit_vector_quantized_amd as sage

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    L = int(c.K).bit_length() - 1
    return sage.pack(t(c.signs), t(c.idx), t(c.rcode), t(c.mu.view(np.float16)),
                     t(c.delta.view(np.float16)), t(c.codebook.view(np.float16)), t(c.pi), L, c.V)


def clone_packed(p):
    import bit_vector_quantized_amd as sage
    return sage.Packed(p.d_out, p.d_in, p.log2K, p.V, p.packed.clone(), p.codebook.clone(),
                       None if p.pi is None else p.pi.clone())


def algorithmic_bytes(p, n_x=1):
    """payload + fp16 grid + codebook + pi (int32) + x + y of one product (SAGE's stored fields
    and the fp16 vectors), the per-unit traffic a perfect kernel reads or writes once."""
    packed = p.d_out * p.d_in * 18 // 64 + p.d_out * (p.d_in // 128) * 4
    return packed + (1 << p.log2K) * 16 + (p.d_in * 4 if p.pi is not None else 0) \
        + n_x * p.d_in * 2 + p.d_out * 2


def packed_weight_bytes(p):
    return p.d_out * p.d_in * 18 // 64 + p.d_out * (p.d_in // 128) * 4


GEMV_SOURCES = ("sage_gemv.hip", "sage_internal.hpp")


def kernel_sources_digest():
    """sha256 (16 hex digits) over the sources the batch-one kernel is built from."""
    h = hashlib.sha256()
    for name in GEMV_SOURCES:
        with open(os.path.join(ROOT, "bit_vector_quantized_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(name):
    """HBM bytes per launch measured with rocprofv3 counters (profiles/), valid only for the
    kernel sources they were measured on."""
    path = os.path.join(ROOT, "profiles", f"{name}.traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_sources") != kernel_sources_digest():
        return None
    return d.get("traffic_bytes")


# ------------------------------------------------------------------------------------------------
# the decoder-layer step
# ------------------------------------------------------------------------------------------------

class LayerBench:
    """The layer step: q|k|v in one launch, o, gate|up in one launch, down (4 launches). Mode
    "compiled": the matrices run with pi = NULL and their inputs arrive already permuted, as the
    producers of the paper's compiled decoding write them (§3.5); mode "eager": each launch
    gathers its input through pi itself."""
    LAUNCHES = (("qkv", ("q", "k", "v"), "attn_in"), ("o", ("o",), "attn_out"),
                ("gateup", ("gate", "up"), "mlp_in"), ("down", ("down",), "mlp_mid"))

    def __init__(self, copies, steps, mode="compiled"):
        import dataclasses
        import numpy as np
        import torch
        import workloads as W
        import bit_vector_quantized_amd as sage
        self.sage = sage
        self.mode = mode
        self.layer = W.decoder_layer()
        base = {n: upload_pack(c) for n, c in self.layer.mats.items()}
        xs = dict(self.layer.xs)
        if mode == "compiled":
            for key, names, inp in self.LAUNCHES:
                pi = self.layer.mats[names[0]].pi
                xs[inp] = np.ascontiguousarray(xs[inp][pi])
            base = {n: dataclasses.replace(p, pi=None) for n, p in base.items()}
        self.bytes_per_layer = sum(packed_weight_bytes(p) for p in base.values())
        if copies <= 0:
            need = max(2, math.ceil(2 * MALL_BYTES / self.bytes_per_layer) + 1)
            divisors = [d for d in range(need, 4 * need) if steps % d == 0]
            copies = divisors[0] if divisors else need
        self.copies = [base] + [{n: clone_packed(p) for n, p in base.items()}
                                for _ in range(copies - 1)]
        self.xs = {k: torch.from_numpy(v).cuda() for k, v in xs.items()}
        self.ys = {n: torch.empty(p.d_out, dtype=torch.float16, device="cuda")
                   for n, p in base.items()}
        self.dom_name = "gemv_kernel (gate|up, 2 x 9728x2560 in one launch)"
        self.dom_bytes = sum(algorithmic_bytes(base[n]) for n in ("gate", "up"))
        self.launches = 4
        self.dom_profile = "gemv_gateup_9728x2560x2"
        self.base = base
        torch.cuda.synchronize()

    def launch(self, key, i):
        names, inp = {k: (n, x) for k, n, x in self.LAUNCHES}[key]
        mats = self.copies[i % len(self.copies)]
        ps = [mats[n] for n in names]
        x = self.xs[inp]
        self.sage.gemv_multi(ps, [x] * len(ps), [self.ys[n] for n in names])

    def dominant(self, i):
        self.launch("gateup", i)

    def step(self, i, ev=None):
        for key, _, _ in self.LAUNCHES:
            self.launch(key, i)


def timed_graph(bench, steps, warmup, eager=False, dominant=True):
    """Returns (wall seconds for `steps` steps, list of dominant-kernel durations in ms)."""
    import torch
    n = len(bench.copies)
    for i in range(warmup):
        bench.step(i)
    torch.cuda.synchronize()
    if eager:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            bench.step(i, evs[i])
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return t1 - t0, [a.elapsed_time(b) for a, b in evs]
    # One graph holds `per` steps over consecutive copies; replayed until `steps` are done.
    per = n
    while steps % per:
        per -= 1
    reps = steps // per
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(per)]

    def capture(with_events):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for i in range(per):
                    bench.step(i, evs[i] if with_events else None)
        torch.cuda.synchronize()
        return g

    # HIP graphs accept captured event records but cannot time them afterwards, so the graph
    # carries only kernels; the dominant launch is timed with HIP events right after.
    g = capture(False)
    g.replay()  # untimed: first replay uploads the graph
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    durs = dominant_graph(bench, per, evs) if dominant else []
    return t1 - t0, durs


def dominant_graph(bench, count, evs, key="gateup"):
    """Average duration of one launch kind (the dominant gate|up by default): a graph of `count`
    such launches over distinct weight copies, replayed between two HIP events on the stream the
    kernels run on. The figure includes the short gap between consecutive kernels of a graph."""
    import torch
    del evs
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(count):
                bench.launch(key, i)
    torch.cuda.synchronize()
    reps = 10
    with torch.cuda.stream(s):
        g.replay()  # upload
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(s)
        for _ in range(reps):
            g.replay()
        b.record(s)
    torch.cuda.synchronize()
    per = a.elapsed_time(b) / (reps * count)
    return [per] * count


def stream_reference(nbytes):
    """The floor for one streaming launch of `nbytes`: sage_stream_read (plain 16-byte loads, no
    decode) over consecutive windows of a 1 GiB buffer, one launch per window, in a graph timed
    like the dominant launch; plus one launch reading the whole GiB."""
    import torch
    import bit_vector_quantized_amd as sage
    pool = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    n = (nbytes + 15) // 16 * 16
    windows = (1 << 30) // n
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for w in range(windows):
                sage.stream_read(pool[w * n:(w + 1) * n], sink=sink)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    reps = 5
    with torch.cuda.stream(s):
        g.replay()
        a.record(s)
        for _ in range(reps):
            g.replay()
        b.record(s)
        torch.cuda.synchronize()
        c = torch.cuda.Event(enable_timing=True)
        d = torch.cuda.Event(enable_timing=True)
        sage.stream_read(pool, sink=sink)
        c.record(s)
        for _ in range(reps):
            sage.stream_read(pool, sink=sink)
        d.record(s)
    torch.cuda.synchronize()
    per_us = a.elapsed_time(b) * 1e3 / (reps * windows)
    gib_us = c.elapsed_time(d) * 1e3 / reps
    del pool
    return {"bytes_per_launch": n, "us_per_launch": round(per_us, 3),
            "gbs": round(n / (per_us * 1e-6) / 1e9, 1),
            "one_gib_launch_gbs": round((1 << 30) / (gib_us * 1e-6) / 1e9, 1)}


def launch_floors(bench):
    """Per-launch floors measured the same way as the layer's launches (a graph of back-to-back
    launches timed with HIP events): an empty launch (sage_stream_read of 16 bytes: dispatch and
    completion only), and for each launch of the step a streaming read of its packed bytes."""
    import torch
    import bit_vector_quantized_amd as sage
    pool = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")

    def graph_us(nbytes):
        n = (nbytes + 15) // 16 * 16
        windows = min(64, (1 << 30) // n)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for w in range(windows):
                    sage.stream_read(pool[w * n:(w + 1) * n], sink=sink)
        torch.cuda.synchronize()
        reps = 10
        with torch.cuda.stream(s):
            g.replay()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(s)
            for _ in range(reps):
                g.replay()
            b.record(s)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / (reps * windows)

    out = {"empty_launch_us": round(graph_us(16), 3), "stream_read_us": {}}
    for key, names, _ in LayerBench.LAUNCHES:
        nb = sum(packed_weight_bytes(bench.base[n]) for n in names)
        out["stream_read_us"][key] = round(graph_us(nb), 3)
    del pool
    return out


# ------------------------------------------------------------------------------------------------
# CPU oracle baseline
# ------------------------------------------------------------------------------------------------

def _oracle_passes(layer, seconds, threads):
    from threadpoolctl import threadpool_limits
    from oracle import decoder
    names = ["q", "k", "v", "o", "gate", "up", "down"]
    done_bytes = 0
    matrices = 0
    t0 = time.perf_counter()
    with threadpool_limits(threads):
        while True:
            for n in names:
                c = layer.mats[n]
                decoder.gemv(c, layer.xs[layer.input_of[n]])
                done_bytes += c.d_out * c.d_in * 18 // 64 + c.d_out * (c.d_in // 128) * 4
                matrices += 1
            if time.perf_counter() - t0 >= seconds:
                break
    return done_bytes, matrices, time.perf_counter() - t0


def cpu_baseline(layer, seconds):
    """The float64 oracle (decode + matrix-vector product per matrix, exactly as the tests use it)
    over whole passes of the layer's seven matrices until `seconds` elapse, single-threaded; then a
    shorter run with the BLAS thread pool on every core this process may use."""
    done_bytes, matrices, dt = _oracle_passes(layer, seconds, 1)
    all_cores = len(os.sched_getaffinity(0))
    b2, m2, dt2 = _oracle_passes(layer, max(2.0, seconds / 4), all_cores)
    return {"value": round(done_bytes / dt / 1e9, 6), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{matrices} matrix products ({matrices // 7} passes over the 7-matrix layer),"
                      f" float64 NumPy decode + matvec, {dt:.1f} s, 1 thread",
            "tokens_per_s": round(matrices / 7 / dt, 4),
            "all_cores": {"value": round(b2 / dt2 / 1e9, 6), "cores": all_cores,
                          "sample": f"{m2} matrix products, {dt2:.1f} s, BLAS threads = cores"}}


# ------------------------------------------------------------------------------------------------
# secondary workloads (one JSON line each, for profiling; not the headline line)
# ------------------------------------------------------------------------------------------------

def bench_single_products(kind, steps, warmup):
    import numpy as np
    import torch
    import workloads as W
    import bit_vector_quantized_amd as sage
    lines = []
    cases = []
    if kind in ("sweep", "all"):
        for K, V in W.SPLITS_FIVE:
            c, x = W.split_sweep_matrix(K, V)
            cases.append((f"sweep_9728x2560_K{K}V{V}", c, x, 1))
    if kind in ("single", "all"):
        for name, c in W.decoder_layer().mats.items():
            cases.append((f"layer_{name}_{c.d_out}x{c.d_in}", c, None, 1))
        # an LM-head-sized product (Qwen3 vocabulary x hidden 2560, 109 MB packed): one launch of
        # several rounds of workgroups
        c = W.draw_codes(W.rng_for(190), 151936, 2560, 64, 4)
        cases.append(("lm_head_151936x2560", c, None, 1))
    if kind in ("gemm", "all"):
        for shape in ((9728, 2560), (2560, 9728)):
            for M in (1, 4, 16, 64):
                c, X = W.small_batch(shape[0], shape[1], M)
                cases.append((f"gemm_{shape[0]}x{shape[1]}_M{M}", c, X, M))
                if M > 1:
                    # compiled decoding: the rows arrive in stored order, the matrix runs with
                    # pi = NULL and no reorder of X runs (SAGE paper §3.5)
                    cases.append((f"gemm_{shape[0]}x{shape[1]}_M{M}_compiled", c,
                                  np.ascontiguousarray(X[:, c.pi]), -M))
    if kind in ("prefill", "all"):
        for shape in ((9728, 2560), (2560, 9728)):
            for M in (128, 256, 512, 1024):
                c, X = W.small_batch(shape[0], shape[1], M)
                cases.append((f"prefill_{shape[0]}x{shape[1]}_M{M}", c, X, M))
    for name, c, x, M in cases:
        log(f"[case] {name}")
        base = upload_pack(c)
        if M < 0:   # compiled decoding (see above)
            M = -M
            base = sage.Packed(base.d_out, base.d_in, base.log2K, base.V, base.packed,
                               base.codebook, None)
        pb = packed_weight_bytes(base)
        copies = max(2, math.ceil(2 * MALL_BYTES / pb) + 1)
        ps = [base] + [clone_packed(base) for _ in range(copies - 1)]
        if M == 1 and (x is None or x.ndim == 1):
            xd = torch.randn(c.d_in, dtype=torch.float16, device="cuda") if x is None \
                else torch.from_numpy(x).cuda()
            y = torch.empty(c.d_out, dtype=torch.float16, device="cuda")
            ws = sage.workspace(sage.gemv_workspace_bytes(base), "cuda")
            fn = lambda p: sage.gemv(p, xd, y, ws=ws)
        else:
            Xd = torch.from_numpy(x).cuda()
            Y = torch.empty((M, c.d_out), dtype=torch.float16, device="cuda")
            ws = sage.workspace(sage.gemm_small_workspace_bytes(base, M), "cuda")
            fn = lambda p: sage.gemm_small(p, Xd, Y, ws=ws)
        for i in range(warmup):
            fn(ps[i % copies])
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for i in range(copies):
                    fn(ps[i])
        g.replay()
        torch.cuda.synchronize()
        reps = max(1, steps // copies)
        t0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / (reps * copies)
        alg = algorithmic_bytes(base, n_x=M) + (M - 1) * c.d_out * 2
        line = {"workload": name, "us_per_call": round(dt * 1e6, 3),
                "packed_gbs": round(pb / dt / 1e9, 1), "effective_gbs": round(alg / dt / 1e9, 1),
                "pct_hbm_peak": round(100 * alg / dt / 1e9 / HBM_PEAK_GBS, 1), "copies": copies}
        if M > 1:
            fl = 2.0 * M * c.d_out * c.d_in
            line["tflops"] = round(fl / dt / 1e12, 2)
            line["pct_mfma_peak"] = round(100 * fl / dt / 1e12 / MFMA_F16_PEAK_TFLOPS, 2)
        print(json.dumps(line), flush=True)
        lines.append(line)
        del ps, base
        torch.cuda.empty_cache()
    return lines


def bench_decode(layers=36, ctx=1024, warmup=5, measure=10):
    """The synthetic end-to-end decode step (bit_vector_quantized_amd/decode_step.py): a
    Qwen3-4B-shaped stack of 36 decoder layers on SAGE-packed synthetic weights, a 1024-token
    context in the key/value caches, timed with the pages' protocol (SAGE paper App. A.2):
    5 warmup steps, then 10 steps each timed with GPU events, median. The step launches every
    kernel from Python (PyTorch attention around the libsage products), so it is also timed as
    one HIP graph replay of the same step (same position, checked bit for bit against the eager
    step) to separate the GPU time from the host's launch time."""
    import torch
    from bit_vector_quantized_amd import decode_step as ds
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20260)
    log(f"[decode] building {layers} synthetic layers")
    lws = [ds.random_layer(gen) for _ in range(layers)]
    packed = sum(packed_weight_bytes(getattr(lw, n)) for lw in lws
                 for n in ("q", "k", "v", "o", "gate", "up", "down"))
    stack = ds.DecodeStack(lws, ctx=ctx, max_new=warmup + measure + 8, gen=gen)
    h0 = (torch.randn(ds.QWEN3_4B.hidden, device="cuda", generator=gen) * 0.5).half()
    times, h = ds.time_steps(stack, h0, warmup, measure)
    eager_ms = ds.median(times)
    # the same step as one graph (fixed position); checked against the eager step
    pos = stack.pos
    h_in = h.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        stack.pos = pos
        stack.step(h_in)
        graph = torch.cuda.CUDAGraph()
        stack.pos = pos
        with torch.cuda.graph(graph, stream=side):
            h_graph = stack.step(h_in)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    stack.pos = pos
    h_eager = stack.step(h_in)
    graph_ok = True
    gtimes = []
    for i in range(warmup + measure):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        e1.synchronize()
        graph_ok = graph_ok and bool(torch.equal(h_graph, h_eager))
        if i >= warmup:
            gtimes.append(e0.elapsed_time(e1))
    graph_ms = ds.median(gtimes)
    line = {"workload": f"decode_step_qwen3_4b_{layers}_layers_ctx{ctx}",
            "protocol": f"{warmup} warmup steps, {measure} measured, median, GPU events",
            "tpot_ms_eager": round(eager_ms, 4), "tokens_per_s_eager": round(1e3 / eager_ms, 1),
            "tpot_ms_graph": round(graph_ms, 4) if graph_ok else None,
            "tokens_per_s_graph": round(1e3 / graph_ms, 1) if graph_ok else None,
            "graph_matches_eager": graph_ok,
            "packed_bytes_per_step": packed,
            "packed_gbs_graph": round(packed / (graph_ms * 1e-3) / 1e9, 1) if graph_ok else None,
            "eager_ms_all": [round(t, 4) for t in times],
            "finite": bool(torch.isfinite(h).all()),
            "data": "synthetic (device-random fields, seeded)"}
    print(json.dumps(line), flush=True)
    return line


def bench_encode(steps, warmup):
    """The fixed-codebook encoder on a 9728x2560 fp32 weight (synthetic: random permutation and
    positive position weights). Cost per subvector: for each of the K codewords 16 multiplies and
    14 adds (numerator and denominator of Eq. (6)), one square and one division, all float64."""
    import numpy as np
    import torch
    import workloads as W
    import bit_vector_quantized_amd as sage
    d_out, d_in = 9728, 2560
    rng = W.rng_for(160)
    Wm, e = W.encoder_matrix(rng, d_out, d_in)
    Wd = torch.from_numpy(Wm).cuda()
    pi = torch.from_numpy(W.draw_perm(rng, d_in)).cuda()
    om = torch.from_numpy(rng.lognormal(size=d_in)).cuda()
    n_sub = d_out * d_in // 8
    for K, V in ((16, 6), (64, 4), (256, 2)):
        cb = torch.from_numpy(W.draw_codebook(rng, K)).cuda()
        fn = lambda: sage.encode_fields(Wd, pi, om, cb, K.bit_length() - 1, V)
        for _ in range(max(1, warmup // 10)):
            fn()
        torch.cuda.synchronize()
        n = max(3, steps // 20)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        dt = e0.elapsed_time(e1) / 1e3 / n
        flops = n_sub * (K * 32 + 8)
        line = {"workload": f"encode_{d_out}x{d_in}_K{K}V{V}", "us_per_call": round(dt * 1e6, 1),
                "subvectors_per_s": round(n_sub / dt), "fp64_tflops": round(flops / dt / 1e12, 2),
                "pct_fp64_peak": round(100 * flops / dt / 1e12 / FP64_PEAK_TFLOPS, 1)}
        print(json.dumps(line), flush=True)


def bench_moe(steps, warmup):
    import numpy as np
    import torch
    import workloads as W
    import bit_vector_quantized_amd as sage
    log("[case] moe")
    moe = W.moe_layer(experts_to_build=range(128))
    packs = [[upload_pack(moe.experts[e][n]) for n in ("gate", "up", "down")] for e in range(128)]
    all_bytes = sum(packed_weight_bytes(p) for ex in packs for p in ex)
    copies = max(2, math.ceil(2 * MALL_BYTES / all_bytes) + 1)
    # every copy's matrices stay referenced here (and by their table) while any launch can run
    copy_packs = [packs] + [[[clone_packed(p) for p in ex] for ex in packs]
                            for _ in range(copies - 1)]
    tables = [sage.expert_table(cp, "cuda")[0] for cp in copy_packs]
    ids = torch.from_numpy(moe.ids).cuda()
    x = torch.from_numpy(moe.x).cuda()
    h = torch.from_numpy(np.ascontiguousarray(moe.h)).cuda()
    k = len(moe.ids)
    yg = torch.empty((k, W.MOE_INTER), dtype=torch.float16, device="cuda")
    yu = torch.empty_like(yg)
    yd = torch.empty((k, W.MOE_HIDDEN), dtype=torch.float16, device="cuda")
    ID, IH = W.MOE_INTER, W.MOE_HIDDEN
    # tables: gate|up pairs and down per copy (the layer as it runs: two launches, since down
    # reads silu(gate) * up), and all three per copy (one grouped launch, down on synthetic h)
    gu = [sage.expert_table([[ex[0], ex[1]] for ex in cp], "cuda")[0] for cp in copy_packs]
    dn = [sage.expert_table([ex[2] for ex in cp], "cuda")[0] for cp in copy_packs]

    def two_launches(i):
        sage.moe_gemv_grouped(gu[i], ids, [x, x], [0, 0], [yg.view(-1), yu.view(-1)], [ID, ID])
        sage.moe_gemv(dn[i], ids, h.view(-1), ID, yd.view(-1), IH)

    def one_launch(i):
        sage.moe_gemv_grouped(tables[i], ids, [x, x, h.view(-1)], [0, 0, ID],
                              [yg.view(-1), yu.view(-1), yd.view(-1)], [ID, ID, IH])

    def timed(fn):
        for i in range(warmup):
            fn(i % copies)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for i in range(copies):
                    fn(i)
        g.replay()
        torch.cuda.synchronize()
        reps = max(1, steps // copies)
        t0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / (reps * copies)

    dt2 = timed(two_launches)
    dt1 = timed(one_launch)
    routed = [packs[int(e)] for e in moe.ids]
    pb = sum(packed_weight_bytes(p) for ex in routed for p in ex)
    alg = sum(algorithmic_bytes(p) for ex in routed for p in ex)
    line = {"workload": "moe_qwen3_30b_a3b_top8_of_128",
            "us_per_layer_two_launches": round(dt2 * 1e6, 3),
            "us_per_call_one_grouped_launch": round(dt1 * 1e6, 3),
            "packed_gbs_one_launch": round(pb / dt1 / 1e9, 1),
            "effective_gbs_one_launch": round(alg / dt1 / 1e9, 1),
            "pct_hbm_peak_one_launch": round(100 * alg / dt1 / 1e9 / HBM_PEAK_GBS, 1),
            "packed_gbs_two_launches": round(pb / dt2 / 1e9, 1),
            "tokens_per_s": round(1.0 / dt2, 1), "copies": copies}
    print(json.dumps(line), flush=True)
    return line


# ------------------------------------------------------------------------------------------------

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the SAGE decode path here runs on a single MI355X)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import bit_vector_quantized_amd as sage
    sage.lib()  # fails loudly when the HIP library is missing

    if args.workload in ("sweep", "gemm", "prefill", "single", "all"):
        bench_single_products(args.workload, args.steps, args.warmup)
    if args.workload in ("moe", "all"):
        bench_moe(args.steps, args.warmup)
    if args.workload in ("encode", "all"):
        bench_encode(args.steps, args.warmup)
    if args.workload in ("decode", "all"):
        bench_decode()
    if args.workload != "layer":
        return

    if args.copy_calibration:
        src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] calibration copy: 268435456 bytes read, 268435456 bytes written")
        del src, dst
    log("[bench] building the decoder layer copies")
    bench = LayerBench(args.copies, args.steps, mode=args.mode)
    log(f"[bench] {len(bench.copies)} copies x {bench.bytes_per_layer} packed bytes; "
        f"timing {args.steps} steps after {args.warmup} warmup steps ({args.mode} decoding)")
    wall, durs = timed_graph(bench, args.steps, args.warmup, eager=args.eager)
    ms_per_step = wall * 1e3 / args.steps
    value = bench.bytes_per_layer / (ms_per_step * 1e-3) / 1e9
    dom_ms = sum(durs) / len(durs) if durs else None
    launch_us = {k: round(dominant_graph(bench, len(bench.copies), None, k)[0] * 1e3, 3)
                 for k, _, _ in LayerBench.LAUNCHES}
    other = LayerBench(args.copies, args.steps, mode="eager" if args.mode == "compiled" else "compiled")
    other_wall, _ = timed_graph(other, args.steps, args.warmup, dominant=False)
    other_ms = other_wall * 1e3 / args.steps
    other_launch_us = {k: round(dominant_graph(other, len(other.copies), None, k)[0] * 1e3, 3)
                       for k, _, _ in LayerBench.LAUNCHES}
    del other
    roofline = None
    if dom_ms:
        achieved = bench.dom_bytes / (dom_ms * 1e-3) / 1e9
        roofline = {"kernel": bench.dom_name,
                    "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": load_traffic(bench.dom_profile + "_" + args.mode),
                    "avg_launch_us": round(dom_ms * 1e3, 3),
                    "algorithmic_bytes_per_launch": bench.dom_bytes}
    line = {
        "metric": "batch-1 VQ GEMV effective packed-weight GB/s and % of HBM peak; tokens/s",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp16 (fp32 accumulate)",
        "data": "synthetic",
        "config": {"workload": "qwen3_4b_decoder_layer_batch1", "split_K_V": [64, 4],
                   "matrices": 7, "launches_per_step": bench.launches,
                   "decoding": args.mode,
                   "packed_bytes_per_step": bench.bytes_per_layer,
                   "weight_copies": len(bench.copies),
                   "timing": "eager" if args.eager else "hip_graph",
                   "launch_us": launch_us,
                   "source_digest": sage.source_digest(),
                   ("eager" if args.mode == "compiled" else "compiled") + "_decoding": {
                       "ms_per_step": round(other_ms, 5),
                       "packed_gbs": round(bench.bytes_per_layer / (other_ms * 1e-3) / 1e9, 1),
                       "launch_us": other_launch_us}},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(1e3 / ms_per_step, 1),
        "roofline": roofline,
        "cpu_baseline": None,
    }
    log("[bench] timing the per-launch floors")
    line["config"]["floors"] = launch_floors(bench)
    log("[bench] timing the streaming-read reference")
    ref = stream_reference(bench.dom_bytes)
    if roofline is not None:
        roofline["stream_read_reference"] = ref
        roofline["frac_of_stream_read"] = round(roofline["achieved"] / ref["gbs"], 4)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        line["cpu_baseline"] = cpu_baseline(bench.layer, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
