#!/usr/bin/env python3
"""Throughput of Transformer-XL relative-position memory attention on one MI355X.

One step = the whole hot path over one batch of synthetic input: for each of
S segments, each of N layers runs txl_layer_step (q/k/v/r projections over
[memory ; h], relative attention, output projection + residual + LayerNorm)
followed by txl_mem_update of that layer's memory.  Default workload: the
12-layer character model shape (batch 22, d_model 512, 8 heads of 64, segment
and memory length 512, 4 segments), bf16, every input resident in HBM before
the timed region.  Prints one JSON line.

value = query tokens per second through the N-layer stack = B * L * S / step time.
The attention kernel (the largest single kernel) is also timed on its own with
HIP events on the step's stream, on the last layer's real q/k/v/r, for the
roofline figure.  The CPU baseline is the fp64 oracle on the host cores.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "rel-pos memory attention fwd: query tokens/s + TFLOP/s vs bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
MI355X_XCDS, MI355X_SIMDS = 8, 1024   # accelerator dies; 256 CUs x 4 SIMDs
ATTN_SRC = os.path.join(ROOT, "relative_position_memory_amd", "csrc", "attn_mfma.hip")
WORKLOAD_NAMES = ("charlm", "wordlm", "large_eval", "large_train")


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="charlm", choices=WORKLOAD_NAMES + ("tiny",))
    p.add_argument("--attn-reps", type=int, default=50)
    p.add_argument("--attn-variant", type=int, default=0, choices=(0, 1, 2),
                   help="attention kernel (txl_attn_variant): 0 by shape, 1 the 64-query "
                        "kernel, 2 the 128-query kernel with key splits")
    p.add_argument("--streams", type=int, default=4,
                   help="HIP streams the stack's segments go round (txl_stack_fwd); 1 = serial")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--train", action="store_true",
                   help="time a training step (forward + backward, stop-gradient memory) at the "
                        "Large train-shape instead")
    p.add_argument("--main-only", action="store_true",
                   help="skip the cached-K/V stack and the feed-forward timing (profiling runs)")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle sample")
    p.add_argument("--eval-speed", action="store_true",
                   help="instead of the throughput line, print the per-token evaluation time "
                        "with memory against the vanilla recompute of the window (the pages' "
                        "Table 9 comparison) at attention lengths 800 .. 3800")
    p.add_argument("--vendor-sdpa", action="store_true",
                   help="instead of the throughput line, time this library's attention and "
                        "torch's fused scaled-dot-product attention (no position term) on the "
                        "same causal-over-memory pairs of the workload's shape")
    p.add_argument("--calib-copy", action="store_true",
                   help="also run a plain 256 MiB device copy (reads 256 MiB, writes 256 MiB) "
                        "so that a counter run can calibrate FETCH_SIZE / WRITE_SIZE")
    p.add_argument("--no-drift", action="store_true",
                   help="skip the deep-stack bf16 drift report (batch row 0 against the oracle)")
    p.add_argument("--traffic-summary", nargs=3, metavar=("WORKLOAD", "FETCH_CSV", "WRITE_CSV"),
                   help="print the attention's HBM traffic summary from two rocprofv3 --pmc "
                        "runs (FETCH_SIZE, WRITE_SIZE) of bench.py --calib-copy")
    p.add_argument("--trace-summary", nargs="+", metavar="CSV",
                   help="print the per-kernel table of a rocprofv3 --kernel-trace --stats run")
    p.add_argument("--pmc-summary", nargs="+", metavar="CSV",
                   help="no GPU work: summarise rocprofv3 --pmc counter CSVs (per kernel: "
                        "MFMA busy fraction, bf16 MFMA FLOPs, HBM bytes) and exit")
    return p.parse_args()


def attn_flops(w):
    """Algorithmic FLOPs of one attention call: 6 d per causal (query, key) pair
    (q.k, (q+v).r and p.v), P = L*M + L(L+1)/2 pairs per (batch, head)."""
    P = w.L * w.M + w.L * (w.L + 1) // 2
    return 6 * w.d * P * w.B * w.H


def attn_bytes(w):
    """Algorithmic HBM bytes of one attention call: q, out, k, v and r once each."""
    es = 2 if w.dtype == "bf16" else 4
    T = w.M + w.L
    return es * (2 * w.B * w.L * w.H * w.d + 2 * w.B * T * w.H * w.d + T * w.H * w.d)


def attn_bound(w):
    """The roofline that bounds the attention at this shape: whichever ideal time
    (FLOPs at the bf16 MFMA peak, bytes at the HBM peak) is longer."""
    t_mfma = attn_flops(w) / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = attn_bytes(w) / (PEAK_HBM_GBS * 1e9)
    return "mfma" if t_mfma >= t_hbm else "hbm"


def layer_flops(w):
    T = w.M + w.L
    HD = w.H * w.d
    gemm = 2 * (w.B * w.L * HD * w.D + w.B * T * 2 * HD * w.D + T * HD * w.D
                + w.B * w.L * w.D * HD)
    return gemm + attn_flops(w)


def layer_bwd_flops(w):
    """Algorithmic FLOPs of one layer's backward (txl_layer_step_bwd) with its
    forward recompute: the forward (layer_flops), then per projection y = x W^T
    the two products dX = dY W and dW = dY^T X (dX only for the current rows: the
    memory's gradient is stopped; none for R), and the attention backward at 16 d
    per causal pair (scores' content and position terms, dP, dV, dq's two terms,
    dk, dr)."""
    T = w.M + w.L
    HD = w.H * w.d
    BL = w.B * w.L
    dW = 2 * (BL * HD * w.D + 2 * w.B * T * HD * w.D + T * HD * w.D + BL * w.D * HD)
    dX = 2 * (BL * HD * w.D + 2 * BL * HD * w.D + BL * w.D * HD)
    P = w.L * w.M + w.L * (w.L + 1) // 2
    return layer_flops(w) + dW + dX + 16 * w.d * P * w.B * w.H


def cpu_baseline_train(w, x, target_s):
    """The backward oracle, as it stands, on the host cores: one layer's forward +
    backward (oracle_bwd.layer_step_bwd) on a sample of the batch rows, scaled to
    query tokens/s of the training step (every layer once per segment)."""
    import numpy as np
    from oracle import oracle as O
    from oracle import oracle_bwd as OB
    g = np.random.default_rng(1).standard_normal((w.B, w.L, w.D))

    def run(b, n):
        t0 = time.perf_counter()
        for r in range(n):
            Wl = x["weights"][r % len(x["weights"])]
            OB.layer_step_bwd(x["h0"][0][:b], x["mem"][0][:b], Wl, x["u"], x["v"], x["R"],
                              g[:b])
        return time.perf_counter() - t0

    t1 = run(1, 1)
    n = max(1, int(round(target_s / max(t1, 1e-3))))
    t = run(1, n) if n > 1 else t1
    return {
        "value": n * w.L / (t * w.n_layers),
        "unit": "query tokens/s",
        "cores": O.num_threads(),
        "kind": "oracle",
        "sample": (f"{n} fp64 layer forward + backward passes (oracle_bwd.layer_step_bwd) over "
                   f"1 of the {w.B} batch rows at full memory ({w.M} rows), {t:.1f} s in all; "
                   f"rate scaled by 1/{w.n_layers} layers to match the stack"),
    }


def traffic_file(workload):
    return os.path.join(ROOT, "profiles", f"attn_mfma_{workload}_traffic.txt")


def read_traffic(workload):
    """HBM bytes per attention launch at this workload from the committed rocprofv3
    counter summary, or None when there is none or the kernel source changed since
    the counters were taken."""
    try:
        kv = {}
        for ln in open(traffic_file(workload)):
            if ":" in ln and not ln.startswith("#"):
                k, v = ln.split(":", 1)
                kv[k.strip()] = v.strip()
        sha = hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()
        if kv.get("kernel_source_sha256") != sha:
            return None
        return float(kv["hbm_bytes_per_dispatch"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_info():
    """CPU model and core counts of the host that runs the oracle."""
    model = None
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"cpu_model": model, "nproc": usable, "cpu_count": os.cpu_count()}


def cpu_baseline(w, x, target_s):
    """The oracle, as it stands, on the host cores: one layer step on a sample of
    the batch rows, scaled to query tokens/s through the N-layer stack (all
    threads, the headline), then the same on one thread, then the attention
    alone (oracle rel_attn at the workload's shape) on all threads.  The oracle
    is compiled with -O3 -march=native on this host first."""
    from oracle import oracle as O
    from relative_position_memory_amd import inputs as I
    flags = O.use_native_build()
    threads = O.num_threads()

    def run(b, n):
        t0 = time.perf_counter()
        for r in range(n):
            Wl = x["weights"][r % len(x["weights"])]
            O.layer_step(x["h0"][0][:b], x["mem"][0][:b], Wl, x["u"], x["v"], x["R"])
        return time.perf_counter() - t0

    def sample(budget, b_max):
        t1 = run(1, 1)
        b = max(1, min(b_max, int(budget / max(t1, 1e-3))))
        tb = run(b, 1) if b > 1 else t1
        n = max(1, int(round(budget / max(tb, 1e-3))))
        t = run(b, n) if n > 1 else tb
        return b, n, t

    b, n, t = sample(target_s * 0.6, w.B)
    res = {
        "value": n * b * w.L / (t * w.n_layers),
        "unit": "query tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{n} fp64 layer steps (projections, attention, LayerNorm) over {b} of the "
                   f"{w.B} batch rows at full memory ({w.M} rows), {t:.1f} s in all on {threads} "
                   f"threads; rate scaled by 1/{w.n_layers} layers to match the stack"),
        "build": f"gcc {flags}",
    }
    res.update(cpu_info())
    O.set_num_threads(1)
    try:
        b1, n1, t1 = sample(target_s * 0.2, w.B)
    finally:
        O.set_num_threads(threads)
    res["single_thread"] = {"value": n1 * b1 * w.L / (t1 * w.n_layers), "unit": "query tokens/s",
                            "sample": f"{n1} layer steps over {b1} batch rows, {t1:.1f} s, 1 thread"}
    # attention alone: the oracle's rel_attn over batch rows of the workload's shape
    c = I.attention_inputs(1, w.H, w.L, w.M, w.d, seed=0, sigma=1.0, sigma_uv=0.1)
    t0 = time.perf_counter()
    O.rel_attn(c["q"], c["k"], c["v"], c["r"], c["u"], c["vb"], w.M)
    ta = time.perf_counter() - t0
    na = max(1, int(round(target_s * 0.2 / max(ta, 1e-3))))
    if na > 1:
        t0 = time.perf_counter()
        for _ in range(na):
            O.rel_attn(c["q"], c["k"], c["v"], c["r"], c["u"], c["vb"], w.M)
        ta = (time.perf_counter() - t0) / na
    row_flops = attn_flops(w) / w.B
    res["attention_alone"] = {
        "query_tokens_per_s": w.L / ta, "gflops": row_flops / ta / 1e9,
        "ms_per_call_full_batch": ta * w.B * 1e3,
        "sample": f"{na} oracle rel_attn calls on 1 batch row ({w.H} heads, L {w.L}, memory "
                  f"{w.M}), {ta * 1e3:.1f} ms each on {threads} threads; full batch = x{w.B}"}
    return res


def pos_ff_time(w, reps, stream):
    """txl_pos_ff over the B*L rows of a segment (d_inner = 4 d_model), HIP events."""
    import numpy as np
    import torch
    from relative_position_memory_amd import txl
    rows, D, Di = w.B * w.L, w.D, 4 * w.D
    rng = np.random.default_rng(3)
    t = lambda shape, std: torch.from_numpy(
        (rng.standard_normal(shape) * std).astype(np.float32)).to(torch.bfloat16).cuda()
    x = t((rows, D), 1.0)
    W1, b1, W2, b2 = t((Di, D), D ** -0.5), t((Di,), 0.1), t((D, Di), Di ** -0.5), t((D,), 0.1)
    g, b = torch.ones(D, dtype=torch.bfloat16).cuda(), torch.zeros(D, dtype=torch.bfloat16).cuda()
    out = torch.empty_like(x)
    ws = torch.empty(txl.pos_ff_workspace_bytes(rows, D, Di, x.dtype), dtype=torch.uint8,
                     device="cuda")
    run = lambda: txl.pos_ff(x, W1, b1, W2, b2, g, b, out, ws, stream=stream)
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / reps * 1e3
    flop = 2.0 * 2 * rows * D * Di
    return {"rows": rows, "d_model": D, "d_inner": Di, "launch_us": us,
            "achieved": flop / (us * 1e-6) / 1e12, "unit": "TFLOP/s",
            "frac": flop / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS}


def kv_stack_ms(w, x, Ws, lws, u, vb, R, h0, steps, warmup, stream, n_streams=1):
    """ms per step of the stack run with txl_layer_step_kv, on the stack's segment
    schedule: segment s on stream s % n_streams, layer n of segment s waiting for
    layer n of segment s - 1 (which appended to the same key/value ring)."""
    import torch
    from relative_position_memory_amd import txl
    tdt = h0.dtype
    dims = txl.layer_dims(w.B, w.L, w.D, w.H, w.d)
    dims_m = txl.layer_dims(w.B, w.M, w.D, w.H, w.d)
    rs = [txl.pos_proj(dims, R, Wl["W_kR"], stream=stream) for Wl in Ws]
    rings = []
    nws = max(txl.kv_workspace_bytes(dims, w.M, tdt), txl.kv_workspace_bytes(dims_m, w.M, tdt))
    wss = [torch.empty(nws, dtype=torch.uint8, device="cuda") for _ in range(n_streams)]
    for n, Wl in enumerate(Ws):
        kv, kb, vbuf = txl.make_kv_ring(dims, w.M, tdt, capacity=w.M + max(w.L, w.M))
        kv.mem_max = w.M
        m = torch.from_numpy(x["mem"][n]).to(tdt).cuda()
        # prefill: the initial memory rows as one segment over an empty memory
        txl.layer_step_kv(dims_m, m, kv, Wl, u, vb, rs[n], torch.empty_like(m), wss[0],
                          stream=stream)
        rings.append((kv, kb, vbuf))
    streams = [stream] + [torch.cuda.Stream() for _ in range(n_streams - 1)]
    bufs = [[torch.empty((w.B, w.L, w.D), dtype=tdt, device="cuda") for _ in range(2)]
            for _ in range(n_streams)]

    def step():
        done = [[None] * w.n_layers for _ in range(2)]
        start = torch.cuda.Event()
        start.record(stream)
        for st in streams[1:]:
            st.wait_event(start)
        for s_ in range(w.n_segments):
            k = s_ % n_streams
            st = streams[k]
            h = h0[s_]
            for n in range(w.n_layers):
                if n_streams > 1 and s_ > 0:
                    st.wait_event(done[(s_ - 1) % 2][n])
                out = bufs[k][n % 2]
                txl.layer_step_kv(dims, h, rings[n][0], lws[n], u, vb, rs[n], out, wss[k],
                                  stream=st)
                if n_streams > 1:
                    ev = torch.cuda.Event()
                    ev.record(st)
                    done[s_ % 2][n] = ev
                h = out
        for st in streams[1:]:
            fin = torch.cuda.Event()
            fin.record(st)
            stream.wait_event(fin)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def train_runner(w, x, streams):
    """The training step's work over all segments of workload w, on one stream or
    two (streams: a list of one or two torch streams).  Per segment: the forward
    through every layer (txl_layer_step_save), then the backward from the top
    (txl_layer_step_bwd_saved; the upstream gradient of the top layer is a fixed
    synthetic tensor, the gradient of each layer's input feeds the layer below).
    The memory of segment s + 1 at layer n is the last M rows of segment s's
    memory and input there ([XL] section 3.2).

    With two streams the backward of segment s runs on the second stream while the
    forward of segment s + 1 runs on the first (stop-gradient memory: the forward
    of s + 1 needs segment s's hidden states, not its gradients).  Activations,
    saved states and rings are held twice (segment parity); the forward of segment
    s waits for the backward of segment s - 2, the last reader of its parity's
    buffers, and segment s's rings are built at the top of each of its layers
    (a copy of segment s - 1's ring and txl_mem_update), beside the backward of
    s - 1, which reads the same data.  Returns (step, grads, outputs)."""
    import numpy as np
    import torch
    from relative_position_memory_amd import txl

    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(tdt).cuda()
    Ws = [{k: dev(v) for k, v in lw.items()} for lw in x["weights"]]
    lws = [txl.layer_weights(Wl) for Wl in Ws]
    u, vb, R = dev(x["u"]), dev(x["v"]), dev(x["R"])
    h0 = dev(x["h0"])
    dims = txl.layer_dims(w.B, w.L, w.D, w.H, w.d)
    N, S = w.n_layers, w.n_segments
    mem0 = [dev(m) for m in x["mem"]]
    ring_data = [[m.clone() for m in mem0], [m.clone() for m in mem0]]
    rings = [[txl.make_ring(dd, 0, w.M) for dd in ring_data[p]] for p in range(2)]
    bws = torch.empty(txl.layer_bwd_workspace_bytes(dims, w.M, tdt), dtype=torch.uint8,
                      device="cuda")
    nsv = txl.layer_saved_bytes(dims, w.M, tdt)
    sbufs = [[torch.empty(nsv, dtype=torch.uint8, device="cuda") for _ in range(N)]
             for _ in range(2)]
    saved = [[None] * N for _ in range(2)]
    hs = [[torch.empty((w.B, w.L, w.D), dtype=tdt, device="cuda") for _ in range(N + 1)]
          for _ in range(2)]
    rng = np.random.default_rng(1)
    g_top = dev(rng.standard_normal((w.B, w.L, w.D)).astype(np.float32))
    g_cur = torch.empty((w.B, w.L, w.D), dtype=tdt, device="cuda")
    outputs = torch.empty((S, w.B, w.L, w.D), dtype=tdt, device="cuda")
    # lws holds raw pointers into Ws: the weight tensors live as long as the step
    box = {"grads": None, "weights": Ws}
    F = streams[0]
    Bk = streams[1] if len(streams) > 1 else streams[0]

    def step():
        # a step starts from the initial memories, so that every step does the same work
        for n in range(N):
            rings[0][n].start, rings[0][n].len = 0, w.M
        with torch.cuda.stream(F):
            for n in range(N):
                ring_data[0][n].copy_(mem0[n])
        bwd_done = [None] * S
        start = torch.cuda.Event()
        start.record(F)
        Bk.wait_stream(F) if Bk is not F else None
        for s in range(S):
            p, q = s % 2, (s - 1) % 2
            if s >= 2 and Bk is not F:
                F.wait_event(bwd_done[s - 2])
            with torch.cuda.stream(F):
                hs[p][0].copy_(h0[s])
                for n in range(N):
                    if s > 0:  # this segment's memory at layer n
                        ring_data[p][n].copy_(ring_data[q][n])
                        rings[p][n].start, rings[p][n].len = rings[q][n].start, rings[q][n].len
                        txl.mem_update(rings[p][n], hs[q][n], stream=F)
                    saved[p][n] = txl.layer_step_save(dims, hs[p][n], rings[p][n], lws[n], u,
                                                      vb, R, hs[p][n + 1], sbufs[p][n], stream=F)
                outputs[s].copy_(hs[p][N])
            fwd_done = torch.cuda.Event()
            fwd_done.record(F)
            if Bk is not F:
                Bk.wait_event(fwd_done)
            with torch.cuda.stream(Bk):
                g = g_top
                for n in reversed(range(N)):
                    box["grads"] = txl.layer_step_bwd(dims, hs[p][n], rings[p][n], lws[n], u, vb,
                                                      R, g, bws, grads=box["grads"], stream=Bk,
                                                      saved=saved[p][n])
                    g_cur.copy_(box["grads"]["dh"])  # the next layer down takes dh in the layers' dtype
                    g = g_cur
            ev = torch.cuda.Event()
            ev.record(Bk)
            bwd_done[s] = ev
        if Bk is not F:
            F.wait_event(bwd_done[S - 1])
    return step, box, outputs, (dims, hs, rings, lws, u, vb, R, g_top, bws)


def train_step(args):
    """Training step with a stop-gradient memory ([XL] section 3.2) at the Large
    train-shape (batch 8, d_model 1024, 16 heads of 64, L = M = 384, 18 layers,
    4 segments, bf16): every segment's forward and backward through the stack
    (train_runner), the backward of a segment beside the next segment's forward on
    a second stream.  The weight gradients are written per layer (no optimizer
    update is part of the step).  value = B * L * segments / step time."""
    import torch
    from relative_position_memory_amd import inputs as I
    from relative_position_memory_amd import txl

    w = I.workload("large_train")
    x = I.make_inputs(w, seed=0)
    stream = torch.cuda.current_stream()
    streams = [stream, torch.cuda.Stream()] if args.streams > 1 else [stream]
    step, box, outputs, (dims, hs, rings, lws, u, vb, R, g_top, bws) = train_runner(w, x, streams)

    def timed(fn, steps, warmup):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    steps = max(1, min(args.steps, 3))
    ms = timed(step, steps, max(args.warmup, 1))
    if len(streams) > 1:
        step1, _, _, _ = train_runner(w, x, [stream])
        ms_serial = timed(step1, 1, 1)
    else:
        ms_serial = ms
    # one layer's backward alone, with its forward recomputed (txl_layer_step_bwd),
    # HIP events on the same stream
    grads = box["grads"]
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b0.record(stream)
    for _ in range(5):
        txl.layer_step_bwd(dims, hs[0][0], rings[0][0], lws[0], u, vb, R, g_top, bws, grads=grads,
                           stream=stream)
    b1.record(stream)
    torch.cuda.synchronize()
    bwd_ms = b0.elapsed_time(b1) / 5
    bwd_tflops = layer_bwd_flops(w) / (bwd_ms / 1e3) / 1e12
    tokens = w.B * w.L * w.n_segments
    res = {
        "metric": "training step (forward + backward, stop-gradient memory): query tokens/s",
        "value": tokens / (ms / 1e3), "unit": "query tokens/s", "n_gpus": 1, "steps": steps,
        "ms_per_step": ms, "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "large_train: 18 layers x 4 segments, forward + backward",
                   "batch": w.B, "d_model": w.D, "n_head": w.H, "d_head": w.d,
                   "segment_len": w.L, "mem_len": w.M, "n_layers": w.n_layers,
                   "n_segments": w.n_segments},
        "schedule": {"streams": len(streams), "serial_ms_per_step": ms_serial,
                     "note": "the backward of segment s beside the forward of segment s+1"},
        "layer_bwd_ms": bwd_ms,
        "roofline": {"bound": "mfma", "kernel": "txl_layer_step_bwd (one layer, all kernels)",
                     "achieved": bwd_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": bwd_tflops / PEAK_BF16_TFLOPS, "traffic": None,
                     "flop_per_call": layer_bwd_flops(w)},
        "note": "forward = txl_layer_step_save, backward = txl_layer_step_bwd_saved per layer "
                "(no recompute); layer_bwd_ms and the roofline time txl_layer_step_bwd, which "
                "recomputes the layer's forward; the upstream gradient of the top layer is "
                "synthetic; no optimizer update"}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_train(w, x, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def vendor_sdpa(args):
    """Context for the attention kernel: torch's fused attention (the vendor
    stack's flash / memory-efficient kernels, selected explicitly so that no
    unfused fallback runs) on the same (query, key) pairs -- L queries over
    M + L keys, query i seeing keys 0 .. M + i -- but without the position term,
    against txl_rel_attn_fwd with it, both bf16 with HIP events.  Rates are given
    per causal pair, since the two compute different amounts per pair."""
    import numpy as np
    import torch
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel
    from torch.nn.attention.bias import causal_lower_right
    from relative_position_memory_amd import inputs as I
    from relative_position_memory_amd import txl

    w = I.workload(args.workload)
    B, H, L, M, d = w.B, w.H, w.L, w.M, w.d
    T = M + L
    pairs = (L * M + L * (L + 1) // 2) * B * H
    rng = np.random.default_rng(0)
    bf = lambda *shape: torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(
        torch.bfloat16).cuda()
    q, k, v, r = bf(B, L, H, d), bf(B, T, H, d), bf(B, T, H, d), bf(T, H, d)
    u, vb = bf(H, d) * 0.1, bf(H, d) * 0.1
    out = torch.empty_like(q)
    nws = txl.rel_attn_workspace_bytes(torch.bfloat16, B, H, L, M, d)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda") if nws else None
    qh, kh, vh = (x.transpose(1, 2).contiguous() for x in (q, k, v))  # [B, H, rows, d]
    mask = causal_lower_right(L, T)

    def timed(fn, reps):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3

    res = {"workload": w.name, "batch": B, "n_head": H, "d_head": d, "segment_len": L,
           "mem_len": M, "causal_pairs": pairs}
    us = timed(lambda: txl.rel_attn_fwd(q, k, v, r, u, vb, M, out, workspace=ws), args.attn_reps)
    res["txl_rel_attn_fwd"] = {"us": us, "Gpairs_per_s": pairs / us / 1e3,
                               "note": "content and position terms, bf16 MFMA"}
    for name, be in (("sdpa_flash", SDPBackend.FLASH_ATTENTION),
                     ("sdpa_efficient", SDPBackend.EFFICIENT_ATTENTION)):
        try:
            with sdpa_kernel([be]):
                us = timed(lambda: F.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask),
                           args.attn_reps)
            res[name] = {"us": us, "Gpairs_per_s": pairs / us / 1e3,
                         "note": "content term only (no position term, no biases)"}
        except RuntimeError as ex:  # backend not built for this shape or device
            res[name] = {"unavailable": str(ex)[:200]}
    print(json.dumps(res), flush=True)


def eval_speed(args):
    """Per-token evaluation time with memory against the vanilla model that
    recomputes the whole window for every prediction ([XL] section 4.5, Table 9):
    the long-memory evaluation shape (d_model 1024, 16 heads of 64, 18 layers),
    one sequence, attention lengths 800 .. 3800.  Three ways per length:
      vanilla      txl_layer_step over the attn_len tokens of the window with an
                   empty memory, every layer: the cost of one prediction;
      state reuse  one new token (L = 1) over a memory of attn_len - 1 cached
                   hidden states, re-projected every step (txl_layer_step), plus
                   the memory update;
      kv cache     one new token over cached keys and values (txl_layer_step_kv)."""
    import numpy as np
    import torch
    from relative_position_memory_amd import inputs as I
    from relative_position_memory_amd import txl

    w = I.workload("large_eval")
    lens = [800, 1800, 2800, 3800]
    rng = np.random.default_rng(0)
    tdt = torch.bfloat16
    HD = w.H * w.d

    def normal(shape, std):
        return torch.from_numpy((rng.standard_normal(shape) * std).astype(np.float32)).to(
            tdt).cuda()

    Ws = [{"W_q": normal((HD, w.D), 0.02), "W_kE": normal((HD, w.D), 0.02),
           "W_v": normal((HD, w.D), 0.02), "W_kR": normal((HD, w.D), 0.02),
           "W_o": normal((w.D, HD), 0.02), "gamma": torch.ones(w.D, dtype=tdt).cuda(),
           "beta": torch.zeros(w.D, dtype=tdt).cuda()} for _ in range(w.n_layers)]
    lws = [txl.layer_weights(Wl) for Wl in Ws]
    u, vb = normal((w.H, w.d), 0.02), normal((w.H, w.d), 0.02)
    R = torch.from_numpy(I.sinusoid_table(max(lens), w.D)).to(tdt).cuda()
    stream = torch.cuda.current_stream()

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    rows = []
    for n_att in lens:
        M = n_att - 1
        # vanilla: the whole window, empty memory
        dv = txl.layer_dims(1, n_att, w.D, w.H, w.d)
        wsv = torch.empty(txl.workspace_bytes(dv, 1, tdt), dtype=torch.uint8, device="cuda")
        hv = normal((1, n_att, w.D), 1.0)
        ov = [torch.empty_like(hv) for _ in range(2)]
        empty = txl.make_ring(torch.zeros((1, 1, w.D), dtype=tdt, device="cuda"), 0, 0)

        def vanilla():
            h = hv
            for n in range(w.n_layers):
                txl.layer_step(dv, h, empty, lws[n], u, vb, R, ov[n % 2], wsv, stream=stream)
                h = ov[n % 2]
        t_van = timed(vanilla, 3)
        # state reuse: L = 1 over attn_len - 1 cached hidden states per layer
        d1 = txl.layer_dims(1, 1, w.D, w.H, w.d)
        ws1 = torch.empty(txl.workspace_bytes(d1, M, tdt), dtype=torch.uint8, device="cuda")
        mems = [normal((1, M, w.D), 1.0) for _ in range(w.n_layers)]
        rings = [txl.make_ring(m, 0, M) for m in mems]
        h1 = normal((1, 1, w.D), 1.0)
        o1 = [torch.empty_like(h1) for _ in range(2)]

        def reuse():
            h = h1
            for n in range(w.n_layers):
                txl.layer_step(d1, h, rings[n], lws[n], u, vb, R, o1[n % 2], ws1, stream=stream)
                txl.mem_update(rings[n], h, stream=stream)
                h = o1[n % 2]
        t_reuse = timed(reuse, 20)
        # cached keys and values
        rs = [txl.pos_proj(d1, R[:n_att], Wl["W_kR"], stream=stream) for Wl in Ws]
        kvs = []
        for _ in range(w.n_layers):
            kv, kb, vbuf = txl.make_kv_ring(d1, M, tdt)
            kb.zero_()
            vbuf.zero_()
            kv.len = M
            kvs.append((kv, kb, vbuf))
        wsk = torch.empty(txl.kv_workspace_bytes(d1, M, tdt), dtype=torch.uint8, device="cuda")

        def kvstep():
            h = h1
            for n in range(w.n_layers):
                txl.layer_step_kv(d1, h, kvs[n][0], lws[n], u, vb, rs[n], o1[n % 2], wsk,
                                  stream=stream)
                h = o1[n % 2]
        t_kv = timed(kvstep, 20)
        rows.append({"attn_len": n_att, "vanilla_ms_per_token": t_van,
                     "state_reuse_ms_per_token": t_reuse, "kv_cache_ms_per_token": t_kv,
                     "speedup_state_reuse": t_van / t_reuse, "speedup_kv_cache": t_van / t_kv})
        print(f"# attn_len {n_att}: vanilla {t_van:.3f} ms, state reuse {t_reuse:.3f} ms, "
              f"kv cache {t_kv:.3f} ms per token", file=sys.stderr, flush=True)
    print(json.dumps({
        "metric": "evaluation time per token: memory vs vanilla window recompute",
        "unit": "ms per token", "higher_is_better": False, "dtype": "bf16",
        "data": "synthetic, random-init weights",
        "config": {"workload": "long-memory evaluation shape without feed-forward",
                   "batch": 1, "d_model": w.D, "n_head": w.H, "d_head": w.d,
                   "n_layers": w.n_layers},
        "rows": rows,
        "pages_table9_speedup": {"3800": 1874, "2800": 1409, "1800": 773, "800": 363},
        "note": "the pages' speed-ups are ratios on their own hardware and full models; "
                "context, not a target"}), flush=True)


def hip_time_us(fn, reps, stream):
    """Average time of fn() in us over reps back-to-back calls, HIP events on stream."""
    import torch
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps * 1e3


def stack_drift(w, x, lws, u, vb, R, dims, ws, tdt, stream, segments):
    """Deep-stack bf16 drift, reported and not gated: the stack (every layer, the
    first `segments` segments, memory updates) from the initial memory on the
    GPU, and the oracle's fp64 recurrence on batch row 0 (batch rows are
    independent).  Max-abs difference of the top layer's output per segment."""
    import numpy as np
    import torch
    from oracle import oracle as O
    from relative_position_memory_amd import txl
    dev = lambda a: torch.from_numpy(a).to(tdt).cuda()
    datas = [dev(m) for m in x["mem"]]
    rings = [txl.make_ring(dd, 0, w.M) for dd in datas]
    bufs = [torch.empty((w.B, w.L, w.D), dtype=tdt, device="cuda") for _ in range(2)]
    gpu_top = []
    for s_ in range(segments):
        h = dev(x["h0"][s_])
        for n in range(w.n_layers):
            out = bufs[n % 2]
            txl.layer_step(dims, h, rings[n], lws[n], u, vb, R, out, ws, stream=stream)
            txl.mem_update(rings[n], h, stream=stream)
            h = out
        gpu_top.append(h[:1].float().cpu().numpy().astype(np.float64))
    mems = [m[:1] for m in x["mem"]]
    per_seg = []
    t0 = time.perf_counter()
    for s_ in range(segments):
        h = x["h0"][s_][:1].astype(np.float64)
        for n in range(w.n_layers):
            out = O.layer_step(h, mems[n], x["weights"][n], x["u"], x["v"], x["R"])
            mems[n] = O.mem_update(mems[n], h, w.M)
            h = out
        per_seg.append(float(np.abs(gpu_top[s_] - h).max()))
    return {"max_abs_per_segment": per_seg, "layers": w.n_layers, "segments": segments,
            "rows": f"batch row 0, all {w.L} positions, top layer output",
            "oracle_s": time.perf_counter() - t0,
            "note": "reported, not gated: the oracle runs fp64 throughout, the GPU stores every "
                    "layer's output and memory in bf16 (half an ulp of |x| in [4, 8) is 0.0156)"}


def pmc_summary(paths):
    """Per-kernel summary of rocprofv3 --pmc CSVs (kernel-serialised counters, one
    row per dispatch and counter, each the sum over the counter's hardware
    instances).  MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES (matrix-core cycles summed over
    all SIMDs: 16 per 16x16x32 and 32 per 32x32x16 bf16 instruction) / (the kernel's
    busy cycles x 1024 SIMDs), the kernel's busy cycles being GRBM_GUI_ACTIVE / 8
    (one instance per XCD); bf16 MFMA FLOPs = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512;
    FETCH_SIZE / WRITE_SIZE in KiB."""
    import collections
    import csv
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in paths:
        per_dispatch = collections.defaultdict(dict)
        for r in csv.DictReader(open(path)):
            key = (r["Kernel_Name"], r["Grid_Size"])
            per_dispatch[(key, r.get("Dispatch_Id", r.get("Correlation_Id", "")))][
                r["Counter_Name"]] = float(r["Counter_Value"])
        for (key, _), cs in per_dispatch.items():
            for c, v in cs.items():
                agg[key][c].append(v)
    print(f"{'kernel':58s} {'grid':>9s} {'n':>4s}  counters (mean per dispatch)")
    for (name, grid), cs in sorted(agg.items(), key=lambda kv: -len(kv[1])):
        mean = {c: sum(v) / len(v) for c, v in cs.items()}
        n = max(len(v) for v in cs.values())
        parts = [f"{c}={m:.4g}" for c, m in sorted(mean.items())]
        if "SQ_VALU_MFMA_BUSY_CYCLES" in mean and mean.get("GRBM_GUI_ACTIVE"):
            busy = mean["GRBM_GUI_ACTIVE"] / MI355X_XCDS
            parts.append(f"busy_us={busy / 2.4e3:.1f}")
            parts.append(f"MFMA_busy={mean['SQ_VALU_MFMA_BUSY_CYCLES'] / (busy * MI355X_SIMDS):.3f}")
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in mean:
            parts.append(f"bf16_MFMA_GFLOP={mean['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512 / 1e9:.3f}")
        print(f"{name[:58]:58s} {grid:>9s} {n:4d}  " + "  ".join(parts))


def _pmc_per_dispatch(path, counter):
    """{(kernel name, grid size): [counter value per dispatch]} of a --pmc CSV."""
    import collections
    import csv
    out = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            out[(r["Kernel_Name"], r["Grid_Size"])].append(float(r["Counter_Value"]))
    return out


def traffic_summary(workload, fetch_csv, write_csv):
    """HBM bytes per attention launch (attn_mfma_kernel or attn_q64_kernel, plus
    attn_part_merge_kernel when the plan splits keys) from FETCH_SIZE and WRITE_SIZE (KiB per dispatch),
    each scaled by what the same counter reads for the 256 MiB device copy that
    --calib-copy adds to the run."""
    fetch = _pmc_per_dispatch(fetch_csv, "FETCH_SIZE")
    write = _pmc_per_dispatch(write_csv, "WRITE_SIZE")
    copy_kib = float(64 << 20) * 4 / 1024
    mean = lambda v: sum(v) / len(v)

    def calib(tab):
        for (name, grid), v in tab.items():
            if "copyBuffer" in name and int(grid) * 2048 == 64 << 22:  # 256 MiB / 2 KiB per item
                return mean(v)
        cand = [mean(v) for (name, _), v in tab.items() if "copyBuffer" in name]
        return max(cand)
    cf, cw = calib(fetch), calib(write)
    fs, wsc = copy_kib / cf, copy_kib / cw

    def kern(tab, key):
        hits = [(n, g, v) for (n, g), v in tab.items() if key in n]
        if not hits:
            return 0, 0.0
        n, g, v = max(hits, key=lambda t: len(t[2]))
        return len(v), mean(v)
    # the attention kernel the workload runs (the 128- or the 64-query one)
    akey = max(("attn_mfma_kernel", "attn_q64_kernel"), key=lambda k: kern(fetch, k)[0])
    na_f, af = kern(fetch, akey)
    na_w, aw = kern(write, akey)
    nm_f, mf = kern(fetch, "attn_part_merge_kernel")
    nm_w, mw = kern(write, "attn_part_merge_kernel")
    hbm = (af * fs + aw * wsc + mf * fs + mw * wsc) * 1024
    from relative_position_memory_amd import inputs as I
    w = I.workload(workload)
    src = os.path.relpath(ATTN_SRC, ROOT)
    sha = hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()
    R = "$R"
    cmd = (f"python3 {R}/bench.py --workload {workload} --steps 1 --warmup 0 --no-cpu-baseline "
           f"--main-only --attn-reps 3 --calib-copy")
    lines = [
        f"# HBM traffic of the attention ({w.name}: B {w.B}, H {w.H}, d {w.d}, L {w.L}, "
        f"M {w.M}, {w.dtype}) per launch",
        "# counter pass 1 (run from /tmp with TMPDIR=/tmp, repo root $R, output folder $OUT):",
        f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/pmc_fetch_{workload} "
        f"-o run -- {cmd}",
        "# counter pass 2:",
        f"#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/pmc_write_{workload} "
        f"-o run -- {cmd}",
        "# summary: python3 bench.py --traffic-summary " + workload +
        f" $OUT/pmc_fetch_{workload}/run_counter_collection.csv"
        f" $OUT/pmc_write_{workload}/run_counter_collection.csv",
        "# FETCH_SIZE / WRITE_SIZE are KiB per dispatch.  Calibration: a plain device copy of",
        "# 256 MiB (reads 262144 KiB, writes 262144 KiB) in the same runs.",
        f"copy_fetch_kib: {cf:.1f}",
        f"copy_write_kib: {cw:.1f}",
        f"fetch_scale: {fs:.4f}",
        f"write_scale: {wsc:.4f}",
        f"attn_kernel: {akey}",
        f"attn_dispatches: {na_f} (fetch run), {na_w} (write run)",
        f"attn_fetch_kib_raw: {af:.1f}",
        f"attn_write_kib_raw: {aw:.1f}",
        f"merge_dispatches: {nm_f} (fetch run), {nm_w} (write run)",
        f"merge_fetch_kib_raw: {mf:.1f}",
        f"merge_write_kib_raw: {mw:.1f}",
        f"hbm_bytes_per_dispatch: {hbm:.0f}",
        f"algorithmic_bytes_per_dispatch: {attn_bytes(w)}  # q, out, k, v, r once each",
        f"traffic_over_algorithmic: {hbm / attn_bytes(w):.3f}",
        f"kernel_source: {src}",
        f"kernel_source_sha256: {sha}",
        "# other kernels of the same runs (scaled KiB per dispatch: fetch, write)",
    ]
    for (name, grid), v in sorted(fetch.items(), key=lambda kv: -mean(kv[1]))[:10]:
        wv = write.get((name, grid))
        lines.append(f"#   {name[:60]:60s} grid {grid:>9s}: {mean(v) * fs:12.1f} "
                     f"{(mean(wv) * wsc if wv else float('nan')):12.1f}")
    print("\n".join(lines), flush=True)


def trace_summary(path, trace=None, top=14):
    """Per-kernel table of rocprofv3's kernel stats CSV: calls, mean, min, max, share.
    With the per-dispatch kernel trace CSV as well, a second table splits each
    kernel's dispatches into those that ran alone on the GPU (no other dispatch
    overlapping them in time) and those that shared it with another stream's work."""
    import csv
    rows = list(csv.DictReader(open(path)))
    print(f"{'kernel':78s} {'calls':>6s} {'mean_us':>9s} {'min_us':>8s} {'max_us':>8s} "
          f"{'share':>6s}")
    for r in rows[:top]:
        print(f"{r['Name'][:78]:78s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} "
              f"{float(r['MinNs']) / 1e3:8.2f} {float(r['MaxNs']) / 1e3:8.2f} "
              f"{float(r['Percentage']):5.1f}%")
    if not trace:
        return
    ds = sorted(((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"])
                 for r in csv.DictReader(open(trace))), key=lambda t: t[0])
    alone = {}
    end_max = -1
    for i, (t0, t1, name) in enumerate(ds):
        nxt = ds[i + 1][0] if i + 1 < len(ds) else None
        solo = t0 >= end_max and (nxt is None or t1 <= nxt)
        end_max = max(end_max, t1)
        alone.setdefault(name, ([], []))[0 if solo else 1].append((t1 - t0) / 1e3)
    names = [r["Name"] for r in rows[:top]]
    print()
    print(f"{'kernel (dispatches alone on the GPU | overlapping another)':78s} {'alone':>6s} "
          f"{'mean_us':>9s} {'shared':>7s} {'mean_us':>9s}")
    for n in names:
        a, b = alone.get(n, ([], []))
        ma = f"{sum(a) / len(a):9.2f}" if a else f"{'-':>9s}"
        mb = f"{sum(b) / len(b):9.2f}" if b else f"{'-':>9s}"
        print(f"{n[:78]:78s} {len(a):6d} {ma} {len(b):7d} {mb}")


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary)
        return
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.trace_summary:
        trace_summary(*args.trace_summary)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this benchmark runs on exactly one GPU (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); no multi-GPU path is built", file=sys.stderr, flush=True)
        sys.exit(2)

    if args.eval_speed:
        eval_speed(args)
        return
    if args.vendor_sdpa:
        vendor_sdpa(args)
        return
    if args.train:
        train_step(args)
        return

    import torch
    from relative_position_memory_amd import inputs as I
    from relative_position_memory_amd import txl

    w = I.workload(args.workload)
    x = I.make_inputs(w, seed=0)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    es = 2 if w.dtype == "bf16" else 4
    txl.attn_variant(args.attn_variant)
    dev = lambda a: torch.from_numpy(a).to(tdt).cuda()
    Ws = [{k: dev(v) for k, v in lw.items()} for lw in x["weights"]]
    lws = [txl.layer_weights(Wl) for Wl in Ws]
    u, vb, R = dev(x["u"]), dev(x["v"]), dev(x["R"])
    ring_data = [dev(m) for m in x["mem"]]
    rings = [txl.make_ring(dd, 0, w.M) for dd in ring_data]
    h0 = dev(x["h0"])
    dims = txl.layer_dims(w.B, w.L, w.D, w.H, w.d)
    ws = torch.empty(txl.workspace_bytes(dims, w.M, tdt), dtype=torch.uint8, device="cuda")
    bufs = [torch.empty((w.B, w.L, w.D), dtype=tdt, device="cuda") for _ in range(2)]
    stream = torch.cuda.current_stream()

    # A step: every segment through every layer with its memory update
    # (txl_stack_fwd).  Segment s goes to streams[s % n]; layer n of segment s + 1
    # waits only for layer n of segment s, so consecutive segments overlap one
    # layer apart, with results bit-identical to the serial order.
    def make_step(n_streams):
        streams = [stream] + [torch.cuda.Stream() for _ in range(n_streams - 1)]
        sws = torch.empty(txl.stack_workspace_bytes(dims, w.M, tdt, n_streams),
                          dtype=torch.uint8, device="cuda")
        h_in = h0[:w.n_segments]
        h_out = torch.empty_like(h_in)

        def step():
            txl.stack_fwd(streams, dims, h_in, rings, lws, u, vb, R, h_out, sws)
        return step

    def timed_ms(step, steps, warmup):
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms = timed_ms(make_step(args.streams), args.steps, args.warmup)
    # the same stack in the serial order on one stream, for comparison
    ms_serial = ms if args.streams == 1 else timed_ms(make_step(1), max(3, args.steps // 4), 1)
    # the layer step behind the attention timing below: full memory, q, k, v, r
    # left in ws
    txl.layer_step(dims, h0[0], rings[0], lws[0], u, vb, R, bufs[0], ws, stream=stream)

    # the attention kernel alone, on the last layer step's q, k, v, r (HIP events, same
    # stream); with the memory full (every ring holds M rows after the first segment)
    # A head size that is not a multiple of 8 (the word model's 41): the layer step's
    # attention reads its head rows padded to d_pad with zeros, and this times that
    # same launch -- d_pad-wide views, u and v zero-padded, scale 1/sqrt(d).
    dpad = txl.d_pad(w.d)
    views = txl.workspace_views(dims, w.M, ws, tdt, padded=True)
    ua = torch.zeros((w.H, dpad), dtype=tdt, device="cuda")
    va = torch.zeros((w.H, dpad), dtype=tdt, device="cuda")
    ua[:, :w.d], va[:, :w.d] = u, vb
    out_a = torch.empty((w.B, w.L, w.H, dpad), dtype=tdt, device="cuda")
    nws = txl.rel_attn_workspace_bytes(tdt, w.B, w.H, w.L, w.M, dpad)
    aws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda") if nws else None

    def attn():
        txl.rel_attn_fwd(views["q"], views["k"], views["v"], views["r"], ua, va, w.M, out_a,
                         scale=1.0 / math.sqrt(w.d), stream=stream, workspace=aws)

    attn_s = hip_time_us(attn, args.attn_reps, stream) / 1e6
    af, ab = attn_flops(w), attn_bytes(w)
    attn_tflops = af / attn_s / 1e12
    attn_gbs = ab / attn_s / 1e9
    bound = attn_bound(w)
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": attn_tflops, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": attn_tflops / PEAK_BF16_TFLOPS,
                "hbm_frac": attn_gbs / PEAK_HBM_GBS}
    else:
        roof = {"bound": "hbm", "achieved": attn_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": attn_gbs / PEAK_HBM_GBS, "mfma_frac": attn_tflops / PEAK_BF16_TFLOPS}
    roof.update({"traffic": read_traffic(w.name),
                 "kernel": txl.attn_kernel(tdt, w.B, w.H, w.L, w.M, dpad),
                 "launch_us": attn_s * 1e6, "flop_per_launch": af, "bytes_per_launch": ab})

    # one layer step alone (full memory; projections, attention, output projection +
    # LayerNorm), and one memory update alone on a scratch ring
    ls_us = hip_time_us(lambda: txl.layer_step(dims, h0[0], rings[0], lws[0], u, vb, R, bufs[0],
                                               ws, stream=stream), 20, stream)
    lf = layer_flops(w)
    scratch = torch.empty_like(ring_data[0])
    sring = txl.make_ring(scratch, 0, w.M)
    mu_us = hip_time_us(lambda: txl.mem_update(sring, h0[0], stream=stream), 20, stream)
    mu_bytes = 2 * w.B * min(w.L, w.M) * w.D * es

    # the same stack with cached keys and values (txl_layer_step_kv): each layer's
    # ring is filled from its initial memory first (untimed), then the segments run
    kv_ms = None if args.main_only else kv_stack_ms(w, x, Ws, lws, u, vb, R, h0, args.steps,
                                                    args.warmup, stream, args.streams)

    # the position-wise feed-forward (not part of the step above) at the same rows,
    # d_inner = 4 d_model
    ff = None if args.main_only else pos_ff_time(w, args.attn_reps, stream)

    tokens = w.B * w.L * w.n_segments
    step_flops = layer_flops(w) * w.n_layers * w.n_segments
    res = {
        "metric": METRIC,
        "value": tokens / (ms / 1e3),
        "unit": "query tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.n_layers} layers x {w.n_segments} segments "
                               f"with memory update", "batch": w.B, "d_model": w.D,
                   "n_head": w.H, "d_head": w.d, "segment_len": w.L, "mem_len": w.M,
                   "n_layers": w.n_layers, "n_segments": w.n_segments},
        "roofline": roof,
        "layer_step": {"us": ls_us, "flop": lf, "achieved": lf / (ls_us * 1e-6) / 1e12,
                       "unit": "TFLOP/s", "frac": lf / (ls_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS,
                       "bound": "mfma"},
        "mem_update": {"us": mu_us, "bytes": mu_bytes, "achieved": mu_bytes / (mu_us * 1e-6) / 1e9,
                       "unit": "GB/s", "frac": mu_bytes / (mu_us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                       "bound": "hbm", "kernel": "ring_copy_kernel"},
        "step_tflops": step_flops / (ms / 1e3) / 1e12,
        "attn_variant": args.attn_variant,
        "schedule": {"entry_point": "txl_stack_fwd", "streams": args.streams,
                     "serial_ms_per_step": ms_serial,
                     "note": "segments go round the streams, segment s+1 one layer behind "
                             "segment s; outputs bit-identical to the one-stream order"},
    }
    if not args.main_only:
        res["pos_ff"] = ff
        res["eval_kv_cache"] = {
            "value": tokens / (kv_ms / 1e3), "unit": "query tokens/s", "ms_per_step": kv_ms,
            "note": "same stack and inputs with cached keys/values (txl_layer_step_kv): only "
                    "the L new rows are projected per segment, r is projected once; the same "
                    "segment schedule over the same streams; outputs equal the step above up "
                    "to rounding"}
    if args.calib_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    if not args.no_drift and not args.main_only:
        res["stack_drift"] = stack_drift(w, x, lws, u, vb, R, dims, ws, tdt, stream,
                                         min(w.n_segments, 4))
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, x, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
