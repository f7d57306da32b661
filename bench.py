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
ATTN_SRC = os.path.join(ROOT, "relative_position_memory_amd", "csrc", "attn_mfma.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_mfma_charlm_traffic.txt")


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="charlm")
    p.add_argument("--attn-reps", type=int, default=50)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle sample")
    p.add_argument("--calib-copy", action="store_true",
                   help="also run a plain 256 MiB device copy (reads 256 MiB, writes 256 MiB) "
                        "so that a counter run can calibrate FETCH_SIZE / WRITE_SIZE")
    return p.parse_args()


def attn_flops(w):
    """Algorithmic FLOPs of one attention call: 6 d per causal (query, key) pair
    (q.k, (q+v).r and p.v), P = L*M + L(L+1)/2 pairs per (batch, head)."""
    P = w.L * w.M + w.L * (w.L + 1) // 2
    return 6 * w.d * P * w.B * w.H


def layer_flops(w):
    T = w.M + w.L
    HD = w.H * w.d
    gemm = 2 * (w.B * w.L * HD * w.D + w.B * T * 2 * HD * w.D + T * HD * w.D
                + w.B * w.L * w.D * HD)
    return gemm + attn_flops(w)


def read_traffic():
    """HBM bytes per attention launch from the committed rocprofv3 counter summary,
    or None when the kernel source changed since the counters were taken."""
    try:
        kv = {}
        for ln in open(TRAFFIC_FILE):
            if ":" in ln and not ln.startswith("#"):
                k, v = ln.split(":", 1)
                kv[k.strip()] = v.strip()
        sha = hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()
        if kv.get("kernel_source_sha256") != sha:
            return None
        return float(kv["hbm_bytes_per_dispatch"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(w, x, target_s):
    """The oracle, as it stands, on the host cores: one layer step on a sample of
    the batch rows, scaled to query tokens/s through the N-layer stack."""
    from oracle import oracle as O
    W0 = x["weights"][0]

    def run(b, n):
        t0 = time.perf_counter()
        for r in range(n):
            Wl = x["weights"][r % len(x["weights"])]
            O.layer_step(x["h0"][0][:b], x["mem"][0][:b], Wl, x["u"], x["v"], x["R"])
        return time.perf_counter() - t0

    t1 = run(1, 1)
    b = max(1, min(w.B, int(target_s / max(t1, 1e-3))))
    tb = run(b, 1) if b > 1 else t1
    n = max(1, int(round(target_s / max(tb, 1e-3))))
    t = run(b, n) if n > 1 else tb
    return {
        "value": n * b * w.L / (t * w.n_layers),
        "unit": "query tokens/s",
        "cores": O.num_threads(),
        "kind": "oracle",
        "sample": (f"{n} fp64 layer steps (projections, attention, LayerNorm) over {b} of the "
                   f"{w.B} batch rows at full memory ({w.M} rows), {t:.1f} s in all; rate scaled "
                   f"by 1/{w.n_layers} layers to match the stack"),
    }


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this build runs on exactly one GPU (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); no multi-GPU path is built", file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    from relative_position_memory_amd import inputs as I
    from relative_position_memory_amd import txl

    w = I.workload(args.workload)
    x = I.make_inputs(w, seed=0)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
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

    def step():
        for s in range(w.n_segments):
            h = h0[s]
            for n in range(w.n_layers):
                out = bufs[n % 2]
                txl.layer_step(dims, h, rings[n], lws[n], u, vb, R, out, ws, stream=stream)
                txl.mem_update(rings[n], h, stream=stream)
                h = out

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps

    # the attention kernel alone, on the last layer step's q, k, v, r (HIP events, same stream)
    views = txl.workspace_views(dims, w.M, ws, tdt)
    out_a = torch.empty((w.B, w.L, w.H, w.d), dtype=tdt, device="cuda")
    nws = txl.rel_attn_workspace_bytes(tdt, w.B, w.H, w.L, w.M, w.d)
    aws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda") if nws else None

    def attn():
        txl.rel_attn_fwd(views["q"], views["k"], views["v"], views["r"], u, vb, w.M, out_a,
                         stream=stream, workspace=aws)

    for _ in range(3):
        attn()
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record(stream)
    for _ in range(args.attn_reps):
        attn()
    a1.record(stream)
    torch.cuda.synchronize()
    attn_s = a0.elapsed_time(a1) / args.attn_reps / 1e3
    af = attn_flops(w)
    attn_tflops = af / attn_s / 1e12

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
        "roofline": {"bound": "mfma", "kernel": "attn_mfma_kernel",
                     "achieved": attn_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": attn_tflops / PEAK_BF16_TFLOPS, "traffic": read_traffic(),
                     "launch_us": attn_s * 1e6, "flop_per_launch": af},
        "step_tflops": step_flops / (ms / 1e3) / 1e12,
    }
    if args.calib_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, x, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
