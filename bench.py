#!/usr/bin/env python3
"""Benchmark of the QLoRA frozen-base hot path on one MI355X.

Headline workload (the largest configuration that fits one GPU): one decoder
layer of a 70B-shaped model, seven projections q, o 8192x8192; k, v
1024x8192; gate, up 28672x8192; down 8192x28672 (855.6M weights), bf16
weights ~ N(0, 0.015), M = 2048 tokens, LoRA r = 64, alpha = 16. One step:
  1. quantize the seven bf16 weights to NF4 + double-quantized constants,
  2. for each projection the forward y = x W_hat^T + (alpha/r) (x A) B with
     u = x A saved (the weight dequantized to bf16 inside the call),
  3. and its backward dX, dA, dB given dY ~ N(0, 1),
on resident synthetic inputs (x ~ N(0,1) per projection: the attention,
norms and activations between them are not part of the path). y and dX are
bf16, the activations' compute dtype (fp32 accumulation); dA, dB fp32.
`value` = the step's multiply-add work (2 flops per MAC, 2MNK + 2Mr(K+N)
forward, 2MNK + 2Mr(N+K) + 2MKr + 2MNr backward; quantization and
dequantization count none) over the host-clock time of exactly K steps
replayed from one captured HIP graph, bracketed by device synchronisation.
One replay must first reproduce the eager step's outputs bit for bit.

`roofline`: the dequant-GEMM forward call on the 28672x8192 projection
(the dominant call of the step; the whole call: the adapter down
projection, the dequantization and the GEMM), its algorithmic flops
2MNK + 2Mr(K+N) over its average duration from HIP events around
back-to-back calls on the stream the library launches on.
`traffic`: that call's HBM bytes from rocprofv3 FETCH_SIZE / WRITE_SIZE
counters (per dispatch, summed over the call's kernels, scaled by the same
counters' reading for an elementwise copy of known size), or null when a
kernel source no longer matches the one the counters were taken on.

Sections beside the step (skipped with --no-extras), one per configuration
of the workload list: the 1024x1024 layer (microseconds per call, and
quantize / dequantize bandwidth over a ring of 512 distinct weights), the
Llama-7B decode GEMV (weight GB/s on a ring of 24 distinct 11008x4096 weights,
tokens/s), the Llama-7B training layer (M = 4096: forward through both routes,
backward, TFLOP/s and tokens/s), bulk quantize / dequantize of 8192x28672
Student-t tensors in each second-level format, merge + requantize, and the
AdamW step on a Llama-7B adapter arena. `cpu_baseline` times the oracle
(single-threaded C) per operation on one core and extrapolates the step; an
all-cores quantize/dequantize run uses P independent oracle processes.

Counter helpers: `--only CALL` runs one call of the step (e.g. fwd_up,
quantize_up) for the timed iterations, or one of the extra calls
fwd_up_lean (the same forward with the smallest workspace, so the fused
kernel that keeps no bf16 copy of the weight runs), dequant_up (row-major
dequantization of the 28672x8192 projection) and
decode_up7b_m1 (the decode forward, M = 1, r = 16, on one 11008x4096
weight); `--copy-calibration BYTES` runs an elementwise copy of BYTES bytes
(the reference reading for the counter scale).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "NF4 dequant-GEMM TFLOP/s & GEMV weight GB/s (fraction of roofline) per layer"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
ACT_DTYPE_NAME = "bfloat16"  # y and dX: the activations' compute dtype

# HBM traffic of the roofline call (the forward on the 28672x8192 projection,
# M 2048, r 64, y bf16) from rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per
# dispatch, summed over the call's kernels) scaled by the counters' reading
# for an elementwise copy of known size. Valid while every listed source
# hashes to the recorded value; None: not measured for these sources.
TRAFFIC = {"call": "fwd_up", "sources": ["api.cpp", "quantize.hip", "gemm_nt.hip", "lora.hip"],
           "src_sha256": "b52528a396a93c197443523b4742383f62e78845e78abb1c0813b0237145cf5d",
           "fetch_bytes": 1710805415, "write_bytes": 601358362}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def nf4_bytes(N, K):
    n = N * K
    nb = n // 64
    return n // 2 + nb + 4 * ((nb + 255) // 256)


def fwd_flops(M, N, K, r):
    return 2 * M * N * K + 2 * M * r * (K + N)


def bwd_flops(M, N, K, r):
    return 2 * M * N * K + 2 * M * r * (N + K) + 2 * M * K * r + 2 * M * N * r


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--no-extras", action="store_true", help="skip the per-configuration sections")
    ap.add_argument("--only", default=None, help="run only this call of the step (counter runs)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="time an elementwise copy of BYTES bytes and exit (counter scale)")
    return ap.parse_args()


def src_sha(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "qlora_fine_tuning_blockwise_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def copy_calibration(nbytes, steps):
    import torch
    dev = torch.device("cuda:0")
    # an elementwise kernel (not a DMA copy) so that the L2 counters see it
    src = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        torch.bitwise_xor(src, 0, out=dst)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        torch.bitwise_xor(src, 0, out=dst)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "steps": steps,
                      "ms": round(ms, 5), "gbps": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}),
          flush=True)


def event_ms(torch, fn, iters, stream, warm=2):
    """Average duration of fn over `iters` back-to-back calls, from HIP events
    recorded on `stream` (the stream the library launches on)."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(iters):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def rate(flops=0, nbytes=0, ms=1.0):
    e = {"ms": round(ms, 5)}
    if flops:
        tf = flops / (ms * 1e-3) / 1e12
        e["tflops"] = round(tf, 2)
        e["frac_bf16_peak"] = round(tf / PEAK_BF16_TFLOPS, 4)
    if nbytes:
        gb = nbytes / (ms * 1e-3) / 1e9
        e["gbps"] = round(gb, 1)
        e["frac_hbm_peak"] = round(gb / PEAK_HBM_GBPS, 4)
    return e


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, args.steps)
        return
    import torch

    import qlora_fine_tuning_blockwise_amd as q
    from qlora_fine_tuning_blockwise_amd import synthetic as syn

    act = getattr(torch, ACT_DTYPE_NAME)
    q._lib.load()  # fail loudly if the HIP library is not built
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    cfg = syn.LAYER_70B
    M, r, alpha = cfg["M"], cfg["r"], cfg["alpha"]
    names = list(cfg["weights"])

    # ------------------------------------------------------------ inputs (resident)
    L = {}
    for t, name in enumerate(names):
        N, K = cfg["weights"][name]
        Wb = syn.torch_normal_bf16((N, K), cfg["w_std"], syn.seed_of(4, t), dev)
        L[name] = dict(
            N=N, K=K, W=Wb, w=q.qlora_quantize_nf4_dq(Wb),
            A=syn.torch_normal_bf16((K, r), 1.0 / K ** 0.5, syn.seed_of(4, 10 + t), dev),
            B=syn.torch_normal_bf16((r, N), 0.01, syn.seed_of(4, 20 + t), dev),
            x=syn.torch_normal_bf16((M, K), 1.0, syn.seed_of(4, 30 + t), dev),
            dY=syn.torch_normal_bf16((M, N), 1.0, syn.seed_of(4, 40 + t), dev),
            y=torch.empty((M, N), dtype=act, device=dev),
            u=torch.empty((M, r), dtype=torch.float32, device=dev),
            dX=torch.empty((M, K), dtype=act, device=dev))
    ws_bytes = max(q.qlora_workspace_bytes(op, M, p["N"], p["K"], r) for op in (0, 1)
                   for p in L.values())
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    log("70B layer inputs ready; workspace", round(ws_bytes / 2 ** 20, 1), "MiB")

    calls = []  # (label, fn, flops, algorithmic bytes)
    for name in names:
        p = L[name]
        calls.append((f"quantize_{name}", lambda p=p: q.qlora_quantize_nf4_dq(p["W"], out=p["w"]),
                      0, 2 * p["N"] * p["K"] + nf4_bytes(p["N"], p["K"])))
    for name in names:
        p = L[name]
        calls.append((f"fwd_{name}", lambda p=p: q.qlora_linear_fwd(
            p["w"], p["x"], p["A"], p["B"], alpha, y=p["y"], u_out=p["u"], workspace=ws),
            fwd_flops(M, p["N"], p["K"], r), 0))
        calls.append((f"bwd_{name}", lambda p=p: p.__setitem__("g", q.qlora_linear_bwd(
            p["w"], p["x"], p["dY"], p["A"], p["B"], alpha, u_saved=p["u"], dx_dtype=act,
            workspace=ws)), bwd_flops(M, p["N"], p["K"], r), 0))
    step_flops = sum(c[2] for c in calls)
    roof_call = "fwd_up"

    if args.only == "fwd_up_lean":
        p = L["up"]
        ws_lean = torch.empty(q.qlora_workspace_bytes(3, M, p["N"], p["K"], r), dtype=torch.uint8,
                              device=dev)
        calls.append(("fwd_up_lean", lambda p=p: q.qlora_linear_fwd(
            p["w"], p["x"], p["A"], p["B"], alpha, y=p["y"], u_out=p["u"], workspace=ws_lean),
            fwd_flops(M, p["N"], p["K"], r), 0))
    deq = None
    if args.only == "dequant_up":
        p = L["up"]
        deq = torch.empty((p["N"], p["K"]), dtype=torch.bfloat16, device=dev)
        calls.append(("dequant_up", lambda p=p: q.qlora_dequant_bf16(p["w"], out=deq), 0,
                      nf4_bytes(p["N"], p["K"]) + 2 * p["N"] * p["K"]))
    if args.only == "decode_up7b_m1":
        dc = syn.LLAMA7B_DECODE
        N7, K7 = dc["weights"]["up"]
        r7 = dc["r"]
        w7 = q.qlora_quantize_nf4_dq(syn.torch_normal_bf16((N7, K7), dc["w_std"],
                                                           syn.seed_of(2, 11), dev))
        A7 = syn.torch_normal_bf16((K7, r7), 1.0 / K7 ** 0.5, syn.seed_of(2, 30), dev)
        B7 = syn.torch_normal_bf16((r7, N7), 0.01, syn.seed_of(2, 31), dev)
        x7 = syn.torch_normal_bf16((1, K7), 1.0, syn.seed_of(2, 41), dev)
        y7 = torch.empty((1, N7), dtype=torch.float32, device=dev)
        ws7 = torch.empty(q.qlora_workspace_bytes(0, 1, N7, K7, r7), dtype=torch.uint8,
                          device=dev)
        calls.append(("decode_up7b_m1", lambda: q.qlora_linear_fwd(
            w7, x7, A7, B7, dc["alpha"], y=y7, workspace=ws7), fwd_flops(1, N7, K7, r7),
            nf4_bytes(N7, K7) + 2 * (K7 * r7 + r7 * N7)))
    if args.only:
        sel = [c for c in calls if c[0] == args.only]
        if not sel:
            sys.exit(f"--only: no call named {args.only}; calls: {[c[0] for c in calls]}")
        label, fn, flops, nbytes = sel[0]
        ms = event_ms(torch, fn, args.steps, stream, warm=args.warmup)
        print(json.dumps({"call": label, "steps": args.steps, **rate(flops, nbytes, ms)}),
              flush=True)
        return

    def step(ev=None):
        for i, (_, fn, _, _) in enumerate(calls):
            if ev is not None:
                ev[i][0].record(stream)
            fn()
            if ev is not None:
                ev[i][1].record(stream)

    log("warmup", args.warmup)
    for _ in range(args.warmup):
        step()
    # Eager steps, every call bracketed by its own pair of events.
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in calls] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    ms_step_eager = (time.perf_counter() - t0) * 1e3 / args.steps
    per_call = [sum(evs[k][i][0].elapsed_time(evs[k][i][1]) for k in range(args.steps))
                / args.steps for i in range(len(calls))]

    # The step captured once as a HIP graph; one replay must reproduce the
    # eager step's outputs bit for bit before it is timed.
    def outputs():
        res = []
        for p in L.values():
            res += [p["w"].codes, p["w"].absmax_q, p["w"].absmax_scale, p["y"], p["u"],
                    *p["g"]]
        return [t.clone() for t in res]

    torch.cuda.synchronize()
    ref = outputs()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    graph.replay()
    torch.cuda.synchronize()
    got = outputs()
    if not all(torch.equal(a, b) for a, b in zip(ref, got)):
        sys.exit("bench.py: the captured step's outputs differ from the eager step's")
    del ref, got
    for _ in range(args.warmup):
        graph.replay()
    # Timed region: exactly K replays, bracketed by device synchronisation.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    log("timed", args.steps, "graph replays:", round(ms_step, 3), "ms per step")
    value = step_flops / (ms_step * 1e-3) / 1e12

    breakdown = {lab: rate(fl, nb, ms) for (lab, _, fl, nb), ms in zip(calls, per_call)}
    proj = {}
    for name in names:
        p = L[name]
        tf, tb = breakdown[f"fwd_{name}"]["ms"], breakdown[f"bwd_{name}"]["ms"]
        proj[name] = {"shape": [p["N"], p["K"]], "fwd_ms": tf, "bwd_ms": tb,
                      "tokens_per_s": round(M / ((tf + tb) * 1e-3), 1)}
    t_fb = sum(v["fwd_ms"] + v["bwd_ms"] for v in proj.values())

    # Roofline: the dominant call (forward on the 28672x8192 projection) alone.
    lab, rfn, rflops, _ = [c for c in calls if c[0] == roof_call][0]
    rms = event_ms(torch, rfn, max(args.steps, 10), stream)
    achieved = rflops / (rms * 1e-3) / 1e12
    traffic = None
    if TRAFFIC["src_sha256"] and TRAFFIC["src_sha256"] == src_sha(TRAFFIC["sources"]):
        traffic = TRAFFIC["fetch_bytes"] + TRAFFIC["write_bytes"]
    pu = L["up"]
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic, "call": "qlora_linear_fwd (whole call)", "label": lab,
                "kernels": ["transpose_kernel", "lora_down_stream_kernel", "lora_down_finalize_kernel",
                            "dequant_kernel<true> (K-slab)", "gemm_nt_kernel"],
                "shape": {"M": M, "N": pu["N"], "K": pu["K"], "r": r},
                "flops_per_call": rflops, "flops_formula": "2MNK + 2Mr(K+N)",
                "avg_ms": round(rms, 5)}

    result = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "ms_per_step_eager": round(ms_step_eager, 4),
        "ms_per_step_device_calls": round(sum(per_call), 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama70b_layer: seven projections (q, o 8192x8192; k, v "
                               "1024x8192; gate, up 28672x8192; down 8192x28672) bf16 "
                               "N(0,0.015) -> NF4+DQ each step; fwd + bwd (dX, dA, dB) at "
                               "M=2048, r=64, alpha=16; y and dX bf16, dA and dB fp32",
                   "weights": {n: list(cfg["weights"][n]) for n in names}, "M": M, "r": r,
                   "alpha": alpha},
        "tokens_per_s": round(M / (t_fb * 1e-3), 1),
        "roofline": roofline, "projections": proj, "breakdown": breakdown,
    }
    del graph, L, ws
    torch.cuda.empty_cache()

    if not args.no_extras:
        log("1024x1024 layer")
        result["linear_1024"] = linear_1024(q, syn, torch, dev, stream)
        log("7B decode GEMV ring")
        result["decode_7b"] = decode_7b(q, syn, torch, dev, stream)
        log("7B training layer")
        result["train_7b"] = train_7b(q, syn, torch, dev, stream, act)
        log("bulk quantize/dequant")
        result["bulk_quantize"] = bulk_quantize(q, syn, torch, dev, stream)
        log("merge + requantize")
        result["merge"] = merge_section(q, syn, torch, dev, stream)
        log("adamw step on the adapter arena")
        result["adamw"] = adamw_section(q, syn, torch, dev, stream)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(syn, cfg, step_flops, ms_step)
    print(json.dumps(result), flush=True)


def graph_of(torch, fn):
    """fn captured as a HIP graph (after one eager call)."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def linear_1024(q, syn, torch, dev, stream):
    """The 1024x1024 layer (fp32 weight ~ N(0, 0.02), M = 16, r = 16, alpha =
    32). Latency-bound: microseconds per call of quantize, dequantize,
    forward and backward (HIP events around a graph of 50 back-to-back calls
    of the same inputs). Bandwidth: the
    quantize and dequantize of a ring of 512 distinct weights (2.1 GB of fp32
    in, past the Infinity Cache), replayed from a captured graph."""
    cfg = syn.LINEAR_1024
    N, K = cfg["weights"]["w"]
    Mq, r, alpha = cfg["M"], cfg["r"], cfg["alpha"]
    W = torch.empty((N, K), device=dev).normal_(0.0, cfg["w_std"])
    w = q.qlora_quantize_nf4_dq(W)
    x = syn.torch_normal_bf16((Mq, K), 1.0, syn.seed_of(1, 3), dev)
    A = syn.torch_normal_bf16((K, r), 1.0 / K ** 0.5, syn.seed_of(1, 1), dev)
    B = syn.torch_normal_bf16((r, N), 0.01, syn.seed_of(1, 2), dev)
    dY = syn.torch_normal_bf16((Mq, N), 1.0, syn.seed_of(1, 4), dev)
    u = torch.empty((Mq, r), dtype=torch.float32, device=dev)
    ws = torch.empty(max(q.qlora_workspace_bytes(op, Mq, N, K, r) for op in (0, 1)),
                     dtype=torch.uint8, device=dev)
    deq = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    y = torch.empty((Mq, N), dtype=torch.float32, device=dev)
    res = {"weight": [N, K], "M": Mq, "r": r}
    for label, fn, fl, nb in (
            ("quantize", lambda: q.qlora_quantize_nf4_dq(W, out=w), 0, 4 * N * K + nf4_bytes(N, K)),
            ("dequant", lambda: q.qlora_dequant_bf16(w, out=deq), 0, nf4_bytes(N, K) + 2 * N * K),
            ("fwd", lambda: q.qlora_linear_fwd(w, x, A, B, alpha, y=y, u_out=u, workspace=ws),
             fwd_flops(Mq, N, K, r), 0),
            ("bwd", lambda: q.qlora_linear_bwd(w, x, dY, A, B, alpha, u_saved=u, workspace=ws),
             bwd_flops(Mq, N, K, r), 0)):
        # device time per call: 50 back-to-back calls captured in one graph
        # (one graph launch costs more than these kernels take)
        def fifty(fn=fn):
            for _ in range(50):
                fn()
        g = graph_of(torch, fifty)
        ms = event_ms(torch, g.replay, 5, stream) / 50
        e = rate(fl, nb, ms)
        e["us_per_call"] = round(ms * 1e3, 2)
        res[label] = e
    # ring of 512 distinct weights
    ring_n = 512
    Ws = torch.empty((ring_n, N, K), device=dev).normal_(0.0, cfg["w_std"])
    ring = [q.qlora_quantize_nf4_dq(Ws[i]) for i in range(ring_n)]
    outs = torch.empty((ring_n, N, K), dtype=torch.bfloat16, device=dev)

    def qring():
        for i in range(ring_n):
            q.qlora_quantize_nf4_dq(Ws[i], out=ring[i])

    def dring():
        for i in range(ring_n):
            q.qlora_dequant_bf16(ring[i], out=outs[i])
    for label, fn, nb in (("quantize_ring", qring, 4 * N * K + nf4_bytes(N, K)),
                          ("dequant_ring", dring, nf4_bytes(N, K) + 2 * N * K)):
        g = graph_of(torch, fn)
        ms = event_ms(torch, g.replay, 5, stream) / ring_n
        e = rate(0, nb, ms)
        e["us_per_call"] = round(ms * 1e3, 3)
        e["ring_weights"] = ring_n
        res[label] = e
    del Ws, ring, outs
    torch.cuda.empty_cache()
    return res


def decode_7b(q, syn, torch, dev, stream):
    """Llama-7B decode (M = 1, 4, 16; r = 16, alpha = 32) on a ring of 24
    distinct 11008x4096 weights (558 MB of NF4, past the 256 MB Infinity
    Cache) and on the 4096x4096 weight: microseconds per call (the adapter
    down projection and the fused GEMV), weight GB/s (codes + 8-bit scale
    codes + second-level scales + A + B per call) and total GB/s with the
    fractions of HBM peak, tokens/s. Also quantize and dequantize of both
    weights (GB/s), each call on another input (rings past the Infinity
    Cache)."""
    cfg = syn.LLAMA7B_DECODE
    r, alpha = cfg["r"], cfg["alpha"]
    res = {"r": r}
    for name, nw in (("up", 24), ("q", 64)):
        N, K = cfg["weights"][name]
        base = syn.torch_normal_bf16((N, K), cfg["w_std"], syn.seed_of(2, 10 + (name == "up")),
                                     dev)
        ring = [q.qlora_quantize_nf4_dq(base) for _ in range(nw)]
        for i, w in enumerate(ring[1:], 1):  # distinct contents: rotate the codes
            w.codes.copy_(ring[0].codes.roll(i))
        deq = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
        sec = {"weight": [N, K], "ring_weights": nw,
               "ring_mb": round(nw * nf4_bytes(N, K) / 1e6, 1)}
        # Quantize and dequantize read distinct tensors call after call (bf16
        # inputs: a ring of at least 512 MB, past the Infinity Cache), so the
        # rates are HBM rates rather than cache rates.
        nb16 = -(-512 * 10 ** 6 // (2 * N * K))
        bases = [base] + [base.roll(i, 1) for i in range(1, nb16)]
        cnt = [0]

        def quant_next():
            cnt[0] += 1
            q.qlora_quantize_nf4_dq(bases[cnt[0] % nb16], out=ring[cnt[0] % nw])

        def deq_next():
            cnt[0] += 1
            q.qlora_dequant_bf16(ring[cnt[0] % nw], out=deq)
        for label, fn, nb in (("quantize", quant_next, 2 * N * K + nf4_bytes(N, K)),
                              ("dequant", deq_next, nf4_bytes(N, K) + 2 * N * K)):
            sec[label] = rate(0, nb, event_ms(torch, fn, 48, stream))
        sec["quantize_ring_mb"] = round(nb16 * 2 * N * K / 1e6, 1)
        del bases
        A = syn.torch_normal_bf16((K, r), 1.0 / K ** 0.5, syn.seed_of(2, 30), dev)
        B = syn.torch_normal_bf16((r, N), 0.01, syn.seed_of(2, 31), dev)
        for Md in cfg["M"]:
            x = syn.torch_normal_bf16((Md, K), 1.0, syn.seed_of(2, 40 + Md), dev)
            y = torch.empty((Md, N), dtype=torch.float32, device=dev)
            ws = torch.empty(q.qlora_workspace_bytes(0, Md, N, K, r), dtype=torch.uint8,
                             device=dev)

            def ring_fwd():
                for w in ring:
                    q.qlora_linear_fwd(w, x, A, B, alpha, y=y, workspace=ws)
            g = graph_of(torch, ring_fwd)
            ms = event_ms(torch, g.replay, 4, stream) / nw
            wbytes = nf4_bytes(N, K) + 2 * (K * r + r * N)
            tbytes = wbytes + 2 * Md * K + 4 * Md * N
            gb = wbytes / (ms * 1e-3) / 1e9
            sec[f"M{Md}"] = {"us_per_call": round(ms * 1e3, 2), "weight_gbps": round(gb, 1),
                             "frac_hbm_peak": round(gb / PEAK_HBM_GBPS, 4),
                             "total_gbps": round(tbytes / (ms * 1e-3) / 1e9, 1),
                             "tflops": round(fwd_flops(Md, N, K, r) / (ms * 1e-3) / 1e12, 3),
                             "tokens_per_s": round(Md / (ms * 1e-3), 1)}
        res[name] = sec
        del ring, base, deq
        torch.cuda.empty_cache()
    return res


def train_7b(q, syn, torch, dev, stream, act):
    """Llama-7B training layer (M = 4096 tokens, r = 16, alpha = 32) on the
    4096x4096 and 11008x4096 weights: the forward through the fast route (one
    bf16 copy of the weight in the workspace, then the dense GEMM) and the
    lean route (the fused kernel that dequantizes in registers), the
    backward (dX, dA, dB); TFLOP/s with the bf16-peak fraction and tokens/s
    = M / (t_fwd + t_bwd)."""
    cfg = syn.LLAMA7B_TRAIN
    M, r, alpha = cfg["M"], cfg["r"], cfg["alpha"]
    res = {"M": M, "r": r}
    for i, name in enumerate(cfg["weights"]):
        N, K = cfg["weights"][name]
        W = syn.torch_normal_bf16((N, K), cfg["w_std"], syn.seed_of(3, i), dev)
        w = q.qlora_quantize_nf4_dq(W)
        del W
        A = syn.torch_normal_bf16((K, r), 1.0 / K ** 0.5, syn.seed_of(3, 10 + i), dev)
        B = syn.torch_normal_bf16((r, N), 0.01, syn.seed_of(3, 20 + i), dev)
        x = syn.torch_normal_bf16((M, K), 1.0, syn.seed_of(3, 40), dev)
        dY = syn.torch_normal_bf16((M, N), 1.0, syn.seed_of(3, 30 + i), dev)
        y = torch.empty((M, N), dtype=act, device=dev)
        u = torch.empty((M, r), dtype=torch.float32, device=dev)
        ws = torch.empty(max(q.qlora_workspace_bytes(op, M, N, K, r) for op in (0, 1)),
                         dtype=torch.uint8, device=dev)
        wsl = torch.empty(q.qlora_workspace_bytes(3, M, N, K, r), dtype=torch.uint8, device=dev)
        ff, bf = fwd_flops(M, N, K, r), bwd_flops(M, N, K, r)
        tf = event_ms(torch, lambda: q.qlora_linear_fwd(w, x, A, B, alpha, y=y, u_out=u,
                                                        workspace=ws), 10, stream)
        tl = event_ms(torch, lambda: q.qlora_linear_fwd(w, x, A, B, alpha, y=y, u_out=u,
                                                        workspace=wsl), 10, stream)
        tb = event_ms(torch, lambda: q.qlora_linear_bwd(w, x, dY, A, B, alpha, u_saved=u,
                                                        dx_dtype=act, workspace=ws), 10, stream)
        res[name] = {"shape": [N, K], "fwd": rate(ff, 0, tf), "fwd_lean": rate(ff, 0, tl),
                     "bwd": rate(bf, 0, tb), "tokens_per_s": round(M / ((tf + tb) * 1e-3), 1)}
        del w, x, dY, ws, wsl, y
        torch.cuda.empty_cache()
    return res


def merge_section(q, syn, torch, dev, stream):
    """Adapter merge on the 11008x4096 weight (r 16): the merge into the 4-bit
    base (dequantize + s (AB)^T in binary32, fp32 out) and its requantization,
    with the relative Frobenius error of the requantized weight against the
    exact 16-bit merge for the 4-bit path and for the clean path (merge into
    the bf16 weight, quantize once)."""
    N, K, r, alpha = 11008, 4096, 16, 32.0
    W = syn.torch_normal_bf16((N, K), 0.02, syn.seed_of(3, 1), dev)
    w = q.qlora_quantize_nf4_dq(W)
    A = syn.torch_normal_bf16((K, r), 1.0 / K ** 0.5, syn.seed_of(3, 11), dev)
    B = syn.torch_normal_bf16((r, N), 0.01, syn.seed_of(3, 21), dev)
    merged = torch.empty((N, K), dtype=torch.float32, device=dev)
    ws = torch.empty(q.qlora_workspace_bytes(2, 0, N, K, r), dtype=torch.uint8, device=dev)
    wq = q.qlora_quantize_nf4_dq(merged)
    ms_m = event_ms(torch, lambda: q.qlora_merge_lora(A, B, alpha, w=w, out=merged, workspace=ws),
                    10, stream)
    ms_q = event_ms(torch, lambda: q.qlora_quantize_nf4_dq(merged, out=wq), 10, stream)
    q.qlora_merge_lora(A, B, alpha, w=w, out=merged, workspace=ws)
    q.qlora_quantize_nf4_dq(merged, out=wq)
    back4 = q.qlora_dequant_bf16(wq).float()
    exact = q.qlora_merge_lora(A, B, alpha, W=W, workspace=ws)
    wc = q.qlora_quantize_nf4_dq(exact)
    backc = q.qlora_dequant_bf16(wc).float()
    nrm = torch.linalg.norm(exact)
    res = {"weight": [N, K], "r": r,
           "merge_4bit_base": rate(0, nf4_bytes(N, K) + 2 * r * (N + K) + 4 * N * K, ms_m),
           "requantize_f32": rate(0, 4 * N * K + nf4_bytes(N, K), ms_q),
           "rel_err_vs_16bit_merge": {
               "merge_into_4bit_then_requantize": round(float(torch.linalg.norm(back4 - exact)
                                                              / nrm), 5),
               "merge_into_bf16_then_quantize": round(float(torch.linalg.norm(backc - exact)
                                                            / nrm), 5)}}
    del W, w, merged, wq, back4, exact, wc, backc
    torch.cuda.empty_cache()
    return res


def adamw_section(q, syn, torch, dev, stream):
    """AdamW on every adapter of a Llama-7B decoder at rank 16 (one flat
    arena, bf16 gradients, bf16 copy written): 28 bytes per parameter, with
    the state in HBM and with the master values and moments in pinned host
    memory (the paged state)."""
    n = syn.adapter_arena_params()
    g = torch.empty(n, dtype=torch.bfloat16, device=dev).normal_(0.0, 1e-2)
    pb = torch.empty(n, dtype=torch.bfloat16, device=dev)
    res = {"params": n, "bytes_per_param": 28}

    def run(where, P, Mo, V, iters):
        st = [0]

        def one():
            st[0] += 1
            q.qlora_adamw_step(P, g, Mo, V, step=st[0], lr=2e-4, weight_decay=0.01, param_bf16=pb)
        ms = event_ms(torch, one, iters, stream)
        e = rate(0, 28 * n, ms)
        e["params_per_s"] = round(n / (ms * 1e-3), 1)
        if where != "hbm":
            e.pop("frac_hbm_peak")
        res[where] = e

    P = torch.empty(n, dtype=torch.float32, device=dev).normal_(0.0, 0.02)
    Mo = torch.zeros(n, dtype=torch.float32, device=dev)
    V = torch.zeros(n, dtype=torch.float32, device=dev)
    run("hbm", P, Mo, V, 10)
    Ph, Mh, Vh = (t.cpu().pin_memory() for t in (P, Mo, V))
    del P, Mo, V
    run("pinned_host", Ph, Mh, Vh, 3)
    return res


def bulk_quantize(q, syn, torch, dev, stream):
    """Quantize and dequantize bandwidth on one 8192x28672 bf16 tensor (the
    65B bulk workload's tensor, 470 MB in, past the Infinity Cache), in each
    second-level format, with the format's error on that heavy-tailed tensor:
    the relative error of the reconstructed block constants c1_hat against
    the exact block absmax (median and 99th percentile over non-zero blocks)
    and the relative Frobenius error of the dequantized weight."""
    N, K = syn.BULK_65B["tensor"]
    Wt = syn.torch_student_t_outliers_bf16((N, K), 4242, dev)
    out = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    c1 = Wt.float().abs().view(-1, 64).amax(dim=1)  # measurement only
    nz = c1 > 0
    wnorm = torch.linalg.norm(Wt.float())
    res = {"tensor": [N, K], "tensors_in_65b": syn.BULK_65B["n_tensors"]}
    for fmt, name in ((q.DQ_INT8, None), (q.DQ_UINT8, "uint8"), (q.DQ_E4M3, "e4m3")):
        w = q.qlora_quantize_nf4_dq(Wt, dq_format=fmt)
        sec = res if name is None else res.setdefault(name, {})
        for label, fn, nbytes in (("quantize", lambda: q.qlora_quantize_nf4_dq(Wt, out=w),
                                   2 * N * K + nf4_bytes(N, K)),
                                  ("dequant", lambda: q.qlora_dequant_bf16(w, out=out),
                                   nf4_bytes(N, K) + 2 * N * K)):
            ms = event_ms(torch, fn, 10, stream, warm=3)
            e = rate(0, nbytes, ms)
            e["params_per_s"] = round(N * K / (ms * 1e-3), 1)
            sec[label] = e
        qb = w.absmax_q
        if fmt == q.DQ_E4M3:
            val = qb.view(torch.float8_e4m3fn).float()
        elif fmt == q.DQ_UINT8:
            val = qb.view(torch.uint8).float()
        else:
            val = qb.float()
        chat = val * w.absmax_scale.repeat_interleave(256)[: val.numel()]
        rel = ((chat - c1).abs() / c1.clamp_min(1e-30))[nz]
        sec["c1_rel_err_p50"] = round(float(rel.median()), 5)
        sec["c1_rel_err_p99"] = round(float(torch.quantile(rel[:: max(1, rel.numel() // 4000000)],
                                                           0.99)), 5)
        q.qlora_dequant_bf16(w, out=out)
        sec["weight_rel_frob_err"] = round(float(torch.linalg.norm(out.float() - Wt.float())
                                                 / wnorm), 5)
        del w
    res["65b_extrapolated_s"] = {
        "quantize": round(res["quantize"]["ms"] * syn.BULK_65B["n_tensors"] / 1e3, 3),
        "dequant": round(res["dequant"]["ms"] * syn.BULK_65B["n_tensors"] / 1e3, 3)}
    del Wt, out, c1, nz
    torch.cuda.empty_cache()
    return res


_CPU_WORKER = r"""
import json, sys, time
sys.path.insert(0, sys.argv[1])
import oracle
from qlora_fine_tuning_blockwise_amd import synthetic as syn
N, K, seed = int(sys.argv[2]), int(sys.argv[3]), int(sys.argv[4])
Wb = syn.normal_bf16((N, K), 0.015, seed)
t0 = time.perf_counter()
c, q8, s2 = oracle.quantize_nf4_dq(Wb, "bf16")
t1 = time.perf_counter()
oracle.dequant_dq(c, q8, s2)
t2 = time.perf_counter()
print(json.dumps({"quantize_s": t1 - t0, "dequant_s": t2 - t1}))
"""


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(syn, cfg, step_flops, ms_step):
    """The oracle (single-threaded C, -O2, no SIMD intrinsics, GEMMs in fp64)
    timed on this host. Per operation on one core, on the 70B layer's
    1024x8192 projection: quantize and dequantize in full (params/s), forward
    and backward on 128 of the 2048 token rows (GFLOP/s). The step's oracle
    time is extrapolated from those rates (quantize of all seven weights,
    a dequantization per forward and per backward, the forward and backward
    MAC work at the measured GFLOP/s); value = step flops / that time. The
    all-cores run starts P independent oracle processes (P = the host's CPU
    count, at most 16), each quantizing and dequantizing its own 1024x8192
    tensor; the aggregate rate uses the slowest process's time."""
    import oracle

    r, alpha, M = cfg["r"], cfg["alpha"], cfg["M"]
    N, K = cfg["weights"]["k"]
    Ms = 128
    Wb = syn.normal_bf16((N, K), cfg["w_std"], syn.seed_of(4, 1))
    x = syn.normal_bf16((Ms, K), 1.0, syn.seed_of(4, 31))
    A = syn.normal_bf16((K, r), 1.0 / K ** 0.5, syn.seed_of(4, 11))
    B = syn.normal_bf16((r, N), 0.01, syn.seed_of(4, 21))
    dY = syn.normal_bf16((Ms, N), 1.0, syn.seed_of(4, 41))
    t0 = time.perf_counter()
    codes, q8, s2 = oracle.quantize_nf4_dq(Wb, "bf16")
    t1 = time.perf_counter()
    What = oracle.dequant_dq(codes, q8, s2)[1].reshape(N, K)
    t2 = time.perf_counter()
    oracle.linear_fwd(x, What, A, B, r, alpha)
    t3 = time.perf_counter()
    oracle.linear_bwd(x, dY, What, A, B, r, alpha)
    t4 = time.perf_counter()
    q_rate, d_rate = N * K / (t1 - t0), N * K / (t2 - t1)
    f_rate = fwd_flops(Ms, N, K, r) / (t3 - t2)
    b_rate = bwd_flops(Ms, N, K, r) / (t4 - t3)
    t_step = 0.0
    for (Nw, Kw) in cfg["weights"].values():
        t_step += Nw * Kw / q_rate + 2 * Nw * Kw / d_rate
        t_step += fwd_flops(M, Nw, Kw, r) / f_rate + bwd_flops(M, Nw, Kw, r) / b_rate
    P = max(1, min(os.cpu_count() or 1, 16))
    procs = [subprocess.Popen([sys.executable, "-c", _CPU_WORKER, ROOT, str(N), str(K),
                               str(syn.seed_of(4, 100 + i))], stdout=subprocess.PIPE)
             for i in range(P)]
    outs = [json.loads(p.communicate()[0].decode().strip().splitlines()[-1]) for p in procs]
    tq = max(o["quantize_s"] for o in outs)
    td = max(o["dequant_s"] for o in outs)
    return {"value": round(step_flops / t_step / 1e12, 6), "unit": "TFLOP/s", "cores": 1,
            "kind": "oracle", "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"one core: quantize + dequantize of the 1024x8192 projection in full, "
                      f"fwd + bwd (dX, dA, dB) on {Ms} of 2048 token rows; the step "
                      f"(7 projections, quantize + 2 dequantizations + fwd + bwd each) "
                      f"extrapolated from those rates to {t_step:.1f} s",
            "extrapolated_step_s": round(t_step, 2), "gpu_speedup": round(t_step / (ms_step * 1e-3), 1),
            "per_op_one_core": {"quantize_params_per_s": round(q_rate, 1),
                                "quantize_gbps": round((2 + 0.515869) * q_rate / 1e9, 3),
                                "dequant_params_per_s": round(d_rate, 1),
                                "dequant_gbps": round(2.515869 * d_rate / 1e9, 3),
                                "fwd_gflops": round(f_rate / 1e9, 3),
                                "bwd_gflops": round(b_rate / 1e9, 3)},
            "all_cores": {"processes": P, "tensor": [N, K],
                          "quantize_params_per_s": round(P * N * K / tq, 1),
                          "dequant_params_per_s": round(P * N * K / td, 1)}}


if __name__ == "__main__":
    main()
