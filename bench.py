#!/usr/bin/env python3
"""Benchmark of the QLoRA frozen-base hot path on one MI355X.

One step = every row of the path over one batch of synthetic input, on the
two Llama-7B-shaped weights (q 4096x4096 and up 11008x4096, bf16 ~N(0,0.02)):
  1. quantize both weights (bf16 -> NF4 codes + 8-bit absmax codes + scales),
  2. dequantize both to bf16,
  3. decode forward (GEMV path) at M = 1, 4 and 16 tokens, each weight,
  4. training forward at M = 4096 tokens (batch 4 x seq 1024), each weight,
  5. backward dX, dA, dB at M = 4096, each weight (dY ~ N(0,1)),
with LoRA r = 16, alpha = 32, A ~ N(0, 1/K), B ~ N(0, 0.01). The layer
outputs y and the input gradients dX are written in bf16, the compute dtype
of the activations (products accumulate in fp32); dA and dB in fp32. The
same up-weight forward writing an fp32 y is timed beside the step.
`value` is the step's multiply-add work (2 flops per MAC; dequantization and
quantization count no flops) over the host-clock time of exactly K steps
bracketed by device synchronisation, inputs resident in HBM. The timed steps
are replays of the step captured once as a HIP graph (every kernel of the
step runs in each replay; one replay must first match the eager step's
outputs bit for bit); the same K steps called one by one from Python are
timed before it and reported as ms_per_step_eager. Per-call durations (the
breakdown) come from HIP events around each call of the eager steps on the
stream the library launches on; their sum is reported as
ms_per_step_device_calls.
The roofline entry is the dominant kernel: the bf16 MFMA GEMM of
the training forward on the 11008x4096 weight (gemm_nt_kernel, the longest
single dispatch of the step), launched alone through qlora_gemm_bf16_nt on the
same operands (x, the dequantized weight, the rank-r extension) and timed by
HIP events around back-to-back launches; `traffic` is that kernel's HBM bytes per
launch from rocprofv3 FETCH_SIZE / WRITE_SIZE counters scaled by the same
counters' reading for a copy of known size, and null when the kernel source no
longer matches the one the counters were taken on. The CPU baseline times the
oracle on a bounded sample of the same workload. Extra sections (skipped
with --no-extras): the decode GEMV on a ring of distinct weights, bulk
quantize/dequant throughput, merge + requantize, the AdamW step, and the
70B-shaped layer (seven projections, M = 2048, r = 64) forward + backward.

Counter helpers: `--only CALL` runs one call of the step (e.g. fwd_train_up)
or the roofline launch (gemm_nt_up) for the timed iterations and prints its
mean time; `--copy-calibration BYTES` runs a device-to-device copy of BYTES
bytes (the reference reading for the counter scale).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "NF4 dequant-GEMM TFLOP/s & GEMV weight GB/s (fraction of roofline) per layer"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E

# HBM traffic of gemm_nt_kernel per launch at x [4096,4096], W [11008,4096]
# bf16, y fp32, from rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch)
# scaled by the counters' reading for a copy of known size. Valid while the
# kernel source hashes to `src_sha256` (None: not measured for this source).
# Layer outputs y and input gradients dX are produced in bf16, the compute
# dtype of the activations; products accumulate in fp32 either way.
ACT_DTYPE_NAME = "bfloat16"

TRAFFIC = {"kernel": "gemm_nt_kernel", "call": "gemm_nt_up", "src": "gemm_nt.hip",
           "y_dtype": "torch.bfloat16",
           "src_sha256": "bd18272f248079780132020c565b3573d3670bae25308ad6f52d9974951eea0f",
           "fetch_bytes": 591671954,   # 288929 KiB x 2.000 (copy reference)
           "write_bytes": 90177536}    # 88064 KiB x 1.000 (copy reference)


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def nf4_bytes(N, K):
    n = N * K
    nb = n // 64
    return n // 2 + nb + 4 * ((nb + 255) // 256)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the GEMV ring and bulk quantize/dequant bandwidth runs")
    ap.add_argument("--only", default=None, help="run only this call of the step (counter runs)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="time a device copy of BYTES bytes and exit (counter scale reference)")
    return ap.parse_args()


def kernel_src_sha(name):
    import hashlib
    path = os.path.join(ROOT, "qlora_fine_tuning_blockwise_amd", "csrc", name)
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


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


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, args.steps)
        return
    import numpy as np
    import torch

    import qlora_fine_tuning_blockwise_amd as q
    from qlora_fine_tuning_blockwise_amd import synthetic as syn

    ACT_DTYPE = getattr(torch, ACT_DTYPE_NAME)

    q._lib.load()  # fail loudly if the HIP library is not built
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = syn.LLAMA7B_TRAIN
    r, alpha, Mt = cfg["r"], cfg["alpha"], cfg["M"]
    Mdec = syn.LLAMA7B_DECODE["M"]
    names = list(cfg["weights"])

    # ------------------------------------------------------------ inputs (resident)
    W, A, B, dY, nf4, deq, yb = {}, {}, {}, {}, {}, {}, {}
    for i, name in enumerate(names):
        N, K = cfg["weights"][name]
        W[name] = syn.torch_normal_bf16((N, K), cfg["w_std"], syn.seed_of(3, i), dev)
        A[name] = syn.torch_normal_bf16((K, r), 1.0 / K ** 0.5, syn.seed_of(3, 10 + i), dev)
        B[name] = syn.torch_normal_bf16((r, N), 0.01, syn.seed_of(3, 20 + i), dev)
        dY[name] = syn.torch_normal_bf16((Mt, N), 1.0, syn.seed_of(3, 30 + i), dev)
        nf4[name] = q.qlora_quantize_nf4_dq(W[name])
        deq[name] = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    K0 = cfg["weights"][names[0]][1]
    x_train = syn.torch_normal_bf16((Mt, K0), 1.0, syn.seed_of(3, 40), dev)
    x_dec = {M: syn.torch_normal_bf16((M, K0), 1.0, syn.seed_of(2, 40 + M), dev) for M in Mdec}
    ws_bytes = max(max(q.qlora_workspace_bytes(0, M, *cfg["weights"][n], r) for M in Mdec + (Mt,))
                   for n in names)
    ws_bytes = max(ws_bytes, max(q.qlora_workspace_bytes(1, Mt, *cfg["weights"][n], r)
                                 for n in names))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = {}
    for name in names:
        N, K = cfg["weights"][name]
        out[name] = dict(
            ydec={M: torch.empty((M, N), dtype=ACT_DTYPE, device=dev) for M in Mdec},
            y=torch.empty((Mt, N), dtype=ACT_DTYPE, device=dev),
            u=torch.empty((Mt, r), dtype=torch.float32, device=dev))

    # ------------------------------------------------------------ flops per call
    def fwd_flops(M, N, K):
        return 2 * M * N * K + 2 * M * r * (K + N)

    def bwd_flops(M, N, K):
        return 2 * M * N * K + 2 * M * r * (N + K) + 2 * M * K * r + 2 * M * N * r

    calls = []  # (label, fn, flops, bytes)
    for name in names:
        N, K = cfg["weights"][name]
        w = nf4[name]
        o = out[name]
        calls.append((f"quantize_{name}", lambda w=w, name=name: q.qlora_quantize_nf4_dq(W[name], out=w),
                      0, 2 * N * K + nf4_bytes(N, K)))
        calls.append((f"dequant_{name}", lambda w=w, name=name: q.qlora_dequant_bf16(w, out=deq[name]),
                      0, nf4_bytes(N, K) + 2 * N * K))
    for name in names:
        N, K = cfg["weights"][name]
        w = nf4[name]
        o = out[name]
        for M in Mdec:
            calls.append((f"fwd_decode_M{M}_{name}",
                          lambda w=w, o=o, M=M, name=name: q.qlora_linear_fwd(
                              w, x_dec[M], A[name], B[name], alpha, y=o["ydec"][M], workspace=ws),
                          fwd_flops(M, N, K),
                          nf4_bytes(N, K) + 2 * (M * K + K * r + r * N) + 4 * M * N))
    for name in names:
        N, K = cfg["weights"][name]
        w = nf4[name]
        o = out[name]
        calls.append((f"fwd_train_{name}",
                      lambda w=w, o=o, name=name: q.qlora_linear_fwd(
                          w, x_train, A[name], B[name], alpha, y=o["y"], u_out=o["u"],
                          workspace=ws),
                      fwd_flops(Mt, N, K), 0))
        calls.append((f"bwd_train_{name}",
                      lambda w=w, o=o, name=name: o.__setitem__("grads", q.qlora_linear_bwd(
                          w, x_train, dY[name], A[name], B[name], alpha, u_saved=o["u"],
                          dx_dtype=ACT_DTYPE, workspace=ws)),
                      bwd_flops(Mt, N, K), 0))
    step_flops = sum(c[2] for c in calls)

    # The roofline launch: the forward's dense stage on the up weight alone.
    Nu, Ku = cfg["weights"]["up"]
    # The weight in the K-slab layout the forward's large-M path dequantizes to.
    w_up_slab = q.qlora_dequant_bf16(nf4["up"], layout=q.LAYOUT_KSLAB32)
    e_up = syn.torch_normal_bf16((Mt, 2 * r), 0.01, syn.seed_of(3, 50), dev)
    f_up = B["up"].t().contiguous()
    y_up = torch.empty((Mt, Nu), dtype=ACT_DTYPE, device=dev)
    roof = ("gemm_nt_up",
            lambda: q.qlora_gemm_bf16_nt(x_train, w_up_slab, e_up, f_up, y=y_up,
                                         b_layout=q.LAYOUT_KSLAB32),
            2 * Mt * Nu * Ku + 2 * Mt * (2 * r) * Nu, 0)
    if args.only:
        sel = [c for c in calls + [roof] if c[0] == args.only]
        if not sel:
            sys.exit(f"--only: no call named {args.only}; "
                     f"calls: {[c[0] for c in calls + [roof]]}")
        label, fn, flops, _ = sel[0]
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        print(json.dumps({"call": label, "steps": args.steps, "ms": round(ms, 5),
                          "tflops": round(flops / (ms * 1e-3) / 1e12, 2) if flops else None}),
              flush=True)
        return

    stream = torch.cuda.current_stream()

    def step(ev=None):
        for i, (label, fn, _, _) in enumerate(calls):
            if ev is not None:
                ev[i][0].record(stream)
            fn()
            if ev is not None:
                ev[i][1].record(stream)

    log("inputs ready; warmup", args.warmup)
    for _ in range(args.warmup):
        step()
    # Timed region: exactly K steps, bracketed by device synchronisation; the
    # host does not wait inside it (the stream stays full), every call of
    # every step is bracketed by its own pair of events.
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in calls] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    log("timed", args.steps, "steps")
    per_call = [sum(evs[k][i][0].elapsed_time(evs[k][i][1]) for k in range(args.steps))
                for i in range(len(calls))]
    ms_step_eager = (t1 - t0) * 1e3 / args.steps
    ms_step_dev = sum(per_call) / args.steps

    # The step captured once as a HIP graph. Called one by one, the small
    # calls cost the host more time (argument handling, 30-50 us each) than
    # their kernels take, and the device idles in between; the replay issues
    # the same kernels with the same arguments back to back. Before it is
    # timed, one replay must reproduce the eager step's outputs bit for bit.
    def outputs():
        res = []
        for n in names:
            o = out[n]
            res += [nf4[n].codes, nf4[n].absmax_q, nf4[n].absmax_scale, deq[n], o["y"], o["u"],
                    *o["ydec"].values(), *o["grads"]]
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
    # Timed region: exactly K replays of the step, bracketed by device
    # synchronisation. `value` is the step work over their host-clock time.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    log("timed", args.steps, "graph replays")
    ms_step_host = (t1 - t0) * 1e3 / args.steps
    value = step_flops / (ms_step_host * 1e-3) / 1e12

    breakdown = {}
    for (label, _, flops, nbytes), tot in zip(calls, per_call):
        ms = tot / args.steps
        e = {"ms": round(ms, 5)}
        if flops:
            e["tflops"] = round(flops / (ms * 1e-3) / 1e12, 2)
            e["frac_bf16_peak"] = round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
        if nbytes:
            e["gbps"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
            e["frac_hbm_peak"] = round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)
        breakdown[label] = e
    # dominant kernel: the forward GEMM on the larger weight, launched alone
    _, rfn, dflops, _ = roof
    for _ in range(args.warmup):
        rfn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        rfn()
    e1.record(stream)
    torch.cuda.synchronize()
    dms = e0.elapsed_time(e1) / args.steps
    achieved = dflops / (dms * 1e-3) / 1e12
    traffic = None
    if (TRAFFIC["src_sha256"] and TRAFFIC["src_sha256"] == kernel_src_sha(TRAFFIC["src"])
            and TRAFFIC["y_dtype"] == str(ACT_DTYPE)):
        traffic = TRAFFIC["fetch_bytes"] + TRAFFIC["write_bytes"]
    # The forward on the up weight with an fp32 y, beside the bf16-y step.
    o_up = out["up"]
    y_f32 = torch.empty((Mt, Nu), dtype=torch.float32, device=dev)
    f32fn = lambda: q.qlora_linear_fwd(nf4["up"], x_train, A["up"], B["up"], alpha, y=y_f32,
                                       u_out=o_up["u"], workspace=ws)
    for _ in range(args.warmup):
        f32fn()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        f32fn()
    e1.record(stream)
    torch.cuda.synchronize()
    f32ms = e0.elapsed_time(e1) / args.steps
    breakdown["fwd_train_up_y_f32"] = {
        "ms": round(f32ms, 5), "tflops": round(fwd_flops(Mt, Nu, Ku) / (f32ms * 1e-3) / 1e12, 2),
        "note": "outside the step: the same forward writing y in fp32"}
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic, "kernel": TRAFFIC["kernel"], "kernel_call": roof[0],
                "shape": {"M": Mt, "N": Nu, "K": Ku, "r": r}, "flops_per_launch": dflops,
                "avg_ms": round(dms, 5)}

    result = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step_host, 4),
        "ms_per_step_device_calls": round(ms_step_dev, 4),
        "ms_per_step_eager": round(ms_step_eager, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "llama7b_nf4_layer_pair: q 4096x4096 + up 11008x4096 bf16 "
                               "N(0,0.02) -> NF4+DQ; decode M=1,4,16; train M=4096 fwd+bwd; "
                               "y and dX bf16 (fp32 accumulation), dA and dB fp32",
                   "weights": {n: list(cfg["weights"][n]) for n in names},
                   "M_decode": list(Mdec), "M_train": Mt, "r": r, "alpha": alpha},
        "roofline": roofline, "breakdown": breakdown,
    }

    if not args.no_extras:
        log("gemv ring")
        result["gemv_ring"] = gemv_ring(q, syn, torch, dev, r, alpha)
        log("bulk quantize/dequant")
        result["bulk_quantize"] = bulk_quantize(q, syn, torch, dev)
        log("merge + requantize")
        result["merge"] = merge_section(q, syn, torch, dev, cfg, nf4, W, A, B, r, alpha)
        log("adamw step on the adapter arena")
        result["adamw"] = adamw_section(q, syn, torch, dev)
        log("70B-shaped layer fwd + bwd")
        result["layer_70b"] = layer_70b(q, syn, torch, dev, ACT_DTYPE)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(np, syn, cfg, step_flops, ms_step_host)
    print(json.dumps(result), flush=True)


def merge_section(q, syn, torch, dev, cfg, nf4, W, A, B, r, alpha, iters=10):
    """Adapter merge on the up weight: the merge into the 4-bit base
    (dequantize + s (AB)^T in binary32, fp32 out) and its requantization, each
    timed with HIP events; plus the relative Frobenius error of the
    requantized weight against the exact 16-bit merge W + s (AB)^T, for the
    4-bit path and for the clean path (merge into the bf16 weight, quantize
    once) that the pages recommend."""
    N, K = cfg["weights"]["up"]
    w = nf4["up"]
    merged = torch.empty((N, K), dtype=torch.float32, device=dev)
    ws = torch.empty(q.qlora_workspace_bytes(2, 0, N, K, r), dtype=torch.uint8, device=dev)
    wq = q.qlora_quantize_nf4_dq(merged)

    def timed(fn):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    ms_m = timed(lambda: q.qlora_merge_lora(A["up"], B["up"], alpha, w=w, out=merged, workspace=ws))
    ms_q = timed(lambda: q.qlora_quantize_nf4_dq(merged, out=wq))
    m_bytes = nf4_bytes(N, K) + 2 * r * (N + K) + 4 * N * K
    q_bytes = 4 * N * K + nf4_bytes(N, K)
    # errors against the exact 16-bit merge (measurement only)
    q.qlora_merge_lora(A["up"], B["up"], alpha, w=w, out=merged, workspace=ws)
    q.qlora_quantize_nf4_dq(merged, out=wq)
    back4 = q.qlora_dequant_bf16(wq).float()
    exact = q.qlora_merge_lora(A["up"], B["up"], alpha, W=W["up"], workspace=ws)
    wc = q.qlora_quantize_nf4_dq(exact)
    backc = q.qlora_dequant_bf16(wc).float()
    nrm = torch.linalg.norm(exact)
    e4 = float(torch.linalg.norm(back4 - exact) / nrm)
    ec = float(torch.linalg.norm(backc - exact) / nrm)
    return {"weight": [N, K], "r": r,
            "merge_4bit_base": {"ms": round(ms_m, 5), "gbps": round(m_bytes / (ms_m * 1e-3) / 1e9, 1),
                                "frac_hbm_peak": round(m_bytes / (ms_m * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)},
            "requantize_f32": {"ms": round(ms_q, 5), "gbps": round(q_bytes / (ms_q * 1e-3) / 1e9, 1),
                               "frac_hbm_peak": round(q_bytes / (ms_q * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)},
            "rel_err_vs_16bit_merge": {"merge_into_4bit_then_requantize": round(e4, 5),
                                       "merge_into_bf16_then_quantize": round(ec, 5)}}


def adamw_section(q, syn, torch, dev, iters=10):
    """AdamW on every adapter of a Llama-7B decoder at rank 16 (one flat
    arena, bf16 gradients, bf16 copy written): 28 bytes per parameter. Timed
    with HIP events with the state in HBM, then with the master values and
    moments in pinned host memory (the paged state; 24 of the 28 bytes cross
    the host link)."""
    n = syn.adapter_arena_params()
    g = torch.empty(n, dtype=torch.bfloat16, device=dev).normal_(0.0, 1e-2)
    pb = torch.empty(n, dtype=torch.bfloat16, device=dev)
    res = {"params": n, "bytes_per_param": 28}

    def run(where, P, M, V):
        step = [0]

        def one():
            step[0] += 1
            q.qlora_adamw_step(P, g, M, V, step=step[0], lr=2e-4, weight_decay=0.01,
                               param_bf16=pb)
        for _ in range(2):
            one()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        k = iters if where == "hbm" else 3
        e0.record()
        for _ in range(k):
            one()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / k
        gbps = 28 * n / (ms * 1e-3) / 1e9
        res[where] = {"ms": round(ms, 4), "gbps": round(gbps, 1),
                      "params_per_s": round(n / (ms * 1e-3), 1)}
        if where == "hbm":
            res[where]["frac_hbm_peak"] = round(gbps / PEAK_HBM_GBPS, 4)

    P = torch.empty(n, dtype=torch.float32, device=dev).normal_(0.0, 0.02)
    M = torch.zeros(n, dtype=torch.float32, device=dev)
    V = torch.zeros(n, dtype=torch.float32, device=dev)
    run("hbm", P, M, V)
    Ph, Mh, Vh = (t.cpu().pin_memory() for t in (P, M, V))
    del P, M, V
    run("pinned_host", Ph, Mh, Vh)
    return res


def layer_70b(q, syn, torch, dev, act_dtype, iters=5):
    """The 70B-shaped decoder layer: all seven projections (q, o 8192x8192;
    k, v 1024x8192; gate, up 28672x8192; down 8192x28672) quantized to NF4 +
    DQ from bf16 N(0, 0.015), then forward and backward (dX, dA, dB) of each
    at M = 2048 tokens, LoRA r = 64, alpha = 16, y and dX in the activations'
    bf16. Timed by HIP events around `iters` passes over the seven
    projections (after one warmup pass)."""
    cfg = syn.LAYER_70B
    M, r, alpha = cfg["M"], cfg["r"], cfg["alpha"]
    names = list(cfg["weights"])
    ws_bytes = max(max(q.qlora_workspace_bytes(op, M, N, K, r) for op in (0, 1))
                   for N, K in cfg["weights"].values())
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    layer = {}
    for t, name in enumerate(names):
        N, K = cfg["weights"][name]
        Wb = syn.torch_normal_bf16((N, K), cfg["w_std"], syn.seed_of(4, t), dev)
        w = q.qlora_quantize_nf4_dq(Wb)
        del Wb
        layer[name] = dict(
            w=w, A=syn.torch_normal_bf16((K, r), 1.0 / K ** 0.5, syn.seed_of(4, 10 + t), dev),
            B=syn.torch_normal_bf16((r, N), 0.01, syn.seed_of(4, 20 + t), dev),
            x=syn.torch_normal_bf16((M, K), 1.0, syn.seed_of(4, 30 + t), dev),
            dY=syn.torch_normal_bf16((M, N), 1.0, syn.seed_of(4, 40 + t), dev),
            y=torch.empty((M, N), dtype=act_dtype, device=dev),
            u=torch.empty((M, r), dtype=torch.float32, device=dev))
    flops = 0
    for name in names:
        N, K = cfg["weights"][name]
        flops += 2 * M * N * K + 2 * M * r * (K + N)  # forward
        flops += 2 * M * N * K + 2 * M * r * (N + K) + 2 * M * K * r + 2 * M * N * r  # backward

    def one_pass():
        for name in names:
            L = layer[name]
            q.qlora_linear_fwd(L["w"], L["x"], L["A"], L["B"], alpha, y=L["y"], u_out=L["u"],
                               workspace=ws)
            q.qlora_linear_bwd(L["w"], L["x"], L["dY"], L["A"], L["B"], alpha, u_saved=L["u"],
                               dx_dtype=act_dtype, workspace=ws)

    one_pass()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        one_pass()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    tf = flops / (ms * 1e-3) / 1e12
    del layer, ws
    torch.cuda.empty_cache()
    return {"projections": {n: list(cfg["weights"][n]) for n in names}, "M": M, "r": r,
            "alpha": alpha, "ms_fwd_bwd": round(ms, 4), "tflops": round(tf, 2),
            "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "tokens_per_s": round(M / (ms * 1e-3), 1)}


def gemv_ring(q, syn, torch, dev, r, alpha):
    """Decode GEMV weight bandwidth on a ring of distinct 11008x4096 weights
    (> 512 MB of NF4, past the 256 MB Infinity Cache)."""
    N, K = 11008, 4096
    nw = 24
    base = syn.torch_normal_bf16((N, K), 0.02, 777, dev)
    ring = [q.qlora_quantize_nf4_dq(base) for _ in range(nw)]
    for w in ring[1:]:  # distinct contents: perturb the codes bytes
        w.codes.copy_(ring[0].codes.roll(1))
    del base
    A = syn.torch_normal_bf16((K, r), 1.0 / K ** 0.5, 778, dev)
    B = syn.torch_normal_bf16((r, N), 0.01, 779, dev)
    res = {"weight": [N, K], "ring_weights": nw, "ring_mb": round(nw * nf4_bytes(N, K) / 1e6, 1)}
    for M in (1, 4, 16):
        x = syn.torch_normal_bf16((M, K), 1.0, 780 + M, dev)
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
        ws = torch.empty(q.qlora_workspace_bytes(0, M, N, K, r), dtype=torch.uint8, device=dev)
        for w in ring:
            q.qlora_linear_fwd(w, x, A, B, alpha, y=y, workspace=ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 4
        e0.record()
        for _ in range(reps):
            for w in ring:
                q.qlora_linear_fwd(w, x, A, B, alpha, y=y, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / (reps * nw)
        wbytes = nf4_bytes(N, K) + 2 * (K * r + r * N)
        gbps = wbytes / (ms * 1e-3) / 1e9
        res[f"M{M}"] = {"us_per_call": round(ms * 1e3, 2), "weight_gbps": round(gbps, 1),
                        "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4),
                        "tokens_per_s": round(M / (ms * 1e-3), 1)}
    del ring
    torch.cuda.empty_cache()
    return res


def bulk_quantize(q, syn, torch, dev):
    """Quantize and dequantize bandwidth on one 8192x28672 bf16 tensor (470 MB
    in, past the Infinity Cache), in each second-level format, with the
    format's error on that heavy-tailed tensor: the relative error of the
    reconstructed block constants c1_hat against the exact block absmax
    (median and 99th percentile over non-zero blocks) and the relative
    Frobenius error of the dequantized weight."""
    N, K = syn.BULK_65B["tensor"]
    Wt = syn.torch_student_t_outliers_bf16((N, K), 4242, dev)
    out = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    # measurement only: the exact block constants and the norm of W
    c1 = Wt.float().abs().view(-1, 64).amax(dim=1)
    nz = c1 > 0
    wnorm = torch.linalg.norm(Wt.float())
    res = {"tensor": [N, K]}
    for fmt, name in ((q.DQ_INT8, None), (q.DQ_UINT8, "uint8"), (q.DQ_E4M3, "e4m3")):
        w = q.qlora_quantize_nf4_dq(Wt, dq_format=fmt)
        sec = res if name is None else res.setdefault(name, {})
        for label, fn, nbytes in (("quantize", lambda: q.qlora_quantize_nf4_dq(Wt, out=w),
                                   2 * N * K + nf4_bytes(N, K)),
                                  ("dequant", lambda: q.qlora_dequant_bf16(w, out=out),
                                   nf4_bytes(N, K) + 2 * N * K)):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 10
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            gbps = nbytes / (ms * 1e-3) / 1e9
            sec[label] = {"ms": round(ms, 4), "gbps": round(gbps, 1),
                          "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4),
                          "params_per_s": round(N * K / (ms * 1e-3), 1)}
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
    del Wt, out, c1, nz
    torch.cuda.empty_cache()
    return res


def cpu_baseline(np, syn, cfg, step_flops, ms_step):
    """The oracle (single-threaded C) on a bounded sample of the step: quantize
    and dequantize both weights in full, then forward and backward (dX, dA, dB)
    on 32 of the 4096 token rows for both weights. Rate = sample flops / time."""
    import oracle

    r, alpha = cfg["r"], cfg["alpha"]
    Ms = 32
    flops = 0
    dt = 0.0
    for i, (name, (N, K)) in enumerate(cfg["weights"].items()):
        Wb = syn.normal_bf16((N, K), cfg["w_std"], syn.seed_of(3, i))
        x = syn.normal_bf16((Ms, K), 1.0, syn.seed_of(3, 50))
        A = syn.normal_bf16((K, r), 1.0 / K ** 0.5, syn.seed_of(3, 10 + i))
        B = syn.normal_bf16((r, N), 0.01, syn.seed_of(3, 20 + i))
        dY = syn.normal_bf16((Ms, N), 1.0, syn.seed_of(3, 30 + i))
        t0 = time.perf_counter()
        codes, q8, s2 = oracle.quantize_nf4_dq(Wb, "bf16")
        What = oracle.dequant_dq(codes, q8, s2)[1].reshape(N, K)
        oracle.linear_fwd(x, What, A, B, r, alpha)
        oracle.linear_bwd(x, dY, What, A, B, r, alpha)
        dt += time.perf_counter() - t0
        flops += 2 * Ms * N * K + 2 * Ms * r * (K + N)
        flops += 2 * Ms * N * K + 2 * Ms * r * (N + K) + 2 * Ms * K * r + 2 * Ms * N * r
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"quantize+dequantize both weights in full, then fwd + bwd (dX, dA, dB) on "
                      f"{Ms} of 4096 token rows per weight; {flops / 1e9:.2f} GFLOP in "
                      f"{dt:.1f} s on one host core"}


if __name__ == "__main__":
    main()
