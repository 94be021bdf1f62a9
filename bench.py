#!/usr/bin/env python3
"""Benchmark of the routed top-k MoE layer on codebook-quantized experts (MI355X).

One step = one pass of the whole hot path over one batch: router top-k + renormalised
softmax, token-to-expert grouping, the fused dequant gate/up + SiLU and down kernels,
and the weighted accumulation.  Default workload: the field-shape decode layer
(hidden 2048, 512 experts + 1 shared, expert intermediate 512, IQ2_XS-like weights,
1 token, top-10).  Inputs are resident in HBM before timing starts.  To keep the
256 MB last-level cache from serving the weights, each step reads a different copy of
the layer (--rotate copies, distinct device buffers with identical bytes; by default
enough copies that no byte is read again before at least 256 MB of other weights have
been) and a fresh batch (distinct seeded activations and logits per step).

One-token decode runs the whole layer in one launch (moe_layer_decode_q); the
three-call path (route, gate/up, down fused with the accumulation) is timed beside it.
Multi-token decode runs the three-call path; batched workloads run route -> gate/up ->
down -> accumulate, the experts with many tokens on the matrix cores.

Prints one JSON line.  Usage: python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

WORKLOADS = {
    # name: (bank list, T, k, shared, zipf, path, description)
    "decode_iq2": ([(1, 512)], 1, 10, 1, 0.0, "decode",
                   "decode layer, IQ2_XS-like experts, hidden 2048, 512 experts + 1 shared, inter 512, 1 token, top-10"),
    "decode_iq1_t8": ([(2, 512)], 8, 10, 1, 0.0, "decode",
                      "decode layer, IQ1_M-like experts, hidden 2048, 512 experts + 1 shared, inter 512, 8 tokens, top-10"),
    "prefill_mixed_t256": ([(1, 256), (2, 256)], 256, 10, 0, 0.0, "prefill",
                           "prefill layer, experts 0-255 IQ2_XS-like and 256-511 IQ1_M-like, hidden 2048, inter 512, "
                           "256 tokens, top-10"),
    "prefill_mixed_t256_zipf": ([(1, 256), (2, 256)], 256, 10, 0, 1.1, "prefill",
                                "as prefill_mixed_t256 with Zipf(1.1)-skewed router logits"),
    "decode_iq1s": ([(4, 512)], 1, 10, 1, 0.0, "decode",
                    "decode layer, IQ1_S-like experts (repacked to the IQ1_M-like layout when loaded), hidden 2048, "
                    "512 experts + 1 shared, inter 512, 1 token, top-10; algorithmic bytes of the IQ1_S-like format"),
    "stack48": (None, 1, 10, 1, 0.0, "stack",
                "stack of 48 routed layers (11 IQ2_XS-like, 37 IQ1_M-like), 512 experts + 1 shared each, hidden 2048, "
                "inter 512, top-10, h <- h + MoE(RMSNorm(h)); 1024-token prefill, then 64 single-token decode steps"),
}
METRIC = "tokens/sec per routed MoE layer + achieved HBM GB/s (% of peak) at top-10/512"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0  # dense fp16
H, I, E = 2048, 512, 512
ROOT = os.path.dirname(os.path.abspath(__file__))
# Sources of the kernels whose traffic the counter summaries record, with the digest of their code.
KERNEL_SOURCES = ("codebook_quantized_routed_amd/csrc/common.hpp", "codebook_quantized_routed_amd/csrc/decode.hpp",
                  "codebook_quantized_routed_amd/csrc/matvec_common.hpp",
                  "codebook_quantized_routed_amd/csrc/gemv_dev.hpp", "codebook_quantized_routed_amd/csrc/route_dev.hpp",
                  "codebook_quantized_routed_amd/csrc/k_fused.hip", "codebook_quantized_routed_amd/csrc/k_gemv.hip",
                  "codebook_quantized_routed_amd/csrc/k_router.hip")
TRAFFIC_FILES = {"decode_iq2": "profiles/hbm_traffic_decode_iq2_t1.txt",
                 "stack48": "profiles/hbm_traffic_stack48_decode.txt"}


# Bytes the last-level cache (256 MB) and the eight 4 MB L2s can hold together: a weight
# read again only after more than this many bytes of other weights comes from HBM.
LLC_REUSE_BYTES = 288 << 20


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def rotation_copies(layer, T, k, shared, max_copies=64):
    """Copies of the layer to cycle through so that no weight is read again within
    LLC_REUSE_BYTES of other steps' weights: a step reads at most min(E, T k) routed
    experts plus the shared one; the smallest step is bounded below by k distinct experts
    (one token) and the shared one."""
    E = layer.n_experts
    per_expert = min(layer.expert_bytes(e) for e in range(E + shared))
    step_min = (min(E, k) + shared) * per_expert
    return int(min(max_copies, max(2, -(-LLC_REUSE_BYTES // step_min) + 1)))


def percentiles(samples_ms):
    a = np.sort(np.asarray(samples_ms, dtype=np.float64)) * 1e3
    return {"p10_us": round(float(np.percentile(a, 10)), 3), "p50_us": round(float(np.percentile(a, 50)), 3),
            "p90_us": round(float(np.percentile(a, 90)), 3), "n": int(a.size)}


def step_distribution(step, first, n):
    """Per-step times of n consecutive steps (step(i) for i = first .. first+n-1), from an
    event recorded between every two steps on the launch stream, with the steps queued
    behind a GPU sleep so that the host does not starve the queue.  Each interval holds
    one step plus one event record."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    torch.cuda._sleep(50_000_000)
    ev[0].record()
    for j in range(n):
        step(first + j)
        ev[j + 1].record()
    torch.cuda.synchronize()
    return [ev[j].elapsed_time(ev[j + 1]) for j in range(n)]


def stream_probe(gb, dev, reps=20):
    """Plain streaming kernels over gb GB of fp32, timed with events over reps passes after
    a warm one: a read-only pass (a sum reduction) and a device-to-device copy (read and
    write).  Their rates are what simple streaming code reaches on this GPU, the
    practical ceiling under the 8 TB/s peak."""
    import torch
    n = int(gb * 1e9) // 4
    x = torch.ones(n, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        fn()
        torch.cuda.synchronize(dev)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize(dev)
        return e0.elapsed_time(e1) / reps

    ms_sum = timed(lambda: x.sum())
    ms_copy = timed(lambda: y.copy_(x))
    assert float(y[-1].item()) == 1.0
    out = {"bytes": n * 4, "passes": reps, "peak_gbs": HBM_PEAK_GBS}
    for name, ms, moved in (("sum", ms_sum, n * 4), ("copy", ms_copy, 2 * n * 4)):
        gbs = moved / (ms * 1e-3) / 1e9
        out[name] = {"ms_per_pass": round(ms, 4), "bytes_moved": moved, "achieved_gbs": round(gbs, 1),
                     "frac": round(gbs / HBM_PEAK_GBS, 4)}
    return out


def cpu_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity": len(os.sched_getaffinity(0))}


def oracle_threads():
    """Threads for the oracle's all-core run: the cores this process may use, capped by
    OMP_NUM_THREADS when it is set (the CPU share the machine gives this job)."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    return max(1, min(n, int(env))) if env.isdigit() else n


def _code_only(src: str) -> str:
    """The source without comments and blank space: what the compiler sees of it."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def kernel_digest() -> str:
    """Digest of the code (comments and spacing excluded) of the kernel sources."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f)) as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` (FETCH_SIZE + WRITE_SIZE counters, each scaled by
    the reading of the same counter for a copy of known size) from the committed counter
    summary of this workload; None when there is none or the kernel sources changed after
    the counters were taken."""
    rel = TRAFFIC_FILES.get(workload)
    if rel is None or not os.path.exists(os.path.join(ROOT, rel)):
        return None
    kv = {}
    with open(os.path.join(ROOT, rel)) as fh:
        for line in fh:
            if ":" in line and not line.startswith((" ", "#", "\t")):
                key, val = line.split(":", 1)
                kv[key.strip()] = val.strip()
    if kv.get("kernel_sources_sha256") != kernel_digest():
        return None
    v = kv.get(f"{kernel}.traffic_bytes_per_launch")
    return int(v) if v else None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_iq2", choices=list(WORKLOADS))
    ap.add_argument("--rotate", type=int, default=0,
                    help="distinct copies of the layer cycled through (0: enough that a copy is read again only "
                         "after more than LLC_REUSE_BYTES of other weights)")
    ap.add_argument("--dist-steps", type=int, default=256,
                    help="steps timed one by one for the p10 / p50 / p90 of the step time")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of a captured graph")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle CPU-baseline sample")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="run three device-to-device copies of this size first (counter calibration)")
    ap.add_argument("--stream-probe-gb", type=float, default=0.0,
                    help="only time one read-only pass over this many GB (the reachable HBM read rate) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the layer is data-parallel and needs no exchange between GPUs, "
              "so only --gpus 1 is supported", file=sys.stderr)
        sys.exit(2)

    import torch

    import codebook_quantized_routed_amd as moe
    import synth

    banks, T, k, shared, zipf, path, desc = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.stream_probe_gb > 0:
        print(json.dumps(stream_probe(args.stream_probe_gb, dev)))
        return
    if args.calib_copy_mb:
        src = torch.ones(args.calib_copy_mb << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if path == "stack":
        return run_stack(args, desc)
    kp = k + shared
    n_ids = E + shared

    t0 = time.time()
    layer = synth.make_layer(banks, hidden=H, inter=I, n_experts=E, has_shared=shared, tag="bench/layer")
    c2, c1 = synth.grid_compact(1), synth.grid_compact(2)
    grids = torch.empty(moe.grids_bytes(), dtype=torch.uint8, device=dev)
    moe.grids_expand(torch.from_numpy(c2.view(np.int16)).to(dev), torch.from_numpy(c1.view(np.int16)).to(dev), grids)
    layers = [moe.DeviceLayer(H, I, E, shared, layer.banks, grids)]
    if args.rotate <= 0:  # a copy's bytes come back only after LLC_REUSE_BYTES of other steps' weights
        args.rotate = rotation_copies(layer, T, k, shared)
    for _ in range(args.rotate - 1):  # distinct buffers, identical bytes
        layers.append(layers[0].copy())
    n_in = max(args.steps, args.dist_steps) + args.warmup
    xs = torch.from_numpy(synth.activations(n_in * T, H, tag="bench/x")).to(dev).view(n_in, T, H)
    lgs = torch.from_numpy(synth.logits(n_in * T, E, tag="bench/l", zipf_alpha=zipf)).to(dev).view(n_in, T, E)
    log(f"inputs ready in {time.time() - t0:.1f}s: {args.rotate} x {layers[0].bytes / 1e6:.1f} MB layers")

    i32 = dict(dtype=torch.int32, device=dev)

    def buffers():
        return dict(ids=torch.zeros((T, kp), **i32), w=torch.zeros((T, kp), dtype=torch.float32, device=dev),
                    counts=torch.zeros(n_ids, **i32), offsets=torch.zeros(n_ids + 1, **i32),
                    ss=torch.zeros(T * kp, **i32), sp=torch.zeros(T * kp, **i32),
                    work=torch.zeros(moe.work_ints(T, kp, n_ids), **i32),
                    h=torch.zeros((T * kp, I), dtype=torch.float32, device=dev),
                    y=torch.zeros((T * kp, H), dtype=torch.float32, device=dev) if path == "prefill" else None)

    acc = torch.zeros((n_in, T, H), dtype=torch.float32, device=dev)

    # the steps of the path, each a function of (step index, buffers)
    def k_route(i, b):
        moe.route_group(lgs[i], T, E, k, shared, b["ids"], b["w"], b["counts"], b["offsets"], b["ss"], b["sp"],
                        b["work"])

    def k_gateup(i, b):
        moe.expert_gateup_q(layers[i % len(layers)].desc, xs[i], T, kp, b["ss"], b["work"], b["h"])

    def k_down_acc(i, b):
        moe.expert_down_accumulate_q(layers[i % len(layers)].desc, b["h"], T, kp, b["ids"], b["w"], b["sp"], acc[i])

    def k_down(i, b):
        moe.expert_down_q(layers[i % len(layers)].desc, b["h"], T, kp, b["work"], b["y"])

    def k_accumulate(i, b):
        moe.accumulate(b["y"], b["w"], b["ids"], b["sp"], T, kp, H, acc[i])

    fused = path == "decode" and T == 1
    ws = torch.zeros(moe.decode_workspace_bytes(kp, I) // 4, dtype=torch.int32, device=dev) if fused else None

    def k_layer_decode(i, b):
        moe.layer_decode_q(layers[i % len(layers)].desc, lgs[i], xs[i], k, shared, b["ids"], b["w"], b["counts"],
                           b["offsets"], b["ss"], b["sp"], b["work"], acc[i], ws)

    split = [("route_group", k_route), ("gateup", k_gateup), ("down_accumulate", k_down_acc)]
    if fused:
        kernels = [("layer_decode", k_layer_decode)]
    elif path == "decode":
        kernels = split
    else:
        kernels = [("route_group", k_route), ("gateup", k_gateup), ("down", k_down), ("accumulate", k_accumulate)]

    shared_buf = buffers()

    def step(i):
        for _, fn in kernels:
            fn(i, shared_buf)

    # ---- parity of the first step against the oracle (sampled tokens)
    step(0)
    torch.cuda.synchronize()
    parity = check_parity(layer, c2, c1, xs[0].cpu().numpy(), lgs[0].cpu().numpy(), k, shared,
                          acc[0].cpu().numpy(), shared_buf["ids"].cpu().numpy())
    log(f"parity: {parity}")

    # ---- algorithmic bytes and useful flops per step (from a CPU routing of the same
    # logits, integer-exact): quantized bytes of the distinct experts a step touches
    import oracle as O
    lg_host = lgs.cpu().numpy()
    gu_bytes, dn_bytes, step_bytes = [], [], []
    for i in range(args.warmup, n_in):
        sel, _ = O.route(lg_host[i], k, shared)
        distinct = [int(e) for e in np.unique(sel)]
        gu = sum(2 * synth.matrix_bytes(layer.bank_of(e)[0].qtype, I, H) for e in distinct)
        dn_distinct = sum(synth.matrix_bytes(layer.bank_of(e)[0].qtype, H, I) for e in distinct)
        # the fused decode kernel reads each selected expert's down matrix once per token
        dn = (sum(synth.matrix_bytes(layer.bank_of(int(e))[0].qtype, H, I) for e in sel.ravel())
              if path == "decode" else dn_distinct)
        gu_bytes.append(gu)
        dn_bytes.append(dn)
        step_bytes.append(gu + dn_distinct)
    flops_step = 2.0 * T * kp * 3 * H * I  # useful multiply-adds of the three projections, x2

    # ---- per-kernel timing.  Every timed step is routed first into buffers of its own;
    # then each kernel runs once per step, back to back, queued behind a GPU sleep so the
    # host never starves the queue, between two events on the launch stream.  The same
    # launches appear in a kernel trace of this command.
    K = args.steps
    per = [buffers() for _ in range(K)]
    for j in range(K):
        k_route(args.warmup + j, per[j])
        if path == "prefill":
            k_gateup(args.warmup + j, per[j])
            k_down(args.warmup + j, per[j])

    def back_to_back(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(50_000_000)
        e0.record()
        for j in range(K):
            fn(args.warmup + j, per[j])
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K

    back_to_back(kernels[-1][1])  # warm: code objects and first touches
    kms = {name: back_to_back(fn) for name, fn in kernels}
    if fused:  # the three-call path of the same steps, for comparison
        kms.update({name: back_to_back(fn) for name, fn in split})

    # ---- the router projection in front of the path (logits from the token's x), timed
    # alone over ROUTER_COPIES copies of the fp32 router matrix (more bytes than the
    # last-level cache holds, so each launch reads its matrix from HBM)
    wr_host = synth.router_weights(E, H, tag="bench/router")
    wsg_host = synth.shared_gate_weights(H, tag="bench/router/gate")
    wrs = [torch.from_numpy(wr_host).to(dev) for _ in range(ROUTER_COPIES)]
    wsg = torch.from_numpy(wsg_host).to(dev) if shared else None
    rlg = torch.zeros((T, E), dtype=torch.float32, device=dev)
    rsw = torch.zeros(T, dtype=torch.float32, device=dev) if shared else None

    def k_router(i, b):
        moe.router_logits(xs[i], wrs[i % ROUTER_COPIES], T, H, E, rlg, wsg, rsw)

    k_router(0, None)
    torch.cuda.synchronize()
    router_parity = check_router_parity(xs[0].cpu().numpy(), wr_host, wsg_host if shared else None,
                                        rlg.cpu().numpy(), None if rsw is None else rsw.cpu().numpy())
    log(f"router parity: {router_parity}")
    kms["router"] = back_to_back(k_router)
    router_bytes = (E + (1 if shared else 0)) * H * 4

    # ---- whole-step timing
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    mode = "eager"
    if not args.no_graph:
        try:
            g = torch.cuda.CUDAGraph()
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                with torch.cuda.graph(g, stream=s):
                    for j in range(args.steps):
                        step(args.warmup + j)
            torch.cuda.synchronize()
            g.replay()  # warm replay
            torch.cuda.synchronize()
            start.record()
            g.replay()
            end.record()
            torch.cuda.synchronize()
            mode = "hip-graph"
        except Exception as exc:  # pragma: no cover - reported, then eager timing
            log(f"graph capture failed ({exc}); timing eager launches")
            mode = "eager"
    if mode == "eager":
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        start.record()
        for j in range(args.steps):
            step(args.warmup + j)
        end.record()
        torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    tok_s = T / (ms * 1e-3)
    # the same steps one by one (fresh inputs, the layer copies in rotation), for the
    # spread of the step time
    dist = percentiles(step_distribution(step, args.warmup, args.dist_steps))
    status = 0
    if fused:  # a timed-out wait in any of the one-launch calls above leaves its word set
        status = moe.decode_error(ws)
        if status:
            log("one-launch decode reported a timed-out wait: its results are undefined")

    gu_b, dn_b, st_b = float(np.mean(gu_bytes)), float(np.mean(dn_bytes)), float(np.mean(step_bytes))
    if fused:  # the dominant (only) kernel: the whole layer in one launch
        rl_kernel, rl_b, rl_ms = "k_layer_decode (route + gate/up + down + accumulate, one launch)", gu_b + dn_b, \
            kms["layer_decode"]
        traffic = measured_traffic(args.workload, "k_layer_decode")
    else:
        rl_kernel, rl_b, rl_ms = "gate/up (dequant mat-vec / MFMA + SiLU*up)", gu_b, kms["gateup"]
        traffic = measured_traffic(args.workload, "k_gateup_wide")
    achieved = rl_b / (rl_ms * 1e-3) / 1e9
    dn_name = "down_accumulate" if path == "decode" else "down"
    out = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tokens/s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": desc, "tokens_per_step": T, "experts": E, "shared_experts": shared, "top_k": k,
                   "hidden": H, "inter": I, "rotation_copies": args.rotate,
                   "rotation_bytes": int(args.rotate * layers[0].bytes), "timing": mode},
        "step_time": dict(dist, over="steps timed one by one, an event between every two (each interval holds "
                                      "one step and one event record)"),
        "step_hbm_gbs": round(st_b / (ms * 1e-3) / 1e9, 1),
        "step_hbm_frac": round(st_b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "algorithmic_bytes_per_step": int(st_b),
        "roofline": {"bound": "hbm", "kernel": rl_kernel,
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "bytes_per_launch": int(rl_b), "launch_us": round(rl_ms * 1e3, 3)},
        "gateup": {"achieved_gbs": round(gu_b / (kms["gateup"] * 1e-3) / 1e9, 1), "bytes_per_launch": int(gu_b),
                   "launch_us": round(kms["gateup"] * 1e3, 3)},
        dn_name: {"achieved_gbs": round(dn_b / (kms[dn_name] * 1e-3) / 1e9, 1), "bytes_per_launch": int(dn_b),
                  "launch_us": round(kms[dn_name] * 1e3, 3)},
        "route_group": {"launch_us": round(kms["route_group"] * 1e3, 3)},
        "router": {"kernel": "k_router (logits = x W_r^T, fp32 weights; shared-expert gate)",
                   "launch_us": round(kms["router"] * 1e3, 3), "bytes_per_launch": router_bytes,
                   "achieved_gbs": round(router_bytes / (kms["router"] * 1e-3) / 1e9, 1),
                   "frac_of_hbm_peak": round(router_bytes / (kms["router"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                   "traffic": measured_traffic(args.workload, "k_router"), "parity": router_parity},
        "parity": parity,
        "decode_status": status,
    }
    if path == "prefill":
        ffn_ms = kms["gateup"] + kms["down"]
        tf = flops_step / (ffn_ms * 1e-3) / 1e12
        out["accumulate"] = {"launch_us": round(kms["accumulate"] * 1e3, 3)}
        out["mfma"] = {"useful_tflops": round(tf, 2), "peak": MFMA_PEAK_TFLOPS, "frac": round(tf / MFMA_PEAK_TFLOPS, 4),
                       "flops_per_step": flops_step, "over": "gate/up + down launches"}
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(layer, c2, c1, xs.cpu().numpy(), lgs.cpu().numpy(), k, shared, T,
                                           args.cpu_seconds)
    print(json.dumps(out), flush=True)
    if status or not parity["pass"]:
        sys.exit(1)


def check_router_parity(x, wr, wsg, lg_gpu, sw_gpu, bound=64 * 2.0 ** -24):
    """GPU logits (and gate) against the oracle's fp64 dots, per element relative to
    sum_c |x_c w_c| (the scale of an fp32 dot's rounding error)."""
    import oracle as O
    l64, s64 = O.router_f64(x, wr, wsg)
    scale = O.dot_abs(x, wr)
    worst = float((np.abs(lg_gpu.astype(np.float64) - l64) / scale).max())
    ok = worst <= bound
    out = {"logits_checked": int(l64.size), "max_err_over_abs_dot": float(f"{worst:.3e}"), "bound": bound}
    if wsg is not None:
        gs = O.dot_abs(x, wsg.reshape(1, -1))[:, 0]
        gerr = float(np.max(np.abs(sw_gpu.astype(np.float64) - s64) - 0.25 * bound * gs))
        ok = ok and gerr <= 2.0 ** -23
        out["gate_checked"] = int(s64.size)
    out["pass"] = bool(ok)
    return out


ROUTER_COPIES = 80
STACK_PREFILL_T = 1024
STACK_DECODE_STEPS = 64


def run_stack(args, desc):
    """The 48-layer chain: a 1024-token prefill, then 64 single-token decode steps, each
    layer h <- h + MoE_l(RMSNorm(h)) with its own seeded logits.  The decode steps are
    captured in one graph; each step works in place on its own residual row."""
    import torch

    import codebook_quantized_routed_amd as moe
    import synth
    from codebook_quantized_routed_amd import stack as S

    k, shared = 10, 1
    kp = k + shared
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    host = {qt: synth.make_layer([(qt, E)], hidden=H, inter=I, n_experts=E, has_shared=shared, tag=f"stack/q{qt}")
            for qt in (1, 2)}
    c2, c1 = synth.grid_compact(1), synth.grid_compact(2)
    grids = torch.empty(moe.grids_bytes(), dtype=torch.uint8, device=dev)
    moe.grids_expand(torch.from_numpy(c2.view(np.int16)).to(dev), torch.from_numpy(c1.view(np.int16)).to(dev), grids)
    formats = S.stack_formats(48)
    layers = S.device_stack(formats, {qt: host[qt].banks for qt in host}, grids, H, I, E, shared, dev)
    st = S.LayerStack(layers, k)
    nl = len(layers)
    TP, ND = STACK_PREFILL_T, STACK_DECODE_STEPS
    lg_pre = torch.from_numpy(synth.logits(nl * TP, E, tag="stack/prefill/l")).to(dev).view(nl, TP, E)
    h_pre0 = torch.from_numpy(synth.activations(TP, H, tag="stack/prefill/h")).to(dev)
    lg_dec = torch.from_numpy(synth.logits(ND * nl, E, tag="stack/decode/l")).to(dev).view(ND, nl, 1, E)
    h_dec0 = torch.from_numpy(synth.activations(ND, H, tag="stack/decode/h")).to(dev).view(ND, 1, H)
    log(f"stack ready in {time.time() - t0:.1f}s: {nl} layers, {sum(l.bytes for l in layers) / 1e9:.2f} GB")

    # ---- parity: decode step 0 layer by layer against the oracle, each layer fed the
    # GPU's own input (so the check covers every layer without compounding)
    h = h_dec0[0].clone()
    ins, outs, ids_gpu = [], [], []
    for l in range(nl):
        ins.append(h.cpu().numpy().copy())
        st.layer(l, h, lg_dec[0, l])
        outs.append(h.cpu().numpy().copy())
        ids_gpu.append(st.buffers(1)["ids"].cpu().numpy().copy())
    parity = check_stack_parity(host, formats, c2, c1, ins, outs, ids_gpu, lg_dec[0].cpu().numpy(), k, shared)
    log(f"parity: {parity}")

    # ---- algorithmic bytes of a decode step: each layer's distinct selected experts
    import oracle as O
    lg_host = lg_dec.cpu().numpy()
    step_bytes = []
    for s in range(ND):
        tot = 0
        for l in range(nl):
            sel, _ = O.route(lg_host[s, l], k, shared)
            tot += sum(host[formats[l]].expert_bytes(int(e)) for e in np.unique(sel))
        step_bytes.append(tot)
    dec_bytes = float(np.mean(step_bytes))

    # ---- prefill: warm once, then timed runs
    hp = h_pre0.clone()
    st.step(hp, lg_pre)
    torch.cuda.synchronize()
    n_pre = max(1, min(3, args.steps))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n_pre):
        hp.copy_(h_pre0)
        st.step(hp, lg_pre)
    e1.record()
    torch.cuda.synchronize()
    pre_ms = e0.elapsed_time(e1) / n_pre

    # ---- the one-launch decode of all layers: the same bits as the per-layer chain
    hd_out = torch.zeros_like(h_dec0)
    st.decode(h_dec0[0], hd_out[0], lg_dec[0])
    torch.cuda.synchronize()
    one_launch_exact = bool(np.array_equal(hd_out[0].cpu().numpy().view(np.uint32), outs[-1].view(np.uint32)))
    parity["one_launch_bit_exact_vs_chain"] = one_launch_exact
    log(f"one-launch decode bit-exact against the per-layer chain: {one_launch_exact}")

    # ---- decode: 64 steps captured in one graph, per-layer chain and one launch
    hd = h_dec0.clone()
    chain_ms, mode = time_decode_steps(args, lambda s: st.step(hd[s], lg_dec[s]), ND)
    dec_ms, mode = time_decode_steps(args, lambda s: st.decode(h_dec0[s], hd_out[s], lg_dec[s]), ND)
    dist = percentiles(step_distribution(lambda s: st.decode(h_dec0[s % ND], hd_out[s % ND], lg_dec[s % ND]), 0,
                                         max(ND, args.dist_steps)))
    status = max(st.stack_error(), st.decode_error(1))
    if status:
        log("one-launch decode reported a timed-out wait: its results are undefined")
    per_layer_tok_s = nl / (dec_ms * 1e-3)
    achieved = dec_bytes / (dec_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(per_layer_tok_s, 1),
        "unit": "tokens/s/layer",
        "n_gpus": 1,
        "steps": ND,
        "warmup": 1,
        "ms_per_step": round(dec_ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": desc, "layers": nl, "iq2_layers": formats.count(1), "iq1_layers": formats.count(2),
                   "experts": E, "shared_experts": shared, "top_k": k, "hidden": H, "inter": I,
                   "prefill_tokens": TP, "decode_steps": ND, "timing": mode},
        "decode": {"us_per_step": round(dec_ms * 1e3, 2), "stack_tokens_per_s": round(1e3 / dec_ms, 1),
                   "kernel": "k_stack_decode (one launch, 48 layers)",
                   "per_layer_chain_us_per_step": round(chain_ms * 1e3, 2),
                   "algorithmic_bytes_per_step": int(dec_bytes), "achieved_gbs": round(achieved, 1),
                   "frac_of_hbm_peak": round(achieved / HBM_PEAK_GBS, 4),
                   "step_time": dict(dist, over="decode steps timed one by one, an event between every two")},
        "prefill": {"ms": round(pre_ms, 3), "tokens_per_s_per_layer": round(TP * nl / (pre_ms * 1e-3), 1),
                    "stack_tokens_per_s": round(TP / (pre_ms * 1e-3), 1)},
        "roofline": {"bound": "hbm", "kernel": "k_stack_decode",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic("stack48", "k_stack_decode"),
                     "bytes_per_launch": int(dec_bytes), "launch_us": round(dec_ms * 1e3, 3)},
        "parity": parity,
        "decode_status": status,
    }
    if not args.no_cpu:
        out["cpu_baseline"] = stack_cpu_baseline(host, formats, c2, c1, h_dec0.cpu().numpy(), lg_host, k, shared,
                                                 args.cpu_seconds)
    print(json.dumps(out), flush=True)
    if status or not parity["pass"]:
        sys.exit(1)


def time_decode_steps(args, step, n):
    """Mean time of one decode step: the n steps captured in one graph and replayed once
    after a warm replay (eager launches with --no-graph or when capture fails)."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if not args.no_graph:
        try:
            g = torch.cuda.CUDAGraph()
            s_ = torch.cuda.Stream()
            s_.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s_):
                with torch.cuda.graph(g, stream=s_):
                    for s in range(n):
                        step(s)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / n, "hip-graph"
        except Exception as exc:  # pragma: no cover - reported, then eager timing
            log(f"graph capture failed ({exc}); timing eager launches")
    for s in range(n):
        step(s)
    torch.cuda.synchronize()
    e0.record()
    for s in range(n):
        step(s)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n, "eager"


def check_stack_parity(host, formats, c2, c1, ins, outs, ids_gpu, lg, k, shared, bound=2e-5, bound_delta=3e-5):
    """Each layer l of one decode step: the oracle's h + MoE_l(RMSNorm(h)) from the GPU's
    input h to layer l, against the GPU's output: max |error| within bound of the layer
    output's L2 norm, and within bound_delta of the layer's MoE output (output - input)."""
    import oracle as O
    g = O.grids(c2, c1)
    tabs = {qt: O.ExpertTable(host[qt]) for qt in host}
    worst, worst_d, ok = 0.0, 0.0, True
    for l, (hin, hout) in enumerate(zip(ins, outs)):  # [1][H] each
        x = O.rmsnorm(hin)
        r = O.moe_layer(tabs[formats[l]], g, x, k, shared, logits=lg[l], acc=hin, n_threads=oracle_threads())
        ok &= bool(np.array_equal(r["ids"][0], ids_gpu[l][0]))
        err = float(np.abs(hout[0].astype(np.float64) - r["acc"][0]).max())
        delta = r["acc"][0].astype(np.float64) - hin[0]
        worst = max(worst, err / float(np.linalg.norm(r["acc"][0].astype(np.float64))))
        worst_d = max(worst_d, err / float(np.linalg.norm(delta)))
    return {"layers_checked": len(ins), "ids_bit_exact": ok, "max_err_rel_l2": float(f"{worst:.3e}"),
            "bound": bound, "max_err_rel_delta_l2": float(f"{worst_d:.3e}"), "bound_delta": bound_delta,
            "pass": bool(ok and worst <= bound and worst_d <= bound_delta)}


def stack_cpu_baseline(host, formats, c2, c1, h0, lg, k, shared, budget_s):
    """The oracle's decode step through the whole stack (RMSNorm + layer per layer), on
    all the cores this job may use, over a bounded number of steps; then one thread on
    a sample of layers (every fourth layer of the first step, so both formats)."""
    import oracle as O
    cores = oracle_threads()
    g = O.grids(c2, c1)
    tabs = {qt: O.ExpertTable(host[qt]) for qt in host}
    t0 = time.monotonic()
    n = 0
    while n < 1 or time.monotonic() - t0 < budget_s:
        h = h0[n % len(h0)].astype(np.float32).reshape(1, -1).copy()
        for l in range(len(formats)):
            x = O.rmsnorm(h)
            h = O.moe_layer(tabs[formats[l]], g, x, k, shared, logits=lg[n % len(lg), l], acc=h,
                            n_threads=cores)["acc"]
        n += 1
    dt = time.monotonic() - t0
    sample = list(range(0, len(formats), 4))
    h = h0[0].astype(np.float32).reshape(1, -1).copy()
    t1 = time.monotonic()
    for l in sample:
        O.moe_layer(tabs[formats[l]], g, O.rmsnorm(h), k, shared, logits=lg[0, l], acc=h, n_threads=1)
    dt1 = time.monotonic() - t1
    return {"value": round(n * len(formats) / dt, 3), "unit": "tokens/s/layer", "cores": cores, "kind": "oracle",
            "sample": f"{n} decode step(s) through {len(formats)} layers, {dt:.1f} s, OpenMP over output rows",
            "single_thread": {"value": round(len(sample) / dt1, 3), "unit": "tokens/s/layer", "cores": 1,
                              "sample": f"{len(sample)} layers (every fourth) of one decode step, {dt1:.1f} s"},
            **cpu_info()}


def check_parity(layer, c2, c1, x, lg, k, shared, acc_gpu, ids_gpu, max_tokens=4):
    import oracle as O
    g = O.grids(c2, c1)
    tab = O.ExpertTable(layer)
    T = x.shape[0]
    toks = sorted(set([0, T // 3, (2 * T) // 3, T - 1]))[:max_tokens]
    worst = 0.0
    ok = True
    for t in toks:
        r = O.moe_layer(tab, g, x[t:t + 1], k, shared, logits=lg[t:t + 1], n_threads=oracle_threads())
        ok &= bool(np.array_equal(r["ids"][0], ids_gpu[t]))
        err = np.abs(acc_gpu[t].astype(np.float64) - r["acc"][0]).max() / np.linalg.norm(r["acc"][0])
        worst = max(worst, float(err))
    return {"tokens_checked": len(toks), "ids_bit_exact": ok, "max_err_rel_l2": float(f"{worst:.3e}"),
            "bound": 2e-5, "pass": bool(ok and worst <= 2e-5)}


def time_oracle(run, n_threads, budget_s):
    """Steps of run(i, n_threads) until budget_s has passed (at least one); returns
    (steps, seconds).  Wall clock (CLOCK_MONOTONIC)."""
    t0 = time.monotonic()
    n = 0
    while n < 1 or time.monotonic() - t0 < budget_s:
        run(n, n_threads)
        n += 1
    return n, time.monotonic() - t0


def cpu_baseline(layer, c2, c1, xs, lgs, k, shared, T, budget_s):
    """The oracle as it stands, on the host cores, over a bounded sample of steps: all
    cores this job may use (the reported value), then one thread."""
    import oracle as O
    cores = oracle_threads()
    g = O.grids(c2, c1)
    tab = O.ExpertTable(layer)

    def run(n, threads):  # cycles over the steps' inputs
        O.moe_layer(tab, g, xs[n % len(xs)], k, shared, logits=lgs[n % len(lgs)], n_threads=threads)

    n, dt = time_oracle(run, cores, budget_s)
    n1, dt1 = time_oracle(run, 1, 0.5 * budget_s)
    return {"value": round(n * T / dt, 3), "unit": "tokens/s/layer", "cores": cores, "kind": "oracle",
            "sample": f"{n} steps x {T} token(s) of the same workload, {dt:.1f} s, OpenMP over output rows",
            "single_thread": {"value": round(n1 * T / dt1, 3), "unit": "tokens/s/layer", "cores": 1,
                              "sample": f"{n1} steps, {dt1:.1f} s"},
            **cpu_info()}


if __name__ == "__main__":
    main()
