#!/usr/bin/env python3
"""Decode benchmark for one HFQ4 top-k MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--mode graph|eager]

A step is one pass of the whole decode hot path for one token through one
MoE layer (d=2048, expert FFN 512, 256 experts, top-8): router GEMV, top-k
and renormalised softmax, grouped gate/up dequant-GEMV, SiLU(gate)*up, down
dequant-GEMV with the routing-weighted combine -- one moe_layer_decode
call.  Inputs are seeded synthetic weights (HFQ4-packed on the device) and
activations, resident in HBM before timing starts.  To keep the 256 MB
Infinity Cache from serving repeats, steps cycle over 32 distinct layer
replicas (each with its own router, 13.8 GB in all) and a pool of 4096
fresh activation vectors.

Prints one JSON line: expert-weight GB/s (metric value), tokens/s, the
dominant kernel's roofline and the CPU oracle timed on a bounded sample.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer decode expert-weight GB/s (% of HBM peak) and tokens/s at top-8"
HBM_PEAK_GBS = 8000.0
D, F, E, K_TOP = 2048, 512, 256, 8
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic_moe_layer_c2.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sources_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_moe_decode_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def load_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    or None if absent or taken on other kernel sources."""
    try:
        with open(PROFILE_TRAFFIC) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sources_sha256") != kernel_sources_digest():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(torch, layers_f32_seed, xs_host, routers_host, budget_s):
    """The oracle (numpy float64) on the first tokens of the same workload,
    timed on the host cores; experts are quantized by the oracle before
    timing starts, as the GPU path gets pre-packed weights."""
    import numpy as np
    from oracle import moe
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    spent, n, t_total = 0.0, 0, 0.0
    seed = layers_f32_seed
    while spent < budget_s and n < len(xs_host):
        r = n % len(routers_host)
        x = xs_host[n:n + 1]
        Wr = routers_host[r]
        idx, _, _ = moe.route(Wr, x, K_TOP)
        exps = {}
        for e in idx[0]:
            g, u, dn = synth.expert_f32(torch, "cuda", seed, r, int(e), D, F)
            exps[int(e)] = moe.PackedExpert.from_f32(g.cpu().numpy(), u.cpu().numpy(),
                                                     dn.cpu().numpy())
        t0 = time.perf_counter()
        moe.moe_layer(x, Wr, exps, K_TOP)
        dt = time.perf_counter() - t0
        t_total += dt
        spent += dt
        n += 1
    per_tok = t_total / n
    return {"value": round(K_TOP * 1671168 / per_tok / 1e9, 4), "unit": "GB/s",
            "cores": threads, "kind": "oracle",
            "sample": "%d single-token layer calls of the same workload (replica r = token mod 32), "
                      "%.1f s of oracle time, %.3f s per token-layer; quantization untimed" %
                      (n, t_total, per_tok),
            "tokens_per_s": round(1.0 / per_tok, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20000)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--mode", choices=["graph", "eager"], default="graph")
    ap.add_argument("--path", choices=["fused", "split"], default="fused")
    ap.add_argument("--replicas", type=int, default=32)
    ap.add_argument("--pool", type=int, default=4096)
    ap.add_argument("--graph-steps", type=int, default=512)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--kernel-samples", type=int, default=40)
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one device copy of 1 GiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import quantized_moe_decode_amd as q
    import quantized_moe_decode_amd.synthetic as syn
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda"
    torch.cuda.set_device(0)

    t0 = time.time()
    layers = [syn.build_layer(torch, seed=0, layer_id=r, E=E, d=D, F=F, device=dev)
              for r in range(args.replicas)]
    xs = synth.activations(torch, dev, 1, args.pool, D)
    torch.cuda.synchronize()
    log("built %d replicas in %.1f s" % (args.replicas, time.time() - t0))

    ws = q.new_workspace(layers[0], 1, K_TOP, dev)
    idx = torch.empty((1, K_TOP), dtype=torch.int32, device=dev)
    wts = torch.empty((1, K_TOP), dtype=torch.float32, device=dev)
    y = torch.empty((1, D), dtype=torch.float32, device=dev)
    if args.path == "split":
        ws2 = q.new_workspace(layers[0], 1, K_TOP, dev)

    def step(i):
        L = layers[i % args.replicas]
        x = xs[i % args.pool:i % args.pool + 1]
        if args.path == "fused":
            q.moe_layer_decode(L, x, K_TOP, ws, y=y, idx=idx, wts=wts)
        else:
            q.moe_route_topk(L.Wr, x, K_TOP, ws=ws2, idx=idx, wts=wts)
            q.moe_expert_decode(L, x, idx, wts, ws, y=y)

    stream = torch.cuda.current_stream()
    if args.mode == "graph":
        G = args.graph_steps
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(stream)
        with torch.cuda.stream(s):
            for i in range(2):
                step(i)
        stream.wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(G):
                step(i)
        torch.cuda.synchronize()
        reps_w = max(1, args.warmup // G)
        reps = max(1, args.steps // G)
        steps = reps * G
        warm = reps_w * G
        run = lambda: [g.replay() for _ in range(reps)]
        run_w = lambda: [g.replay() for _ in range(reps_w)]
    else:
        steps, warm = args.steps, args.warmup
        run = lambda: [step(i) for i in range(steps)]
        run_w = lambda: [step(i) for i in range(warm)]

    run_w()
    torch.cuda.synchronize()
    err = q.workspace_error(ws)
    if err:
        raise SystemExit("device error word %d after warmup" % err)
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    run()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    gpu_ms = ev0.elapsed_time(ev1)
    err = q.workspace_error(ws)
    if err:
        raise SystemExit("device error word %d after timed run" % err)

    # Live duration of each kernel of the step, from the library's phase
    # stamps (s_memrealtime at 100 MHz, thread 0 of every workgroup): a second
    # graph of the same steps is captured with stamping on, and after each
    # replay the last step's kernels give first-workgroup-start to
    # last-workgroup-end.  The stamps cost a few stores per workgroup.
    kern = None
    if args.mode == "graph" and args.path == "fused":
        import ctypes
        tr = torch.zeros(4 * 1024 * 8, dtype=torch.int64, device=dev)
        q.lib.hfq4_debug_set_trace(ctypes.c_void_p(tr.data_ptr()), tr.numel() * 8)
        gt = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gt):
            for i in range(G):
                step(i)
        q.lib.hfq4_debug_set_trace(None, 0)
        samples = {"logits": [], "gateup": [], "down": [], "step": []}
        nwg = {0: E, 1: torch.cuda.get_device_properties(0).multi_processor_count, 2: D // 8}
        for rep in range(args.kernel_samples):
            gt.replay()
            torch.cuda.synchronize()
            t = tr.view(4, 1024, 8).cpu().numpy()
            st, en = {}, {}
            for kk, last in ((0, 1), (1, 5), (2, 3)):
                n = min(nwg[kk], 1024)
                st[kk] = int(t[kk, :n, 0].min())
                en[kk] = int(t[kk, :n, last].max())
            samples["logits"].append((en[0] - st[0]) / 100.0)
            samples["gateup"].append((en[1] - st[1]) / 100.0)
            samples["down"].append((en[2] - st[2]) / 100.0)
            samples["step"].append((en[2] - st[0]) / 100.0)
        kern = {k: (sum(v) / len(v), sorted(v)[len(v) // 2]) for k, v in samples.items()}
        del gt

    if args.calib_copy:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    per_step_s = gpu_ms / 1e3 / steps
    expert_bytes = K_TOP * layers[0].expert_bytes()
    router_bytes = E * D * 4
    algo_bytes = expert_bytes + router_bytes + 2 * D * 4 + 2 * K_TOP * 4
    value = expert_bytes / per_step_s / 1e9
    achieved = algo_bytes / per_step_s / 1e9
    traffic = load_traffic()
    # algorithmic bytes of one gate/up launch: the selected experts' gate and
    # up rows, the logits, x, and the h it writes (plus idx/wts)
    gu_bytes = K_TOP * 2 * q.hfq4_packed_bytes(F, D) + E * 4 + D * 4 + K_TOP * F * 4 + 2 * K_TOP * 4
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": round(per_step_s * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u4 weights, f16 products, f32 accumulate (router f32)",
        "data": "synthetic (seeded N(0,0.02) weights HFQ4-packed on device; x ~ N(0,1))",
        "config": {"workload": "single MoE layer decode, d=2048, expert FFN 512, 256 experts, "
                               "top-8, 1 token, HFQ4 experts; %d replicas, %d-token x pool" %
                               (args.replicas, args.pool),
                   "global_batch": 1, "mode": args.mode, "path": args.path},
        "tokens_per_s": round(1.0 / per_step_s, 1),
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "wall_s_timed": round(wall, 4),
        "roofline": ({"bound": "hbm",
                      "achieved": round(gu_bytes / (kern["gateup"][0] * 1e-6) / 1e9, 2),
                      "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": round(gu_bytes / (kern["gateup"][0] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                      "traffic": traffic,
                      "kernel": "gateup_fast_kernel<true> (top-k + grouped gate/up dequant-GEMV)",
                      "algorithmic_bytes_per_launch": gu_bytes,
                      "avg_launch_us": round(kern["gateup"][0], 3),
                      "median_launch_us": round(kern["gateup"][1], 3),
                      "samples": args.kernel_samples,
                      "kernel_us": {k: round(v[0], 3) for k, v in kern.items()}}
                     if kern else None),
        "layer_roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                           "algorithmic_bytes_per_step": algo_bytes,
                           "kernels_per_step": 3 if args.path == "fused" else 4},
    }
    if not args.no_cpu:
        xs_host = xs[:64].cpu().numpy()
        routers_host = [L.Wr.cpu().numpy() for L in layers]
        out["cpu_baseline"] = cpu_baseline(torch, 0, xs_host, routers_host, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
