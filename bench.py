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
import ctypes
import json
import math
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
    from quantized_moe_decode_amd.profiling import kernel_sources_digest as digest
    return digest(ROOT)


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


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(torch, layers_f32_seed, xs_host, routers_host, budget_s):
    """The oracle (numpy float64) on the first tokens of the same workload,
    timed on the host cores: once with the BLAS pool at the cores this
    process may run on (capped by OMP_NUM_THREADS when set, the machine's CPU
    share), once single-threaded on a shorter sample.  Experts are quantized
    by the oracle before timing starts, as the GPU path gets pre-packed
    weights."""
    from oracle import moe
    import synth
    from threadpoolctl import threadpool_limits
    avail = len(os.sched_getaffinity(0))
    want = int(os.environ.get("OMP_NUM_THREADS") or avail)
    threads = max(1, min(avail, want))
    seed = layers_f32_seed
    exps_cache = {}

    def experts_of(r, idx):
        exps = {}
        for e in idx:
            key = (r, int(e))
            if key not in exps_cache:
                g, u, dn = synth.expert_f32(torch, "cuda", seed, r, int(e), D, F)
                exps_cache[key] = moe.PackedExpert.from_f32(g.cpu().numpy(), u.cpu().numpy(),
                                                            dn.cpu().numpy())
            exps[int(e)] = exps_cache[key]
        return exps

    def run(nthreads, budget, max_tokens):
        spent, n = 0.0, 0
        with threadpool_limits(limits=nthreads):
            while spent < budget and n < min(len(xs_host), max_tokens):
                r = n % len(routers_host)
                x = xs_host[n:n + 1]
                Wr = routers_host[r]
                idx, _, _ = moe.route(Wr, x, K_TOP)
                exps = experts_of(r, idx[0])
                t0 = time.perf_counter()
                moe.moe_layer(x, Wr, exps, K_TOP)
                spent += time.perf_counter() - t0
                n += 1
        return n, spent

    n, t_total = run(threads, budget_s, len(xs_host))
    per_tok = t_total / n
    n1, t1 = run(1, budget_s / 4, n)
    per_tok1 = t1 / n1
    return {"value": round(K_TOP * 1671168 / per_tok / 1e9, 4), "unit": "GB/s",
            "cores": threads, "kind": "oracle",
            "sample": "%d single-token layer calls of the same workload (replica r = token mod 32), "
                      "%.1f s of oracle time, %.3f s per token-layer; quantization untimed" %
                      (n, t_total, per_tok),
            "tokens_per_s": round(1.0 / per_tok, 4),
            "cores_available": avail, "cpu_model": _cpu_model(),
            "single_thread": {"value": round(K_TOP * 1671168 / per_tok1 / 1e9, 4), "unit": "GB/s",
                              "tokens_per_s": round(1.0 / per_tok1, 4),
                              "sample": "%d of the same calls, %.1f s" % (n1, t1)}}


def _warm_translations(torch, tensors):
    """Read one byte of every 4 KiB page of each tensor once (about 1.6 % of
    its cache lines).  Decode touches the whole model every token, so its
    address translations are warm after the first pass; this puts the
    benchmark's weight replicas in that state without bringing their bytes
    into the caches."""
    total = 0.0
    for t in tensors:
        v = t.view(-1)
        total += float(v[::max(1, 4096 // v.element_size())].float().sum())
    return total


def _graph_upload(torch, g):
    """Upload an instantiated graph to the device (hipGraphUpload) so that
    its first timed replay carries no upload cost."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    ex = g.raw_cuda_graph_exec()
    rc = hip.hipGraphUpload(ctypes.c_void_p(ex), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    if rc != 0:
        raise SystemExit("hipGraphUpload failed: %d" % rc)


def _calib_copy(torch):
    """One 1 GiB device copy: the reference the counter runs scale by."""
    a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    del a, b


def _base(args, steps, warm, per_step_s, value, workload, extra_cfg=None):
    cfg = {"workload": workload, "global_batch": 1, "mode": "graph"}
    cfg.update(extra_cfg or {})
    return {"metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
            "steps": steps, "warmup": warm, "ms_per_step": round(per_step_s * 1e3, 6),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "u4 weights, f16 products, f32 accumulate (router f32)",
            "data": "synthetic (seeded N(0,0.02) weights HFQ4-packed on device; x ~ N(0,1))",
            "config": cfg, "cpu_baseline": None}


def _graphs(torch, step, n_steps, per_graph):
    """Capture n_steps calls of step(i) into graphs of per_graph steps."""
    s = torch.cuda.Stream()
    cur = torch.cuda.current_stream()
    s.wait_stream(cur)
    with torch.cuda.stream(s):
        step(0)
    cur.wait_stream(s)
    torch.cuda.synchronize()
    gs = []
    for g0 in range(0, n_steps, per_graph):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(g0, min(n_steps, g0 + per_graph)):
                step(i)
        gs.append(g)
    torch.cuda.synchronize()
    return gs


def _time_graphs(torch, gs, reps_warm, reps):
    for _ in range(reps_warm):
        for g in gs:
            g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(reps):
        for g in gs:
            g.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / 1e3


def bench_stack(args, torch, q):
    """40 MoE layers (d=2048, F=512, E=256, top-8), each preceded by a dense
    2048 x 2048 HFQ4 GEMV with residual; 1 token; 256 fresh tokens cycled."""
    from quantized_moe_decode_amd.stack import build_stack
    import synth
    NL, POOL = 40, 256
    t0 = time.time()
    st = build_stack(torch, 0, NL, E, D, F, K_TOP, 1, dense=True)
    xs = synth.activations(torch, "cuda", 2, POOL, D)
    outs = torch.empty((POOL, D), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    log("built the %d-layer stack in %.1f s" % (NL, time.time() - t0))

    def step(i):
        outs[i:i + 1].copy_(st.step(xs[i:i + 1]))

    gs = _graphs(torch, step, POOL, 32)
    reps = max(1, args.steps // POOL)
    secs = _time_graphs(torch, gs, 1, reps)
    steps = reps * POOL
    err = q.workspace_error(st.ws)
    if err or not bool(torch.isfinite(outs).all()):
        raise SystemExit("stack run: device error word %d, finite outputs %s"
                         % (err, bool(torch.isfinite(outs).all())))
    per = secs / steps
    eb = NL * K_TOP * st.layers[0].expert_bytes()
    dense_b = NL * q.hfq4_packed_bytes(D, D)
    router_b = NL * E * D * 4
    algo = eb + dense_b + router_b
    out = _base(args, steps, POOL, per, eb / per / 1e9,
                "40-layer expert stack decode: per layer a dense 2048x2048 HFQ4 GEMV + residual, "
                "then a MoE layer (d=2048, FFN 512, 256 experts, top-8) + residual; 1 token; "
                "%d fresh tokens cycled" % POOL)
    out["tokens_per_s"] = round(1.0 / per, 2)
    out["pct_hbm_peak"] = round(100.0 * eb / per / 1e9 / HBM_PEAK_GBS, 2)
    out["roofline"] = {"bound": "hbm", "achieved": round(algo / per / 1e9, 2),
                       "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": round(algo / per / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                       "kernel": "whole step: 40 x (dense GEMV, router logits, top-k + gate/up, "
                                 "down + combine)",
                       "algorithmic_bytes_per_step": algo,
                       "expert_bytes_per_step": eb, "dense_bytes_per_step": dense_b,
                       "router_bytes_per_step": router_b, "kernels_per_step": 4 * NL}
    return out


def _zero_copy_rate(torch, q, nbytes):
    """PCIe rates: a kernel reading a pinned host HFQ4 matrix zero-copy
    (hfq4_gemv over it, batch 1) and a host-to-device DMA copy."""
    rows = nbytes // q.hfq4_packed_bytes(1, D)
    host = torch.empty(rows * q.hfq4_packed_bytes(1, D), dtype=torch.uint8, pin_memory=True)
    host.zero_()
    x = torch.zeros((1, D), dtype=torch.float32, device="cuda")
    y = torch.empty((1, rows), dtype=torch.float32, device="cuda")
    q.hfq4_gemv(host, rows, D, x, y=y)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    best_zc = 0.0
    for _ in range(3):
        ev0.record()
        q.hfq4_gemv(host, rows, D, x, y=y)
        ev1.record()
        torch.cuda.synchronize()
        best_zc = max(best_zc, host.numel() / (ev0.elapsed_time(ev1) / 1e3) / 1e9)
    dst = torch.empty(host.numel(), dtype=torch.uint8, device="cuda")
    best_dma = 0.0
    for _ in range(3):
        ev0.record()
        dst.copy_(host, non_blocking=True)
        ev1.record()
        torch.cuda.synchronize()
        best_dma = max(best_dma, host.numel() / (ev0.elapsed_time(ev1) / 1e3) / 1e9)
    del host, dst
    return best_zc, best_dma


def _stream_ceiling(torch, q, nbytes):
    """The same dequant-GEMV machinery where it is not latency-bound: one
    token through an nbytes HFQ4 matrix in HBM (hfq4_gemv), best of 5."""
    rows = nbytes // q.hfq4_packed_bytes(1, D)
    W = torch.zeros(rows * q.hfq4_packed_bytes(1, D), dtype=torch.uint8, device="cuda")
    x = torch.randn((1, D), dtype=torch.float32, device="cuda")
    y = torch.empty((1, rows), dtype=torch.float32, device="cuda")
    q.hfq4_gemv(W, rows, D, x, y=y)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    best = 0.0
    for _ in range(5):
        ev0.record()
        q.hfq4_gemv(W, rows, D, x, y=y)
        ev1.record()
        torch.cuda.synchronize()
        best = max(best, W.numel() / (ev0.elapsed_time(ev1) / 1e3) / 1e9)
    del W, y
    return best


def bench_hostmapped(args, torch, q):
    """48 MoE layers (d=2048, F=512, E=512, top-8), residual between layers;
    experts of layers 0-23 in HBM, of layers 24-47 in pinned host memory
    read zero-copy by the same kernels."""
    from quantized_moe_decode_amd.stack import build_stack
    import synth
    NL, HOST_FROM, EH, POOL = 48, 24, 512, 64
    zc, dma = _zero_copy_rate(torch, q, 1 << 32)   # 4 GiB of pinned memory
    log("PCIe: zero-copy kernel read %.1f GB/s, DMA host->device %.1f GB/s" % (zc, dma))
    t0 = time.time()
    st = build_stack(torch, 0, NL, EH, D, F, K_TOP, 1, dense=False, host_from=HOST_FROM)
    xs = synth.activations(torch, "cuda", 2, POOL, D)
    outs = torch.empty((POOL, D), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    log("built the %d-layer host-mapped stack in %.1f s" % (NL, time.time() - t0))

    def step(i):
        outs[i:i + 1].copy_(st.step(xs[i:i + 1]))

    gs = _graphs(torch, step, POOL, 16)
    reps = max(1, min(args.steps, 256) // POOL)
    secs = _time_graphs(torch, gs, 1, reps)
    steps = reps * POOL
    err = q.workspace_error(st.ws)
    if err or not bool(torch.isfinite(outs).all()):
        raise SystemExit("host-mapped run: device error word %d, finite outputs %s"
                         % (err, bool(torch.isfinite(outs).all())))
    per = secs / steps
    eb_layer = K_TOP * st.layers[0].expert_bytes()
    host_b = (NL - HOST_FROM) * eb_layer
    hbm_b = HOST_FROM * eb_layer + NL * EH * D * 4
    pcie_peak = max(zc, dma)
    t_bound = hbm_b / (HBM_PEAK_GBS * 1e9) + host_b / (pcie_peak * 1e9)
    out = _base(args, steps, POOL, per, NL * eb_layer / per / 1e9,
                "host-mapped expert mode: 48 MoE layers (d=2048, FFN 512, 512 experts, top-8) + "
                "residual; experts of layers 0-23 in HBM, 24-47 in pinned host memory read "
                "zero-copy; 1 token; %d fresh tokens cycled" % POOL)
    out["tokens_per_s"] = round(1.0 / per, 2)
    out["roofline"] = {"bound": "hbm+pcie", "achieved": round((hbm_b + host_b) / per / 1e9, 2),
                       "peak": round((hbm_b + host_b) / t_bound / 1e9, 2), "unit": "GB/s",
                       "frac": round(t_bound / per, 4), "traffic": None,
                       "kernel": "whole step: 48 x (router logits, top-k + gate/up, down + combine)",
                       "hbm_bytes_per_step": hbm_b, "host_bytes_per_step": host_b,
                       "pcie_zero_copy_gbs": round(zc, 2), "pcie_dma_gbs": round(dma, 2),
                       "pcie_peak_used_gbs": round(pcie_peak, 2),
                       "bound_ms_per_step": round(t_bound * 1e3, 4),
                       "host_gbs_if_hbm_at_peak": round(
                           host_b / max(per - hbm_b / (HBM_PEAK_GBS * 1e9), 1e-12) / 1e9, 2)}
    return out


def bench_offload(args, torch, q):
    """One host-resident layer of the host-mapped workload's shape (d=2048,
    F=512, E=512, top-8, Zipf-biased router): one decode step timed with the
    experts read over PCIe by the GPU kernels and with the experts computed
    on the host CPU (router on the GPU), and the route the 15% rule picks."""
    import synth
    from quantized_moe_decode_amd.offload import measure_routes
    EH, N = 512, 64
    zc, dma = _zero_copy_rate(torch, q, 1 << 32)
    L = q.synthetic.build_layer(torch, 0, 30, EH, D, F, bias=synth.zipf_bias(0, EH),
                                host_mapped=True)
    xs = synth.activations(torch, "cuda", 6, N, D)
    nthreads = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit() and int(os.environ["OMP_NUM_THREADS"]) > 0:
        nthreads = min(nthreads, int(os.environ["OMP_NUM_THREADS"]))
    m = measure_routes(torch, L, xs, K_TOP, nthreads=nthreads, host_kernels=("avx512", "avx2"))
    best = min(m["pcie_s_per_step"], m["cpu_s_per_step"])
    out = _base(args, N, 3, best, m["expert_bytes_per_step"] / best / 1e9,
                "host-resident expert layer (d=2048, FFN 512, 512 experts, top-8, Zipf router), "
                "experts in pinned host memory; PCIe zero-copy route vs CPU route; 1 token; %d "
                "fresh tokens" % N)
    out["offload"] = {k: (round(v, 8) if isinstance(v, float) else v) for k, v in m.items()}
    out["offload"]["rule"] = "CPU only when at least 15% faster than PCIe"
    out["offload"]["cpu_threads"] = nthreads
    out["offload"]["cpu_model"] = _cpu_model()
    pcie_roof = {"bound": "pcie", "achieved": round(m["pcie_expert_gbs"], 2),
                 "peak": round(max(zc, dma), 2), "unit": "GB/s",
                 "frac": round(m["pcie_expert_gbs"] / max(zc, dma), 4), "traffic": None,
                 "kernel": "PCIe route: whole layer step (router, top-k + gate/up, down)",
                 "pcie_zero_copy_gbs": round(zc, 2), "pcie_dma_gbs": round(dma, 2)}
    host_gbs = _host_read_rate(torch, nthreads)
    cpu_roof = {"bound": "host-dram", "achieved": round(m["cpu_expert_gbs"], 2),
                "peak": round(host_gbs, 2), "unit": "GB/s",
                "frac": round(m["cpu_expert_gbs"] / host_gbs, 4), "traffic": None,
                "kernel": "CPU route: whole layer step (router on the GPU, routing and x to the "
                          "host, experts on %d host threads (%s), y back); peak = a %d-thread "
                          "read of 1 GiB of pinned host memory" % (nthreads, m["host_kernel"],
                                                                    nthreads)}
    if m["route"] == "cpu":
        out["roofline"], out["roofline_other_route"] = cpu_roof, pcie_roof
    else:
        out["roofline"], out["roofline_other_route"] = pcie_roof, cpu_roof
    return out


def _host_read_rate(torch, nthreads):
    """GB/s of a multi-threaded read (a sum) of 1 GiB of pinned host memory."""
    old = torch.get_num_threads()
    torch.set_num_threads(nthreads)
    try:
        buf = torch.ones(1 << 28, dtype=torch.float32, pin_memory=True)
        best = None
        for _ in range(4):
            t0 = time.perf_counter()
            float(buf.sum())
            dt = time.perf_counter() - t0
            best = dt if best is None else min(best, dt)
        del buf
        return (1 << 30) / best / 1e9
    finally:
        torch.set_num_threads(old)


def bench_cache(args, torch, q):
    """An HBM expert cache over host-resident experts: 8 layers of the
    host-mapped workload's shape (d=2048, F=512, E=512, top-8) with a
    Zipf(1.1)-biased router, every expert in pinned host memory; the HBM
    budget holds a quarter of the expert bytes (plus the routers); hot-set
    placement from each layer's routing of 256 calibration tokens, and, for
    comparison, whole-layer placement at the same budget.  Decode steps
    x' = x + MoE(x) through the 8 layers, one token at a time."""
    import numpy as np
    import synth
    import quantized_moe_decode_amd.cache as cache
    NL, EH, POOL = 8, 512, 64
    zc, dma = _zero_copy_rate(torch, q, 1 << 32)
    pcie = max(zc, dma)
    bias = synth.zipf_bias(0, EH)
    t0 = time.time()
    layers = [q.synthetic.build_layer(torch, 0, l, EH, D, F, bias=bias, host_mapped=True)
              for l in range(NL)]
    log("built %d host-resident layers in %.1f s" % (NL, time.time() - t0))
    eb = layers[0].expert_bytes()
    fixed = NL * EH * D * 4                       # the routers stay in HBM
    budget = fixed + NL * EH * eb // 4
    calib = synth.activations(torch, "cuda", 21, 256, D)
    heat = cache.routing_heat(torch, layers, calib, K_TOP)
    xs = synth.activations(torch, "cuda", 22, POOL, D)
    ws = q.new_workspace(layers[0], 1, K_TOP)
    res = {}
    for mode, name in ((q.HFQ4_PLACE_HOTSET, "hotset"), (q.HFQ4_PLACE_LAYERS, "layers")):
        tables, pool, resident, placed = cache.place_and_build(torch, layers, heat, budget, fixed,
                                                               mode=mode)
        hits = torch.zeros(2, dtype=torch.int64, device="cuda")
        bufs = [torch.empty((1, D), dtype=torch.float32, device="cuda") for _ in range(2)]
        outs = torch.empty((POOL, D), dtype=torch.float32, device="cuda")

        def step(i):
            cur = xs[i:i + 1]
            for li, T in enumerate(tables):
                out = bufs[li & 1]
                q.moe_layer_decode_table(T, cur, K_TOP, ws, residual=cur, y=out, hits=hits)
                cur = out
            outs[i:i + 1].copy_(cur)

        gs = _graphs(torch, step, POOL, POOL)
        for g in gs:                       # upload and warm
            g.replay()
        torch.cuda.synchronize()
        hits.zero_()
        secs = _time_graphs(torch, gs, 0, 1)
        h = hits.cpu().numpy().astype(np.float64)
        per = secs / POOL
        sel = h.sum() / POOL                        # expert selections per step (= NL * k)
        hit = h[0] / h.sum()
        hbm_b = hit * sel * eb + NL * EH * D * 4
        host_b = (1 - hit) * sel * eb
        t_bound = hbm_b / (HBM_PEAK_GBS * 1e9) + host_b / (pcie * 1e9)
        res[name] = {"ms_per_step": round(per * 1e3, 4), "tokens_per_s": round(1 / per, 1),
                     "hit_rate": round(hit, 4), "resident_experts": int(resident.sum()),
                     "resident_fraction": round(float(resident.mean()), 4),
                     "hbm_bytes_per_step": int(hbm_b), "pcie_bytes_per_step": int(host_b),
                     "expert_gbs": round(sel * eb / per / 1e9, 2),
                     "bound_ms_per_step": round(t_bound * 1e3, 4),
                     "frac_of_split_bound": round(t_bound / per, 4)}
        log("%s placement: hit rate %.3f, %.3f ms per step (bound %.3f ms)"
            % (name, hit, per * 1e3, t_bound * 1e3))
        del tables, pool, gs
        torch.cuda.empty_cache()
    hs = res["hotset"]
    out = _base(args, POOL, 1, hs["ms_per_step"] / 1e3, hs["expert_gbs"],
                "HBM expert cache over host-resident experts: 8 layers (d=2048, FFN 512, 512 "
                "experts, top-8, Zipf(1.1) router), HBM budget = routers + 1/4 of the expert "
                "bytes, hot-set placement from 256 calibration tokens; 1 token; %d fresh tokens"
                % POOL)
    out["cache"] = res
    out["cache"]["budget_bytes"] = int(budget)
    out["tokens_per_s"] = hs["tokens_per_s"]
    out["roofline"] = {"bound": "hbm+pcie", "achieved": hs["expert_gbs"],
                       "peak": round(sel * eb / (hs["bound_ms_per_step"] / 1e3) / 1e9, 2),
                       "unit": "GB/s", "frac": hs["frac_of_split_bound"], "traffic": None,
                       "kernel": "whole step: 8 table layers (single launch each)",
                       "pcie_zero_copy_gbs": round(zc, 2), "pcie_dma_gbs": round(dma, 2)}
    return out


def bench_turbo(args, torch, q):
    """TurboQuant KV codec: encode and decode of 1 GiB of f32 vectors (2^21
    of 128 values at 2, 3, 4 and 8 bits; 64 and 256 values at 4 bits); both
    kernels are HBM streams, so the roofline is HBM bandwidth over the bytes
    read plus written."""
    res = {}
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    for n, bits in ((128, 4), (128, 3), (128, 2), (128, 8), (64, 4), (256, 4)):
        N = (1 << 28) // n                  # 1 GiB of f32 vectors
        V = torch.randn((N, n), dtype=torch.float32, device="cuda")
        rec = q.turbo_record_bytes(n, bits)
        out = torch.empty((N, rec), dtype=torch.uint8, device="cuda")
        dec = torch.empty((N, n), dtype=torch.float32, device="cuda")
        q.turbo_encode(V, bits, out=out)
        q.turbo_decode(out, n, bits, v=dec)
        torch.cuda.synchronize()
        t = {}
        for name, fn in (("encode", lambda: q.turbo_encode(V, bits, out=out)),
                         ("decode", lambda: q.turbo_decode(out, n, bits, v=dec))):
            best = 1e9
            for _ in range(5):
                ev0.record()
                fn()
                ev1.record()
                torch.cuda.synchronize()
                best = min(best, ev0.elapsed_time(ev1) / 1e3)
            t[name] = best
        moved = N * (4 * n + rec)
        key = str(bits) if n == 128 else "n%d_%d" % (n, bits)
        res[key] = {"n": n, "vectors": N, "record_bytes": rec, "ratio_vs_f32": round(4 * n / rec, 3),
                          "encode_ms": round(t["encode"] * 1e3, 4),
                          "decode_ms": round(t["decode"] * 1e3, 4),
                          "encode_gbs": round(moved / t["encode"] / 1e9, 1),
                          "decode_gbs": round(moved / t["decode"] / 1e9, 1),
                          "encode_frac": round(moved / t["encode"] / 1e9 / HBM_PEAK_GBS, 4),
                          "decode_frac": round(moved / t["decode"] / 1e9 / HBM_PEAK_GBS, 4),
                          "vectors_per_s_decode": round(N / t["decode"], 0)}
        log("turbo n=%d bits=%d: encode %.1f GB/s, decode %.1f GB/s" % (
            n, bits, res[key]["encode_gbs"], res[key]["decode_gbs"]))
        del out, dec, V
    r4 = res["4"]
    out = _base(args, 5, 1, r4["decode_ms"] / 1e3, r4["decode_gbs"],
                "TurboQuant KV codec: 2^21 vectors of 128 f32 (1 GiB), 4-bit records of 68 bytes; "
                "value = decode GB/s (record bytes read + f32 written)")
    out["unit"] = "GB/s"
    out["turbo"] = res
    out["roofline"] = {"bound": "hbm", "achieved": r4["decode_gbs"], "peak": HBM_PEAK_GBS,
                       "unit": "GB/s", "frac": r4["decode_frac"], "traffic": None,
                       "kernel": "turbo_decode_kernel<128, 4, true>"}
    return out


def bench_skewed(args, torch, q):
    """One layer shape (d=2048, F=512, E=512, top-8) with Zipf(1.1)-biased
    router logits; token batches of 1, 4 and 16.  16 replicas of the layer
    (13.7 GB) and a 4096-token pool keep the Infinity Cache from serving
    repeats."""
    import numpy as np
    import quantized_moe_decode_amd.synthetic as syn
    import synth
    EH, NREP, POOL = 512, 16, 4096
    bias = synth.zipf_bias(0, EH)
    t0 = time.time()
    layers = [syn.build_layer(torch, 0, r, EH, D, F, bias=bias) for r in range(NREP)]
    xs = synth.activations(torch, "cuda", 3, POOL, D)
    torch.cuda.synchronize()
    log("built %d skewed replicas in %.1f s" % (NREP, time.time() - t0))
    eb = layers[0].expert_bytes()
    res = {}
    for B in [int(v) for v in args.batches.split(",")]:
        ws = q.new_workspace(layers[0], B, K_TOP)
        y = torch.empty((B, D), dtype=torch.float32, device="cuda")
        idx = torch.empty((B, K_TOP), dtype=torch.int32, device="cuda")
        wts = torch.empty((B, K_TOP), dtype=torch.float32, device="cuda")
        nsteps = POOL // B
        G = 256

        def step(i):
            j = (i * B) % POOL
            q.moe_layer_decode(layers[i % NREP], xs[j:j + B], K_TOP, ws, y=y, idx=idx, wts=wts)

        gs = _graphs(torch, step, G, G)
        reps = max(1, args.steps // (4 * G))
        secs = _time_graphs(torch, gs, 1, reps)
        err = q.workspace_error(ws)
        if err:
            raise SystemExit("device error word %d after the skewed run (B=%d)" % (err, B))
        per = secs / (reps * G)

        # warm mode: the same steps on one replica, so the hot experts of the
        # skewed routing are served again from the Infinity Cache (labelled
        # as such; not the headline)
        def step_warm(i):
            j = (i * B) % POOL
            q.moe_layer_decode(layers[0], xs[j:j + B], K_TOP, ws, y=y, idx=idx, wts=wts)

        gw = _graphs(torch, step_warm, G, G)
        per_warm = _time_graphs(torch, gw, 1, reps) / (reps * G)
        del gw
        # distinct experts per step, from the routing of the same steps
        uni = []
        rws = torch.empty(q.moe_route_workspace_bytes(EH, B), dtype=torch.uint8,
                                             device="cuda")
        for i in range(G):
            j = (i * B) % POOL
            L = layers[i % NREP]
            ii, _ = q.moe_route_topk(L.Wr, xs[j:j + B], K_TOP, bias=L.bias, ws=rws)
            uni.append(len(np.unique(ii.cpu().numpy())))
        u = float(np.mean(uni))
        res[str(B)] = {"ms_per_step": round(per * 1e3, 5), "tokens_per_s": round(B / per, 1),
                       "mean_distinct_experts": round(u, 2),
                       "expert_gbs": round(u * eb / per / 1e9, 2),
                       "pct_hbm_peak": round(100 * u * eb / per / 1e9 / HBM_PEAK_GBS, 2),
                       "steps": reps * G,
                       "warm": {"mode": "one replica, hot set reused from the Infinity Cache",
                                "ms_per_step": round(per_warm * 1e3, 5),
                                "tokens_per_s": round(B / per_warm, 1)}}
        del ws
    if args.calib_copy:
        _calib_copy(torch)
    b1 = res[min(res, key=int)]
    out = _base(args, sum(r["steps"] for r in res.values()), 0, b1["ms_per_step"] / 1e3,
                b1["expert_gbs"],
                "skewed-routing layer: d=2048, FFN 512, 512 experts, top-8, Zipf(s=1.1) router "
                "bias, token batches 1/4/16; %d replicas, %d-token pool" % (NREP, POOL),
                {"global_batch": [int(v) for v in res]})
    out["per_batch"] = res
    out["tokens_per_s"] = b1["tokens_per_s"]
    out["roofline"] = {"bound": "hbm", "achieved": b1["expert_gbs"], "peak": HBM_PEAK_GBS,
                       "unit": "GB/s", "frac": round(b1["expert_gbs"] / HBM_PEAK_GBS, 4),
                       "traffic": None, "kernel": "whole layer step at B=1 (expert bytes of the "
                                                  "distinct selected experts)"}
    return out


def main():
    ap = argparse.ArgumentParser(description="Throughput of the HFQ4 MoE decode path on one MI355X; "
                                             "prints one JSON line.")
    ap.add_argument("--gpus", type=int, default=1, help="GPUs (only 1 is supported)")
    ap.add_argument("--steps", type=int, default=20000, help="timed steps (exactly this many)")
    ap.add_argument("--warmup", type=int, default=2000, help="untimed steps before timing")
    ap.add_argument("--mode", choices=["graph", "eager"], default="graph",
                    help="steps as HIP-graph replays or as eager launches")
    ap.add_argument("--path", choices=["fused", "split"], default="fused",
                    help="moe_layer_decode, or moe_route_topk + moe_expert_decode")
    ap.add_argument("--launches", type=int, choices=[1, 2, 3], default=3,
                    help="one-token layers as the router -> gate/up -> down launch chain (3), "
                         "as one launch whose workgroups exchange the logits, h and the per-slot "
                         "down sums through tagged words (1), or as that launch's routing and "
                         "gate/up phases followed by the down kernel (2); same results")
    ap.add_argument("--xch-min-batch", type=int, default=9,
                    help="batched calls of at least this many tokens route by exchange (one "
                         "router workgroup per token), smaller ones in every gate/up workgroup "
                         "(17: never; same results)")
    ap.add_argument("--replicas", type=int, default=32,
                    help="distinct layer copies cycled through (so caches cannot serve repeats)")
    ap.add_argument("--pool", type=int, default=4096, help="distinct input tokens cycled through")
    ap.add_argument("--graph-steps", type=int, default=512,
                    help="most steps captured in one HIP graph (the graph holds the largest "
                         "divisor of --steps not above this)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="time budget of the oracle's CPU baseline sample")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU baseline")
    ap.add_argument("--kernel-samples", type=int, default=200,
                    help="eager steps (back to back) timed with HIP events for the roofline")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one device copy of 1 GiB (counter calibration)")
    ap.add_argument("--batches", default="1,4,16",
                    help="token batch sizes of the skewed workload")
    ap.add_argument("--no-companions", action="store_true",
                    help="layer workload: skip the short runs of the skewed (4 and 16 tokens) "
                         "and 40-layer stack workloads that follow the headline in the same line")
    ap.add_argument("--workload", choices=["layer", "stack", "hostmapped", "skewed", "floor",
                                           "offload", "cache", "turbo"],
                    default="layer",
                    help="layer: one MoE layer (the headline line); stack: 40 layers with a dense "
                         "GEMV each; hostmapped: 48 layers, experts of 24 in pinned host memory; "
                         "skewed: 512 experts, Zipf-biased routing, token batches 1/4/16; "
                         "floor: the latency and bandwidth probes of the one-token floor model; "
                         "offload: PCIe vs CPU route for host-resident experts; cache: HBM expert "
                         "cache over host-resident experts; turbo: TurboQuant KV codec")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: runs on several GPUs are not supported "
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
    q.lib.hfq4_debug_set_single_launch({3: 0, 1: 1, 2: 2}[args.launches])
    q.lib.hfq4_debug_set_route_exchange(args.xch_min_batch)
    if args.workload == "floor":
        from quantized_moe_decode_amd import probes
        out = {"workload": "latency and bandwidth probes (floor model of the one-token layer)",
               "probes": probes.run_all(torch, log=log)}
        print(json.dumps(out), flush=True)
        return
    if args.workload != "layer":
        out = {"stack": bench_stack, "hostmapped": bench_hostmapped, "skewed": bench_skewed,
               "offload": bench_offload, "cache": bench_cache,
               "turbo": bench_turbo}[args.workload](args, torch, q)
        print(json.dumps(out), flush=True)
        return

    t0 = time.time()
    layers = [syn.build_layer(torch, seed=0, layer_id=r, E=E, d=D, F=F, device=dev)
              for r in range(args.replicas)]
    xs = synth.activations(torch, dev, 1, args.pool, D)
    torch.cuda.synchronize()
    log("built %d replicas in %.1f s" % (args.replicas, time.time() - t0))
    # steady-state address translation for every replica (the timed steps
    # still read every weight byte from HBM: the replicas are 54x the
    # Infinity Cache); without it a short run (--steps 20) pays first-touch
    # translation misses that a decode loop pays only on its first pass
    _warm_translations(torch, [t for L in layers for t in (L.gate, L.up, L.down, L.Wr)])

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
        # exactly K timed steps: one graph of G steps replayed K / G times,
        # uploaded to the device before timing.  When K and W have a common
        # divisor of at least 4 (not above --graph-steps), G is the largest
        # such and the W warmup steps are W / G replays of the same graph, so
        # its one-time first-replay cost (about 1 us per step of a 20-step
        # graph) falls in the warmup, as it does in a decode loop; otherwise
        # G is the largest divisor of K and the W warmup steps run eagerly
        # (the same calls) on other activations of the pool
        K = args.steps
        W = args.warmup
        cw = math.gcd(K, W)
        GW = max(g for g in range(1, min(cw, args.graph_steps) + 1) if cw % g == 0) if W else 0
        G = max(g for g in range(1, min(K, args.graph_steps) + 1) if K % g == 0)
        warm_graph = GW >= 4
        if warm_graph:
            G = GW
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
        _graph_upload(torch, g)
        reps = K // G
        steps, warm = K, args.warmup
        run = lambda: [g.replay() for _ in range(reps)]
        if warm_graph:
            run_w = lambda: [g.replay() for _ in range(warm // G)]
        else:
            run_w = lambda: [step(G + i) for i in range(warm)]
    else:
        G = 0
        steps, warm = args.steps, args.warmup
        run = lambda: [step(i) for i in range(steps)]
        run_w = lambda: [step(steps + i) for i in range(warm)]

    run_w()
    torch.cuda.synchronize()
    err = q.workspace_error(ws)
    if err:
        raise SystemExit("device error word %d after warmup" % err)
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    from quantized_moe_decode_amd import probes
    wall0 = time.perf_counter()
    probes.spin(torch, 200)
    ev0.record(stream)
    run()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    gpu_ms = ev0.elapsed_time(ev1)
    timing = ("HIP events around the replays; a 200 us single-wave spin ahead of the first "
              "event keeps the device busy while the host enqueues them")
    if args.mode == "graph":
        timing += ("; %d steps per graph, %d timed replays; warmup: %s"
                   % (G, reps, "%d replay%s of the same graph" % (warm // G, "" if warm == G else "s")
                      if warm_graph else "%d eager steps" % warm))
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

        tr = torch.zeros(4 * 1024 * 8, dtype=torch.int64, device=dev)
        q.lib.hfq4_debug_set_trace(ctypes.c_void_p(tr.data_ptr()), tr.numel() * 8)
        gt = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gt):
            for i in range(G):
                step(i)
        q.lib.hfq4_debug_set_trace(None, 0)
        samples = {"logits": [], "gateup": [], "down": [], "step": []}
        ncu = torch.cuda.get_device_properties(0).multi_processor_count
        nwg = {0: E, 1: ncu, 2: D // 8}
        for rep in range(args.kernel_samples):
            gt.replay()
            torch.cuda.synchronize()
            t = tr.view(4, 1024, 8).cpu().numpy()
            if int(t[0, :E, 0].max()) == 0:
                n = min(ncu, 1024)
                if int(t[2, :nwg[2], 0].max()) == 0:
                    # one launch per step (the single-launch layer): stamps 0..6
                    span = (int(t[1, :n, 6].max()) - int(t[1, :n, 0].min())) / 100.0
                    samples["gateup"].append(span)
                    samples["step"].append(span)
                    continue
                # two launches: routing + gate/up (stamps 0..4), then down
                st1, en1 = int(t[1, :n, 0].min()), int(t[1, :n, 4].max())
                st2, en2 = int(t[2, :nwg[2], 0].min()), int(t[2, :nwg[2], 3].max())
                samples["gateup"].append((en1 - st1) / 100.0)
                samples["down"].append((en2 - st2) / 100.0)
                samples["step"].append((en2 - st1) / 100.0)
                continue
            st, en = {}, {}
            for kk, last in ((0, 1), (1, 5), (2, 3)):
                n = min(nwg[kk], 1024)
                st[kk] = int(t[kk, :n, 0].min())
                en[kk] = int(t[kk, :n, last].max())
            samples["logits"].append((en[0] - st[0]) / 100.0)
            samples["gateup"].append((en[1] - st[1]) / 100.0)
            samples["down"].append((en[2] - st[2]) / 100.0)
            samples["step"].append((en[2] - st[0]) / 100.0)
        kern = {k: (sum(v) / len(v), sorted(v)[len(v) // 2]) for k, v in samples.items() if v}
        del gt

    # Launch duration of the gate/up kernel by HIP events on the stream the
    # library launches on (the library records a start and a stop event
    # around that launch, hipExtLaunchKernel), over eager steps of the same
    # workload issued back to back (the first 10 are not counted): the
    # duration rocprofv3's kernel trace reports (dispatch to completion),
    # not the in-kernel span above.  Eager steps leave host-side gaps between
    # launches, so single durations vary; the average is reported, with the
    # median beside it.
    ev_us = None
    if args.path == "fused":

        hip = ctypes.CDLL("libamdhip64.so")
        # one event pair per step: the steps go back to back on the stream
        # (no synchronisation between them, as in decode), and the pairs
        # are read once at the end
        n = args.kernel_samples + 10
        evs = []
        for _ in range(n):
            e0, e1 = ctypes.c_void_p(), ctypes.c_void_p()
            if hip.hipEventCreate(ctypes.byref(e0)) or hip.hipEventCreate(ctypes.byref(e1)):
                raise SystemExit("hipEventCreate failed")
            evs.append((e0, e1))
        torch.cuda.synchronize()
        # a spin kernel keeps the device busy while the host enqueues every
        # step, so the steps then run back to back and an event pair times
        # its launch on the device, not the host's enqueue gap before it
        from quantized_moe_decode_amd import probes
        spin_s = 0.02
        probes.spin(torch, spin_s * 1e6)
        t_enq = time.perf_counter()
        for i, (e0, e1) in enumerate(evs):
            q.lib.hfq4_debug_set_events(e0, e1)
            step(i * 7919)
        t_enq = time.perf_counter() - t_enq
        q.lib.hfq4_debug_set_events(None, None)
        torch.cuda.synchronize()
        vals = []
        for i, (e0, e1) in enumerate(evs):
            ms = ctypes.c_float()
            if hip.hipEventElapsedTime(ctypes.byref(ms), e0, e1):
                raise SystemExit("hipEventElapsedTime failed")
            if i >= 10:
                vals.append(ms.value * 1e3)
            hip.hipEventDestroy(e0)
            hip.hipEventDestroy(e1)
        ev_us = (sum(vals) / len(vals), sorted(vals)[len(vals) // 2], t_enq < spin_s)

    if args.calib_copy:
        _calib_copy(torch)

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
                   "global_batch": 1, "mode": args.mode, "path": args.path, "launches": args.launches},
        "tokens_per_s": round(1.0 / per_step_s, 1),
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "wall_s_timed": round(wall, 4),
        "step_timing": timing,
        "translation_warmup": "one byte of every 4 KiB page of every replica's weights read "
                              "once before the warm-up steps",
        "roofline": ({"bound": "hbm",
                      "achieved": round(gu_bytes / (ev_us[0] * 1e-6) / 1e9, 2),
                      "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": round(gu_bytes / (ev_us[0] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                      "traffic": traffic,
                      "kernel": "gateup_fast_kernel<true> (top-k + grouped gate/up dequant-GEMV)",
                      "algorithmic_bytes_per_launch": gu_bytes,
                      "avg_launch_us": round(ev_us[0], 3),
                      "median_launch_us": round(ev_us[1], 3),
                      "launch_timing": "HIP events around the launch, eager steps enqueued behind "
                                       "a 20 ms spin kernel so that they run back to back",
                      "enqueue_covered_by_spin": bool(ev_us[2]),
                      "samples": args.kernel_samples,
                      "in_kernel_span_us": ({k: round(v[0], 3) for k, v in kern.items()}
                                            if kern else None),
                      "in_kernel_span_frac": (round(gu_bytes / (kern["gateup"][0] * 1e-6) / 1e9
                                                    / HBM_PEAK_GBS, 4) if kern else None)}
                     if ev_us else None),
        "layer_roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                           "algorithmic_bytes_per_step": algo_bytes,
                           "kernels_per_step": 3 if args.path == "fused" else 4},
    }
    # secondary ratio against the streaming ceiling of the same kernel family
    ceil = _stream_ceiling(torch, q, 1 << 32)
    out["stream_ceiling"] = {"kernel": "hfq4_gemv, 1 token, 4 GiB HFQ4 matrix in HBM",
                             "gbs": round(ceil, 1), "frac_of_peak": round(ceil / HBM_PEAK_GBS, 4),
                             "layer_value_frac": round(value / ceil, 4)}
    if not args.no_cpu:
        xs_host = xs[:512].cpu().numpy()
        routers_host = [L.Wr.cpu().numpy() for L in layers]
        out["cpu_baseline"] = cpu_baseline(torch, 0, xs_host, routers_host, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    if not args.no_companions:
        del layers, ws
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        out["companion_workloads"] = companions(args, torch, q)
    print(json.dumps(out), flush=True)


def companions(args, torch, q):
    """Short runs of two other workloads after the headline, so that one
    invocation also measures them: the skewed layer (E=512, Zipf router) at
    4 and 16 tokens per step and the 40-layer stack at 1 token, each as its
    own --workload reports it but with fixed step counts (1024 timed steps
    of the skewed layer per batch, 2048 of the stack) instead of --steps."""
    import copy
    res = {"note": "measured in the same process after the headline; fixed step counts "
                   "(skewed: 1024 steps per batch, cold replicas; stack: 2048 steps)"}
    a = copy.copy(args)
    a.steps, a.batches, a.calib_copy = 4096, "4,16", False
    try:
        sk = bench_skewed(a, torch, q)
        res["skewed_E512_zipf"] = {b: {k: r[k] for k in ("ms_per_step", "tokens_per_s",
                                                          "mean_distinct_experts", "expert_gbs",
                                                          "pct_hbm_peak", "steps")}
                                   for b, r in sk["per_batch"].items()}
    except (Exception, SystemExit) as e:
        res["skewed_E512_zipf"] = {"error": str(e)}
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    a.steps = 2048
    try:
        st = bench_stack(a, torch, q)
        res["stack_40_layers"] = {"ms_per_step": st["ms_per_step"], "tokens_per_s": st["tokens_per_s"],
                                  "expert_gbs": st["value"], "pct_hbm_peak": st["pct_hbm_peak"],
                                  "steps": st["steps"]}
    except (Exception, SystemExit) as e:
        res["stack_40_layers"] = {"error": str(e)}
    return res


if __name__ == "__main__":
    main()
