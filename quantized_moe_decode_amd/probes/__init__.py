"""Latency and bandwidth probes behind the one-token floor model.

Runs the kernels of probes/probe.hip (libhfq4probe.so) and returns plain
numbers; `python bench.py --workload floor` prints them as one JSON line.
Measurement only: nothing here is on the decode path.

* chase      dependent-load latency (one lane following a random cyclic
             chain of 128-byte lines) for a footprint that sits in L2, in
             the Infinity Cache, or in HBM;
* boundary   a kernel writing one value per workgroup followed on the
             stream by one reading all of them: the gap between the last
             producer's end and the first consumer's start, and how long
             the consumer's first read takes (data written on other dies);
* empty      back-to-back empty kernels, eager and inside a HIP graph;
* pingpong   a flag bounced between two workgroups with agent-scope
             atomics (one-way latency), on the same die and across dies,
             relaxed and as release/acquire with a payload;
* chain      a graph of dependent minimal launches (each reads what the
             previous one wrote): us per launch, with the default argument
             loads and with the arguments preloaded (libhfq4probe_kp.so);
* read       a plain streaming read of a large buffer (GB/s).
"""

import ctypes
import os

HERE = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_PATH = os.path.join(HERE, "libhfq4probe.so")
LIB_PATH_KP = os.path.join(HERE, "libhfq4probe_kp.so")
TICK_NS = 10.0   # s_memrealtime runs at 100 MHz


def _lib(preload=False):
    path = LIB_PATH_KP if preload else LIB_PATH
    if not os.path.exists(path):
        raise ImportError("%s not built -- run 'python quantized_moe_decode_amd/build.py'" % path)
    lib = ctypes.CDLL(path)
    P, I, U32, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint32, ctypes.c_size_t
    for name, args in {"probe_chase": [P, U32, I, P, P], "probe_empty": [I, I, P],
                       "probe_pingpong": [P, P, I, I, I, I, P, P],
                       "probe_produce": [P, I, P, P], "probe_consume": [P, I, P, P, P],
                       "probe_read": [P, SZ, I, P, P],
                       "probe_exchange": [P, P, I, I, U32, I, P, I, I, P],
                       "probe_spin": [ctypes.c_uint64, P], "probe_chain": [P, P, I, P]}.items():
        f = getattr(lib, name)
        f.restype = I
        f.argtypes = args
    return lib


def _s(torch):
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _ok(rc, what):
    if rc != 0:
        raise RuntimeError("%s: HIP error %d" % (what, rc))


def chase(torch, footprint, hops=20000, seed=0):
    """ns per dependent load over a random cycle of 128-byte lines spanning
    `footprint` bytes."""
    lib = _lib()
    lines = footprint // 128
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    perm = torch.randperm(lines, generator=g, device="cuda", dtype=torch.int64)
    nxt = torch.zeros(lines * 32, dtype=torch.int32, device="cuda")
    # line perm[i] points at line perm[i+1] (one cycle through every line)
    nxt[perm * 32] = (torch.roll(perm, -1) * 32).to(torch.int32)
    out = torch.zeros(2, dtype=torch.int64, device="cuda")
    start = int(perm[0].item()) * 32
    _ok(lib.probe_chase(_p(nxt), start, hops, _p(out), _s(torch)), "probe_chase")
    torch.cuda.synchronize()
    ticks = int(out[0].item())
    del nxt, perm
    return ticks * TICK_NS / hops


def boundary(torch, n=256, reps=50):
    """Producer -> consumer launch pair on one stream, inside a HIP graph:
    (median gap between the last producer store and the first consumer
    start, median time of the consumer's read of the n values, fraction of
    consumer workgroups that ran on another die than value 0's producer)."""
    import numpy as np
    lib = _lib()
    vals = torch.zeros(n, dtype=torch.float32, device="cuda")
    stamps = torch.zeros(4 * n, dtype=torch.int64, device="cuda")
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    gaps, reads = [], []
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            _ok(lib.probe_produce(_p(vals), n, _p(stamps), _s(torch)), "probe_produce")
            _ok(lib.probe_consume(_p(vals), n, _p(stamps), _p(sink), _s(torch)), "probe_consume")
    for _ in range(reps):
        g.replay()
        torch.cuda.synchronize()
        st = stamps.cpu().numpy()
        prod_end = st[:n].max()
        cons_start = st[n:2 * n]
        gaps.append((cons_start.min() - prod_end) * TICK_NS)
        reads.append(np.median(st[2 * n:3 * n] - cons_start) * TICK_NS)
    return float(np.median(gaps)), float(np.median(reads))


def empty(torch, n=2000, grid=256, block=256):
    """us per empty kernel: (eager back to back, inside one HIP graph)."""
    lib = _lib()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(100):
        _ok(lib.probe_empty(grid, block, _s(torch)), "probe_empty")
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(n):
        lib.probe_empty(grid, block, _s(torch))
    ev1.record()
    torch.cuda.synchronize()
    eager = ev0.elapsed_time(ev1) * 1e3 / n
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for _ in range(n):
                lib.probe_empty(grid, block, _s(torch))
    g.replay()
    torch.cuda.synchronize()
    ev0.record()
    g.replay()
    ev1.record()
    torch.cuda.synchronize()
    return eager, ev0.elapsed_time(ev1) * 1e3 / n


def pingpong(torch, partner, rounds=2000, release=False, payload_words=0):
    """One-way flag latency in ns between workgroup 0 and `partner` (half a
    round trip), and the two workgroups' die ids."""
    lib = _lib()
    flags = torch.zeros(64, dtype=torch.int32, device="cuda")
    payload = torch.zeros(max(payload_words, 1), dtype=torch.int32, device="cuda")
    out = torch.zeros(8, dtype=torch.int64, device="cuda")
    _ok(lib.probe_pingpong(_p(flags), _p(payload), payload_words, rounds, partner,
                           1 if release else 0, _p(out), _s(torch)), "probe_pingpong")
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    if o[4]:
        return None, int(o[2]), int(o[3])
    return float(o[0]) * TICK_NS / rounds / 2.0, int(o[2]), int(o[3])


def exchange(torch, per_wg, flags=False, nwg=None, reps=20, replicas=1, stagger=False):
    """All-to-all exchange inside one launch: every workgroup publishes
    per_wg tagged words and polls all of them.  Returns (median over
    launches of: last workgroup done - last publish, in ns; median poll
    rounds; timeouts)."""
    import numpy as np
    lib = _lib()
    nwg = nwg or torch.cuda.get_device_properties(0).multi_processor_count
    words = torch.zeros(replicas * nwg * per_wg, dtype=torch.int64, device="cuda")
    flagw = torch.zeros(nwg, dtype=torch.int32, device="cuda")
    stamps = torch.zeros(4 * nwg, dtype=torch.int64, device="cuda")
    spans, rounds, tos = [], [], 0
    for r in range(reps):
        _ok(lib.probe_exchange(_p(words), _p(flagw), nwg, per_wg, r + 1, 1 if flags else 0,
                               _p(stamps), replicas, 1 if stagger else 0, _s(torch)),
            "probe_exchange")
        torch.cuda.synchronize()
        st = stamps.cpu().numpy()
        spans.append((st[nwg:2 * nwg].max() - st[:nwg].max()) * TICK_NS)
        rounds.append(np.median(st[2 * nwg:3 * nwg]))
        tos += int(st[3 * nwg:].sum())
    return float(np.median(spans)), float(np.median(rounds)), tos


def spin(torch, us):
    """Keep the device busy for `us` microseconds (one wave) on the current
    stream: put in front of a timed region so that the host has enqueued the
    region's work before the device reaches it."""
    _ok(_lib().probe_spin(int(us * 100), _s(torch)), "probe_spin")


def read(torch, nbytes=1 << 32, reps=5):
    """Best GB/s of a plain streaming read of nbytes in HBM."""
    lib = _lib()
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    grid = 8 * torch.cuda.get_device_properties(0).multi_processor_count
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    _ok(lib.probe_read(_p(buf), nbytes, grid, _p(sink), _s(torch)), "probe_read")
    best = 0.0
    for _ in range(reps):
        ev0.record()
        lib.probe_read(_p(buf), nbytes, grid, _p(sink), _s(torch))
        ev1.record()
        torch.cuda.synchronize()
        best = max(best, nbytes / (ev0.elapsed_time(ev1) / 1e3) / 1e9)
    del buf
    return best


def chain(torch, preload=False, launches=400, reps=20, n=256 * 64):
    """us per launch of a HIP graph of dependent minimal launches (256
    workgroups of 64 threads, each element read from the previous launch's
    output), timed over replays after a first one."""
    lib = _lib(preload)
    a = torch.zeros(n, dtype=torch.float32, device="cuda")
    b = torch.zeros(n, dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for i in range(launches):
                src, dst = (a, b) if i % 2 == 0 else (b, a)
                _ok(lib.probe_chain(_p(src), _p(dst), n, _s(torch)), "probe_chain")
    g.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(reps):
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    if float(a[0]) != (reps + 1) * launches:
        raise RuntimeError("chain probe: wrong count %s" % float(a[0]))
    return ev0.elapsed_time(ev1) * 1e3 / (reps * launches)


def run_all(torch, log=print):
    """Every probe once; returns a dict of the numbers."""
    res = {}
    for name, fp in (("l2", 1 << 20), ("infinity_cache", 64 << 20), ("hbm", 4 << 30)):
        res["chase_ns_" + name] = round(chase(torch, fp), 1)
        log("chase %s (%d B footprint): %.1f ns per dependent load" % (name, fp, res["chase_ns_" + name]))
    gap, rd = boundary(torch)
    res["boundary_gap_ns"], res["boundary_first_read_ns"] = round(gap, 1), round(rd, 1)
    log("graph boundary: %.0f ns from last producer store to first consumer start; "
        "consumer read of 256 values written on other dies %.0f ns" % (gap, rd))
    res["chain_us_per_launch"] = round(chain(torch), 3)
    res["chain_us_per_launch_kernarg_preload"] = round(chain(torch, preload=True), 3)
    log("dependent minimal launches in a graph: %.2f us each; with the kernel arguments "
        "preloaded into scalar registers %.2f us"
        % (res["chain_us_per_launch"], res["chain_us_per_launch_kernarg_preload"]))
    eager, graph = empty(torch)
    res["empty_kernel_us_eager"], res["empty_kernel_us_graph"] = round(eager, 3), round(graph, 3)
    log("empty 256x256 kernel: %.2f us eager, %.2f us in a graph" % (eager, graph))
    pp = {}
    for partner in (8, 1, 2, 3, 4, 5, 6, 7):
        ns, a, b = pingpong(torch, partner)
        pp["wg0-wg%d" % partner] = {"ns": None if ns is None else round(ns, 1), "dies": [a, b]}
        log("flag one-way wg0 -> wg%d (dies %d, %d): %s ns" % (partner, a, b, ns))
    res["flag_relaxed_agent"] = pp
    ns, a, b = pingpong(torch, 1, rounds=1000, release=True, payload_words=256)
    res["flag_release_acquire_1KiB_ns"] = None if ns is None else round(ns, 1)
    log("release/acquire message of 1 KiB, one way (dies %d, %d): %s ns" % (a, b, ns))
    for per_wg, fl, rep, stg in ((1, False, 1, False), (1, False, 8, False), (1, False, 32, False),
                                 (16, False, 1, False), (16, False, 1, True), (16, False, 8, False),
                                 (16, False, 8, True), (16, True, 8, True), (2, False, 8, True)):
        ns, rnd, to = exchange(torch, per_wg, flags=fl, replicas=rep, stagger=stg)
        key = "exchange_%dw_r%d%s%s" % (per_wg, rep, "_stagger" if stg else "", "_flags" if fl else "")
        res[key] = {"ns": round(ns, 1), "median_rounds": rnd, "timeouts": to}
        log("all-to-all exchange, %d tagged words per workgroup, %d copies%s%s: %.0f ns after the "
            "last publish (median %.0f poll rounds, %d timeouts)"
            % (per_wg, rep, ", staggered reads" if stg else "",
               ", behind per-workgroup flags" if fl else "", ns, rnd, to))
    res["read_gbs"] = round(read(torch), 1)
    log("streaming read of 4 GiB: %.1f GB/s" % res["read_gbs"])
    return res
