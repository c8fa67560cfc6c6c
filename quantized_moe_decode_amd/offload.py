"""Host-resident experts: the measured choice between reading them over PCIe
from the GPU kernel and computing them on the host CPU.

hipfire expert-offload explainer, section "PCIe 直通": by default the GPU
kernel reads host-mapped experts over PCIe; at load the engine times the
PCIe path against a CPU GEMV on this machine and switches to the CPU only
when the CPU is at least 15% faster (the rule itself is the library's
hfq4_offload_choice).  Strata user report, section "1. Strata 是什么":
experts that are not on the device run on the CPU.

measure_routes times one decode step of a host-resident layer both ways:

* pcie -- moe_layer_decode on the host-mapped layer: the router and every
  expert kernel on the GPU, the expert bytes crossing PCIe;
* cpu  -- the router on the GPU (moe_route_topk), the routing and the
  activation copied to pinned host buffers, the experts on the host CPU
  (moe_expert_decode_host), the output copied back: a host round trip per
  layer, which is what a decode with CPU experts pays.  The host row kernel
  is itself chosen by measurement: which of the CPU's instruction sets
  decodes HFQ4 fastest differs between CPUs (a wider vector does not always
  win).
"""

import time

from . import (Hfq4Error, HostMoeLayer, hfq4_offload_choice, moe_expert_decode_host,
               moe_layer_decode, moe_route_topk, moe_route_workspace_bytes, new_workspace,
               set_host_kernel)


def measure_routes(torch, layer, xs, k, nthreads=0, warm=3,
                   host_kernels=("avx512", "avx2", "portable")):
    """layer: a host-mapped MoeLayer (pinned experts, router on the device);
    xs: device tokens [N, d].  Returns a dict with both per-step times, the
    expert bytes a step moves and the route chosen.  The CPU route is timed
    with each host row kernel of host_kernels that this CPU has, and the
    fastest stays selected (process-wide) for later host calls."""
    N, d = xs.shape
    dev = xs.device
    # PCIe: GPU kernels read the pinned experts zero-copy
    ws = new_workspace(layer, 1, k, dev)
    y = torch.empty((1, d), dtype=torch.float32, device=dev)
    idx = torch.empty((1, k), dtype=torch.int32, device=dev)
    wts = torch.empty((1, k), dtype=torch.float32, device=dev)
    for t in range(warm):
        moe_layer_decode(layer, xs[t:t + 1], k, ws, y=y, idx=idx, wts=wts)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for t in range(N):
        moe_layer_decode(layer, xs[t:t + 1], k, ws, y=y, idx=idx, wts=wts)
    ev1.record()
    torch.cuda.synchronize()
    t_pcie = ev0.elapsed_time(ev1) / 1e3 / N
    # CPU: router on the GPU, experts on the host
    hl = HostMoeLayer(layer.gate, layer.up, layer.down, layer.E, layer.d, layer.F)
    rws = torch.zeros(moe_route_workspace_bytes(layer.E, 1), dtype=torch.uint8, device=dev)
    x_h = torch.empty((1, d), dtype=torch.float32, pin_memory=True)
    i_h = torch.empty((1, k), dtype=torch.int32, pin_memory=True)
    w_h = torch.empty((1, k), dtype=torch.float32, pin_memory=True)
    y_h = torch.empty((1, d), dtype=torch.float32, pin_memory=True)
    y_c = torch.empty((1, d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def cpu_step(x):
        moe_route_topk(layer.Wr, x, k, bias=layer.bias, ws=rws, idx=idx, wts=wts)
        i_h.copy_(idx, non_blocking=True)
        w_h.copy_(wts, non_blocking=True)
        x_h.copy_(x, non_blocking=True)
        stream.synchronize()
        moe_expert_decode_host(hl, x_h, i_h, w_h, y=y_h, nthreads=nthreads)
        y_c.copy_(y_h, non_blocking=True)

    def time_cpu():
        for t in range(warm):
            cpu_step(xs[t:t + 1])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(N):
            cpu_step(xs[t:t + 1])
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / N

    # every host row kernel this CPU has, twice in turn (the first pass also
    # warms the host threads and the experts' page translations); the
    # fastest one stays selected for the CPU route
    kernels = []
    for name in host_kernels:
        try:
            set_host_kernel(name)
            kernels.append(name)
        except Hfq4Error:
            pass
    by_kernel = {name: [] for name in kernels}
    for _ in range(2):
        for name in kernels:
            set_host_kernel(name)
            by_kernel[name].append(time_cpu())
    fastest = min(kernels, key=lambda name: min(by_kernel[name]))
    set_host_kernel(fastest)
    t_cpu = min(by_kernel[fastest])
    eb = k * layer.expert_bytes()
    use_cpu = hfq4_offload_choice(t_pcie, t_cpu)
    return {"pcie_s_per_step": t_pcie, "cpu_s_per_step": t_cpu, "expert_bytes_per_step": eb,
            "pcie_expert_gbs": eb / t_pcie / 1e9, "cpu_expert_gbs": eb / t_cpu / 1e9,
            "route": "cpu" if use_cpu else "pcie", "steps": N, "host_kernel": fastest,
            "cpu_us_per_step_by_host_kernel": {n: [round(v * 1e6, 1) for v in ts]
                                               for n, ts in by_kernel.items()}}
