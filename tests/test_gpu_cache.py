"""GPU parity of the HBM expert cache (pointer-table layers) and of the CPU
route for host-resident experts, through the C ABI.

* A table layer whose experts sit in a shuffled HBM pool, and one whose
  experts are half in the pool and half in pinned host memory, give the
  same bits as the layer holding the same bytes in one HBM tensor each, and
  the oracle's result; the hit counters count exactly the selections of
  resident experts.
* Hot-set placement from a calibration pass keeps the most often selected
  experts of a Zipf-skewed router in HBM (the hit rate on fresh tokens is
  well above the resident fraction).
* The CPU route (router on the GPU, experts on the host CPU) matches the
  GPU's host-mapped layer and the oracle.
"""

import numpy as np
import pytest

import synth
from oracle import moe as om

from _parity import REL_L2_TOL, ExpertCache, oracle_layer_check, rel_l2

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module")
def q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_moe_decode_amd as q
    import quantized_moe_decode_amd.synthetic  # noqa: F401
    import quantized_moe_decode_amd.cache  # noqa: F401
    q.lib.hfq4_debug_set_arch(b"")
    return q


SEED, E, D, F, K = 13, 64, 2048, 512, 8


@pytest.fixture(scope="module")
def layers(q):
    say("building the HBM and pinned copies of a 64-expert layer")
    bias = synth.zipf_bias(5, E)
    hbm = q.synthetic.build_layer(torch, SEED, 0, E, D, F, bias=bias)
    host = q.synthetic.build_layer(torch, SEED, 0, E, D, F, bias=bias, host_mapped=True)
    return hbm, host, bias


@pytest.mark.parametrize("pattern", ["all", "half", "none"])
def test_table_layer_bitwise_and_hits(q, layers, pattern):
    hbm, host, bias = layers
    rng = np.random.default_rng(7)
    resident = np.zeros((1, E), dtype=np.uint8)
    if pattern == "all":
        resident[:] = 1
    elif pattern == "half":
        resident[0, rng.permutation(E)[:E // 2]] = 1
    say("table layer, resident:", pattern)
    tables, pool = q.cache.build_cache(torch, [host], resident)
    T = tables[0]
    hits = torch.zeros(2, dtype=torch.int64, device="cuda")
    ws = q.new_workspace(hbm, 1, K)
    ws_t = q.new_workspace(hbm, 1, K)
    xs = synth.activations(torch, "cuda", 77, 6, D)
    n_res = 0
    cache = ExpertCache(torch, "cuda", SEED, 0, D, F)
    for t in range(xs.shape[0]):
        x = xs[t:t + 1].contiguous()
        i1, w1, y1 = q.moe_layer_decode(hbm, x, K, ws, residual=x)
        i2, w2, y2 = q.moe_layer_decode_table(T, x, K, ws_t, residual=x, hits=hits)
        torch.cuda.synchronize()
        assert torch.equal(i1, i2) and torch.equal(w1, w2) and torch.equal(y1, y2), t
        n_res += int(resident[0, i2.cpu().numpy()[0]].sum())
        if t < 2:
            err, amb = oracle_layer_check(x.cpu().numpy(), hbm.Wr.cpu().numpy(), bias, cache, K,
                                          i2.cpu().numpy(), w2.cpu().numpy(), y2.cpu().numpy(),
                                          residual=x.cpu().numpy())
            assert amb == 0 and err <= REL_L2_TOL, (amb, err)
    assert q.workspace_error(ws_t) == 0
    h = hits.cpu().numpy().tolist()
    assert h == [n_res, xs.shape[0] * K - n_res], (h, n_res)


def test_hotset_placement_hit_rate(q, layers):
    hbm, host, bias = layers
    calib = synth.activations(torch, "cuda", 88, 256, D)
    heat = q.cache.routing_heat(torch, [hbm], calib, K)
    assert int(heat.sum()) == 256 * K
    eb = hbm.expert_bytes()
    budget = 16 * eb + 123          # a quarter of the experts
    tables, pool, resident, placed = q.cache.place_and_build(torch, [host], heat, budget, 0)
    assert resident.sum() == 16 and placed == 16 * eb
    # the placed experts are the 16 hottest
    hottest = np.argsort(-heat[0].astype(np.int64), kind="stable")[:16]
    assert set(np.nonzero(resident[0])[0].tolist()) == set(hottest.tolist())
    hits = torch.zeros(2, dtype=torch.int64, device="cuda")
    ws = q.new_workspace(hbm, 1, K)
    xs = synth.activations(torch, "cuda", 99, 64, D)
    for t in range(xs.shape[0]):
        q.moe_layer_decode_table(tables[0], xs[t:t + 1].contiguous(), K, ws, hits=hits)
    torch.cuda.synchronize()
    h = hits.cpu().numpy()
    rate = h[0] / h.sum()
    say("hot-set hit rate with a quarter of the experts resident: %.3f" % rate)
    assert h.sum() == 64 * K and rate > 0.4


def test_cpu_route_matches_gpu_and_oracle(q, layers):
    hbm, host, bias = layers
    hl = q.HostMoeLayer(host.gate, host.up, host.down, E, D, F)
    xs = synth.activations(torch, "cuda", 55, 3, D)
    cache = ExpertCache(torch, "cuda", SEED, 0, D, F)
    ws = q.new_workspace(host, 1, K)
    rws = torch.zeros(q.moe_route_workspace_bytes(E, 1), dtype=torch.uint8, device="cuda")
    for t in range(xs.shape[0]):
        x = xs[t:t + 1].contiguous()
        i_g, w_g, y_g = q.moe_layer_decode(host, x, K, ws)          # GPU reads over PCIe
        idx, wts = q.moe_route_topk(hbm.Wr, x, K, bias=hbm.bias, ws=rws)
        y_c, err = q.moe_expert_decode_host(hl, x.cpu().numpy(), idx.cpu().numpy(),
                                            wts.cpu().numpy())
        assert err == 0
        assert torch.equal(idx, i_g) and torch.equal(wts, w_g)
        assert rel_l2(y_c[0], y_g.cpu().numpy()[0]) <= REL_L2_TOL
        e2, amb = oracle_layer_check(x.cpu().numpy(), hbm.Wr.cpu().numpy(), bias, cache, K,
                                     idx.cpu().numpy(), wts.cpu().numpy(), y_c)
        assert amb == 0 and e2 <= REL_L2_TOL, e2


def test_measure_routes_choice(q, layers):
    """The load-time route probe: both routes timed, every host row kernel
    the CPU has timed twice, the fastest kept selected, and the route the
    15 % rule gives for the two times."""
    from quantized_moe_decode_amd.offload import measure_routes
    hbm, host, bias = layers
    say("route probe on the 64-expert host-resident layer")
    xs = synth.activations(torch, "cuda", 57, 6, D)
    try:
        m = measure_routes(torch, host, xs, K, nthreads=4, warm=1)
        by = m["cpu_us_per_step_by_host_kernel"]
        assert "portable" in by and m["host_kernel"] in by
        assert all(len(v) == 2 and min(v) > 0 for v in by.values())
        assert min(by[m["host_kernel"]]) == min(min(v) for v in by.values())
        assert abs(m["cpu_s_per_step"] * 1e6 - min(by[m["host_kernel"]])) <= 0.1
        assert m["pcie_s_per_step"] > 0 and m["steps"] == 6
        assert m["expert_bytes_per_step"] == K * host.expert_bytes()
        assert m["route"] == ("cpu" if q.hfq4_offload_choice(m["pcie_s_per_step"],
                                                              m["cpu_s_per_step"]) else "pcie")
        assert q.set_host_kernel(m["host_kernel"]) == m["host_kernel"]
    finally:
        q.set_host_kernel("best")


@pytest.mark.parametrize("En,k", [(256, 8), (100, 4), (1024, 8), (512, 2), (64, 8), (700, 4),
                                  (100, 6)])
def test_single_launch_equals_three_launch(q, En, k):
    """The single-launch one-token kernel (which the table layers run on),
    and its two-launch form (its routing and gate/up phases, then the down
    kernel), give the same bits as the three-launch chain for expert counts
    that take every top-k width and k = 2, 4, 8 (k = 6 runs the chain every
    time), report no device error, and keep doing so when batched calls
    share the workspace between one-token calls."""
    L = q.synthetic.build_layer(torch, 31, 0, En, D, F)
    xs = synth.activations(torch, "cuda", 32, 6, D)
    outs = []
    try:
        for mode in (0, 1, 2):   # three launches, one, two
            q.lib.hfq4_debug_set_single_launch(mode)
            ws = q.new_workspace(L, 4, k)
            got = []
            for t in range(xs.shape[0]):
                if t == 3:   # a batched call on the same workspace
                    q.moe_layer_decode(L, xs[:4], k, ws)
                got.append(tuple(v.clone() for v in q.moe_layer_decode(L, xs[t:t + 1], k, ws,
                                                                        residual=xs[t:t + 1])))
            torch.cuda.synchronize()
            assert q.workspace_error(ws) == 0
            outs.append(got)
    finally:
        q.lib.hfq4_debug_set_single_launch(0)
    for other in outs[1:]:
        for a, b in zip(outs[0], other):
            for u, v in zip(a, b):
                assert torch.equal(u, v)


@pytest.mark.parametrize("k", [2, 4, 8])
def test_single_launch_given_routing(q, k):
    """moe_expert_decode with the routing given: the single launch equals
    the three-launch chain bit for bit, an index out of range is a dead slot
    on both (INDEX error bit, nothing added), and the oracle agrees."""
    En = 128
    L = q.synthetic.build_layer(torch, 41, 0, En, D, F)
    rng = np.random.default_rng(k)
    xs = synth.activations(torch, "cuda", 42, 3, D)
    idx = torch.from_numpy(np.stack([rng.permutation(En)[:k] for _ in range(3)]).astype(np.int32)).cuda()
    wts = torch.from_numpy(rng.uniform(0.05, 1, size=(3, k)).astype(np.float32)).cuda()
    bad = idx.clone()
    bad[0, k - 1] = En + 5            # out of range: a dead slot
    res = []
    try:
        for single in (0, 1):
            q.lib.hfq4_debug_set_single_launch(single)
            ws = q.new_workspace(L, 1, k)
            out = []
            for t in range(3):
                out.append(q.moe_expert_decode(L, xs[t:t + 1], idx[t:t + 1], wts[t:t + 1], ws,
                                               residual=xs[t:t + 1]).clone())
            torch.cuda.synchronize()
            assert q.workspace_error(ws) == 0
            ws2 = q.new_workspace(L, 1, k)
            yb = q.moe_expert_decode(L, xs[0:1], bad[0:1], wts[0:1], ws2).clone()
            torch.cuda.synchronize()
            assert q.workspace_error(ws2) & 1
            res.append((out, yb))
    finally:
        q.lib.hfq4_debug_set_single_launch(0)
    for u, v in zip(res[0][0], res[1][0]):
        assert torch.equal(u, v)
    assert torch.equal(res[0][1], res[1][1])
    cache = ExpertCache(torch, "cuda", 41, 0, D, F)
    for t in range(2):
        x64 = xs[t].cpu().numpy().astype(np.float64)
        outs = [om.expert_forward(cache(int(e)), x64) for e in idx[t].cpu().numpy()]
        ref = om.combine(outs, wts[t].cpu().numpy()) + x64
        assert rel_l2(res[1][0][t].cpu().numpy()[0], ref) <= REL_L2_TOL, t
