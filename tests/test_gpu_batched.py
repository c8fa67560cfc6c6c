"""GPU parity of the batched (2..16 tokens) decode path on MFMA, and of the
single-token path at expert counts other than the benchmark's.

Token batches of the d=2048-class, F=512 layer shape run through matrix-core
kernels that group the (token, slot) pairs by expert.  Every case is checked
against the oracle token by token (routing exact up to the stated tie rule,
weights within 1e-5, output relative L2 <= 2e-3), plus the properties the
grouping must keep: caller-supplied duplicate experts count once per slot,
invalid indices contribute nothing, graph replays match eager runs bit for
bit, and repeated calls are bitwise identical."""

import numpy as np
import pytest

from oracle import moe
import synth

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
    q.lib.hfq4_debug_set_arch(b"")
    return q


_layers = {}


def _layer(q, seed, E, d, F=512, bias=None):
    key = (seed, E, d, F, bias is not None)
    if key not in _layers:
        L = q.synthetic.build_layer(torch, seed=seed, layer_id=0, E=E, d=d, F=F, bias=bias)
        _layers[key] = (L, ExpertCache(torch, "cuda", seed, 0, d, F))
    return _layers[key]


@pytest.mark.parametrize("B,k,d,E", [(2, 8, 2048, 64), (3, 8, 2048, 256), (8, 8, 2048, 512),
                                     (16, 8, 1920, 32), (5, 1, 2048, 16), (4, 4, 2048, 8),
                                     (16, 8, 2048, 16), (6, 8, 2048, 1024), (7, 6, 2000, 100)])
@pytest.mark.parametrize("fused", [True, False])
def test_batched_layer_vs_oracle(q, B, k, d, E, fused):
    say("batched B=%d k=%d d=%d E=%d fused=%s" % (B, k, d, E, fused))
    L, cache = _layer(q, 21, E, d)
    x = synth.activations(torch, "cuda", 100 + B, B, d)
    res = synth.activations(torch, "cuda", 200 + B, B, d)
    ws = q.new_workspace(L, B, k)
    if fused:
        idx, wts, y = q.moe_layer_decode(L, x, k, ws, residual=res)
    else:
        idx, wts = q.moe_route_topk(L.Wr, x, k, ws=ws)
        y = q.moe_expert_decode(L, x, idx, wts, ws, residual=res)
    torch.cuda.synchronize()
    assert q.workspace_error(ws) == 0
    err, amb = oracle_layer_check(x.cpu().numpy(), L.Wr.cpu().numpy(), None, cache, k,
                                  idx.cpu().numpy(), wts.cpu().numpy(), y.cpu().numpy(),
                                  residual=res.cpu().numpy())
    say("max rel-L2 %.3g, tie-ambiguous tokens %d" % (err, amb))
    assert amb == 0 and err <= REL_L2_TOL


@pytest.mark.parametrize("E,k", [(100, 8), (1024, 8), (1024, 1), (64, 5)])
def test_single_token_expert_counts(q, E, k):
    """One token on the VALU path (top-k inside the gate/up kernel) with
    expert counts that are not 256: 100 (not a multiple of the wave), 1024
    (16 logits per lane), 64 (one per lane), against the oracle."""
    d = 2048
    say("single token E=%d k=%d" % (E, k))
    L, cache = _layer(q, 25, E, d)
    x = synth.activations(torch, "cuda", 500 + E + k, 1, d)
    res = synth.activations(torch, "cuda", 600 + E + k, 1, d)
    ws = q.new_workspace(L, 1, k)
    idx, wts, y = q.moe_layer_decode(L, x, k, ws, residual=res)
    torch.cuda.synchronize()
    assert q.workspace_error(ws) == 0
    err, amb = oracle_layer_check(x.cpu().numpy(), L.Wr.cpu().numpy(), None, cache, k,
                                  idx.cpu().numpy(), wts.cpu().numpy(), y.cpu().numpy(),
                                  residual=res.cpu().numpy())
    assert amb == 0 and err <= REL_L2_TOL
    # the two-call form gives the same bits
    i2, w2 = q.moe_route_topk(L.Wr, x, k, ws=ws)
    y2 = q.moe_expert_decode(L, x, i2, w2, ws, residual=res)
    torch.cuda.synchronize()
    assert torch.equal(idx, i2) and torch.equal(wts, w2) and torch.equal(y, y2)


@pytest.mark.parametrize("B,E,skew", [(16, 512, True), (6, 1024, False), (3, 100, False)])
def test_batched_fused_equals_two_call_bitwise(q, B, E, skew):
    """The fused layer routes inside the gate/up kernel; moe_route_topk runs
    the same routing functions in its own kernel.  Indices, weights, logits
    and outputs of the two forms are identical bit for bit."""
    d, k = 2048, 8
    bias = synth.zipf_bias(7, E) if skew else None
    say("fused vs two-call B=%d E=%d skew=%s" % (B, E, skew))
    L, _ = _layer(q, 23, E, d, bias=bias)
    x = synth.activations(torch, "cuda", 300 + B, B, d)
    res = synth.activations(torch, "cuda", 400 + B, B, d)
    ws = q.new_workspace(L, B, k)
    i1, w1, y1 = q.moe_layer_decode(L, x, k, ws, residual=res)
    i1, w1, y1 = i1.clone(), w1.clone(), y1.clone()
    lg = torch.empty(B, E, device="cuda")
    i2, w2 = q.moe_route_topk(L.Wr, x, k, ws=ws, bias=L.bias, logits=lg)
    y2 = q.moe_expert_decode(L, x, i2, w2, ws, residual=res)
    torch.cuda.synchronize()
    assert q.workspace_error(ws) == 0
    assert torch.equal(i1, i2) and torch.equal(w1, w2) and torch.equal(y1, y2)
    # the logits the routing saw: the selected experts are their top k
    top = torch.topk(lg, k, dim=1).values
    sel = torch.gather(lg, 1, i2.long())
    assert torch.equal(torch.sort(sel, dim=1, descending=True).values, top)


@pytest.mark.parametrize("B,E,skew", [(2, 256, False), (5, 512, True), (8, 1024, False),
                                      (12, 512, True), (16, 64, False)])
def test_route_exchange_equals_per_workgroup_routing(q, B, E, skew):
    """Routing by exchange (one router workgroup per token, selections
    gathered through tagged words) and routing in every gate/up workgroup
    give the same bits at every batch size, with batched calls of the other
    mode and one-token calls sharing the workspace in between, and report no
    device error."""
    d, k = 2048, 8
    bias = synth.zipf_bias(9, E) if skew else None
    say("route exchange vs per-workgroup B=%d E=%d skew=%s" % (B, E, skew))
    L, cache = _layer(q, 27, E, d, bias=bias)
    x = synth.activations(torch, "cuda", 500 + B, 3 * B, d)
    res = synth.activations(torch, "cuda", 600 + B, B, d)
    ws = q.new_workspace(L, B, k)
    outs = {}
    try:
        for mb in (2, 17, 2):                     # exchange, per workgroup, exchange again
            q.lib.hfq4_debug_set_route_exchange(mb)
            got = []
            for t in range(3):
                got.append(tuple(v.clone() for v in
                                 q.moe_layer_decode(L, x[t * B:(t + 1) * B], k, ws, residual=res)))
                q.moe_layer_decode(L, x[t:t + 1], k, ws)   # a one-token call in between
            torch.cuda.synchronize()
            assert q.workspace_error(ws) == 0, mb
            outs.setdefault(mb, []).append(got)
    finally:
        q.lib.hfq4_debug_set_route_exchange(9)
    ref = outs[17][0]
    for runs in outs.values():
        for got in runs:
            for a, b in zip(ref, got):
                for u, v in zip(a, b):
                    assert torch.equal(u, v)
    i, w, y = ref[0]
    err, amb = oracle_layer_check(x[:B].cpu().numpy(), L.Wr.cpu().numpy(), bias, cache, k,
                                  i.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy(),
                                  residual=res.cpu().numpy())
    assert amb == 0 and err <= REL_L2_TOL, (amb, err)


def test_batched_duplicates_and_invalid(q):
    """Caller routing with a repeated expert inside a token and an index out
    of range: the repeat counts as its own slot, the bad slot adds nothing
    and sets the index error bit."""
    B, k, d, E = 4, 8, 2048, 32
    L, cache = _layer(q, 21, E, d)
    say("duplicates / invalid")
    x = synth.activations(torch, "cuda", 7, B, d)
    rng = np.random.default_rng(5)
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(B)]).astype(np.int32)
    idx[0, 3] = idx[0, 1]            # repeat inside token 0
    idx[1, :] = idx[2, :]            # tokens 1 and 2 pick the same experts
    idx[3, 5] = E + 3                # invalid
    wts = rng.random((B, k)).astype(np.float32)
    ws = q.new_workspace(L, B, k)
    y = q.moe_expert_decode(L, x, torch.from_numpy(idx).cuda(), torch.from_numpy(wts).cuda(), ws)
    torch.cuda.synchronize()
    assert q.workspace_error(ws) & q.HFQ4_DEV_ERR_INDEX
    xs = x.cpu().numpy().astype(np.float64)
    yg = y.cpu().numpy()
    for b in range(B):
        outs, ws_b = [], []
        for j in range(k):
            e = int(idx[b, j])
            if 0 <= e < E:
                outs.append(moe.expert_forward(cache(e), xs[b]))
                ws_b.append(float(wts[b, j]))
        ref = moe.combine(outs, np.array(ws_b))
        assert rel_l2(yg[b], ref) <= REL_L2_TOL, b


def test_batched_invalid_ignores_stale_h(q):
    """An out-of-range slot adds nothing when the workspace still holds
    non-finite h from an earlier call."""
    B, k, d, E = 3, 8, 2048, 32
    L, cache = _layer(q, 21, E, d)
    say("batched invalid, stale h")
    ws = q.new_workspace(L, B, k)
    idx0 = torch.arange(k, dtype=torch.int32, device="cuda").repeat(B, 1)
    wts = torch.full((B, k), 1.0 / k, dtype=torch.float32, device="cuda")
    xbad = torch.full((B, d), float("nan"), dtype=torch.float32, device="cuda")
    q.moe_expert_decode(L, xbad, idx0, wts, ws)
    torch.cuda.synchronize()
    x = synth.activations(torch, "cuda", 12, B, d)
    idx = idx0.clone()
    idx[1, 2] = -5
    y = q.moe_expert_decode(L, x, idx, wts, ws).cpu().numpy()
    assert q.workspace_error(ws) & q.HFQ4_DEV_ERR_INDEX
    assert np.all(np.isfinite(y))
    xs = x.cpu().numpy().astype(np.float64)
    for b in range(B):
        outs = [moe.expert_forward(cache(j), xs[b]) for j in range(k) if not (b == 1 and j == 2)]
        ref = moe.combine(outs, np.full(len(outs), 1.0 / k))
        assert rel_l2(y[b], ref) <= REL_L2_TOL, b


def test_batched_all_invalid_gives_residual(q):
    B, k, d, E = 3, 8, 2048, 16
    L, _ = _layer(q, 21, E, d)
    say("all invalid")
    x = synth.activations(torch, "cuda", 8, B, d)
    res = synth.activations(torch, "cuda", 9, B, d)
    idx = torch.full((B, k), -1, dtype=torch.int32, device="cuda")
    wts = torch.ones((B, k), dtype=torch.float32, device="cuda")
    ws = q.new_workspace(L, B, k)
    y = q.moe_expert_decode(L, x, idx, wts, ws, residual=res)
    torch.cuda.synchronize()
    assert q.workspace_error(ws) & q.HFQ4_DEV_ERR_INDEX
    assert torch.equal(y, res)


def test_batched_graph_replays_and_determinism(q):
    """Several batched layer calls captured in one graph: every replay (with
    eager work between replays) equals the eager results bit for bit."""
    d, E, k = 2048, 64, 8
    L, _ = _layer(q, 21, E, d)
    say("graph replays")
    xs = synth.activations(torch, "cuda", 11, 3 * 16, d).view(3, 16, d)
    Bs = [4, 16, 2]
    wss = [q.new_workspace(L, B, k) for B in Bs]
    outs = [torch.empty(B, d, device="cuda") for B in Bs]
    ref = []
    for i, B in enumerate(Bs):
        ref.append(q.moe_layer_decode(L, xs[i, :B], k, wss[i])[2].clone())
        again = q.moe_layer_decode(L, xs[i, :B], k, wss[i])[2]
        assert torch.equal(ref[-1], again)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i, B in enumerate(Bs):
            q.moe_layer_decode(L, xs[i, :B], k, wss[i], y=outs[i])
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for i in range(len(Bs)):
            assert torch.equal(outs[i], ref[i]), (rep, i)
        q.moe_layer_decode(L, xs[0, :4], k, wss[0])
        torch.cuda.synchronize()
    for w in wss:
        assert q.workspace_error(w) == 0


def test_batch_matches_single_tokens(q):
    """A token's output in a batch agrees with the same token alone (the
    single-token VALU path) within the bar: the two paths share no kernel."""
    d, E, k, B = 2048, 256, 8, 6
    L, _ = _layer(q, 21, E, d)
    say("batch vs single")
    x = synth.activations(torch, "cuda", 12, B, d)
    wsb = q.new_workspace(L, B, k)
    ib, wb, yb = q.moe_layer_decode(L, x, k, wsb)
    ws1 = q.new_workspace(L, 1, k)
    for b in range(B):
        i1, w1, y1 = q.moe_layer_decode(L, x[b:b + 1].contiguous(), k, ws1)
        torch.cuda.synchronize()
        assert torch.equal(i1[0], ib[b])
        assert rel_l2(yb[b].cpu().numpy(), y1[0].cpu().numpy()) <= REL_L2_TOL
