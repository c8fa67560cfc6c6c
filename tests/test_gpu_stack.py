"""GPU parity of layer stacks and of host-mapped experts.

Stack (per layer t = x + D x, then x' = t + MoE(t)): the GPU chain of C-ABI
calls is compared layer by layer with the oracle's own chain, started from
the same synthetic token (the oracle never sees a GPU value).  Routing must
be identical at every layer and every layer output within the per-token
relative-L2 bar.  Only where the oracle's k-th/(k+1)-th logit gap is within
1e-3 (relative) may the GPU pick the other expert of that pair -- its
choice must then be a valid top-k -- and that token's comparison ends
there, since the two chains legitimately part.

Host-mapped experts (pinned host memory read zero-copy over PCIe) run
through the same kernels, so a host-mapped layer must give the same bits as
the identical layer in HBM.
"""

import numpy as np
import pytest

from oracle import hfq4, moe
import synth

from _parity import REL_L2_TOL, ExpertCache, check_routing, rel_l2, routing_valid

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

GAP_MIN = 1e-3   # smallest oracle logit gap at the top-k boundary the chain check accepts


def say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module")
def q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_moe_decode_amd as q
    q.lib.hfq4_debug_set_arch(b"")
    return q


def _oracle_layers(seed, n, E, d, F, dense, bias=None):
    """Oracle view of the synthetic stack: quantized by the oracle from the
    same seeded f32 draws (drawn on the device that drew the GPU stack's
    weights, then copied to the host)."""
    for l in range(n):
        Wr = synth.router_f32(torch, "cuda", seed, l, E, d).cpu().numpy()
        D = (hfq4.quantize_rows(synth.dense_f32(torch, "cuda", seed, l, d).cpu().numpy())
             if dense else None)
        yield dict(Wr=Wr, bias=bias, dense=D, experts=ExpertCache(torch, "cuda", seed, l, d, F))


def _boundary_gap(logits, k):
    s = np.sort(np.asarray(logits, dtype=np.float64))[::-1]
    return float(s[k - 1] - s[k]) if len(s) > k else np.inf


def _chain_check(q, st, seed, x_rows, E, d, F, k, dense, n_check, bias=None):
    """Run the GPU stack once (eager, capturing every layer) and compare the
    first n_check layers with the oracle chain, token by token."""
    x = torch.from_numpy(np.ascontiguousarray(x_rows, dtype=np.float32)).cuda()
    cap = []
    out = st.step(x, capture=cap)
    torch.cuda.synchronize()
    worst = 0.0
    compared = 0
    for b in range(x_rows.shape[0]):
        tr = []
        moe.stack_step(x_rows[b], _oracle_layers(seed, n_check, E, d, F, dense, bias), k, trace=tr)
        for l, (x_ref, idx_ref, wts_ref, logits) in enumerate(tr):
            y_gpu, idx_gpu, wts_gpu = (c[b].cpu().numpy() for c in cap[l])
            ref = [int(e) for e in idx_ref]
            got = idx_gpu.tolist()
            if got != ref:
                # the two chains' inputs differ by rounding, so experts whose
                # logits are this close may swap; the GPU's choice must still
                # be a valid top-k of the oracle's logits
                assert routing_valid(got, logits, k, rel=GAP_MIN), \
                    (b, l, _boundary_gap(logits, k), got, ref)
                if set(got) != set(ref):
                    say("token %d: near-tie at layer %d (gap %.3g), chain compared up to it"
                        % (b, l, _boundary_gap(logits, k)))
                    break
                say("token %d layer %d: near-equal experts in swapped order" % (b, l))
            # the layer input already differs by the previous layers' rounding,
            # so the weights are held to the output's relative bar
            w_ref = np.array([wts_ref[ref.index(e)] for e in got])
            assert rel_l2(wts_gpu, w_ref) <= REL_L2_TOL, (b, l, wts_gpu, w_ref)
            err = rel_l2(y_gpu, x_ref)
            worst = max(worst, err)
            assert err <= REL_L2_TOL, "token %d layer %d: rel-L2 %.3g" % (b, l, err)
            compared += 1
    # near-ties are rare: most token-layers must have been compared
    assert compared * 2 >= n_check * x_rows.shape[0], compared
    return out, cap, worst


@pytest.mark.parametrize("n,E,d,F,k,B", [(4, 16, 512, 256, 4, 2), (3, 32, 2048, 512, 8, 1),
                                         (3, 24, 1000, 200, 3, 3)])
def test_small_stack_vs_oracle_chain(q, n, E, d, F, k, B):
    from quantized_moe_decode_amd.stack import build_stack
    say("stack", n, E, d, F, k, B)
    seed = 11
    st = build_stack(torch, seed, n, E, d, F, k, B, dense=True)
    x = synth.activations(torch, "cuda", seed, B, d).cpu().numpy()
    _, _, worst = _chain_check(q, st, seed, x, E, d, F, k, True, n)
    say("worst layer rel-L2 %.3g" % worst)


def test_stack_graph_equals_eager(q):
    from quantized_moe_decode_amd.stack import build_stack
    say("stack graph vs eager")
    st = build_stack(torch, 5, 3, 16, 512, 256, 4, 2, dense=True)
    pool = synth.activations(torch, "cuda", 5, 4, 512).view(2, 2, 512)
    outs = torch.empty(2, 2, 512, device="cuda")
    g = torch.cuda.CUDAGraph()
    st.step(pool[0])                       # warm-up outside capture
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(2):
            outs[i].copy_(st.step(pool[i]))
    ref = [st.step(pool[i]).clone() for i in range(2)]
    for rep in range(3):
        outs.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(outs[i], ref[i]), (rep, i)
        st.step(pool[1])                   # eager work between replays
        torch.cuda.synchronize()


def test_c4_stack_full_size(q):
    """The 40-layer stack at its real shape (d=2048, F=512, E=256, k=8, a
    dense 2048 x 2048 per layer) in the launch configuration the benchmark
    times: the first two layers against the oracle chain, the full 40-layer
    output finite and equal to a second run."""
    from quantized_moe_decode_amd.stack import build_stack
    say("c4 stack 40 layers")
    seed = 3
    st = build_stack(torch, seed, 40, 256, 2048, 512, 8, 1, dense=True)
    x = synth.activations(torch, "cuda", seed, 1, 2048).cpu().numpy()
    out, cap, worst = _chain_check(q, st, seed, x, 256, 2048, 512, 8, True, 2)
    say("first layers worst rel-L2 %.3g" % worst)
    first = out.clone()
    again = st.step(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    assert torch.isfinite(first).all()
    assert torch.equal(first, again)
    del st
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B", [1, 4])
def test_host_mapped_layer_bitwise(q, B):
    """c5 layer shape (E=512, d=2048, F=512, k=8): host-mapped == HBM bits,
    and the host-mapped layer against the oracle."""
    from quantized_moe_decode_amd.synthetic import build_layer
    say("host-mapped layer B=%d" % B)
    seed, lid, E, d, F, k = 9, 30, 512, 2048, 512, 8
    hbm = build_layer(torch, seed, lid, E, d, F)
    host = build_layer(torch, seed, lid, E, d, F, host_mapped=True)
    assert not host.gate.is_cuda and host.gate.is_pinned()
    x = synth.activations(torch, "cuda", seed + B, B, d)
    res = []
    for L in (hbm, host):
        ws = q.new_workspace(L, B, k)
        res.append(q.moe_layer_decode(L, x, k, ws, residual=x))
        torch.cuda.synchronize()
        assert q.workspace_error(ws) == 0
    for a, b in zip(res[0], res[1]):
        assert torch.equal(a, b)
    idx, wts, y = (t.cpu().numpy() for t in res[1])
    xs = x.cpu().numpy().astype(np.float64)
    Wr = synth.router_f32(torch, "cuda", seed, lid, E, d).cpu().numpy()
    logits = moe.router_logits(Wr, xs)
    check_routing(idx, wts, logits, k)
    cache = ExpertCache(torch, "cuda", seed, lid, d, F)
    _, _, y_ref, _ = moe.moe_layer(xs, Wr, cache, k, idx=idx)
    for b in range(B):
        assert rel_l2(y[b], y_ref[b] + xs[b]) <= REL_L2_TOL


def test_host_mapped_gemv_bitwise(q):
    say("host-mapped gemv")
    rows, K = 3000, 2048
    w = torch.cat([synth.dense_f32(torch, "cuda", 1, i, K, std=0.02)
                   for i in range(2)])[:rows].contiguous()
    packed = q.hfq4_pack(w)
    hostp = torch.empty(packed.numel(), dtype=torch.uint8, pin_memory=True)
    hostp.copy_(packed)
    x = synth.activations(torch, "cuda", 4, 2, K)
    a = q.hfq4_gemv(packed, rows, K, x)
    b = q.hfq4_gemv(hostp, rows, K, x)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    ref = np.stack([hfq4.matvec(hfq4.quantize_rows(w.cpu().numpy()), rows, K,
                                x[i].cpu().numpy().astype(np.float64)) for i in range(2)])
    for i in range(2):
        assert rel_l2(b[i].cpu().numpy(), ref[i]) <= REL_L2_TOL
