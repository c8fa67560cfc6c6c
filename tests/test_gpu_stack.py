"""GPU parity of layer stacks and of host-mapped experts.

Stack (per layer t = x + D x, then x' = t + MoE(t)): every layer of the GPU
chain of C-ABI calls is checked against the oracle with teacher forcing --
the oracle takes the GPU's input to that layer (its f32 values), so the
rounding of earlier layers does not compound into the comparison:

* the dense step: t_gpu against x_in + D x_in, relative L2 <= 2e-3;
* routing of the MoE layer on t_gpu: indices exactly the oracle's (up to
  the f32 near-tie bound of the parity helpers, and the seeded cases hold
  no such tie), weights within 1e-5;
* the layer output: x'_gpu against t_gpu + MoE(t_gpu), relative L2 <= 2e-3.

The free-running oracle chain (its own input at every layer) is reported
beside it for small stacks, for information only.

Host-mapped experts (pinned host memory read zero-copy over PCIe) run
through the same kernels, so a host-mapped layer must give the same bits as
the identical layer in HBM, and a stack mixing HBM and host-mapped layers
(the host-mapped workload's composition x' = x + MoE(x), no dense step) is
checked like the dense stack.
"""

import numpy as np
import pytest

from oracle import hfq4, moe
import synth

from _parity import REL_L2_TOL, ExpertCache, check_routing, logit_tol, rel_l2

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module")
def q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_moe_decode_amd as q
    q.lib.hfq4_debug_set_arch(b"")
    return q


def _oracle_layer(seed, l, E, d, F, dense, bias=None):
    """Oracle view of stack layer l: quantized by the oracle from the same
    seeded f32 draws (drawn on the device that drew the GPU stack's
    weights, then copied to the host)."""
    Wr = synth.router_f32(torch, "cuda", seed, l, E, d).cpu().numpy()
    D = (hfq4.quantize_rows(synth.dense_f32(torch, "cuda", seed, l, d).cpu().numpy())
         if dense else None)
    return dict(Wr=Wr, bias=bias, dense=D, experts=ExpertCache(torch, "cuda", seed, l, d, F))


def _run_captured(st, x_rows):
    x = torch.from_numpy(np.ascontiguousarray(x_rows, dtype=np.float32)).cuda()
    cap = []
    out = st.step(x, capture=cap)
    torch.cuda.synchronize()
    cap = [tuple(c.cpu().numpy() for c in entry) for entry in cap]
    return out, cap


def _teacher_forced(seed, x_rows, cap, layers, E, d, F, k, dense, bias=None):
    """Check the listed layers of a captured GPU run, each against the
    oracle fed that layer's GPU input.  Returns the worst rel-L2 seen."""
    worst = 0.0
    for l in layers:
        L = _oracle_layer(seed, l, E, d, F, dense, bias)
        x_in = (x_rows if l == 0 else cap[l - 1][1]).astype(np.float64)
        t_gpu, out_gpu, idx_gpu, wts_gpu = cap[l]
        if dense:
            t_ref = x_in + hfq4.matvec(L["dense"], d, d, x_in)
            for b in range(x_in.shape[0]):
                e = rel_l2(t_gpu[b], t_ref[b])
                assert e <= REL_L2_TOL, "layer %d token %d: dense step rel-L2 %.3g" % (l, b, e)
                worst = max(worst, e)
        t = t_gpu.astype(np.float64)
        logits = moe.router_logits(L["Wr"], t, bias)
        amb = check_routing(idx_gpu, wts_gpu, logits, k, logit_tol(L["Wr"], t, bias))
        assert amb == 0, "layer %d: %d tie-ambiguous tokens" % (l, amb)
        _, _, y, _ = moe.moe_layer(t, L["Wr"], L["experts"], k, bias, idx=idx_gpu)
        for b in range(t.shape[0]):
            e = rel_l2(out_gpu[b], t[b] + y[b])
            assert e <= REL_L2_TOL, "layer %d token %d: output rel-L2 %.3g" % (l, b, e)
            worst = max(worst, e)
    return worst


def _free_running(seed, x_rows, cap, n, E, d, F, k, dense, bias=None):
    """End-to-end rel-L2 of the GPU chain against the oracle's own chain
    (information only: near-ties may legitimately part the chains)."""
    errs = []
    for b in range(x_rows.shape[0]):
        layers = [_oracle_layer(seed, l, E, d, F, dense, bias) for l in range(n)]
        ref = moe.stack_step(x_rows[b], layers, k)
        errs.append(rel_l2(cap[-1][1][b], ref))
    return max(errs)


@pytest.mark.parametrize("n,E,d,F,k,B", [(4, 16, 512, 256, 4, 2), (3, 32, 2048, 512, 8, 1),
                                         (3, 24, 1000, 200, 3, 3), (5, 64, 2048, 512, 8, 4)])
def test_small_stack_teacher_forced(q, n, E, d, F, k, B):
    from quantized_moe_decode_amd.stack import build_stack
    say("stack", n, E, d, F, k, B)
    seed = 11
    st = build_stack(torch, seed, n, E, d, F, k, B, dense=True)
    x = synth.activations(torch, "cuda", seed, B, d).cpu().numpy()
    _, cap = _run_captured(st, x)
    worst = _teacher_forced(seed, x, cap, range(n), E, d, F, k, True)
    say("worst layer rel-L2 %.3g; free-running chain end-to-end %.3g"
        % (worst, _free_running(seed, x, cap, n, E, d, F, k, True)))


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


C4_SEED, C4_LAYERS = 3, 40


@pytest.fixture(scope="module")
def c4_run(q):
    """The 40-layer stack at its real shape (d=2048, F=512, E=256, k=8, a
    dense 2048 x 2048 per layer) in the launch configuration the benchmark
    times, run once with every layer captured."""
    from quantized_moe_decode_amd.stack import build_stack
    say("building the 40-layer stack")
    st = build_stack(torch, C4_SEED, C4_LAYERS, 256, 2048, 512, 8, 1, dense=True)
    x = synth.activations(torch, "cuda", C4_SEED, 1, 2048).cpu().numpy()
    out, cap = _run_captured(st, x)
    again = st.step(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    assert torch.equal(out, again)
    yield x, cap
    del st
    torch.cuda.empty_cache()


@pytest.mark.parametrize("l0", [0, 10, 20, 30])
def test_c4_stack_every_layer(q, c4_run, l0):
    """Every one of the 40 layers (ten per case) against the oracle with
    teacher forcing: dense step, routing and layer output."""
    x, cap = c4_run
    say("c4 stack layers %d..%d" % (l0, l0 + 9))
    worst = _teacher_forced(C4_SEED, x, cap, range(l0, l0 + 10), 256, 2048, 512, 8, True)
    say("worst rel-L2 %.3g" % worst)


@pytest.mark.parametrize("B", [1, 2])
def test_c5_mixed_stack_teacher_forced(q, B):
    """The host-mapped workload's composition at its layer shape (E=512,
    d=2048, F=512, k=8, x' = x + MoE(x), no dense step): layers 0-1 in HBM,
    2-3 in pinned host memory, every layer against the oracle with teacher
    forcing, and the host-mapped layers bitwise equal to an all-HBM copy of
    the same stack."""
    from quantized_moe_decode_amd.stack import build_stack
    seed, n, E, d, F, k = 17, 4, 512, 2048, 512, 8
    say("c5 mixed stack, host-mapped from layer 2, B=%d" % B)
    st = build_stack(torch, seed, n, E, d, F, k, B, dense=False, host_from=2)
    assert st.layers[3].c.flags == q.HFQ4_LAYER_HOST_MAPPED and st.layers[1].c.flags == 0
    x = synth.activations(torch, "cuda", seed, B, d).cpu().numpy()
    out, cap = _run_captured(st, x)
    worst = _teacher_forced(seed, x, cap, range(n), E, d, F, k, False)
    say("worst rel-L2 %.3g" % worst)
    del st
    hbm = build_stack(torch, seed, n, E, d, F, k, B, dense=False)
    out2, cap2 = _run_captured(hbm, x)
    for a, b in zip(cap, cap2):
        for u, v in zip(a, b):
            assert np.array_equal(u, v)
    del hbm
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B", [1, 4, 16])
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
    assert check_routing(idx, wts, logits, k, logit_tol(Wr, xs)) == 0
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
