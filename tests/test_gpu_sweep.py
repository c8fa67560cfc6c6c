"""Seeded random sweep of layer shapes through the C ABI, against the oracle.

Each case draws a batch size, top-k, expert count, hidden size, expert width
and options (skew bias, residual, fused or two-call) from a fixed generator,
so the list is the same on every run.  Hidden sizes in (1792, 2048] with
F = 512 take the tuned kernels (VALU for one token, MFMA for 2..16 tokens);
the others take the generic kernels.  Per case: routing and up to three
tokens' outputs against the oracle (the oracle quantizes only the experts
those tokens select, to stay within seconds), the fused and two-call forms
bit-identical, and a repeated call bit-identical."""

import numpy as np
import pytest

from oracle import moe
import synth

from _parity import REL_L2_TOL, ExpertCache, check_routing, logit_tol, oracle_layer_check

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _cases(n=32, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        tuned = i % 3 != 2
        B = int(rng.choice([1, 1, 2, 3, 4, 5, 7, 8, 11, 16]))
        k = int(rng.integers(1, 9))
        E = max(k, int(rng.choice([9, 33, 64, 100, 256, 300, 512, 777, 1024])))
        if tuned:
            d, F = int(rng.choice([1796, 1800, 1920, 2000, 2044, 2048])), 512
        else:
            d, F = int(rng.choice([256, 764, 1024, 1500])), int(rng.choice([128, 256, 300, 512]))
        out.append(dict(i=i, B=B, k=k, E=E, d=d, F=F, skew=bool(rng.random() < 0.5),
                        res=bool(rng.random() < 0.5), fused=bool(rng.random() < 0.5)))
    return out


CASES = _cases()


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


@pytest.mark.parametrize("c", CASES, ids=lambda c: "B%d-k%d-E%d-d%d-F%d" % (c["B"], c["k"], c["E"],
                                                                            c["d"], c["F"]))
def test_sweep_case(q, c):
    say(c)
    seed = 1000 + c["i"]
    B, k, E, d, F = c["B"], c["k"], c["E"], c["d"], c["F"]
    bias = synth.zipf_bias(seed, E) if c["skew"] else None
    L = q.synthetic.build_layer(torch, seed=seed, layer_id=0, E=E, d=d, F=F, bias=bias)
    x = synth.activations(torch, "cuda", seed, B, d)
    res = synth.activations(torch, "cuda", seed + 1, B, d) if c["res"] else None
    ws = q.new_workspace(L, B, k)
    if c["fused"]:
        idx, wts, y = q.moe_layer_decode(L, x, k, ws, residual=res)
    else:
        idx, wts = q.moe_route_topk(L.Wr, x, k, bias=L.bias, ws=ws)
        y = q.moe_expert_decode(L, x, idx, wts, ws, residual=res)
    idx, wts, y = idx.clone(), wts.clone(), y.clone()
    torch.cuda.synchronize()
    assert q.workspace_error(ws) == 0

    # the other form, and a repeat of the same form: identical bits
    if c["fused"]:
        i2, w2 = q.moe_route_topk(L.Wr, x, k, bias=L.bias, ws=ws)
        y2 = q.moe_expert_decode(L, x, i2, w2, ws, residual=res)
        i3, w3, y3 = q.moe_layer_decode(L, x, k, ws, residual=res)
    else:
        i2, w2, y2 = q.moe_layer_decode(L, x, k, ws, residual=res)
        i3, w3 = q.moe_route_topk(L.Wr, x, k, bias=L.bias, ws=ws)
        y3 = q.moe_expert_decode(L, x, i3, w3, ws, residual=res)
    torch.cuda.synchronize()
    for a, b in ((idx, i2), (wts, w2), (y, y2), (idx, i3), (wts, w3), (y, y3)):
        assert torch.equal(a, b)

    # routing of every token, outputs of up to three against the oracle
    xs = x.cpu().numpy()
    Wr = L.Wr.cpu().numpy()
    bnp = None if bias is None else np.asarray(bias, dtype=np.float64)
    logits = moe.router_logits(Wr, xs.astype(np.float64), bnp)
    amb = check_routing(idx.cpu().numpy(), wts.cpu().numpy(), logits, k, logit_tol(Wr, xs, bnp))
    assert amb == 0
    sel = sorted(set([0, B // 2, B - 1]))
    cache = ExpertCache(torch, "cuda", seed, 0, d, F)
    err, amb = oracle_layer_check(xs[sel], Wr, bnp, cache, k, idx.cpu().numpy()[sel],
                                  wts.cpu().numpy()[sel], y.cpu().numpy()[sel],
                                  residual=None if res is None else res.cpu().numpy()[sel])
    say("max rel-L2 %.3g over tokens %s, tie-ambiguous %d" % (err, sel, amb))
    assert amb == 0 and err <= REL_L2_TOL
