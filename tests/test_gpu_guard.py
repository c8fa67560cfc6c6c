"""Canary guard bands around every output buffer of every entry point.

Each output (y, idx, wts, logits, packed bytes) and each workspace sits in
the middle of a larger allocation whose head and tail hold a canary
pattern; after the calls the bands must be intact (a padding-write check:
no kernel writes outside the buffers it was given), and the outputs
themselves must be fully written (no canary left inside, results finite and
matching the oracle elsewhere in the suite).  The shapes take every kernel
family: the tuned one-token and batched kernels, the generic kernels, the
dense GEMV and the packer, with sizes that end in ragged tails.
"""

import numpy as np
import pytest

from oracle import hfq4
import synth

from _parity import CANARY_WORD, REL_L2_TOL, Guarded, rel_l2

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


def _no_canary(t):
    raw = t.contiguous().view(torch.int32).cpu().numpy()
    assert not np.any(raw == CANARY_WORD), "output left unwritten"


@pytest.mark.parametrize("rows,K", [(1, 256), (37, 300), (4096, 2048), (513, 128)])
def test_pack_guard(q, rows, K):
    say("pack guard", rows, K)
    w = synth.activations(torch, "cuda", rows, rows, K, std=0.02)
    g = Guarded(torch, q.hfq4_packed_bytes(rows, K), torch.uint8, guard=256)
    q.hfq4_pack(w, out=g.t)
    torch.cuda.synchronize()
    g.check()
    assert np.array_equal(g.t.cpu().numpy(), hfq4.quantize_rows(w.cpu().numpy()))


@pytest.mark.parametrize("rows,K,batch", [(2048, 2048, 1), (2051, 2048, 1), (129, 1000, 16),
                                          (7, 128, 3), (40000, 2048, 1)])
def test_gemv_guard(q, rows, K, batch):
    say("gemv guard", rows, K, batch)
    w = synth.activations(torch, "cuda", 3, rows, K, std=0.02)
    W = q.hfq4_pack(w)
    x = synth.activations(torch, "cuda", 4, batch, K)
    gy = Guarded(torch, (batch, rows), torch.float32)
    q.hfq4_gemv(W, rows, K, x, y=gy.t)
    torch.cuda.synchronize()
    gy.check()
    _no_canary(gy.t)
    sample = np.unique(np.r_[0, rows - 1, np.arange(0, rows, max(1, rows // 64))])
    ref = hfq4.matvec(hfq4.quantize_rows(w[sample].cpu().numpy()), len(sample), K,
                      x.cpu().numpy().astype(np.float64))
    for b in range(batch):
        assert rel_l2(gy.t[b].cpu().numpy()[sample], ref[b]) <= REL_L2_TOL


# (E, d, F, k, B): tuned one-token, tuned batched, generic shapes
LAYERS = [(256, 2048, 512, 8, 1), (512, 2048, 512, 8, 16), (64, 2000, 512, 6, 3),
          (33, 764, 300, 5, 1), (16, 256, 128, 2, 4)]


@pytest.mark.parametrize("E,d,F,k,B", LAYERS)
@pytest.mark.parametrize("fused", [True, False])
def test_layer_guard(q, E, d, F, k, B, fused):
    say("layer guard", E, d, F, k, B, "fused" if fused else "two-call")
    L = q.synthetic.build_layer(torch, seed=E + d, layer_id=0, E=E, d=d, F=F,
                                bias=synth.zipf_bias(2, E) if B > 1 else None)
    x = synth.activations(torch, "cuda", 8, B, d)
    gws = Guarded(torch, q.moe_workspace_bytes(L, B, k), torch.uint8, guard=256, zero=True)
    gy = Guarded(torch, (B, d), torch.float32)
    gi = Guarded(torch, (B, k), torch.int32)
    gw = Guarded(torch, (B, k), torch.float32)
    gl = Guarded(torch, (B, E), torch.float32)
    gr = None
    for rep in range(2):     # the second call reuses the (no longer fresh) workspace
        if fused:
            q.moe_layer_decode(L, x, k, gws.t, y=gy.t, idx=gi.t, wts=gw.t)
        else:
            rws = Guarded(torch, q.moe_route_workspace_bytes(E, B), torch.uint8, guard=256,
                          zero=True)
            q.moe_route_topk(L.Wr, x, k, bias=L.bias, ws=rws.t, idx=gi.t, wts=gw.t,
                             logits=gl.t)
            q.moe_expert_decode(L, x, gi.t, gw.t, gws.t, y=gy.t)
            gr = rws
        torch.cuda.synchronize()
        assert q.workspace_error(gws.t) == 0
        for g in (gws, gy, gi, gw) + ((gl, gr) if not fused else ()):
            g.check()
        for t in (gy.t, gi.t, gw.t) + ((gl.t,) if not fused else ()):
            _no_canary(t)
        assert torch.isfinite(gy.t).all()
        assert bool(((gi.t >= 0) & (gi.t < E)).all())
