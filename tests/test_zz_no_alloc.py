"""The allocation-free layer entry point (moe_layer_decode_noalloc) against
moe_layer_decode with a caller workspace: the same kernels on the same
inputs, so idx, wts and y must be identical bit for bit.  Two calls in a
row on the library's shared scratch, the second on a smaller input (fewer
tokens, fewer experts, another kernel family), then the first shape again;
one token's output also against the oracle.  Everything goes through the
C ABI."""

import numpy as np
import pytest

import synth

from _parity import REL_L2_TOL, ExpertCache, oracle_layer_check

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


def _pair(q, L, x, k, res):
    """(noalloc outputs, workspace outputs) for one call shape."""
    B, d = x.shape
    outs = []
    for noalloc in (True, False):
        idx = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
        wts = torch.full((B, k), float("nan"), dtype=torch.float32, device="cuda")
        y = torch.full((B, d), float("nan"), dtype=torch.float32, device="cuda")
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        if noalloc:
            q.moe_layer_decode_noalloc(L, x, k, idx, wts, y, residual=res, err=err)
        else:
            ws = q.new_workspace(L, B, k)
            q.moe_layer_decode(L, x, k, ws, residual=res, y=y, idx=idx, wts=wts)
        torch.cuda.synchronize()
        if noalloc:
            assert int(err.item()) == 0
        else:
            assert q.workspace_error(ws) == 0
        outs.append((idx, wts, y))
    return outs


def test_noalloc_matches_workspace_entry_point(q):
    big = q.synthetic.build_layer(torch, seed=41, layer_id=0, E=512, d=2048, F=512,
                                  bias=synth.zipf_bias(4, 512))
    small = q.synthetic.build_layer(torch, seed=42, layer_id=0, E=256, d=2048, F=512)
    tiny, Lh = q.synthetic.tiny_layer(torch, 0)
    cases = [("E=512 skewed, 16 tokens (matrix-core kernels)", big, 16, 8),
             ("E=256, 1 token (one-token kernels), smaller", small, 1, 8),
             ("tiny layer, 1 token (generic kernels), smaller again", tiny, 1, 2),
             ("E=512 skewed, 16 tokens again", big, 16, 8)]
    for i, (name, L, B, k) in enumerate(cases):
        say("noalloc call %d: %s" % (i, name))
        x = synth.activations(torch, "cuda", 50 + i, B, L.d)
        res = synth.activations(torch, "cuda", 60 + i, B, L.d)
        (i1, w1, y1), (i2, w2, y2) = _pair(q, L, x, k, res)
        assert torch.equal(i1, i2) and torch.equal(w1, w2) and torch.equal(y1, y2), name
        assert torch.isfinite(y1).all()
        if i == 1:   # one token against the oracle too
            cache = ExpertCache(torch, "cuda", 42, 0, 2048, 512)
            err, amb = oracle_layer_check(x.cpu().numpy(), L.Wr.cpu().numpy(), None, cache, k,
                                          i1.cpu().numpy(), w1.cpu().numpy(), y1.cpu().numpy(),
                                          residual=res.cpu().numpy())
            assert amb == 0 and err <= REL_L2_TOL, (amb, err)


def test_noalloc_host_mapped_one_token(q):
    """A host-mapped one-token layer stages its selected down matrices in
    the scratch (the largest use of it): same bits as the workspace call."""
    Lh = q.synthetic.build_layer(torch, seed=43, layer_id=0, E=64, d=2048, F=512,
                                 host_mapped=True)
    x = synth.activations(torch, "cuda", 70, 1, 2048)
    (i1, w1, y1), (i2, w2, y2) = _pair(q, Lh, x, 8, None)
    assert torch.equal(i1, i2) and torch.equal(w1, w2) and torch.equal(y1, y2)


def test_noalloc_reports_device_errors(q):
    """A NaN activation makes every logit NaN: the sticky non-finite bit
    reaches the caller's error word."""
    L = q.synthetic.build_layer(torch, seed=44, layer_id=0, E=32, d=2048, F=512)
    x = torch.full((1, 2048), float("nan"), device="cuda")
    idx = torch.empty((1, 8), dtype=torch.int32, device="cuda")
    wts = torch.empty((1, 8), dtype=torch.float32, device="cuda")
    y = torch.empty((1, 2048), dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    q.moe_layer_decode_noalloc(L, x, 8, idx, wts, y, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & q.HFQ4_DEV_ERR_NONFINITE
    assert bool(((idx >= 0) & (idx < 32)).all())
