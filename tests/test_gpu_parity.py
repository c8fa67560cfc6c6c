"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: HFQ4 bytes and routing indices bit-exact (ties inside the stated
tolerance may come in either order, and the alternative must be a valid
top-k); routing weights within 1e-5; layer output relative L2 <= 2e-3 per
token.  Inputs are seeded and synthetic (synth)."""

import numpy as np
import pytest

from oracle import hfq4, moe
import synth

from _parity import (REL_L2_TOL, ExpertCache, Guarded, check_logits, check_routing, logit_tol,
                     oracle_layer_check, rel_l2)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(scope="module")
def q():
    _need_gpu()
    import quantized_moe_decode_amd as q
    q.lib.hfq4_debug_set_arch(b"")
    return q


def say(*a):
    print("[case]", *a, flush=True)


# ------------------------------------------------------------------ pack

@pytest.mark.parametrize("rows,K,std,off", [(1, 256, 0.02, 0.0), (7, 128, 1.0, 0.5),
                                            (33, 300, 0.02, 0.0), (64, 2048, 0.02, 0.0),
                                            (5, 2050, 3.0, -1.0), (512, 2048, 0.02, 0.0),
                                            (2048, 512, 0.02, 0.0), (3, 5000, 1e-3, 0.0)])
def test_pack_bit_exact(q, rows, K, std, off):
    say("hfq4_pack", rows, K)
    rng = np.random.default_rng(rows * 7919 + K)
    W = (rng.standard_normal((rows, K)) * std + off).astype(np.float32)
    W[0, : min(K, 4)] = [0.0, 15.0, 2.5, 3.5][: min(K, 4)] if std == 1.0 else W[0, : min(K, 4)]
    got = q.hfq4_pack(torch.from_numpy(W).cuda()).cpu().numpy()
    ref = hfq4.quantize_rows(W)
    assert got.shape == ref.shape
    assert np.array_equal(got, ref), "first mismatch at byte %d" % int(np.argmax(got != ref))


def test_pack_golden_and_constant_blocks(q):
    say("hfq4_pack golden")
    i = np.arange(256)
    W = np.stack([(i % 16).astype(np.float32), np.full(256, 0.75, np.float32),
                  (np.float32(-0.25) + ((7 * i) % 16).astype(np.float32) / np.float32(64))])
    got = q.hfq4_pack(torch.from_numpy(W).cuda()).cpu().numpy().tobytes()
    assert got[:8] == bytes.fromhex("0000803f00000000")
    assert got[8:136] == bytes.fromhex("1032547698badcfe") * 16
    assert got[136:144] == bytes.fromhex("000000000000403f")
    assert got[272:280] == bytes.fromhex("0000803c000080be")
    assert got[280:408] == bytes.fromhex("705e3c1af8d6b492") * 16


def test_pack_signed_zero_minimum(q):
    # golden blocks F and G: the minimum is a zero stored as -0.0 (F: mixed
    # with +0.0); the zero field holds +0.0, so both pack to block A's bytes
    say("hfq4_pack signed zeros")
    i = np.arange(256)
    rows = []
    for neg in (i % 32 == 0, i % 16 == 0):
        w = (i % 16).astype(np.float32)
        w[neg] = np.float32(-0.0)
        rows.append(w)
    W = np.stack(rows + [rows[0][::-1].copy()])
    got = q.hfq4_pack(torch.from_numpy(W).cuda()).cpu().numpy()
    assert np.array_equal(got, hfq4.quantize_rows(W))
    blkA = bytes.fromhex("0000803f00000000") + bytes.fromhex("1032547698badcfe") * 16
    assert got[:136].tobytes() == blkA and got[136:272].tobytes() == blkA
    assert got[272:280].tobytes() == bytes.fromhex("0000803f00000000")


def test_pack_rejects_nonfinite(q):
    say("hfq4_pack nonfinite")
    W = np.zeros((3, 512), np.float32)
    W[1, 300] = np.inf
    W[2, 5] = np.nan
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = q.hfq4_pack(torch.from_numpy(W).cuda(), bad=bad).cpu().numpy().reshape(3, 2, 136)
    assert int(bad.item()) == 2
    assert np.all(out[1, 1] == 0) and np.all(out[2, 0] == 0)
    with pytest.raises(q.Hfq4Error):
        q.hfq4_pack(torch.from_numpy(W).cuda())


# ------------------------------------------------------------------ gemv

@pytest.mark.parametrize("rows,K,batch,resid", [(1, 256, 1, False), (7, 128, 1, True),
                                                (64, 2048, 1, False), (2051, 2048, 1, True),
                                                (300, 300, 4, False), (129, 1000, 16, True),
                                                (40, 4096, 2, False), (17, 16384, 2, True),
                                                (2048, 512, 16, False), (33, 1001, 3, True),
                                                (5, 257, 1, False), (96, 2046, 1, True)])
def test_gemv(q, rows, K, batch, resid):
    say("hfq4_gemv", rows, K, batch, resid)
    rng = np.random.default_rng(rows + 31 * K + batch)
    W = (rng.standard_normal((rows, K)) * 0.02).astype(np.float32)
    P = hfq4.quantize_rows(W)
    x = rng.standard_normal((batch, K)).astype(np.float32)
    r = rng.standard_normal((batch, rows)).astype(np.float32) if resid else None
    Wd = torch.from_numpy(P).cuda()
    # rows of x padded to a multiple of 4 floats (the ABI's ldx rule)
    ldx = (K + 3) // 4 * 4
    xp = np.full((batch, ldx), 7.0, dtype=np.float32)
    xp[:, :K] = x
    xd = torch.from_numpy(xp).cuda()[:, :K]
    y = q.hfq4_gemv(Wd, rows, K, xd,
                    residual=None if r is None else torch.from_numpy(r).cuda()).cpu().numpy()
    ref = hfq4.matvec(P, rows, K, x)
    if r is not None:
        ref = ref + r
    for b in range(batch):
        assert rel_l2(y[b], ref[b]) <= REL_L2_TOL, (b, rel_l2(y[b], ref[b]))
    # run-to-run bitwise determinism
    y2 = q.hfq4_gemv(Wd, rows, K, xd,
                     residual=None if r is None else torch.from_numpy(r).cuda()).cpu().numpy()
    assert np.array_equal(y, y2)


def test_gemv_long_matrix(q):
    """A matrix past the long-GEMV switch (>= 512 MiB of weights: four row
    loads per wave and group, every wave looping over row groups), with a
    residual and two tokens; 96 sampled rows against the oracle, the first
    and last rows among them.  The rows repeat a 4096-row packed block, so
    the oracle needs only that block."""
    say("hfq4_gemv long matrix")
    K, batch, base = 2048, 2, 4096
    rows = 560_000
    rng = np.random.default_rng(11)
    Wb = (rng.standard_normal((base, K)) * 0.02).astype(np.float32)
    Pb = hfq4.quantize_rows(Wb)
    Wd = torch.from_numpy(Pb.reshape(base, -1)).cuda().repeat((rows + base - 1) // base, 1)
    Wd = Wd[:rows].contiguous()
    assert Wd.numel() * 1 >= (1 << 29)
    x = rng.standard_normal((batch, K)).astype(np.float32)
    r = rng.standard_normal((batch, rows)).astype(np.float32)
    y = q.hfq4_gemv(Wd.view(-1), rows, K, torch.from_numpy(x).cuda(),
                    residual=torch.from_numpy(r).cuda()).cpu().numpy()
    sample = np.unique(np.concatenate([[0, 1, rows - 2, rows - 1],
                                       rng.integers(0, rows, size=92)]))
    ref_base = hfq4.matvec(Pb, base, K, x)          # [batch][base]
    for b in range(batch):
        ref = ref_base[b][sample % base] + r[b][sample]
        assert rel_l2(y[b][sample], ref) <= REL_L2_TOL, b


@pytest.mark.parametrize("rows,K", [(2048, 2048), (300, 1000)])
def test_gemv_residual_in_place(q, rows, K):
    """residual and y the same buffer: y = y + W x."""
    say("hfq4_gemv in place", rows, K)
    rng = np.random.default_rng(rows + K)
    W = (rng.standard_normal((rows, K)) * 0.02).astype(np.float32)
    P = hfq4.quantize_rows(W)
    x = rng.standard_normal((1, K)).astype(np.float32)
    r = rng.standard_normal((1, rows)).astype(np.float32)
    yr = torch.from_numpy(r.copy()).cuda()
    q.hfq4_gemv(torch.from_numpy(P).cuda(), rows, K, torch.from_numpy(x).cuda(), residual=yr, y=yr)
    ref = hfq4.matvec(P, rows, K, x) + r
    assert rel_l2(yr.cpu().numpy()[0], ref[0]) <= REL_L2_TOL


def test_gemv_exact_grid_block(q):
    # block C dequantizes exactly; with x = ones the sum is exactly -34
    say("hfq4_gemv exact")
    i = np.arange(256)
    w = (np.float32(-0.25) + ((7 * i) % 16).astype(np.float32) / np.float32(64))[None, :]
    Wd = torch.from_numpy(hfq4.quantize_rows(w)).cuda()
    y = q.hfq4_gemv(Wd, 1, 256, torch.ones((1, 256), device="cuda")).cpu().numpy()
    assert abs(y[0, 0] + 34.0) < 1e-4


# ------------------------------------------------------------------ routing

@pytest.mark.parametrize("E,d,k,B,zipf", [(8, 256, 2, 1, False), (256, 2048, 8, 16, False),
                                          (512, 2048, 8, 16, True), (1024, 64, 16, 3, False),
                                          (5, 8, 5, 2, False), (1, 4, 1, 1, False)])
def test_route_topk(q, E, d, k, B, zipf):
    say("moe_route_topk", E, d, k, B, zipf)
    rng = np.random.default_rng(E + d + k + B)
    Wr = (rng.standard_normal((E, d)) * 0.02).astype(np.float32)
    x = rng.standard_normal((B, d)).astype(np.float32)
    bias = synth.zipf_bias(1, E) if zipf else None
    gl, gi, gw = (Guarded(torch, (B, E), torch.float32), Guarded(torch, (B, k), torch.int32),
                  Guarded(torch, (B, k), torch.float32))
    gws = Guarded(torch, q.moe_route_workspace_bytes(E, B), torch.uint8, guard=256, zero=True)
    idx, wts = q.moe_route_topk(torch.from_numpy(Wr).cuda(), torch.from_numpy(x).cuda(), k,
                                bias=None if bias is None else torch.from_numpy(bias).cuda(),
                                logits=gl.t, idx=gi.t, wts=gw.t, ws=gws.t)
    torch.cuda.synchronize()
    for g in (gl, gi, gw, gws):
        g.check()
    l64 = moe.router_logits(Wr, x, bias)
    tau = logit_tol(Wr, x, bias)
    check_logits(gl.t.cpu().numpy(), l64, tau)
    amb = check_routing(idx.cpu().numpy(), wts.cpu().numpy(), l64, k, tau)
    assert amb == 0


def test_route_ties_lower_index(q):
    say("moe_route_topk ties")
    E, d, k = 64, 4, 8
    Wr = np.zeros((E, d), np.float32)
    Wr[[3, 10, 20, 40], 0] = 1.0       # four tied top logits
    Wr[[5, 7, 9, 11, 13], 0] = 0.5     # five tied next
    x = np.ones((1, d), np.float32)
    idx, wts = q.moe_route_topk(torch.from_numpy(Wr).cuda(), torch.from_numpy(x).cuda(), k)
    assert idx.cpu().numpy().tolist() == [[3, 10, 20, 40, 5, 7, 9, 11]]
    w = wts.cpu().numpy()[0]
    e1, e2 = 1.0, np.exp(-0.5)
    ref = np.array([e1] * 4 + [e2] * 4) / (4 * e1 + 4 * e2)
    assert np.allclose(w, ref, atol=1e-6)


@pytest.mark.parametrize("E", [64, 200, 300, 512, 700, 1024])
@pytest.mark.parametrize("B", [1, 3])
def test_route_heavy_ties(q, E, B):
    """Logits taking only a few distinct values (ties within a lane's block
    of experts and across lanes, at every block size the top-k uses): the
    selection must be exactly the lower-index top-k."""
    say("moe_route_topk heavy ties", E, B)
    k = 8
    rng = np.random.default_rng(E + B)
    d = 4
    Wr = np.zeros((E, d), np.float32)
    Wr[:, 0] = rng.integers(0, 4, size=E).astype(np.float32) * 0.25
    x = np.zeros((B, d), np.float32)
    x[:, 0] = np.arange(1, B + 1, dtype=np.float32)
    idx, wts = q.moe_route_topk(torch.from_numpy(Wr).cuda(), torch.from_numpy(x).cuda(), k)
    logits = (x.astype(np.float64) @ Wr.astype(np.float64).T).astype(np.float32)
    got = idx.cpu().numpy()
    for b in range(B):
        assert got[b].tolist() == moe.topk_lower_index(logits[b], k), b


# ------------------------------------------------------------------ expert decode + layer

def _tiny_inputs(q, seed=0):
    layer, L = q.synthetic.tiny_layer(torch, seed)
    exps = [moe.PackedExpert.from_f32(L["gate"][e], L["up"][e], L["down"][e]) for e in range(L["E"])]
    return layer, L, exps


@pytest.fixture(scope="module")
def qs(q):
    import quantized_moe_decode_amd.synthetic  # noqa: F401
    return q


def test_tiny_layer_packs_match_oracle(qs):
    say("tiny layer packs")
    layer, L, exps = _tiny_inputs(qs)
    g = layer.gate.cpu().numpy().reshape(8, -1)
    dn = layer.down.cpu().numpy().reshape(8, -1)
    for e in range(8):
        assert np.array_equal(g[e], exps[e].gate)
        assert np.array_equal(dn[e], exps[e].down)


@pytest.mark.parametrize("fused", [False, True])
def test_tiny_layer(qs, fused):
    say("tiny layer fused=%s" % fused)
    q = qs
    layer, L, exps = _tiny_inputs(q)
    x = torch.from_numpy(L["x"]).cuda()
    ws = q.new_workspace(layer, 1, 2)
    if fused:
        idx, wts, y = q.moe_layer_decode(layer, x, 2, ws)
    else:
        idx, wts = q.moe_route_topk(layer.Wr, x, 2, ws=ws)
        y = q.moe_expert_decode(layer, x, idx, wts, ws)
    torch.cuda.synchronize()
    assert q.workspace_error(ws) == 0
    err, amb = oracle_layer_check(L["x"], L["Wr"], None, exps, 2, idx.cpu().numpy(),
                                  wts.cpu().numpy(), y.cpu().numpy())
    assert amb == 0 and err <= REL_L2_TOL, err


def test_tiny_all_k_and_batches(qs):
    q = qs
    layer, L, exps = _tiny_inputs(q, 5)
    rng = np.random.default_rng(9)
    for B in (1, 3, 16):
        for k in (1, 2, 8):
            say("tiny layer B=%d k=%d" % (B, k))
            x = rng.standard_normal((B, 256)).astype(np.float32)
            r = rng.standard_normal((B, 256)).astype(np.float32)
            ws = q.new_workspace(layer, B, k)
            idx, wts, y = q.moe_layer_decode(layer, torch.from_numpy(x).cuda(), k, ws,
                                             residual=torch.from_numpy(r).cuda())
            torch.cuda.synchronize()
            assert q.workspace_error(ws) == 0
            err, amb = oracle_layer_check(x, L["Wr"], None, exps, k, idx.cpu().numpy(),
                                          wts.cpu().numpy(), y.cpu().numpy(), residual=r)
            assert amb == 0 and err <= REL_L2_TOL, (B, k, err)


@pytest.mark.parametrize("E,k,B", [(32, 9, 1), (32, 12, 3), (32, 16, 8), (16, 16, 2), (64, 16, 5),
                                   (48, 11, 11)])
def test_top_k_above_eight(qs, E, k, B):
    """k from 9 to the maximum of 16 (the generic kernels), including k = E
    (every expert selected) and batch * k at its limit of 128 pairs, fused
    and two-call, against the oracle."""
    q = qs
    d, F, seed = 256, 128, 61
    say("top-%d of %d, %d tokens" % (k, E, B))
    layer = q.synthetic.build_layer(torch, seed, 0, E, d, F)
    cache = ExpertCache(torch, "cuda", seed, 0, d, F)
    x = synth.activations(torch, "cuda", 62 + k, B, d)
    r = synth.activations(torch, "cuda", 63 + k, B, d)
    ws = q.new_workspace(layer, B, k)
    i1, w1, y1 = q.moe_layer_decode(layer, x, k, ws, residual=r)
    i1, w1, y1 = i1.clone(), w1.clone(), y1.clone()
    i2, w2 = q.moe_route_topk(layer.Wr, x, k, ws=ws)
    y2 = q.moe_expert_decode(layer, x, i2, w2, ws, residual=r)
    torch.cuda.synchronize()
    assert q.workspace_error(ws) == 0
    assert torch.equal(i1, i2) and torch.equal(w1, w2)
    assert torch.equal(y1, y2)
    err, amb = oracle_layer_check(x.cpu().numpy(), layer.Wr.cpu().numpy(), None, cache, k,
                                  i1.cpu().numpy(), w1.cpu().numpy(), y1.cpu().numpy(),
                                  residual=r.cpu().numpy())
    assert amb == 0 and err <= REL_L2_TOL, (err, amb)


def test_expert_decode_bad_index_skipped(qs):
    q = qs
    say("expert decode bad index")
    layer, L, exps = _tiny_inputs(q)
    x = torch.from_numpy(L["x"]).cuda()
    idx = torch.tensor([[3, 99]], dtype=torch.int32, device="cuda")
    wts = torch.tensor([[0.6, 0.4]], dtype=torch.float32, device="cuda")
    ws = q.new_workspace(layer, 1, 2)
    y = q.moe_expert_decode(layer, x, idx, wts, ws).cpu().numpy()
    assert q.workspace_error(ws) & q.HFQ4_DEV_ERR_INDEX
    ref = 0.6 * moe.expert_forward(exps[3], L["x"][0])
    assert rel_l2(y[0], ref) <= REL_L2_TOL


@pytest.mark.parametrize("E,d,F,k", [(64, 2048, 512, 8), (16, 256, 128, 2), (40, 1024, 300, 5)])
def test_bad_index_ignores_stale_h(qs, E, d, F, k):
    """A slot whose index is out of range adds nothing, also when the
    workspace still holds non-finite h from an earlier call (one token: the
    tuned kernels for d = 2048, F = 512, the generic ones otherwise)."""
    q = qs
    say("bad index, stale h", E, d, F, k)
    layer = q.synthetic.build_layer(torch, seed=3, layer_id=0, E=E, d=d, F=F)
    cache = ExpertCache(torch, "cuda", 3, 0, d, F)
    ws = q.new_workspace(layer, 1, k)
    idx0 = torch.arange(k, dtype=torch.int32, device="cuda").view(1, k)
    wts = torch.full((1, k), 1.0 / k, dtype=torch.float32, device="cuda")
    xbad = torch.full((1, d), float("nan"), dtype=torch.float32, device="cuda")
    q.moe_expert_decode(layer, xbad, idx0, wts, ws)        # every h slot now NaN
    torch.cuda.synchronize()
    assert q.workspace_error(ws) == 0
    x = synth.activations(torch, "cuda", 5, 1, d)
    idx = idx0.clone()
    idx[0, 1] = E + 7
    y = q.moe_expert_decode(layer, x, idx, wts, ws).cpu().numpy()
    assert q.workspace_error(ws) & q.HFQ4_DEV_ERR_INDEX
    assert np.all(np.isfinite(y))
    xs = x.cpu().numpy().astype(np.float64)[0]
    outs = [moe.expert_forward(cache(j), xs) for j in range(k) if j != 1]
    ref = moe.combine(outs, np.full(len(outs), 1.0 / k))
    assert rel_l2(y[0], ref) <= REL_L2_TOL


@pytest.fixture(scope="module")
def c2(qs):
    say("building 256-expert layer d=2048 F=512")
    layer = qs.synthetic.build_layer(torch, seed=0, layer_id=0, E=256, d=2048, F=512)
    return layer, ExpertCache(torch, "cuda", 0, 0, 2048, 512)


def test_c2_packed_experts_match_oracle(qs, c2):
    layer, cache = c2
    gb = qs.hfq4_packed_bytes(512, 2048)
    for e in (0, 137, 255):
        say("c2 pack parity expert", e)
        ex = cache(e)
        assert np.array_equal(layer.gate[e * gb:(e + 1) * gb].cpu().numpy(), ex.gate)
        assert np.array_equal(layer.up[e * gb:(e + 1) * gb].cpu().numpy(), ex.up)
        assert np.array_equal(layer.down[e * gb:(e + 1) * gb].cpu().numpy(), ex.down)


@pytest.mark.parametrize("fused", [True, False])
def test_c2_single_token(qs, c2, fused):
    q = qs
    layer, cache = c2
    T = 8
    xs = synth.activations(torch, "cuda", 1, T, 2048)
    gws = Guarded(torch, q.moe_workspace_bytes(layer, 1, 8), torch.uint8, guard=256, zero=True)
    ws = gws.t
    Wr = layer.Wr.cpu().numpy()
    for t in range(T):
        say("c2 token", t, "fused", fused)
        x = xs[t:t + 1].contiguous()
        gy, gi, gw = (Guarded(torch, (1, 2048), torch.float32), Guarded(torch, (1, 8), torch.int32),
                      Guarded(torch, (1, 8), torch.float32))
        if fused:
            idx, wts, y = q.moe_layer_decode(layer, x, 8, ws, y=gy.t, idx=gi.t, wts=gw.t)
        else:
            idx, wts = q.moe_route_topk(layer.Wr, x, 8, ws=ws, idx=gi.t, wts=gw.t)
            y = q.moe_expert_decode(layer, x, idx, wts, ws, y=gy.t)
        torch.cuda.synchronize()
        assert q.workspace_error(ws) == 0
        for g in (gy, gi, gw, gws):
            g.check()
        err, amb = oracle_layer_check(x.cpu().numpy(), Wr, None, cache, 8, idx.cpu().numpy(),
                                      wts.cpu().numpy(), y.cpu().numpy())
        assert amb == 0 and err <= REL_L2_TOL, (amb, err)


def test_c2_fused_equals_two_call_bitwise(qs, c2):
    q = qs
    layer, _ = c2
    say("c2 fused vs two-call, B=4")
    x = synth.activations(torch, "cuda", 2, 4, 2048)
    ws = q.new_workspace(layer, 4, 8)
    i1, w1, y1 = q.moe_layer_decode(layer, x, 8, ws)
    i2, w2 = q.moe_route_topk(layer.Wr, x, 8, ws=ws)
    y2 = q.moe_expert_decode(layer, x, i2, w2, ws)
    i3, w3, y3 = q.moe_layer_decode(layer, x, 8, ws)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2) and torch.equal(w1, w2) and torch.equal(y1, y2)
    assert torch.equal(y1, y3)


def test_c3_skewed_batch(qs):
    q = qs
    say("building 512-expert zipf layer")
    bias = synth.zipf_bias(7, 512)
    layer = q.synthetic.build_layer(torch, seed=3, layer_id=0, E=512, d=2048, F=512, bias=bias)
    cache = ExpertCache(torch, "cuda", 3, 0, 2048, 512)
    for B in (1, 4, 16):
        say("c3 B=%d" % B)
        x = synth.activations(torch, "cuda", 10 + B, B, 2048)
        gws = Guarded(torch, q.moe_workspace_bytes(layer, B, 8), torch.uint8, guard=256, zero=True)
        gy, gi, gw = (Guarded(torch, (B, 2048), torch.float32), Guarded(torch, (B, 8), torch.int32),
                      Guarded(torch, (B, 8), torch.float32))
        idx, wts, y = q.moe_layer_decode(layer, x, 8, gws.t, y=gy.t, idx=gi.t, wts=gw.t)
        torch.cuda.synchronize()
        assert q.workspace_error(gws.t) == 0
        for g in (gy, gi, gw, gws):
            g.check()
        # every token's routing and output (the skew makes the union small,
        # and the oracle quantizes each selected expert once)
        err, amb = oracle_layer_check(x.cpu().numpy(), layer.Wr.cpu().numpy(), bias, cache, 8,
                                      idx.cpu().numpy(), wts.cpu().numpy(), y.cpu().numpy())
        say("c3 B=%d: %d distinct experts, max rel-L2 %.3g" % (B, len(np.unique(idx.cpu().numpy())), err))
        assert amb == 0 and err <= REL_L2_TOL, (amb, err)
