"""Host CPU execution of HFQ4 experts (hfq4_gemv_host, moe_expert_decode_host,
hfq4_offload_choice) against the oracle, through the C ABI.  No GPU: these
entry points touch host memory only.

The packed weights come from the oracle's quantizer (the only CPU packer;
the product path takes packed bytes as its input), the activations and
weights from the seeded generators.  Bars: relative L2 <= 2e-3 per token
(the stated one; the f32 arithmetic lands near 1e-7), bitwise independence
of the thread count, and the 15% rule of the route choice.
"""

import ctypes
import math

import numpy as np
import pytest

from oracle import hfq4, moe
import synth

from _parity import REL_L2_TOL, rel_l2


@pytest.fixture(scope="module")
def q():
    import quantized_moe_decode_amd as q
    return q


@pytest.fixture(params=["avx512", "avx2", "portable"])
def kern(q, request):
    """Each host row kernel in turn (skipped where the CPU lacks it); the
    best one is restored afterwards."""
    try:
        q.set_host_kernel(request.param)
    except q.Hfq4Error:
        pytest.skip("this CPU lacks the %s kernel" % request.param)
    yield request.param
    q.set_host_kernel("best")


@pytest.mark.parametrize("rows,K,batch,resid", [(1, 256, 1, False), (7, 128, 1, True),
                                                (33, 300, 2, False), (2051, 2048, 1, True),
                                                (129, 1000, 3, True), (5, 5000, 1, False),
                                                (512, 2048, 16, False), (2048, 512, 4, True)])
def test_gemv_host_vs_oracle(q, kern, rows, K, batch, resid):
    rng = np.random.default_rng(rows * 31 + K)
    W = (rng.standard_normal((rows, K)) * 0.02).astype(np.float32)
    P = hfq4.quantize_rows(W)
    x = rng.standard_normal((batch, K)).astype(np.float32)
    r = rng.standard_normal((batch, rows)).astype(np.float32) if resid else None
    y = q.hfq4_gemv_host(P, rows, K, x, residual=r)
    ref = hfq4.matvec(P, rows, K, x)
    if r is not None:
        ref = ref + r
    for b in range(batch):
        e = rel_l2(y[b], ref[b])
        assert e <= REL_L2_TOL and e < 1e-5, (b, e)


def test_gemv_host_exact_grid_and_padding(q, kern):
    # block C dequantizes exactly (sum -34 with x = 1); a K = 128 row pads
    # its block with zeros that must not contribute
    i = np.arange(256)
    wC = (np.float32(-0.25) + ((7 * i) % 16).astype(np.float32) / np.float32(64))[None, :]
    y = q.hfq4_gemv_host(hfq4.quantize_rows(wC), 1, 256, np.ones((1, 256), np.float32))
    assert y[0, 0] == -34.0
    wE = (np.arange(128) % 16).astype(np.float32)[None, :]
    y = q.hfq4_gemv_host(hfq4.quantize_rows(wE), 1, 128, np.ones((1, 128), np.float32))
    assert y[0, 0] == 8 * 120.0


def test_gemv_host_thread_count_independent(q, kern):
    rng = np.random.default_rng(3)
    W = (rng.standard_normal((777, 2048)) * 0.02).astype(np.float32)
    P = hfq4.quantize_rows(W)
    x = rng.standard_normal((2, 2048)).astype(np.float32)
    ys = [q.hfq4_gemv_host(P, 777, 2048, x, nthreads=n) for n in (1, 3, 8)]
    assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[0], ys[2])


def _host_layer(q, seed, E, d, F):
    """A host layer of E experts drawn by the seeded host generator and
    packed by the oracle quantizer; returns (HostMoeLayer, experts dict)."""
    exps, g, u, dn = {}, [], [], []
    for e in range(E):
        ge = synth.host_matrix(seed, F, d, 0.02, e, 0)
        ue = synth.host_matrix(seed, F, d, 0.02, e, 1)
        de = synth.host_matrix(seed, d, F, 0.02, e, 2)
        exps[e] = moe.PackedExpert.from_f32(ge, ue, de)
        g.append(exps[e].gate)
        u.append(exps[e].up)
        dn.append(exps[e].down)
    L = q.HostMoeLayer(np.concatenate(g), np.concatenate(u), np.concatenate(dn), E, d, F)
    return L, exps


@pytest.mark.parametrize("E,d,F,k,B", [(8, 256, 128, 2, 1), (16, 2048, 512, 8, 1),
                                       (12, 1000, 300, 3, 4), (9, 2048, 512, 8, 2)])
def test_expert_decode_host_vs_oracle(q, kern, E, d, F, k, B):
    L, exps = _host_layer(q, E + d, E, d, F)
    rng = np.random.default_rng(E * d)
    x = rng.standard_normal((B, d)).astype(np.float32)
    Wr = (rng.standard_normal((E, d)) * 0.05).astype(np.float32)
    idx, wts, _ = moe.route(Wr, x, k)
    res = rng.standard_normal((B, d)).astype(np.float32)
    y, err = q.moe_expert_decode_host(L, x, idx.astype(np.int32), wts.astype(np.float32),
                                      residual=res)
    assert err == 0
    _, _, y_ref, _ = moe.moe_layer(x, Wr, exps, k, idx=idx)
    for b in range(B):
        e = rel_l2(y[b], y_ref[b] + res[b])
        assert e <= REL_L2_TOL, (b, e)


def test_expert_decode_host_bad_index(q):
    E, d, F = 8, 256, 128
    L, exps = _host_layer(q, 5, E, d, F)
    x = np.random.default_rng(1).standard_normal((1, d)).astype(np.float32)
    idx = np.array([[3, 99]], np.int32)
    wts = np.array([[0.6, 0.4]], np.float32)
    y, err = q.moe_expert_decode_host(L, x, idx, wts)
    assert err & q.HFQ4_DEV_ERR_INDEX
    ref = 0.6 * moe.expert_forward(exps[3], x[0].astype(np.float64))
    assert rel_l2(y[0], ref) <= REL_L2_TOL


def test_host_kernels_agree(q):
    # the row kernels differ only in f32 rounding order
    rng = np.random.default_rng(11)
    W = (rng.standard_normal((300, 2048)) * 0.02).astype(np.float32)
    P = hfq4.quantize_rows(W)
    x = rng.standard_normal((2, 2048)).astype(np.float32)
    ys = {}
    for name in ("avx512", "avx2", "portable"):
        try:
            q.set_host_kernel(name)
        except q.Hfq4Error:
            continue
        ys[name] = q.hfq4_gemv_host(P, 300, 2048, x)
    q.set_host_kernel("best")
    assert "portable" in ys
    for name, y in ys.items():
        assert rel_l2(y, ys["portable"]) < 1e-6, name


def test_host_kernel_selection(q):
    best = q.set_host_kernel("best")
    assert best in ("avx512", "avx2", "portable")
    assert q.set_host_kernel("portable") == "portable"
    assert q.set_host_kernel("best") == best
    used = ctypes.c_int(0)
    for bad in (-1, 4):
        assert q.lib.hfq4_debug_set_host_kernel(bad, ctypes.byref(used)) == q.HFQ4_E_INVALID
    assert q.set_host_kernel("best") == best


def test_offload_choice_rule(q):
    # the CPU path only when it is at least 15% faster
    assert q.hfq4_offload_choice(1.15, 1.0)
    assert not q.hfq4_offload_choice(1.149, 1.0)
    assert not q.hfq4_offload_choice(1.0, 1.0)
    assert q.hfq4_offload_choice(3.0, 1.0)
    for bad in ((0.0, 1.0), (1.0, -1.0), (math.inf, 1.0), (math.nan, 1.0)):
        with pytest.raises(q.Hfq4Error):
            q.hfq4_offload_choice(*bad)
