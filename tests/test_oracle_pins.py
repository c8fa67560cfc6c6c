"""Pins for the CPU oracle (no GPU).

Each test checks the oracle against something other than itself: bytes
worked out by hand, a size the pages print, a closed form, an error bound,
a special case that reduces to a textbook routine, or brute force on tiny
inputs.  Together they are meant to catch the plausible mistakes: swapped
header fields, swapped nibbles, a dropped zero point, truncating instead of
rounding, a transposed operand, padding that leaks into a sum, gate/up
swapped, the wrong softmax normalisation, the wrong tie-break.
"""

import math
import os
import struct

import numpy as np
import pytest

from oracle import hfq4, moe
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------ golden blocks

def _golden_records():
    recs = {}
    with open(os.path.join(GOLDEN, "hfq4_blocks.txt"), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, K, rule, header, pattern, reps = [t.strip() for t in line.split("|")]
            recs[name] = dict(K=int(K), rule=rule, header=bytes.fromhex(header),
                              pattern=bytes.fromhex(pattern), reps=int(reps))
    return recs


def _weights(name, K):
    i = np.arange(K)
    if name in ("A", "E"):
        return (i % 16).astype(np.float32)
    if name == "B":
        return np.full(K, 0.75, np.float32)
    if name == "C":
        return (np.float32(-0.25) + ((7 * i) % 16).astype(np.float32) / np.float32(64)).astype(np.float32)
    if name == "D":
        w = np.zeros(K, np.float32)
        w[:4] = [0, 15, 2.5, 3.5]
        return w
    if name in ("F", "G"):
        w = (i % 16).astype(np.float32)
        neg = (i % 32 == 0) if name == "F" else (i % 16 == 0)
        w[neg] = np.float32(-0.0)
        return w
    raise KeyError(name)


@pytest.mark.parametrize("name", ["A", "B", "C", "D", "E", "F", "G"])
def test_golden_block_bytes(name):
    rec = _golden_records()[name]
    K = rec["K"]
    w = _weights(name, K)
    got = hfq4.quantize_rows(w[None, :]).tobytes()
    assert len(got) == 136
    assert got[:8] == rec["header"]
    codes = rec["pattern"] * rec["reps"]
    assert got[8:8 + len(codes)] == codes
    if name == "E":  # padded half of the block is all zero codes
        assert got[8 + len(codes):] == b"\x00" * 64


def test_golden_A_closed_forms():
    w = _weights("A", 256)
    P = hfq4.quantize_rows(w[None, :])
    assert hfq4.matvec(P, 1, 256, np.ones(256))[0] == 1920.0
    for j in (0, 1, 15, 16, 17, 255):
        e = np.zeros(256)
        e[j] = 1.0
        assert hfq4.matvec(P, 1, 256, e)[0] == float(j % 16)


def test_golden_B_exact():
    P = hfq4.quantize_rows(_weights("B", 256)[None, :])
    assert np.all(hfq4.dequantize(P, 1, 256) == 0.75)


def test_golden_C_roundtrip_and_zero_point():
    w = _weights("C", 256)
    P = hfq4.quantize_rows(w[None, :])
    back = hfq4.dequantize(P, 1, 256)[0]
    assert np.array_equal(back.astype(np.float32), w)
    assert np.array_equal(back, w.astype(np.float64))
    # the zero point must enter every weight: sum w = 256*(-0.25) + 16*(0+..+15)/64
    assert hfq4.matvec(P, 1, 256, np.ones(256))[0] == -34.0


def test_golden_D_ties_to_even_and_bound():
    w = _weights("D", 256)
    P = hfq4.quantize_rows(w[None, :])
    back = hfq4.dequantize(P, 1, 256)[0]
    assert back[2] == 2.0 and back[3] == 4.0
    assert abs(back[2] - 2.5) == 0.5  # exactly scale/2, so the bound is inclusive


def test_golden_FG_signed_zero_minimum():
    # the weights hold -0.0 (F: mixed with +0.0; G: the only zeros), and the
    # zero field is +0.0 whichever zero a min() returns, in either scan order
    for name in "FG":
        w = _weights(name, 256)
        assert np.signbit(w).sum() == (8 if name == "F" else 16)
        for order in (w, w[::-1].copy()):
            s, z, _ = hfq4.quantize_block(order)
            assert struct.pack("<f", z) == b"\x00\x00\x00\x00"
        P = hfq4.quantize_rows(w[None, :])
        assert P.tobytes() == hfq4.quantize_rows(_weights("A", 256)[None, :]).tobytes()
        assert np.array_equal(hfq4.dequantize(P, 1, 256)[0], np.abs(w).astype(np.float64))


def test_golden_E_padding_does_not_contribute():
    P = hfq4.quantize_rows(_weights("E", 128)[None, :])
    assert P.size == 136
    assert hfq4.matvec(P, 1, 128, np.ones(128))[0] == 8 * 120.0


def test_scalar_block_encoder_matches_golden():
    # the one-block scalar quantizer and encoder give the same golden bytes
    for name in "ABCDEFG":
        rec = _golden_records()[name]
        w = _weights(name, rec["K"])
        s, z, q = hfq4.quantize_block(w)
        b = hfq4.encode_block(s, z, q)
        assert b[:8] == rec["header"]
        assert b == hfq4.quantize_rows(w[None, :]).tobytes()


# ------------------------------------------------------------ sizes

def test_size_identity_matches_page_figure():
    with open(os.path.join(GOLDEN, "sizes.txt"), encoding="utf-8") as f:
        rows = [l for l in f if l.strip() and not l.startswith("#")]
    E, d, F, total, mib = [int(t) for t in rows[0].split("|")]
    per_expert = 2 * hfq4.packed_bytes(F, d) + hfq4.packed_bytes(d, F)
    assert per_expert == 1671168
    assert E * per_expert == total
    assert total == mib * 2 ** 20


@pytest.mark.parametrize("rows,K,expect", [(1, 256, 136), (1, 128, 136), (1, 257, 272),
                                           (3, 512, 816), (0, 2048, 0), (2048, 2048, 2228224)])
def test_packed_bytes(rows, K, expect):
    assert hfq4.packed_bytes(rows, K) == expect
    if rows:
        W = np.zeros((rows, K), np.float32)
        assert hfq4.quantize_rows(W).size == expect


# ------------------------------------------------------------ error bound

@pytest.mark.parametrize("seed,std,offset,K", [(1, 0.02, 0.0, 2048), (2, 1.0, 3.0, 512),
                                               (3, 1e-3, -0.5, 300), (4, 50.0, 0.0, 1000)])
def test_dequant_error_bound(seed, std, offset, K):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((16, K)) * std + offset).astype(np.float32)
    P = hfq4.quantize_rows(W)
    scale, zero, q = hfq4.decode_fields(P, 16, K)
    What = hfq4.dequantize(P, 16, K)
    nb = hfq4.blocks_per_row(K)
    s = np.repeat(scale.astype(np.float64), 256, axis=1)[:, :K]
    err = np.abs(W.astype(np.float64) - What)
    assert np.all(err <= s * (0.5 + 2.0 ** -19))
    # min and max of each block are represented (zero = min; max within the bound)
    for r in range(16):
        for b in range(nb):
            blk = W[r, b * 256:min(K, b * 256 + 256)]
            assert zero[r, b] == blk.min()
    # rounding, not truncation: the chosen code is never beaten by a neighbour
    # by more than f32 rounding of (w - zero)/scale
    up = np.abs(W - (What + s))
    dn = np.abs(W - (What - s))
    slack = s * 2.0 ** -19
    assert np.all(err <= up + slack) and np.all(err <= dn + slack)


def test_nonfinite_rejected():
    W = np.zeros((1, 256), np.float32)
    W[0, 7] = np.nan
    with pytest.raises(ValueError):
        hfq4.quantize_rows(W)
    W[0, 7] = np.inf
    with pytest.raises(ValueError):
        hfq4.quantize_rows(W)


# ------------------------------------------------------------ matvec orientation

def test_matvec_orientation_and_linearity():
    K = 512
    rows = np.stack([_weights("A", 256).tolist() * 2, (_weights("C", 256).tolist() * 2)]).astype(np.float32)
    P = hfq4.quantize_rows(rows)
    What = hfq4.dequantize(P, 2, K)
    for j in (0, 3, 255, 256, 300, 511):
        e = np.zeros(K)
        e[j] = 1
        y = hfq4.matvec(P, 2, K, e)
        assert y[0] == float(j % 16)
        assert y[1] == What[1, j] == -0.25 + ((7 * (j % 256)) % 16) / 64
    rng = np.random.default_rng(0)
    x1, x2 = rng.standard_normal(K), rng.standard_normal(K)
    lhs = hfq4.matvec(P, 2, K, 2 * x1 - 3 * x2)
    rhs = 2 * hfq4.matvec(P, 2, K, x1) - 3 * hfq4.matvec(P, 2, K, x2)
    assert np.allclose(lhs, rhs, rtol=0, atol=1e-11)


def _scalar_decode_row(row_bytes, K):
    """Independent scalar decoder (struct + bit shifts), for brute force."""
    out = []
    nb = (K + 255) // 256
    for b in range(nb):
        blk = row_bytes[136 * b:136 * (b + 1)]
        scale, zero = struct.unpack("<ff", bytes(blk[:8]))
        for i in range(256):
            if b * 256 + i >= K:
                break
            byte = blk[8 + i // 2]
            q = (byte >> 4) if (i & 1) else (byte & 15)
            out.append(zero + scale * q)
    return out


def test_dequantize_matches_scalar_decoder():
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((3, 300)) * 0.02).astype(np.float32)
    P = hfq4.quantize_rows(W)
    What = hfq4.dequantize(P, 3, 300)
    rb = hfq4.packed_bytes(1, 300)
    for r in range(3):
        ref = _scalar_decode_row(P[r * rb:(r + 1) * rb], 300)
        assert np.array_equal(np.array(ref), What[r])


# ------------------------------------------------------------ routing

def test_topk_all_equal():
    idx = moe.topk_lower_index([0.5] * 8, 3)
    assert idx == [0, 1, 2]
    assert np.allclose(moe.softmax_renorm([0.5] * 8, idx), [1 / 3] * 3, atol=1e-15)


def test_topk_closed_forms():
    l = [0.0, math.log(3.0)]
    idx = moe.topk_lower_index(l, 2)
    assert idx == [1, 0]
    assert np.allclose(moe.softmax_renorm(l, idx), [0.75, 0.25], atol=1e-15)
    l = [1.0, 3.0, 3.0, 2.0]
    idx = moe.topk_lower_index(l, 2)
    assert idx == [1, 2]
    assert np.allclose(moe.softmax_renorm(l, idx), [0.5, 0.5], atol=1e-15)
    l = [0.0, math.log(2.0), math.log(4.0)]
    assert moe.topk_lower_index(l, 3) == [2, 1, 0]
    assert np.allclose(moe.softmax_renorm(l, [2, 1, 0]), [4 / 7, 2 / 7, 1 / 7], atol=1e-15)
    assert np.allclose(moe.softmax_renorm(l, [2, 1]), [2 / 3, 1 / 3], atol=1e-15)


def test_router_bias_enters_with_its_sign():
    # Wr = 0, so the logits are the bias alone: [0, ln 3] selects expert 1
    # first with weight 3/(1+3) -- a bias subtracted instead of added would
    # select expert 0 first
    d = 16
    Wr = np.zeros((2, d), np.float32)
    x = np.random.default_rng(3).standard_normal((1, d))
    bias = np.array([0.0, math.log(3.0)])
    assert np.array_equal(moe.router_logits(Wr, x, bias), [[0.0, math.log(3.0)]])
    idx, wts, _ = moe.route(Wr, x, 2, bias)
    assert idx.tolist() == [[1, 0]]
    assert np.allclose(wts, [[0.75, 0.25]], rtol=0, atol=1e-15)
    # and in the layer: y = 3/4 y_1 + 1/4 y_0 with closed-form constant experts
    D, F = 256, 128
    xl = np.full((1, D), 1.0 / 256)
    exps = {0: _const_expert(0.5, 0.25, 1.0, D, F), 1: _const_expert(1.0, 1.0, 2.0, D, F)}
    idx, wts, y, _ = moe.moe_layer(xl, np.zeros((2, D), np.float32), exps, 2, bias=bias)
    y0 = F * (0.5 / (1 + math.exp(-0.5)) * 0.25) * 1.0
    y1 = F * (1.0 / (1 + math.exp(-1.0)) * 1.0) * 2.0
    assert idx.tolist() == [[1, 0]]
    assert np.allclose(y[0], 0.75 * y1 + 0.25 * y0, rtol=1e-13, atol=0)


def test_idx_override_recomputes_weights():
    # logits [0, ln 2, ln 4]: the oracle's own selection is [2, 1, 0] with
    # weights [4/7, 2/7, 1/7]; a caller-given order or subset gets the
    # weights of that selection, not the oracle's
    d, F = 256, 128
    x = np.full((1, d), 1.0 / 256)
    Wr = np.zeros((3, d), np.float32)
    Wr[1, :] = math.log(2.0)
    Wr[2, :] = math.log(4.0)
    c = [1.0, 2.0, 4.0]
    exps = {e: _const_expert(0.5, 0.25, c[e], d, F) for e in range(3)}
    yu = F * (0.5 / (1 + math.exp(-0.5)) * 0.25)      # expert e gives c[e] * yu
    l = [0.0, float(np.float32(math.log(2.0))), float(np.float32(math.log(4.0)))]
    p = np.exp(l)
    idx, wts, y, _ = moe.moe_layer(x, Wr, exps, 3)
    assert idx.tolist() == [[2, 1, 0]]
    assert np.allclose(wts[0], p[[2, 1, 0]] / p.sum(), rtol=1e-14, atol=0)
    idx, wts, y, _ = moe.moe_layer(x, Wr, exps, 3, idx=[[0, 1, 2]])
    assert idx.tolist() == [[0, 1, 2]]
    assert np.allclose(wts[0], p / p.sum(), rtol=1e-14, atol=0)
    assert np.allclose(y[0], yu * float(np.dot(p / p.sum(), c)), rtol=1e-13, atol=0)
    idx, wts, y, _ = moe.moe_layer(x, Wr, exps, 2, idx=[[0, 1]])
    assert np.allclose(wts[0], p[:2] / p[:2].sum(), rtol=1e-14, atol=0)
    assert np.allclose(y[0], yu * (p[0] * c[0] + p[1] * c[1]) / (p[0] + p[1]), rtol=1e-13, atol=0)


def test_topk_matches_lexsort_and_k_term_softmax():
    rng = np.random.default_rng(7)
    for trial in range(50):
        E = int(rng.integers(2, 64))
        k = int(rng.integers(1, E + 1))
        l = np.round(rng.standard_normal(E), 1)  # rounding creates exact ties
        idx = moe.topk_lower_index(l, k)
        order = np.lexsort((np.arange(E), -l))[:k]  # key: logit desc, then index asc
        assert idx == order.tolist()
        w = moe.softmax_renorm(l, idx)
        sel = l[idx]
        ref = np.exp(sel - sel.max()) / np.exp(sel - sel.max()).sum()
        assert np.allclose(w, ref, rtol=0, atol=1e-12)
        assert abs(w.sum() - 1.0) < 1e-12
        # shift invariance of both selection and weights
        idx2 = moe.topk_lower_index(l + 7.25, k)
        assert idx2 == idx
        assert np.allclose(moe.softmax_renorm(l + 7.25, idx2), w, atol=1e-12)
        if k == E:
            p = np.exp(l - l.max())
            p /= p.sum()
            assert np.allclose(w, p[idx], atol=1e-12)


# ------------------------------------------------------------ experts

def test_silu_values():
    assert moe.silu(0.0) == 0.0
    assert abs(moe.silu(1.0) - 0.7310585786300049) < 1e-15
    assert abs(moe.silu(-1.0) + 0.2689414213699951) < 1e-15
    assert abs(moe.silu(40.0) - 40.0) < 1e-12
    assert abs(moe.silu(-40.0)) < 1e-15


def _const_expert(a, b, c, d, F):
    """gate rows all a, up rows all b, down rows all c (scale 0 blocks)."""
    return moe.PackedExpert.from_f32(np.full((F, d), a, np.float32),
                                     np.full((F, d), b, np.float32),
                                     np.full((d, F), c, np.float32))


def test_expert_closed_form_gate_up_order():
    d, F = 256, 128
    x = np.full(d, 1.0 / 256)          # sum x = 1
    ex = _const_expert(0.5, 0.25, 1.0, d, F)
    y = moe.expert_forward(ex, x)
    h = 0.5 / (1 + math.exp(-0.5)) * 0.25
    assert np.allclose(y, F * h, rtol=1e-14, atol=0)
    swapped = moe.expert_forward(_const_expert(0.25, 0.5, 1.0, d, F), x)
    assert not np.allclose(swapped, y)


def test_layer_closed_form_combine():
    d, F = 256, 128
    x = np.full((1, d), 1.0 / 256)
    Wr = np.zeros((3, d), np.float32)
    Wr[1, :] = math.log(3.0)              # logits [0, ln 3, -1]
    Wr[2, :] = -1.0
    exps = {0: _const_expert(0.5, 0.25, 1.0, d, F), 1: _const_expert(1.0, 1.0, 2.0, d, F),
            2: _const_expert(9.0, 9.0, 9.0, d, F)}
    idx, wts, y, _ = moe.moe_layer(x, Wr, exps, 2)
    assert idx.tolist() == [[1, 0]]
    assert np.allclose(wts, [[0.75, 0.25]], atol=1e-7)  # Wr is f32: ln3 rounded
    y0 = F * (0.5 / (1 + math.exp(-0.5)) * 0.25) * 1.0
    y1 = F * (1.0 / (1 + math.exp(-1.0)) * 1.0) * 2.0
    l1 = float(np.float32(math.log(3.0)))
    w1 = math.exp(l1) / (math.exp(l1) + 1.0)
    assert np.allclose(y[0], w1 * y1 + (1 - w1) * y0, rtol=1e-13)


def _brute_expert(ex, x):
    """Pure-Python loops over the scalar-decoded matrices."""
    rbg = hfq4.packed_bytes(1, ex.d)
    rbd = hfq4.packed_bytes(1, ex.F)
    g = [sum(w * xi for w, xi in zip(_scalar_decode_row(ex.gate[f * rbg:(f + 1) * rbg], ex.d), x))
         for f in range(ex.F)]
    u = [sum(w * xi for w, xi in zip(_scalar_decode_row(ex.up[f * rbg:(f + 1) * rbg], ex.d), x))
         for f in range(ex.F)]
    h = [gi / (1 + math.exp(-gi)) * ui for gi, ui in zip(g, u)]
    return [sum(w * hi for w, hi in zip(_scalar_decode_row(ex.down[i * rbd:(i + 1) * rbd], ex.F), h))
            for i in range(ex.d)]


def test_tiny_layer_brute_force():
    L = synth.tiny_layer(0)
    d, F, E, k = L["d"], L["F"], L["E"], 2
    exps = [moe.PackedExpert.from_f32(L["gate"][e], L["up"][e], L["down"][e]) for e in range(E)]
    x = L["x"][0].astype(np.float64)
    idx, wts, y, logits = moe.moe_layer(L["x"], L["Wr"], exps, k)
    # enumerate every pair: the selected pair is the one whose smaller logit
    # is >= every other logit
    l = [sum(float(a) * float(b) for a, b in zip(L["Wr"][e], x)) for e in range(E)]
    best = None
    for i in range(E):
        for j in range(i + 1, E):
            rest = [l[m] for m in range(E) if m not in (i, j)]
            if min(l[i], l[j]) >= max(rest):
                best = (i, j)
    assert best is not None and set(best) == set(idx[0].tolist())
    i, j = sorted(best, key=lambda e: -l[e])
    wi = 1.0 / (1.0 + math.exp(l[j] - l[i]))
    yi = _brute_expert(exps[i], x)
    yj = _brute_expert(exps[j], x)
    ref = np.array([wi * a + (1 - wi) * b for a, b in zip(yi, yj)])
    assert np.allclose(y[0], ref, rtol=1e-10, atol=1e-13)
    assert np.allclose(wts[0], [wi, 1 - wi], atol=1e-13)


def test_expert_permutation_invariance():
    L = synth.tiny_layer(3)
    E, k = L["E"], 2
    exps = [moe.PackedExpert.from_f32(L["gate"][e], L["up"][e], L["down"][e]) for e in range(E)]
    idx, wts, y, _ = moe.moe_layer(L["x"], L["Wr"], exps, k)
    perm = np.random.default_rng(1).permutation(E)   # new expert p holds old expert perm[p]
    inv = np.argsort(perm)
    idx2, wts2, y2, _ = moe.moe_layer(L["x"], L["Wr"][perm], [exps[perm[p]] for p in range(E)], k)
    assert np.array_equal(idx2, inv[idx])
    assert np.allclose(wts2, wts, atol=1e-15)
    assert np.allclose(y2, y, rtol=1e-13, atol=1e-15)


def test_stack_step_identity_and_one_layer():
    # zero dense matrix and zero down projections -> x passes through unchanged
    d, F = 256, 128
    rng = np.random.default_rng(2)
    x = rng.standard_normal(d)
    zero_ex = _const_expert(0.1, 0.1, 0.0, d, F)
    dense0 = hfq4.quantize_rows(np.zeros((d, d), np.float32))
    layers = [dict(Wr=rng.standard_normal((4, d)).astype(np.float32),
                   experts=[zero_ex] * 4, dense=dense0)] * 3
    assert np.array_equal(moe.stack_step(x, layers, 2), x)
    # one layer, non-trivial: t = x + D x then x' = t + MoE(t)
    L = synth.tiny_layer(4)
    exps = [moe.PackedExpert.from_f32(L["gate"][e], L["up"][e], L["down"][e]) for e in range(8)]
    D = hfq4.quantize_rows((np.eye(d) * 0.5).astype(np.float32))
    x = L["x"][0].astype(np.float64)
    out = moe.stack_step(x, [dict(Wr=L["Wr"], experts=exps, dense=D)], 2)
    t = x + hfq4.dequantize(D, d, d) @ x
    _, _, y, _ = moe.moe_layer(t, L["Wr"], exps, 2)
    assert np.allclose(out, t + y[0], rtol=1e-14, atol=1e-15)
