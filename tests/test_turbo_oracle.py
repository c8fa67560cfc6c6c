"""Pins for the TurboQuant codec oracle (no GPU).

Each test checks oracle/turbo.py against something other than itself: the
page's compression table, the Hadamard matrix's closed forms, the 1-bit
Lloyd-Max level sqrt(2/pi), the optimality conditions of the other levels
checked by independent quadrature, a bit stream packed by hand, norm
preservation, and brute force over every code vector on a tiny case.
"""

import itertools
import math
import os

import numpy as np
import pytest
from scipy import integrate

from oracle import turbo

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_record_sizes_match_page_ratios():
    rows = [l for l in open(os.path.join(GOLDEN, "turbo_sizes.txt"), encoding="utf-8")
            if l.strip() and not l.startswith("#")]
    assert len(rows) == 4
    for line in rows:
        bits, nbytes, ratio = [t.strip() for t in line.split("|")]
        assert turbo.record_bytes(128, int(bits)) == int(nbytes)
        got = 128 * 4 / int(nbytes)
        # the page prints two or three significant figures
        assert abs(got - float(ratio)) <= 0.5 * 10 ** (-(len(ratio.split(".")[1]))) + 1e-9, (bits, got)


def test_hadamard_closed_forms():
    H2 = turbo.hadamard(2) * math.sqrt(2)
    assert np.array_equal(H2, [[1, 1], [1, -1]])
    H4 = turbo.hadamard(4) * 2
    assert np.array_equal(H4, [[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]])
    for n in (8, 128):
        H = turbo.hadamard(n)
        assert np.allclose(H @ H, np.eye(n), atol=1e-12)          # orthonormal and an involution
        assert np.allclose(H, H.T)
        e0 = np.zeros(n)
        e0[0] = 1
        assert np.allclose(H @ e0, np.full(n, 1 / math.sqrt(n)))
        # Sylvester recursion H_2n = [[H, H], [H, -H]] / sqrt(2)
        H2n = turbo.hadamard(2 * n)
        assert np.allclose(H2n[:n, :n], H / math.sqrt(2)) and np.allclose(H2n[n:, n:], -H / math.sqrt(2))
    with pytest.raises(ValueError):
        turbo.hadamard(6)


def test_lloyd_max_one_bit_closed_form():
    lv = turbo.lloyd_max(1)
    assert np.allclose(lv, [-math.sqrt(2 / math.pi), math.sqrt(2 / math.pi)], atol=1e-12)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_lloyd_max_optimality_by_quadrature(bits):
    lv = turbo.lloyd_max(bits)
    L = len(lv)
    assert L == 1 << bits
    assert np.all(np.diff(lv) > 0)
    assert np.allclose(lv, -lv[::-1], atol=1e-12)                   # symmetric
    pdf = lambda x: math.exp(-x * x / 2) / math.sqrt(2 * math.pi)
    edges = [-np.inf] + [(lv[j] + lv[j + 1]) / 2 for j in range(L - 1)] + [np.inf]
    for j in range(L):
        m, _ = integrate.quad(lambda x: x * pdf(x), edges[j], edges[j + 1])
        p, _ = integrate.quad(pdf, edges[j], edges[j + 1])
        assert abs(m / p - lv[j]) < 1e-9, (j, m / p, lv[j])    # each level is its cell's mean
    # more levels, less distortion
    def mse(levels):
        e = [-np.inf] + [(levels[j] + levels[j + 1]) / 2 for j in range(len(levels) - 1)] + [np.inf]
        return sum(integrate.quad(lambda x, c=c: (x - c) ** 2 * pdf(x), e[j], e[j + 1])[0]
                   for j, c in enumerate(levels))
    assert mse(lv) < mse(turbo.lloyd_max(bits - 1))


def test_pack_by_hand():
    # 3-bit codes 0..7, LSB first: bits 000 100 010 110 001 101 011 111
    # -> stream 0b...: byte0 = 0b10001000 = 0x88, byte1 = 0b11000110 = 0xc6, byte2 = 0xfa
    assert turbo.pack_codes(range(8), 3) == bytes([0x88, 0xC6, 0xFA])
    assert turbo.unpack_codes(bytes([0x88, 0xC6, 0xFA]), 8, 3).tolist() == list(range(8))
    assert turbo.pack_codes([1, 2, 3, 0], 2) == bytes([0b00111001])
    assert turbo.pack_codes([0xA, 0x5], 4) == bytes([0x5A])


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_norm_preserved_and_error_small(bits):
    rng = np.random.default_rng(bits)
    for scale in (1.0, 1e-3, 50.0):
        v = (rng.standard_normal(128) * scale).astype(np.float32)
        rec, codes, s, r = turbo.encode(v, bits)
        assert len(rec) == turbo.record_bytes(128, bits)
        vh = turbo.decode(rec, 128, bits)
        nv = np.linalg.norm(v.astype(np.float64))
        assert abs(np.linalg.norm(vh) / nv - 1) < 2e-7                 # exact up to the f32 of s
        # relative error of the direction within the quantiser's distortion
        assert np.linalg.norm(vh - v) / nv < {2: 0.45, 3: 0.25, 4: 0.14, 8: 0.01}[bits]


def test_zero_vector_and_scale_invariance():
    rec, codes, s, _ = turbo.encode(np.zeros(16, np.float32), 2)
    assert s == 0 and not codes.any() and np.array_equal(turbo.decode(rec, 16, 2), np.zeros(16))
    # codes depend on the direction only; s scales with the norm
    rng = np.random.default_rng(4)
    v = rng.standard_normal(64)
    _, c1, s1, _ = turbo.encode(v, 3)
    _, c2, s2, _ = turbo.encode(v * 8.0, 3)
    assert np.array_equal(c1, c2) and abs(s2 / s1 - 8.0) < 1e-12


def test_codes_minimise_distance_brute_force():
    # n = 4, 2 bits: among all 256 code vectors, the chosen one is closest to
    # the rotated unit vector (the per-coordinate nearest centroid is optimal)
    rng = np.random.default_rng(9)
    cents = turbo.centroids(4, 2)
    for _ in range(20):
        v = rng.standard_normal(4)
        _, codes, _, r = turbo.encode(v, 2)
        best = min(itertools.product(range(4), repeat=4),
                   key=lambda c: float(np.sum((r - cents[list(c)]) ** 2)))
        assert list(best) == codes.tolist()


@pytest.mark.parametrize("n", [64, 128, 256])
@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_library_levels_match_oracle(n, bits):
    # the library computes its level table on the host with its own
    # Lloyd-Max iteration; it must agree with the oracle's to f32 rounding
    import quantized_moe_decode_amd as q
    got = q.turbo_levels(n, bits).astype(np.float64)
    ref = turbo.centroids(n, bits)
    assert np.max(np.abs(got - ref) / np.abs(ref)) < 1e-7
    assert q.turbo_record_bytes(n, bits) == turbo.record_bytes(n, bits)
