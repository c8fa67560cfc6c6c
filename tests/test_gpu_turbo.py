"""GPU parity of the TurboQuant KV codec (turbo_encode / turbo_decode through
the C ABI) against the oracle.

Bars.  Codes: equal to the oracle's, except that a coordinate whose rotated
value lies within the f32 error bound of the kernel's arithmetic of the
threshold between two levels may take either of them (where floating point
decides an integer, the two sides compute the value in different precision:
float64 in the oracle, f32 in the kernel); such coordinates are counted and
must be rare.  The norm ratio s within 2e-6 relative.  Decoding: the GPU
decode of a record against the oracle's decode of the same record,
relative L2 <= 1e-5 per vector, and the decoded norm equal to the input's
within 1e-5 (the page's exact-norm property, up to f32).  Canary bands
around every output.
"""

import math

import numpy as np
import pytest

from oracle import turbo

from _parity import Guarded

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


def _vectors(n, count, seed):
    rng = np.random.default_rng(seed)
    V = rng.standard_normal((count, n)).astype(np.float32)
    V[0] = 0.0                              # zero vector
    V[1] = 0.0
    V[1, 3] = 2.5                           # one-hot: rotates to a flat vector
    V[2] = 1.0                              # constant: rotates to a spike
    V[3] *= np.float32(1e-20)               # tiny
    V[4] *= np.float32(1e15)                # huge
    V[5:9] = (V[5:9] * rng.uniform(0.1, 10, size=(4, 1))).astype(np.float32)
    return V


def _check_records(rows, ids, recs, dec, n, bits, specials=9):
    """Records recs[j] (and their GPU decodes dec[j]) of the vectors rows[j]
    (vector number ids[j]) against the oracle; returns (codes differing at a
    threshold, codes seen) over the vectors numbered past the special ones."""
    cents = turbo.centroids(n, bits)
    thr = (cents[:-1] + cents[1:]) / 2
    near, total = 0, 0
    for j, i in enumerate(ids):
        ref_rec, codes, s, r = turbo.encode(rows[j], bits)
        got_codes = turbo.unpack_codes(recs[j].tobytes(), n, bits)
        got_s = float(np.frombuffer(recs[j, -4:].tobytes(), dtype="<f4")[0])
        diff = np.nonzero(got_codes != codes)[0]
        if diff.size:
            # only where r is within the kernel's f32 error of a threshold
            # between the two levels
            bound = (math.log2(n) + 8) * 2.0 ** -24 * (np.abs(r).sum() / math.sqrt(n) + np.abs(r))
            for e in diff:
                a, b = sorted((int(codes[e]), int(got_codes[e])))
                assert b == a + 1, (i, e, codes[e], got_codes[e])
                assert abs(r[e] - thr[a]) <= bound[e], (i, e, r[e], thr[a], bound[e])
            if i >= specials:   # the special vectors rotate onto exact threshold ties
                near += diff.size
        if i >= specials:
            total += n
        if s == 0:
            assert got_s == 0 and not got_codes.any()
        else:
            assert abs(got_s / s - 1) <= 2e-6 or diff.size, (i, got_s, s)
        # decode of the GPU's own record, by the oracle, against the GPU decode
        ref_dec = turbo.decode(recs[j].tobytes(), n, bits)
        nr = np.linalg.norm(ref_dec)
        if nr == 0:
            assert not dec[j].any()
        else:
            assert np.linalg.norm(dec[j] - ref_dec) / nr <= 1e-5, i
            assert abs(np.linalg.norm(dec[j]) / np.linalg.norm(rows[j].astype(np.float64)) - 1) <= 1e-5, i
    return near, total


@pytest.mark.parametrize("n", [64, 128, 256])
@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_turbo_encode_decode_vs_oracle(q, n, bits):
    say("turbo n=%d bits=%d" % (n, bits))
    count = 300
    V = _vectors(n, count, n * 10 + bits)
    rec = q.turbo_record_bytes(n, bits)
    go = Guarded(torch, (count, rec), torch.uint8, guard=256)
    q.turbo_encode(torch.from_numpy(V).cuda(), bits, out=go.t)
    gv = Guarded(torch, (count, n), torch.float32)
    q.turbo_decode(go.t, n, bits, v=gv.t)
    torch.cuda.synchronize()
    go.check()
    gv.check()
    near, total = _check_records(V, range(count), go.t.cpu().numpy(),
                                 gv.t.cpu().numpy().astype(np.float64), n, bits)
    say("codes of random vectors differing at a threshold: %d of %d" % (near, total))
    assert near <= max(2, total // 10000)


@pytest.mark.parametrize("n", [64, 128, 256])
@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_turbo_search_paths_agree(q, n, bits):
    """The encoder's bucket-table search and its binary search over the
    thresholds give the same records, bit for bit (a ragged count: the last
    wave holds fewer vectors than it takes)."""
    say("turbo search paths n=%d bits=%d" % (n, bits))
    count = 4099
    V = torch.from_numpy(_vectors(n, count, 7 * n + bits)).cuda()
    a = q.turbo_encode(V, bits)
    try:
        q.lib.hfq4_debug_set_turbo_search(1)
        b = q.turbo_encode(V, bits)
    finally:
        q.lib.hfq4_debug_set_turbo_search(0)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("n,bits", [(64, 3), (128, 4), (256, 8)])
def test_turbo_strided_unaligned(q, n, bits):
    """Rows at a stride that is not a multiple of four floats, from a base
    that is not 16-byte aligned (the kernels' element-wise access): the same
    records and the same decoded values as the contiguous, aligned call."""
    say("turbo strided n=%d bits=%d" % (n, bits))
    count, ld = 777, n + 3
    V = torch.from_numpy(_vectors(n, count, 3 * n + bits)).cuda()
    big = torch.zeros(count * ld + 1, dtype=torch.float32, device="cuda")
    Vs = big[1:].view(count, ld)[:, :n]
    Vs.copy_(V)
    a = q.turbo_encode(V, bits)
    b = q.turbo_encode(Vs, bits)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    d = q.turbo_decode(a, n, bits)
    outb = torch.full((count * ld + 1,), 7.0, dtype=torch.float32, device="cuda")
    Ds = outb[1:].view(count, ld)[:, :n]
    q.turbo_decode(a, n, bits, v=Ds)
    torch.cuda.synchronize()
    assert torch.equal(d, Ds)
    gaps = outb[1:].view(count, ld)[:, n:]
    assert bool((gaps == 7.0).all()) and float(outb[0]) == 7.0


@pytest.mark.parametrize("n", [64, 128, 256])
def test_turbo_tiny_counts(q, n):
    """Calls with fewer vectors than a wave takes (1, 3, 17) against the
    oracle, and a call with none writes nothing."""
    bits = 4
    rec = q.turbo_record_bytes(n, bits)
    for count in (1, 3, 17):
        say("turbo tiny n=%d count=%d" % (n, count))
        V = np.random.default_rng(count * n).standard_normal((count, n)).astype(np.float32)
        go = Guarded(torch, (count, rec), torch.uint8, guard=256)
        q.turbo_encode(torch.from_numpy(V).cuda(), bits, out=go.t)
        gv = Guarded(torch, (count, n), torch.float32)
        q.turbo_decode(go.t, n, bits, v=gv.t)
        torch.cuda.synchronize()
        go.check()
        gv.check()
        near, _ = _check_records(V, range(count), go.t.cpu().numpy(),
                                 gv.t.cpu().numpy().astype(np.float64), n, bits, specials=0)
        assert near <= 2
    empty = torch.zeros((0, n), dtype=torch.float32, device="cuda")
    out = torch.full((rec,), 0x5A, dtype=torch.uint8, device="cuda")
    q.turbo_encode(empty, bits, out=out)
    torch.cuda.synchronize()
    assert bool((out == 0x5A).all())


def test_turbo_full_size_sampled(q):
    """The benchmarked workload, 2^21 vectors of 128 values (1 GiB of f32)
    at 4 bits in one call each way: 96 sampled records (the first, the
    last and random ones) against the oracle."""
    say("turbo full size n=128 bits=4")
    n, bits, count = 128, 4, 1 << 21
    g = torch.Generator(device="cuda")
    g.manual_seed(2024)
    V = torch.randn((count, n), dtype=torch.float32, device="cuda", generator=g)
    recs = q.turbo_encode(V, bits)
    dec = q.turbo_decode(recs, n, bits)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    idx = np.unique(np.concatenate([[0, 1, count - 2, count - 1], rng.integers(0, count, 92)]))
    it = torch.from_numpy(idx).cuda()
    near, total = _check_records(V[it].cpu().numpy(), idx, recs[it].cpu().numpy(),
                                 dec[it].cpu().numpy().astype(np.float64), n, bits, specials=0)
    say("sampled codes differing at a threshold: %d of %d" % (near, total))
    assert near <= 2


def test_turbo_refusals(q):
    v = torch.zeros((4, 96), dtype=torch.float32, device="cuda")
    with pytest.raises(q.Hfq4Error):
        q.turbo_encode(v, 4)                                  # n = 96 unsupported
    v = torch.zeros((4, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(q.Hfq4Error):
        q.turbo_encode(v, 5)                                  # 5 bits unsupported
    out = torch.empty(10, dtype=torch.uint8, device="cuda")
    with pytest.raises(q.Hfq4Error):
        q.turbo_encode(v, 4, out=out)                         # too small
