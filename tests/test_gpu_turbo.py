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
    recs = go.t.cpu().numpy()
    dec = gv.t.cpu().numpy().astype(np.float64)
    cents = turbo.centroids(n, bits)
    thr = (cents[:-1] + cents[1:]) / 2
    near, total = 0, 0
    for i in range(count):
        ref_rec, codes, s, r = turbo.encode(V[i], bits)
        got_codes = turbo.unpack_codes(recs[i].tobytes(), n, bits)
        got_s = float(np.frombuffer(recs[i, -4:].tobytes(), dtype="<f4")[0])
        diff = np.nonzero(got_codes != codes)[0]
        if diff.size:
            # only where r is within the kernel's f32 error of a threshold
            # between the two levels
            bound = (math.log2(n) + 8) * 2.0 ** -24 * (np.abs(r).sum() / math.sqrt(n) + np.abs(r))
            for j in diff:
                a, b = sorted((int(codes[j]), int(got_codes[j])))
                assert b == a + 1, (i, j, codes[j], got_codes[j])
                assert abs(r[j] - thr[a]) <= bound[j], (i, j, r[j], thr[a], bound[j])
            if i >= 9:   # the special vectors above rotate onto exact threshold ties
                near += diff.size
        if i >= 9:
            total += n
        if s == 0:
            assert got_s == 0 and not got_codes.any()
        else:
            assert abs(got_s / s - 1) <= 2e-6 or diff.size, (i, got_s, s)
        # decode of the GPU's own record, by the oracle, against the GPU decode
        ref_dec = turbo.decode(recs[i].tobytes(), n, bits)
        nr = np.linalg.norm(ref_dec)
        if nr == 0:
            assert not dec[i].any()
        else:
            assert np.linalg.norm(dec[i] - ref_dec) / nr <= 1e-5, i
            assert abs(np.linalg.norm(dec[i]) / np.linalg.norm(V[i].astype(np.float64)) - 1) <= 1e-5, i
    say("codes of random vectors differing at a threshold: %d of %d" % (near, total))
    assert near <= max(2, total // 10000)


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
