"""Comparison helpers for the GPU parity tests (no method arithmetic here:
expected values come from the oracle).

Routing near-ties.  The oracle's logits are float64; the kernels sum each
logit in f32.  Where floating point decides the selection, both sides take
the decision in the kernels' precision: the oracle selects on its float64
logits rounded to f32.  The kernels' own f32 rounding can still move a logit
by up to the f32 summation error bound

    tau[e] = (n + 1) * 2^-24 * (sum_i |Wr[e, i] * x[i]| + |bias[e]|),

n being the longest chain of roundings any logit goes through in the
kernels: the one-wave-per-row router sums d/64 products per lane and then
64 lanes in 6 levels, the matrix-core router 4 products per step over d/16
elements per wave (at most d/16 roundings) and then 4 waves and 4 K-splits,
and the bias adds one: n = d/16 + 8 bounds both.  Two experts whose oracle
logits are closer than tau[a] + tau[c] may therefore legitimately come out
in either order.  Such tokens are counted ("tie-ambiguous"), the GPU's
selection must still be a valid top-k under that bound, and the seeded
cases are required to contain none.
"""

import numpy as np

from oracle import hfq4, moe
import synth

REL_L2_TOL = 2e-3          # layer output, per token (the stated bar)
WTS_ATOL = 1e-5            # routing weights, absolute
WTS_SUM_TOL = 1e-6         # |sum of a token's weights - 1|
U32 = 2.0 ** -24           # f32 unit roundoff


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def logit_tol(Wr, x, bias=None):
    """Per-logit f32 error bound tau [B, E] (see the module docstring)."""
    Wr = np.asarray(Wr, dtype=np.float64)
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    n = Wr.shape[1] / 16.0 + 8.0
    mag = np.abs(x) @ np.abs(Wr).T
    if bias is not None:
        mag = mag + np.abs(np.asarray(bias, dtype=np.float64))
    return (n + 1.0) * U32 * mag


def routing_valid(sel, logits, k, tau):
    """Is `sel` (k expert ids, in order) a top-k of `logits` (float64) when
    two logits closer than tau[a] + tau[c] may come in either order?"""
    sel = [int(e) for e in sel]
    E = len(logits)
    if len(sel) != k or len(set(sel)) != k or min(sel) < 0 or max(sel) >= E:
        return False
    for a, c in zip(sel, sel[1:]):          # order: non-increasing up to ties
        if logits[a] < logits[c] - (tau[a] + tau[c]):
            return False
    chosen = set(sel)
    for u in range(E):                      # no unselected expert strictly better
        if u in chosen:
            continue
        for s in sel:
            if logits[u] > logits[s] + (tau[u] + tau[s]):
                return False
    return True


def check_routing(idx_gpu, wts_gpu, logits64, k, tau):
    """Compare GPU routing with the oracle's.  Returns the number of
    tie-ambiguous tokens (GPU selection differs from the oracle's only
    inside the f32 bound tau [B, E]); raises AssertionError otherwise."""
    idx_gpu = np.asarray(idx_gpu)
    wts_gpu = np.asarray(wts_gpu, dtype=np.float64)
    tau = np.atleast_2d(tau)
    amb = 0
    for b in range(idx_gpu.shape[0]):
        l = logits64[b]
        ref = moe.topk_lower_index(l.astype(np.float32), k)
        got = idx_gpu[b].tolist()
        if got != ref:
            assert routing_valid(got, l, k, tau[b]), "token %d: gpu %s oracle %s" % (b, got, ref)
            amb += 1
        w_ref = moe.softmax_renorm(l, got)
        assert np.max(np.abs(wts_gpu[b] - w_ref)) <= WTS_ATOL, (b, wts_gpu[b], w_ref)
        assert abs(wts_gpu[b].sum() - 1.0) <= WTS_SUM_TOL, (b, wts_gpu[b].sum() - 1.0)
    return amb


def check_logits(logits_gpu, logits64, tau):
    """GPU f32 logits within the f32 summation bound of the float64 ones."""
    d = np.abs(np.asarray(logits_gpu, dtype=np.float64) - logits64)
    assert np.all(d <= tau), float(np.max(d / np.maximum(tau, 1e-300)))


class ExpertCache:
    """Oracle-quantized experts of a device-drawn layer, regenerated on
    demand from the seeded generator (only selected experts are drawn)."""

    def __init__(self, torch, device, seed, layer_id, d, F):
        self.t, self.dev, self.seed, self.layer, self.d, self.F = torch, device, seed, layer_id, d, F
        self.cache = {}

    def f32(self, e):
        g, u, dn = synth.expert_f32(self.t, self.dev, self.seed, self.layer, e, self.d, self.F)
        return g.cpu().numpy(), u.cpu().numpy(), dn.cpu().numpy()

    def __call__(self, e):
        if e not in self.cache:
            g, u, dn = self.f32(e)
            self.cache[e] = moe.PackedExpert.from_f32(g, u, dn)
        return self.cache[e]


def oracle_layer_check(x, Wr, bias, experts, k, idx_gpu, wts_gpu, y_gpu, residual=None):
    """Full check of one layer call: routing (with tie handling) and the
    per-token rel-L2 of y.  Returns (max rel-L2, n ambiguous)."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    logits = moe.router_logits(Wr, x, bias)
    amb = check_routing(idx_gpu, wts_gpu, logits, k, logit_tol(Wr, x, bias))
    # evaluate the oracle on the GPU's (validated) selection
    _, _, y_ref, _ = moe.moe_layer(x, Wr, experts, k, bias, idx=np.asarray(idx_gpu))
    if residual is not None:
        y_ref = y_ref + np.atleast_2d(np.asarray(residual, dtype=np.float64))
    errs = [rel_l2(y_gpu[b], y_ref[b]) for b in range(x.shape[0])]
    return max(errs), amb


# ------------------------------------------------------------ canary bands

CANARY_WORD = 0x7FC0DEAD        # a quiet-NaN pattern no kernel writes
GUARD = 64                      # elements of canary on each side (256 B for 4-byte types)


class Guarded:
    """A device tensor of `shape` with `guard` canary elements before and
    after it in one allocation (the inside starts 256-byte aligned when
    guard * element size is a multiple of 256).  `.t` is the inside, filled
    with the canary too unless `zero` (workspaces start zeroed); `check()`
    after the calls asserts that no kernel wrote outside it."""

    def __init__(self, torch, shape, dtype, device="cuda", guard=GUARD, zero=False):
        self.torch = torch
        shape = (shape,) if isinstance(shape, int) else tuple(shape)
        self.n = int(np.prod(shape))
        self.esize = torch.empty((), dtype=dtype).element_size()
        self.guard = guard
        self.full = torch.empty(self.n + 2 * guard, dtype=dtype, device=device)
        if self.esize == 4:
            self.full.view(torch.int32).fill_(CANARY_WORD)
        else:
            self.full.view(torch.uint8).fill_(0xA5)
        self.t = self.full[guard:guard + self.n].view(*shape)
        if zero:
            self.t.zero_()

    def check(self):
        raw = self.full.view(self.torch.uint8).cpu().numpy()
        g = self.guard * self.esize
        ref = np.empty(g, dtype=np.uint8)
        if self.esize == 4:
            ref.view(np.uint32)[:] = CANARY_WORD
        else:
            ref[:] = 0xA5
        head, tail = raw[:g], raw[g + self.n * self.esize:]
        assert np.array_equal(head, ref), "a kernel wrote before the buffer"
        assert tail.size == g and np.array_equal(tail, ref), "a kernel wrote past the buffer"
