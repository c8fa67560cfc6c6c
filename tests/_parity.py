"""Comparison helpers for the GPU parity tests (no method arithmetic here:
expected values come from the oracle)."""

import numpy as np

from oracle import hfq4, moe
import synth

REL_L2_TOL = 2e-3          # layer output, per token (the stated bar)
WTS_ATOL = 1e-5            # routing weights, absolute
TIE_REL = 1e-4             # logit gap below which either order is accepted


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def tie_tol(l, rel=TIE_REL):
    return rel * max(1.0, abs(float(l)))


def routing_valid(sel, logits, k, rel=TIE_REL):
    """Is `sel` (k expert ids, in order) a top-k of `logits` (float64) when
    logits closer than the tie tolerance may come in either order?"""
    sel = [int(e) for e in sel]
    E = len(logits)
    if len(sel) != k or len(set(sel)) != k or min(sel) < 0 or max(sel) >= E:
        return False
    for a, c in zip(sel, sel[1:]):          # order: non-increasing up to ties
        if logits[a] < logits[c] - tie_tol(logits[c], rel):
            return False
    chosen = set(sel)
    worst = min(logits[s] for s in sel)
    for u in range(E):                      # no unselected expert strictly better
        if u not in chosen and logits[u] > worst + tie_tol(worst, rel):
            return False
    return True


def check_routing(idx_gpu, wts_gpu, logits64, k):
    """Compare GPU routing with the oracle's.  Returns the number of
    tie-ambiguous tokens (GPU order differs from the oracle's only inside
    the tie tolerance); raises AssertionError otherwise."""
    idx_gpu = np.asarray(idx_gpu)
    wts_gpu = np.asarray(wts_gpu, dtype=np.float64)
    amb = 0
    for b in range(idx_gpu.shape[0]):
        l = logits64[b]
        ref = moe.topk_lower_index(l.astype(np.float32), k)
        got = idx_gpu[b].tolist()
        if got != ref:
            assert routing_valid(got, l, k), "token %d: gpu %s oracle %s" % (b, got, ref)
            amb += 1
        w_ref = moe.softmax_renorm(l, got)
        assert np.max(np.abs(wts_gpu[b] - w_ref)) <= WTS_ATOL, (b, wts_gpu[b], w_ref)
        assert abs(wts_gpu[b].sum() - 1.0) <= 1e-6 * k
    return amb


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
    amb = check_routing(idx_gpu, wts_gpu, logits, k)
    # evaluate the oracle on the GPU's (validated) selection
    _, _, y_ref, _ = moe.moe_layer(x, Wr, experts, k, bias, idx=np.asarray(idx_gpu))
    if residual is not None:
        y_ref = y_ref + np.atleast_2d(np.asarray(residual, dtype=np.float64))
    errs = [rel_l2(y_gpu[b], y_ref[b]) for b in range(x.shape[0])]
    return max(errs), amb
