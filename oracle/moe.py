"""Top-k routed MoE layer decode (oracle; test infrastructure).

Steps, in the order the decode path takes them:

1. router logits  l[e] = sum_i Wr[e, i] x[i] + bias[e]          (float64)
2. top-k selection: the k largest logits, ties to the lower expert index
   (top-8 per token: hipfire expert-offload explainer, section "125GB 的 MoE
   模型，为什么 32GB 显卡也有得跑？"; the tie rule is a reading)
3. routing weights: full softmax over all E logits, then the k selected
   probabilities renormalised to sum 1 (reading: softmax, then renormalised
   top-k)
4. per selected expert e (gate/up/down tensors: Strata user report, section
   "3. 模型与引擎"):  g = Wg_e x,  u = Wu_e x,  h = SiLU(g) * u,
   y_e = Wd_e h, with every W an HFQ4 matrix dequantized exactly
   (reading: SiLU(gate) * up)
5. combine  y = sum_j w_j y_{e_j}, j in selection order.

A token batch is B independent tokens: grouping tokens by expert is a
speed-up only and does not appear here.

The stacked and host-mapped compositions (stack_step) follow readings, not
passages: parity unpinned against the pages.
"""

import numpy as np

from . import hfq4


# ---------------------------------------------------------------- routing

def router_logits(Wr, x, bias=None):
    """l[b, e] = sum_i Wr[e, i] * x[b, i] + bias[e] in float64.  x: [d] or [B, d]."""
    Wr = np.asarray(Wr, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    l = x @ Wr.T
    if bias is not None:
        l = l + np.asarray(bias, dtype=np.float64)
    return l


def topk_lower_index(logits, k):
    """Brute-force top-k of one token's logits: k passes, each scanning
    e = 0..E-1 over the not-yet-selected experts and keeping the first
    strict maximum, so equal logits go to the lower index.  Returns a list
    of k expert indices in selection order (logit descending, index
    ascending)."""
    logits = [float(v) for v in np.asarray(logits).reshape(-1)]
    E = len(logits)
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    taken = [False] * E
    out = []
    for _ in range(k):
        best = -1
        for e in range(E):
            if taken[e]:
                continue
            if best < 0 or logits[e] > logits[best]:
                best = e
        taken[best] = True
        out.append(best)
    return out


def softmax_renorm(logits, idx):
    """Full softmax p = exp(l - max l) / sum exp(l - max l) over all E
    experts, then w_j = p[idx_j] / sum_sel p.  float64."""
    l = np.asarray(logits, dtype=np.float64).reshape(-1)
    p = np.exp(l - l.max())
    p = p / p.sum()
    sel = p[np.asarray(idx, dtype=np.int64)]
    return sel / sel.sum()


def route(Wr, x, k, bias=None, logit_dtype=np.float64):
    """Route a batch: returns (idx int32 [B, k], wts float64 [B, k], logits
    float64 [B, E]).  With logit_dtype=np.float32 the selection is taken on
    the float64 logits rounded to f32 (the kernel's precision); the weights
    always come from the float64 logits."""
    x = np.atleast_2d(np.asarray(x))
    l = router_logits(Wr, x, bias)
    B = l.shape[0]
    idx = np.zeros((B, k), dtype=np.int32)
    wts = np.zeros((B, k), dtype=np.float64)
    for b in range(B):
        ls = l[b].astype(logit_dtype)
        sel = topk_lower_index(ls, k)
        idx[b] = sel
        wts[b] = softmax_renorm(l[b], sel)
    return idx, wts, l


# ---------------------------------------------------------------- experts

def silu(g):
    """SiLU(g) = g / (1 + exp(-g)), float64."""
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(-g))


class PackedExpert:
    """One expert's three HFQ4 matrices: gate [F, d], up [F, d], down [d, F]."""

    def __init__(self, gate, up, down, d, F):
        self.gate = np.asarray(gate, dtype=np.uint8).reshape(-1)
        self.up = np.asarray(up, dtype=np.uint8).reshape(-1)
        self.down = np.asarray(down, dtype=np.uint8).reshape(-1)
        self.d = d
        self.F = F
        assert self.gate.size == hfq4.packed_bytes(F, d)
        assert self.up.size == hfq4.packed_bytes(F, d)
        assert self.down.size == hfq4.packed_bytes(d, F)

    @classmethod
    def from_f32(cls, gate, up, down):
        """Quantize f32 matrices with the oracle quantizer."""
        F, d = np.shape(gate)
        return cls(hfq4.quantize_rows(gate), hfq4.quantize_rows(up),
                   hfq4.quantize_rows(down), d, F)


def expert_forward(ex, x):
    """y_e = Wd (SiLU(Wg x) * (Wu x)) for one token x [d] -> float64 [d]."""
    g = hfq4.matvec(ex.gate, ex.F, ex.d, x)
    u = hfq4.matvec(ex.up, ex.F, ex.d, x)
    h = silu(g) * u
    return hfq4.matvec(ex.down, ex.d, ex.F, h)


def combine(outputs, wts):
    """y = sum_j wts[j] * outputs[j], in j order, float64."""
    y = np.zeros_like(np.asarray(outputs[0], dtype=np.float64))
    for yj, wj in zip(outputs, wts):
        y = y + float(wj) * np.asarray(yj, dtype=np.float64)
    return y


def moe_layer(x, Wr, experts, k, bias=None, logit_dtype=np.float64, idx=None):
    """One MoE layer over a batch x [B, d] (or [d]).

    experts: a mapping/callable e -> PackedExpert (only the selected experts
    are ever requested).  If idx is given ([B, k]) it replaces the selection
    (used to re-evaluate an alternative, equally valid selection); the
    weights are then recomputed for that selection, in its order: the
    renormalised softmax of the float64 logits of the given experts.
    Returns (idx int32 [B, k], wts float64 [B, k], y float64 [B, d], logits).
    """
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    get = experts if callable(experts) else experts.__getitem__
    r_idx, r_wts, logits = route(Wr, x, k, bias, logit_dtype)
    if idx is not None:
        idx = np.asarray(idx, dtype=np.int32).reshape(r_idx.shape)
        r_wts = np.stack([softmax_renorm(logits[b], idx[b]) for b in range(x.shape[0])])
        r_idx = idx
    B, d = x.shape
    y = np.zeros((B, d), dtype=np.float64)
    for b in range(B):
        outs = [expert_forward(get(int(e)), x[b]) for e in r_idx[b]]
        y[b] = combine(outs, r_wts[b])
    return r_idx, r_wts, y, logits


def stack_step(x, layers, k, trace=None):
    """One decode step through a stack (reading; parity unpinned against the
    pages).  layers: iterable of dicts with keys 'Wr', 'experts', optional
    'bias', optional 'dense' (packed HFQ4 d x d).  Per layer:
    t = x + D x (when a dense matrix is present), then x' = t + MoE(t).
    With trace (a list), every layer appends (x', idx, wts, logits)."""
    x = np.asarray(x, dtype=np.float64).reshape(-1)
    d = x.size
    for L in layers:
        if L.get("dense") is not None:
            x = x + hfq4.matvec(L["dense"], d, d, x)
        idx, wts, y, logits = moe_layer(x, L["Wr"], L["experts"], k, L.get("bias"))
        x = x + y[0]
        if trace is not None:
            trace.append((x.copy(), idx[0], wts[0], logits[0]))
    return x
