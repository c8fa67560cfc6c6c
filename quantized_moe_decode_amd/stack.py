"""Decode through a stack of MoE layers by chaining C-ABI calls.

Per layer (a reading: the pages give no layer composition):
    t  = x + D x          (hfq4_gemv with the residual, when the layer has a
                           dense HFQ4 matrix D)
    x' = t + MoE(t)       (moe_layer_decode with the residual)
Buffers ping-pong between two vectors per token batch so that no call's
output overlaps its input.  Everything is enqueued on the current stream and
can be captured in a HIP graph.  Layers whose experts live in pinned host
memory (HFQ4_LAYER_HOST_MAPPED) run through the same kernels; their weight
reads cross PCIe (hipfire expert-offload explainer, section "PCIe 直通").
"""

import synth

from . import hfq4_gemv, hfq4_pack, moe_layer_decode, moe_workspace_bytes, new_workspace
from .synthetic import build_layer


class Stack:
    def __init__(self, layers, dense, k, batch, device="cuda"):
        import torch
        self.layers = layers          # list of MoeLayer (with Wr)
        self.dense = dense            # list of packed HFQ4 d x d tensors, or None entries
        self.k = k
        self.batch = batch
        d = layers[0].d
        self.d = d
        self.buf = [torch.empty((batch, d), dtype=torch.float32, device=device) for _ in range(2)]
        # one workspace serves every layer: size it for the largest need
        # (host-mapped layers also stage their selected down matrices)
        big = max(layers, key=lambda L: moe_workspace_bytes(L, batch, k))
        self.ws = new_workspace(big, batch, k, device)
        self.idx = torch.empty((batch, k), dtype=torch.int32, device=device)
        self.wts = torch.empty((batch, k), dtype=torch.float32, device=device)

    def step(self, x, capture=None):
        """One decode step of the token batch x [batch, d]; returns the tensor
        holding the output.  With capture (a list), every layer appends
        (input to the MoE layer, output, idx, wts) copies (for checks; not
        for timing)."""
        cur = x
        flip = 0
        for li, L in enumerate(self.layers):
            D = self.dense[li] if self.dense is not None else None
            if D is not None:
                t = self.buf[flip]
                hfq4_gemv(D, self.d, self.d, cur, residual=cur, y=t)
                flip ^= 1
            else:
                t = cur
            out = self.buf[flip]
            moe_layer_decode(L, t, self.k, self.ws, residual=t, y=out, idx=self.idx, wts=self.wts)
            flip ^= 1
            cur = out
            if capture is not None:
                capture.append((t.clone(), out.clone(), self.idx.clone(), self.wts.clone()))
        return cur


def build_stack(torch, seed, n_layers, E, d, F, k, batch, dense=True, host_from=None,
                device="cuda", bias=None):
    """Synthetic stack: layer l draws its experts/router with layer id l and,
    when dense, a d x d HFQ4 matrix.  Layers l >= host_from keep their experts
    in pinned host memory."""
    layers, dmats = [], []
    for l in range(n_layers):
        host = host_from is not None and l >= host_from
        layers.append(build_layer(torch, seed, l, E, d, F, device=device, bias=bias,
                                  host_mapped=host))
        if dense:
            w = synth.dense_f32(torch, device, seed, l, d)
            dmats.append(hfq4_pack(w))
            del w
        else:
            dmats.append(None)
    return Stack(layers, dmats if dense else None, k, batch, device)
