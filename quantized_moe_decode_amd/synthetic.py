"""Seeded synthetic MoE layers on the device (weights drawn by `synth`,
packed by hfq4_pack).  Used by the benchmark and the GPU tests; draws no
numbers itself and computes nothing beyond packing.
"""

import synth

from . import MoeLayer, hfq4_pack, hfq4_packed_bytes, Hfq4Error, HFQ4_E_INVALID


def build_layer(torch, seed, layer_id, E, d, F, device="cuda", router=True, bias=None,
                host_mapped=False, wstd=0.02, rstd=0.02):
    """A full layer: E experts of gate [F, d], up [F, d], down [d, F] HFQ4,
    router Wr [E, d] f32 (optional) and optional bias [E].  With
    host_mapped the expert buffers are pinned host memory (packed on the
    device, then copied)."""
    gb = hfq4_packed_bytes(F, d)
    db = hfq4_packed_bytes(d, F)
    gate = torch.empty(E * gb, dtype=torch.uint8, device=device)
    up = torch.empty(E * gb, dtype=torch.uint8, device=device)
    down = torch.empty(E * db, dtype=torch.uint8, device=device)
    bad = torch.zeros(1, dtype=torch.int32, device=device)
    for e in range(E):
        g, u, dn = synth.expert_f32(torch, device, seed, layer_id, e, d, F, wstd)
        hfq4_pack(g, out=gate[e * gb:(e + 1) * gb], bad=bad)
        hfq4_pack(u, out=up[e * gb:(e + 1) * gb], bad=bad)
        hfq4_pack(dn, out=down[e * db:(e + 1) * db], bad=bad)
    if int(bad.item()):
        raise Hfq4Error(HFQ4_E_INVALID, "non-finite synthetic weights")
    if host_mapped:
        hg = torch.empty(gate.numel(), dtype=torch.uint8, pin_memory=True)
        hu = torch.empty(up.numel(), dtype=torch.uint8, pin_memory=True)
        hd = torch.empty(down.numel(), dtype=torch.uint8, pin_memory=True)
        hg.copy_(gate)
        hu.copy_(up)
        hd.copy_(down)
        del gate, up, down
        gate, up, down = hg, hu, hd
    Wr = synth.router_f32(torch, device, seed, layer_id, E, d, rstd) if router else None
    if bias is not None:
        bias = torch.as_tensor(bias, dtype=torch.float32, device=device)
    return MoeLayer(gate, up, down, E, d, F, Wr=Wr, bias=bias, host_mapped=host_mapped)


def tiny_layer(torch, seed=0, device="cuda"):
    """The tiny layer (d=256, F=128, E=8) drawn on the host; returns
    (MoeLayer, host dict of the f32 draws)."""
    L = synth.tiny_layer(seed)
    d, F, E = L["d"], L["F"], L["E"]
    gb = hfq4_packed_bytes(F, d)
    db = hfq4_packed_bytes(d, F)
    gate = torch.empty(E * gb, dtype=torch.uint8, device=device)
    up = torch.empty(E * gb, dtype=torch.uint8, device=device)
    down = torch.empty(E * db, dtype=torch.uint8, device=device)
    for e in range(E):
        hfq4_pack(torch.from_numpy(L["gate"][e]).to(device), out=gate[e * gb:(e + 1) * gb])
        hfq4_pack(torch.from_numpy(L["up"][e]).to(device), out=up[e * gb:(e + 1) * gb])
        hfq4_pack(torch.from_numpy(L["down"][e]).to(device), out=down[e * db:(e + 1) * db])
    Wr = torch.from_numpy(L["Wr"]).to(device)
    return MoeLayer(gate, up, down, E, d, F, Wr=Wr), L
