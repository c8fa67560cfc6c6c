"""HBM expert cache over host-resident experts (argument marshalling and
buffer bookkeeping; the placement rule and every step of the decode run in
the library).

hipfire expert-offload explainer, section "放置算法：auto 自动放置…": fixed
weights first, then routed experts fill the device budget -- layer by layer
by default, or by a decode-heat ranking (the hot set) -- and what does not
fit stays in pinned host memory, read by the GPU kernel over PCIe (section
"PCIe 直通").  Strata user report, sections "1. Strata 是什么" and "5. 实测
速度": the most routed experts cached on the device, with the cache's hit
rate as the figure of merit.

A model here is a list of host-resident layers (MoeLayer with pinned
gate/up/down tensors and a router in HBM).  build_cache copies the experts
the placement marks resident into one HBM pool (gate | up | down per slot)
and gives every layer a pointer table: a resident expert's entry points at
its slot, the others at their pinned host bytes (mapped for the device).
"""

import numpy as np

from . import (HFQ4_PLACE_HOTSET, MoeLayerTableC, host_device_pointer, hfq4_packed_bytes,
               moe_place_experts, moe_route_topk, moe_route_workspace_bytes)


class TableLayer:
    """One layer reached through its pointer table (device int64 [E, 3]) and
    resident mask (device uint8 [E]); keeps the tensors it points into
    alive."""

    def __init__(self, ptr, resident, E, d, F, Wr, bias, keep):
        self.ptr, self.resident = ptr, resident
        self.E, self.d, self.F = E, d, F
        self.Wr, self.bias = Wr, bias
        self._keep = keep
        self.c = MoeLayerTableC(ptr.data_ptr(), resident.data_ptr(), E, d, F)

    def expert_bytes(self):
        return 2 * hfq4_packed_bytes(self.F, self.d) + hfq4_packed_bytes(self.d, self.F)


def routing_heat(torch, layers, xs, k):
    """Selection counts [len(layers), E] of each layer's router over the
    calibration tokens xs [N, d] (device), routed 16 at a time."""
    heat = np.zeros((len(layers), layers[0].E), dtype=np.uint64)
    ws = torch.zeros(moe_route_workspace_bytes(layers[0].E, 16), dtype=torch.uint8,
                     device=xs.device)
    for li, L in enumerate(layers):
        for t0 in range(0, xs.shape[0], 16):
            idx, _ = moe_route_topk(L.Wr, xs[t0:t0 + 16], k, bias=L.bias, ws=ws)
            heat[li] += torch.bincount(idx.view(-1).long(), minlength=L.E).cpu().numpy().astype(
                np.uint64)
    return heat


def build_cache(torch, layers, resident, device="cuda"):
    """HBM pool holding the experts marked resident ([len(layers), E]) and a
    TableLayer per layer.  Returns (table layers, pool tensor)."""
    E, d, F = layers[0].E, layers[0].d, layers[0].F
    gb, db = hfq4_packed_bytes(F, d), hfq4_packed_bytes(d, F)
    eb = 2 * gb + db
    n_res = int(resident.sum())
    pool = torch.empty(max(n_res, 1) * eb, dtype=torch.uint8, device=device)
    base = pool.data_ptr()
    slot = 0
    tables = []
    for li, L in enumerate(layers):
        hg, hu, hd = (host_device_pointer(t) for t in (L.gate, L.up, L.down))
        ptr = np.zeros((E, 3), dtype=np.uint64)
        for e in range(E):
            if resident[li, e]:
                o = slot * eb
                pool[o:o + gb].copy_(L.gate[e * gb:(e + 1) * gb], non_blocking=True)
                pool[o + gb:o + 2 * gb].copy_(L.up[e * gb:(e + 1) * gb], non_blocking=True)
                pool[o + 2 * gb:o + eb].copy_(L.down[e * db:(e + 1) * db], non_blocking=True)
                ptr[e] = (base + o, base + o + gb, base + o + 2 * gb)
                slot += 1
            else:
                ptr[e] = (hg + e * gb, hu + e * gb, hd + e * db)
        tptr = torch.from_numpy(ptr.view(np.int64)).to(device)
        tres = torch.from_numpy(np.ascontiguousarray(resident[li], dtype=np.uint8)).to(device)
        tables.append(TableLayer(tptr, tres, E, d, F, L.Wr, L.bias, (L, pool)))
    torch.cuda.synchronize()
    return tables, pool


def place_and_build(torch, layers, heat, budget_bytes, fixed_bytes, mode=HFQ4_PLACE_HOTSET,
                    device="cuda"):
    """Placement by the library's rule, then the cache.  Returns (tables,
    pool, resident, placed expert bytes)."""
    eb = layers[0].expert_bytes()
    resident, placed = moe_place_experts(mode, len(layers), layers[0].E, eb, fixed_bytes,
                                         budget_bytes, heat=heat)
    tables, pool = build_cache(torch, layers, resident, device)
    return tables, pool, resident, placed
