"""C-ABI checks that need no GPU: the library loads, exports every entry
point include/hfq4moe.h declares, and refuses bad arguments on the host
before touching a device.

No call here ever reaches a kernel launch: every call either fails host
validation or has the device check forced to refuse (hfq4_debug_set_arch),
so the file is safe to run on a machine with a GPU as well.
"""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hfq4moe.h")


@pytest.fixture(scope="module")
def q():
    import quantized_moe_decode_amd as q
    q.lib.hfq4_debug_set_arch(b"gfx942")   # any call that passes validation is refused
    yield q
    q.lib.hfq4_debug_set_arch(b"")


def header_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


def test_header_declares_the_boundary():
    fns = header_functions()
    for name in ["hfq4_pack", "hfq4_gemv", "moe_route_topk", "moe_expert_decode",
                 "moe_layer_decode", "moe_workspace_bytes", "hfq4_packed_bytes", "hfq4_last_error"]:
        assert name in fns


def test_every_declared_symbol_is_exported(q):
    out = subprocess.run(["nm", "-D", "--defined-only", q.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    missing = [f for f in header_functions() if f not in exported]
    assert not missing, missing
    assert set(q.EXPORTS) <= exported


def test_no_oracle_import_in_product():
    # the product path never imports the oracle
    pkg = os.path.join(ROOT, "quantized_moe_decode_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith(".py"):
                src = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b", src, flags=re.M), f


def test_packed_bytes(q):
    assert q.hfq4_packed_bytes(512, 2048) == 557056
    assert q.hfq4_packed_bytes(2048, 512) == 557056
    assert q.hfq4_packed_bytes(1, 128) == 136
    assert q.hfq4_packed_bytes(0, 7) == 0
    with pytest.raises(q.Hfq4Error) as e:
        q.hfq4_packed_bytes(1, 0)
    assert e.value.code == q.HFQ4_E_INVALID and "K" in str(e.value)


P = ctypes.c_void_p
A = 0x7F0000000000        # fake, 256-aligned; never dereferenced


def test_pack_validation(q):
    L = q.lib
    assert L.hfq4_pack(P(A), 4, 0, 4, P(A + 4096), 10 ** 6, None, None) == q.HFQ4_E_INVALID
    assert L.hfq4_pack(P(A), 4, 256, 100, P(A + 4096), 10 ** 6, None, None) == q.HFQ4_E_INVALID
    r = L.hfq4_pack(P(A), 4, 256, 256, P(A + 8192), 100, None, None)
    assert r == q.HFQ4_E_INVALID and "needs 544 bytes, got 100" in q.last_error()
    assert L.hfq4_pack(P(A), 4, 256, 256, P(A + 8193), 544, None, None) == q.HFQ4_E_ALIGN
    assert L.hfq4_pack(P(A), 4, 256, 256, P(A + 16), 544, None, None) == q.HFQ4_E_INVALID  # overlap
    assert L.hfq4_pack(P(A), 4, 256, 256, P(A + 8192), 544, None, None) == q.HFQ4_E_DEVICE
    assert "gfx950" in q.last_error()
    assert L.hfq4_pack(None, 0, 256, 256, None, 0, None, None) == q.HFQ4_OK  # empty is a no-op


def test_gemv_validation(q):
    L = q.lib
    W, x, y = P(A), P(A + (1 << 24)), P(A + (1 << 25))
    assert L.hfq4_gemv(W, 8, 0, x, 256, 1, None, 0, y, 8, None) == q.HFQ4_E_UNSUPPORTED
    assert L.hfq4_gemv(W, 8, 256, x, 256, 0, None, 0, y, 8, None) == q.HFQ4_E_INVALID
    assert L.hfq4_gemv(W, 8, 256, x, 256, 17, None, 0, y, 8, None) == q.HFQ4_E_INVALID
    assert L.hfq4_gemv(W, 8, 256, x, 255, 1, None, 0, y, 8, None) == q.HFQ4_E_ALIGN
    assert L.hfq4_gemv(W, 8, 256, P(A + (1 << 24) + 4), 256, 1, None, 0, y, 8, None) == q.HFQ4_E_ALIGN
    assert L.hfq4_gemv(W, 8, 256, x, 256, 1, None, 0, P(A + (1 << 24) + 64), 8, None) == q.HFQ4_E_INVALID
    assert L.hfq4_gemv(W, 8, 256, x, 256, 1, None, 0, P(A + 64), 8, None) == q.HFQ4_E_INVALID  # y in W
    assert L.hfq4_gemv(W, 8, 256, x, 256, 1, None, 0, y, 4, None) == q.HFQ4_E_INVALID   # ldy < rows
    assert L.hfq4_gemv(W, 8, 256, x, 256, 1, None, 0, y, 8, None) == q.HFQ4_E_DEVICE


def test_route_validation(q):
    L = q.lib
    Wr, x, idx, wts, ws = P(A), P(A + (1 << 24)), P(A + (2 << 24)), P(A + (3 << 24)), P(A + (4 << 24))
    need = q.moe_route_workspace_bytes(256, 1)
    args = lambda E=256, d=2048, B=1, k=8, wsb=need, wsp=ws: (Wr, None, E, d, x, d, B, k, idx, wts, None,
                                                               wsp, wsb, None)
    assert L.moe_route_topk(*args(k=0)) == q.HFQ4_E_INVALID
    assert L.moe_route_topk(*args(E=4, k=8)) == q.HFQ4_E_INVALID
    assert L.moe_route_topk(*args(k=17)) == q.HFQ4_E_INVALID
    assert L.moe_route_topk(*args(E=2000)) == q.HFQ4_E_INVALID
    assert L.moe_route_topk(*args(d=2046)) == q.HFQ4_E_UNSUPPORTED
    assert L.moe_route_topk(*args(B=17)) == q.HFQ4_E_INVALID
    r = L.moe_route_topk(*args(wsb=need - 1))
    assert r == q.HFQ4_E_WORKSPACE and ("needs %d bytes, got %d" % (need, need - 1)) in q.last_error()
    assert L.moe_route_topk(*args(wsp=P(A + (4 << 24) + 16))) == q.HFQ4_E_ALIGN
    assert L.moe_route_topk(*args()) == q.HFQ4_E_DEVICE


def _layer(q, E=256, d=2048, F=512, gate=A, flags=0, sg=None):
    gb = q.hfq4_packed_bytes(F, d)
    db = q.hfq4_packed_bytes(d, F)
    return q.MoeLayerC(gate, A + (1 << 30), A + (2 << 30), E, d, F, sg or gb, gb, db, flags, 0)


def test_layer_validation(q):
    L = q.lib
    out = ctypes.c_size_t()
    by = ctypes.byref
    assert L.moe_workspace_bytes(by(_layer(q)), 1, 8, by(out)) == q.HFQ4_OK
    need = out.value
    assert L.moe_workspace_bytes(by(_layer(q, E=0)), 1, 8, by(out)) == q.HFQ4_E_INVALID
    assert L.moe_workspace_bytes(by(_layer(q, d=4096)), 1, 8, by(out)) == q.HFQ4_E_UNSUPPORTED
    assert L.moe_workspace_bytes(by(_layer(q, F=510)), 1, 8, by(out)) == q.HFQ4_E_UNSUPPORTED
    assert L.moe_workspace_bytes(by(_layer(q, sg=1000)), 1, 8, by(out)) == q.HFQ4_E_INVALID
    assert "557056" in q.last_error()
    assert L.moe_workspace_bytes(by(_layer(q, gate=A + 8)), 1, 8, by(out)) == q.HFQ4_E_ALIGN
    assert L.moe_workspace_bytes(by(_layer(q, flags=8)), 1, 8, by(out)) == q.HFQ4_E_INVALID
    x, idx, wts, y, ws = (P(A + (3 << 30)), P(A + (4 << 30)), P(A + (5 << 30)), P(A + (6 << 30)),
                          P(A + (7 << 30)))
    lay = by(_layer(q))
    dec = L.moe_expert_decode
    assert dec(lay, x, 2048, 1, idx, wts, 8, None, y, 2048, ws, need, None) == q.HFQ4_E_DEVICE
    assert dec(lay, x, 2048, 1, idx, wts, 8, None, y, 2048, ws, need - 4, None) == q.HFQ4_E_WORKSPACE
    assert dec(lay, x, 2048, 1, idx, wts, 0, None, y, 2048, ws, need, None) == q.HFQ4_E_INVALID
    assert dec(lay, x, 2048, 16, idx, wts, 16, None, y, 2048, ws, 1 << 30, None) == q.HFQ4_E_UNSUPPORTED
    assert dec(lay, x, 2048, 1, None, wts, 8, None, y, 2048, ws, need, None) == q.HFQ4_E_INVALID
    assert dec(lay, x, 2048, 1, idx, wts, 8, None, x, 2048, ws, need, None) == q.HFQ4_E_INVALID  # y == x
    assert dec(lay, x, 2046, 1, idx, wts, 8, None, y, 2048, ws, need, None) == q.HFQ4_E_ALIGN
    lay_dec = L.moe_layer_decode
    assert lay_dec(lay, None, None, x, 2048, 1, 8, idx, wts, None, y, 2048, ws, need, None) == q.HFQ4_E_INVALID
    assert lay_dec(lay, P(A + (8 << 30)), None, x, 2048, 1, 8, idx, wts, None, y, 2048, ws, need,
                   None) == q.HFQ4_E_DEVICE


def test_workspace_sizes_scale(q):
    lay = _layer(q)
    s1 = q.moe_workspace_bytes(type("L", (), {"c": lay})(), 1, 8)
    s16 = q.moe_workspace_bytes(type("L", (), {"c": lay})(), 16, 8)
    assert s16 > s1 >= 256 + 4 * 256 + 4 * 8 * 512


def test_device_refusal_names_arch(q):
    q.lib.hfq4_debug_set_arch(b"gfx90a")
    r = q.lib.moe_workspace_init(P(A), 1024, None)
    assert r == q.HFQ4_E_DEVICE and "gfx90a" in q.last_error()
    q.lib.hfq4_debug_set_arch(b"gfx942")


def test_noalloc_refuses_beyond_its_scratch(q):
    # a host-mapped one-token layer with F = 2048 and k = 16 stages 16 down
    # matrices of 2048 x 2048 (35.7 MB): beyond the fixed scratch, refused on
    # the host before any device work
    E, d, F, k = 64, 2048, 2048, 16
    gb = 2048 * 8 * 136
    L = q.MoeLayerC(16, 16, 16, E, d, F, gb, gb, gb, q.HFQ4_LAYER_HOST_MAPPED, 0)
    P = ctypes.c_void_p
    rc = q.lib.moe_layer_decode_noalloc(ctypes.byref(L), P(16), None, P(4096), d, 1, k,
                                        P(1 << 20), P(1 << 21), None, P(1 << 22), d, None, None)
    assert rc == q.HFQ4_E_WORKSPACE
    msg = q.last_error()
    assert "scratch" in msg and str(q.NOALLOC_SCRATCH_BYTES) in msg
    # within the scratch, validation passes and the (forced) device check refuses
    L = q.MoeLayerC(16, 16, 16, 256, 2048, 512, 557056, 557056, 557056, 0, 0)
    rc = q.lib.moe_layer_decode_noalloc(ctypes.byref(L), P(16), None, P(4096), 2048, 16, 8,
                                        P(1 << 20), P(1 << 21), None, P(1 << 22), 2048, None, None)
    assert rc == q.HFQ4_E_DEVICE


def test_turbo_validation(q):
    L = q.lib
    by = ctypes.byref
    sz = ctypes.c_size_t()
    assert L.turbo_record_bytes(96, 4, by(sz)) == q.HFQ4_E_UNSUPPORTED
    assert L.turbo_record_bytes(128, 5, by(sz)) == q.HFQ4_E_UNSUPPORTED
    assert L.turbo_record_bytes(128, 4, None) == q.HFQ4_E_INVALID
    assert L.turbo_record_bytes(128, 4, by(sz)) == 0 and sz.value == 68
    levels = (ctypes.c_float * 16)()
    assert L.turbo_levels(128, 4, None) == q.HFQ4_E_INVALID
    assert L.turbo_levels(128, 4, levels) == 0
    lv = list(levels)
    assert all(a < b for a, b in zip(lv, lv[1:]))
    n, bits, count, rec = 128, 4, 1000, 68
    v, out = A, A + (1 << 30)

    def enc(v=v, count=count, ldv=n, out=out, ob=rec * count, bits=bits):
        return L.turbo_encode(P(v) if v else None, count, n, ldv, bits, P(out), ob, None)

    assert enc(count=-1) == q.HFQ4_E_INVALID
    assert enc(count=0) == 0                      # nothing to do: no device is touched
    assert enc(v=0) == q.HFQ4_E_INVALID
    assert enc(ldv=n - 1) == q.HFQ4_E_INVALID
    assert enc(ob=rec * count - 1) == q.HFQ4_E_INVALID
    assert enc(v=A + 2) == q.HFQ4_E_ALIGN
    assert enc(out=A + 4 * 64) == q.HFQ4_E_INVALID   # the records would overlap v
    assert enc(bits=5) == q.HFQ4_E_UNSUPPORTED
    assert enc() == q.HFQ4_E_DEVICE

    def dec(inp=out, ib=rec * count, count=count, vv=v, ldv=n, bits=bits):
        return L.turbo_decode(P(inp) if inp else None, ib, count, n, bits, P(vv), ldv, None)

    assert dec(count=-1) == q.HFQ4_E_INVALID
    assert dec(count=0) == 0
    assert dec(inp=0) == q.HFQ4_E_INVALID
    assert dec(ldv=n - 1) == q.HFQ4_E_INVALID
    assert dec(ib=rec * count - 1) == q.HFQ4_E_INVALID
    assert dec(inp=out + 2) == q.HFQ4_E_ALIGN
    assert dec(vv=out + 64) == q.HFQ4_E_INVALID        # v would overlap the records
    assert dec(bits=8) == q.HFQ4_E_INVALID             # 132-byte records: 68000 bytes hold 515
    assert dec() == q.HFQ4_E_DEVICE
    assert L.hfq4_debug_set_turbo_search(1) == 0 and L.hfq4_debug_set_turbo_search(0) == 0
