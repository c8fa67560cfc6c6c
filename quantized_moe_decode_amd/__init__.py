"""Python binding of libhfq4moe.so (HFQ4 top-k MoE decode on MI355X / gfx950).

Argument marshalling only: every step of the decode path runs in the HIP
kernels behind the C ABI (include/hfq4moe.h).  torch supplies device
memory and the current stream; nothing here computes.  If the shared
library is missing the import fails loudly -- there is no fallback.

Functions keep the C names: hfq4_packed_bytes, hfq4_pack, hfq4_gemv,
moe_route_workspace_bytes, moe_route_topk, moe_workspace_bytes,
moe_workspace_init, moe_expert_decode, moe_layer_decode.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhfq4moe.so")

HFQ4_OK = 0
HFQ4_E_INVALID = -1
HFQ4_E_ALIGN = -2
HFQ4_E_WORKSPACE = -3
HFQ4_E_DEVICE = -4
HFQ4_E_HIP = -5
HFQ4_E_UNSUPPORTED = -6
HFQ4_DEV_ERR_INDEX = 1
HFQ4_DEV_ERR_TIMEOUT = 2
HFQ4_DEV_ERR_NONFINITE = 4
HFQ4_LAYER_HOST_MAPPED = 1
MAX_BATCH = 16
MAX_TOPK = 16
MAX_EXPERTS = 1024

EXPORTS = [
    "hfq4_last_error", "hfq4_version", "hfq4_debug_set_arch", "hfq4_packed_bytes", "hfq4_pack",
    "hfq4_gemv", "moe_route_workspace_bytes", "moe_route_topk", "moe_workspace_bytes",
    "moe_workspace_init", "moe_expert_decode", "moe_layer_decode", "hfq4_host_device_pointer",
    "hfq4_debug_set_trace", "hfq4_debug_set_events",
]


class Hfq4Error(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("hfq4 status %d: %s" % (code, msg))
        self.code = code


class MoeLayerC(ctypes.Structure):
    _fields_ = [("gate", ctypes.c_void_p), ("up", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("E", ctypes.c_int64), ("d", ctypes.c_int64), ("F", ctypes.c_int64),
                ("stride_gate", ctypes.c_int64), ("stride_up", ctypes.c_int64),
                ("stride_down", ctypes.c_int64), ("flags", ctypes.c_uint32),
                ("reserved", ctypes.c_uint32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libhfq4moe.so not built at %s -- run quantized_moe_decode_amd.build "
                          "(no CPU fallback exists)" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    sig = {
        "hfq4_last_error": (ctypes.c_char_p, []),
        "hfq4_version": (I32, []),
        "hfq4_debug_set_arch": (I32, [ctypes.c_char_p]),
        "hfq4_packed_bytes": (I32, [I64, I64, ctypes.POINTER(SZ)]),
        "hfq4_pack": (I32, [P, I64, I64, I64, P, SZ, P, P]),
        "hfq4_gemv": (I32, [P, I64, I64, P, I64, I32, P, I64, P, I64, P]),
        "moe_route_workspace_bytes": (I32, [I64, I32, ctypes.POINTER(SZ)]),
        "moe_route_topk": (I32, [P, P, I64, I64, P, I64, I32, I32, P, P, P, P, SZ, P]),
        "moe_workspace_bytes": (I32, [ctypes.POINTER(MoeLayerC), I32, I32, ctypes.POINTER(SZ)]),
        "moe_workspace_init": (I32, [P, SZ, P]),
        "moe_expert_decode": (I32, [ctypes.POINTER(MoeLayerC), P, I64, I32, P, P, I32, P, P, I64,
                                    P, SZ, P]),
        "moe_layer_decode": (I32, [ctypes.POINTER(MoeLayerC), P, P, P, I64, I32, I32, P, P, P, P,
                                   I64, P, SZ, P]),
        "hfq4_host_device_pointer": (I32, [P, ctypes.POINTER(P)]),
        "hfq4_debug_set_trace": (I32, [P, SZ]),
        "hfq4_debug_set_events": (I32, [P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


lib = _load()


def last_error():
    return lib.hfq4_last_error().decode()


def _check(code):
    if code != HFQ4_OK:
        raise Hfq4Error(code, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


# ------------------------------------------------------------------ format

def hfq4_packed_bytes(rows, K):
    out = ctypes.c_size_t()
    _check(lib.hfq4_packed_bytes(rows, K, ctypes.byref(out)))
    return out.value


def hfq4_pack(w, out=None, bad=None, stream=None):
    """Quantize a contiguous f32 device matrix [rows, K] into HFQ4 bytes.
    Returns the uint8 tensor; raises if any block was rejected."""
    import torch
    rows, K = w.shape
    ldw = w.stride(0)
    assert w.dtype == torch.float32 and w.stride(1) == 1
    nbytes = hfq4_packed_bytes(rows, K)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    own_bad = bad is None
    if own_bad:
        bad = torch.zeros(1, dtype=torch.int32, device=w.device)
    _check(lib.hfq4_pack(_ptr(w), rows, K, ldw, _ptr(out), out.numel(), _ptr(bad), _stream(stream)))
    if own_bad:
        n = int(bad.item())
        if n:
            raise Hfq4Error(HFQ4_E_INVALID, "%d HFQ4 block(s) held non-finite values" % n)
    return out


def hfq4_gemv(W, rows, K, x, residual=None, y=None, stream=None):
    """y[b] = residual[b] + W x[b] for x [batch, K] f32 (device).  W is a
    device tensor or a pinned host tensor (read zero-copy over PCIe)."""
    import torch
    x2 = x if x.dim() == 2 else x.view(1, -1)
    batch = x2.shape[0]
    if y is None:
        y = torch.empty((batch, rows), dtype=torch.float32, device=x.device)
    ldr = residual.stride(0) if (residual is not None and residual.dim() == 2) else rows
    wp = _ptr(W) if W.is_cuda else ctypes.c_void_p(host_device_pointer(W))
    _check(lib.hfq4_gemv(wp, rows, K, _ptr(x2), x2.stride(0), batch, _ptr(residual), ldr,
                         _ptr(y), y.stride(0) if y.dim() == 2 else rows, _stream(stream)))
    return y


# ------------------------------------------------------------------ routing

def moe_route_workspace_bytes(E, batch):
    out = ctypes.c_size_t()
    _check(lib.moe_route_workspace_bytes(E, batch, ctypes.byref(out)))
    return out.value


def moe_route_topk(Wr, x, k, bias=None, ws=None, logits=None, idx=None, wts=None, stream=None):
    """Router GEMV + top-k + renormalised softmax.  Returns (idx, wts)."""
    import torch
    E, d = Wr.shape
    x2 = x if x.dim() == 2 else x.view(1, -1)
    B = x2.shape[0]
    if ws is None:
        ws = torch.zeros(moe_route_workspace_bytes(E, B), dtype=torch.uint8, device=x.device)
    if idx is None:
        idx = torch.empty((B, k), dtype=torch.int32, device=x.device)
    if wts is None:
        wts = torch.empty((B, k), dtype=torch.float32, device=x.device)
    _check(lib.moe_route_topk(_ptr(Wr), _ptr(bias), E, d, _ptr(x2), x2.stride(0), B, k, _ptr(idx),
                              _ptr(wts), _ptr(logits), _ptr(ws), ws.numel(), _stream(stream)))
    return idx, wts


def host_device_pointer(t):
    """Device address of a pinned host tensor (torch pin_memory=True)."""
    if t.is_cuda or not t.is_pinned():
        raise Hfq4Error(HFQ4_E_INVALID, "host-mapped tensors must be pinned host memory")
    out = ctypes.c_void_p()
    _check(lib.hfq4_host_device_pointer(ctypes.c_void_p(t.data_ptr()), ctypes.byref(out)))
    return out.value


# ------------------------------------------------------------------ experts

class MoeLayer:
    """Tensors of one MoE layer: gate/up [E * packed(F, d)] and down
    [E * packed(d, F)] uint8 buffers (device or pinned host), router Wr
    [E, d] f32 and optional bias [E]."""

    def __init__(self, gate, up, down, E, d, F, Wr=None, bias=None, host_mapped=False,
                 stride_gate=None, stride_up=None, stride_down=None):
        self.gate, self.up, self.down = gate, up, down
        self.E, self.d, self.F = E, d, F
        self.Wr, self.bias = Wr, bias
        gb = hfq4_packed_bytes(F, d)
        db = hfq4_packed_bytes(d, F)
        if host_mapped:
            ptrs = [host_device_pointer(t) for t in (gate, up, down)]
        else:
            for t in (gate, up, down):
                if not t.is_cuda:
                    raise Hfq4Error(HFQ4_E_INVALID, "expert tensors must be on the device "
                                    "(or pinned host memory with host_mapped=True)")
            ptrs = [t.data_ptr() for t in (gate, up, down)]
        self.c = MoeLayerC(ptrs[0], ptrs[1], ptrs[2], E, d, F,
                           stride_gate or gb, stride_up or gb, stride_down or db,
                           HFQ4_LAYER_HOST_MAPPED if host_mapped else 0, 0)

    def expert_bytes(self):
        return 2 * hfq4_packed_bytes(self.F, self.d) + hfq4_packed_bytes(self.d, self.F)


def moe_workspace_bytes(layer, batch, k):
    out = ctypes.c_size_t()
    _check(lib.moe_workspace_bytes(ctypes.byref(layer.c), batch, k, ctypes.byref(out)))
    return out.value


def moe_workspace_init(ws, stream=None):
    _check(lib.moe_workspace_init(_ptr(ws), ws.numel(), _stream(stream)))


def new_workspace(layer, batch, k, device="cuda"):
    import torch
    return torch.zeros(moe_workspace_bytes(layer, batch, k), dtype=torch.uint8, device=device)


def moe_expert_decode(layer, x, idx, wts, ws, residual=None, y=None, stream=None):
    import torch
    x2 = x if x.dim() == 2 else x.view(1, -1)
    B = x2.shape[0]
    k = idx.shape[-1]
    if y is None:
        y = torch.empty((B, layer.d), dtype=torch.float32, device=x.device)
    _check(lib.moe_expert_decode(ctypes.byref(layer.c), _ptr(x2), x2.stride(0), B, _ptr(idx),
                                 _ptr(wts), k, _ptr(residual), _ptr(y), y.stride(0), _ptr(ws),
                                 ws.numel(), _stream(stream)))
    return y


def moe_layer_decode(layer, x, k, ws, residual=None, y=None, idx=None, wts=None, stream=None):
    """Route + experts in one enqueue.  Returns (idx, wts, y)."""
    import torch
    x2 = x if x.dim() == 2 else x.view(1, -1)
    B = x2.shape[0]
    if y is None:
        y = torch.empty((B, layer.d), dtype=torch.float32, device=x.device)
    if idx is None:
        idx = torch.empty((B, k), dtype=torch.int32, device=x.device)
    if wts is None:
        wts = torch.empty((B, k), dtype=torch.float32, device=x.device)
    _check(lib.moe_layer_decode(ctypes.byref(layer.c), _ptr(layer.Wr), _ptr(layer.bias), _ptr(x2),
                                x2.stride(0), B, k, _ptr(idx), _ptr(wts), _ptr(residual), _ptr(y),
                                y.stride(0), _ptr(ws), ws.numel(), _stream(stream)))
    return idx, wts, y


def workspace_error(ws):
    """Sticky device error word of a workspace (synchronises the device)."""
    return int(ws[:4].view(__import__("torch").int32).item())
