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
HFQ4_E_NOFIT = -7
HFQ4_PLACE_LAYERS = 0
HFQ4_PLACE_HOTSET = 1
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
    "hfq4_debug_set_trace", "hfq4_debug_set_events", "moe_layer_decode_noalloc",
    "hfq4_gemv_host", "moe_expert_decode_host", "hfq4_offload_choice",
    "hfq4_debug_set_single_launch", "hfq4_debug_set_route_exchange", "moe_place_experts",
    "moe_layer_decode_table", "hfq4_debug_set_host_kernel", "hfq4_debug_set_turbo_search",
    "turbo_record_bytes", "turbo_levels", "turbo_encode", "turbo_decode",
]
NOALLOC_SCRATCH_BYTES = 8 << 20


class Hfq4Error(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("hfq4 status %d: %s" % (code, msg))
        self.code = code


class MoeLayerTableC(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("resident", ctypes.c_void_p), ("E", ctypes.c_int64),
                ("d", ctypes.c_int64), ("F", ctypes.c_int64)]


class MoeLayerC(ctypes.Structure):
    _fields_ = [("gate", ctypes.c_void_p), ("up", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("E", ctypes.c_int64), ("d", ctypes.c_int64), ("F", ctypes.c_int64),
                ("stride_gate", ctypes.c_int64), ("stride_up", ctypes.c_int64),
                ("stride_down", ctypes.c_int64), ("flags", ctypes.c_uint32),
                ("reserved", ctypes.c_uint32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libhfq4moe.so not built at %s -- build it with "
                          "'python quantized_moe_decode_amd/build.py' (no CPU fallback exists)"
                          % LIB_PATH)
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
        "moe_layer_decode_noalloc": (I32, [ctypes.POINTER(MoeLayerC), P, P, P, I64, I32, I32, P, P,
                                           P, P, I64, P, P]),
        "hfq4_gemv_host": (I32, [P, I64, I64, P, I64, I32, P, I64, P, I64, I32]),
        "moe_expert_decode_host": (I32, [ctypes.POINTER(MoeLayerC), P, I64, I32, P, P, I32, P, P,
                                         I64, I32, ctypes.POINTER(ctypes.c_uint32)]),
        "hfq4_offload_choice": (I32, [ctypes.c_double, ctypes.c_double, ctypes.POINTER(I32)]),
        "hfq4_debug_set_single_launch": (I32, [I32]),
        "hfq4_debug_set_route_exchange": (I32, [I32]),
        "hfq4_debug_set_turbo_search": (I32, [I32]),
        "hfq4_debug_set_host_kernel": (I32, [I32, ctypes.POINTER(I32)]),
        "moe_place_experts": (I32, [I32, I64, I64, P, ctypes.c_uint64, ctypes.c_uint64,
                                    ctypes.c_uint64, P, ctypes.POINTER(ctypes.c_uint64)]),
        "moe_layer_decode_table": (I32, [ctypes.POINTER(MoeLayerTableC), P, P, P, I32, I32, P, P, P,
                                         P, P, P, SZ, P]),
        "turbo_record_bytes": (I32, [I32, I32, ctypes.POINTER(SZ)]),
        "turbo_levels": (I32, [I32, I32, P]),
        "turbo_encode": (I32, [P, I64, I32, I64, I32, P, SZ, P]),
        "turbo_decode": (I32, [P, SZ, I64, I32, I32, P, I64, P]),
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


def _need(cond, msg):
    """Argument checks the C ABI cannot make (it sees pointers, not tensor
    sizes or dtypes): refuse before anything is enqueued."""
    if not cond:
        raise Hfq4Error(HFQ4_E_INVALID, msg)


def _f32(t, name):
    import torch
    _need(t.dtype == torch.float32, "%s must be float32, got %s" % (name, t.dtype))
    _need(t.dim() <= 1 or t.stride(-1) == 1, "%s must have unit stride along its rows" % name)


def _rows(t, name, n, width):
    """t holds n rows of at least `width` elements at its row stride."""
    t2 = t if t.dim() == 2 else t.view(1, -1)
    _need(t2.shape[0] == n, "%s has %d rows, expected %d" % (name, t2.shape[0], n))
    _need(t2.shape[1] >= width, "%s rows hold %d elements, need %d" % (name, t2.shape[1], width))


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
    _f32(x2, "x")
    _need(x2.shape[1] >= K, "x rows hold %d elements, need K = %d" % (x2.shape[1], K))
    _need(W.dtype == torch.uint8 and W.is_contiguous(), "W must be a contiguous uint8 tensor")
    _need(W.numel() >= hfq4_packed_bytes(rows, K),
          "W holds %d bytes, a %d x %d HFQ4 matrix needs %d" % (W.numel(), rows, K,
                                                               hfq4_packed_bytes(rows, K)))
    if y is None:
        y = torch.empty((batch, rows), dtype=torch.float32, device=x.device)
    _f32(y, "y")
    _rows(y, "y", batch, rows)
    if residual is not None:
        _f32(residual, "residual")
        _rows(residual, "residual", batch, rows)
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
    _f32(Wr, "Wr")
    _need(Wr.is_contiguous(), "Wr must be contiguous [E, d]")
    _f32(x2, "x")
    _need(x2.shape[1] >= d, "x rows hold %d elements, need d = %d" % (x2.shape[1], d))
    if bias is not None:
        _f32(bias, "bias")
        _need(bias.numel() >= E, "bias holds %d values, need E = %d" % (bias.numel(), E))
    if ws is None:
        ws = torch.zeros(moe_route_workspace_bytes(E, B), dtype=torch.uint8, device=x.device)
    if idx is None:
        idx = torch.empty((B, k), dtype=torch.int32, device=x.device)
    if wts is None:
        wts = torch.empty((B, k), dtype=torch.float32, device=x.device)
    _check_routing_out(idx, wts, B, k)
    if logits is not None:
        _f32(logits, "logits")
        _need(logits.is_contiguous() and logits.numel() >= B * E,
              "logits must be a contiguous [B, E] float32 tensor")
    _need(ws.dtype == torch.uint8, "ws must be a uint8 tensor")
    _check(lib.moe_route_topk(_ptr(Wr), _ptr(bias), E, d, _ptr(x2), x2.stride(0), B, k, _ptr(idx),
                              _ptr(wts), _ptr(logits), _ptr(ws), ws.numel(), _stream(stream)))
    return idx, wts


def _check_routing_out(idx, wts, B, k):
    import torch
    _need(idx.dtype == torch.int32 and idx.is_contiguous() and idx.numel() == B * k,
          "idx must be a contiguous [B, k] int32 tensor")
    _need(wts.dtype == torch.float32 and wts.is_contiguous() and wts.numel() == B * k,
          "wts must be a contiguous [B, k] float32 tensor")


def _check_io(layer, x2, y, residual, ws):
    """Shapes, dtypes and strides of a layer call's activations."""
    import torch
    B = x2.shape[0]
    _f32(x2, "x")
    _need(x2.shape[1] >= layer.d, "x rows hold %d elements, need d = %d" % (x2.shape[1], layer.d))
    _f32(y, "y")
    _rows(y, "y", B, layer.d)
    if residual is not None:
        r2 = residual if residual.dim() == 2 else residual.view(1, -1)
        _f32(r2, "residual")
        _rows(r2, "residual", B, layer.d)
        # the C ABI reads the residual at y's row stride
        _need(B == 1 or r2.stride(0) == y.stride(0),
              "residual row stride %d differs from y's %d" % (r2.stride(0), y.stride(0)))
    _need(ws.dtype == torch.uint8, "ws must be a uint8 tensor")


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
        import torch
        self.gate, self.up, self.down = gate, up, down
        self.E, self.d, self.F = E, d, F
        self.Wr, self.bias = Wr, bias
        gb = hfq4_packed_bytes(F, d)
        db = hfq4_packed_bytes(d, F)
        # the kernels address E * stride bytes of each tensor
        for t, name, st in ((gate, "gate", stride_gate or gb), (up, "up", stride_up or gb),
                            (down, "down", stride_down or db)):
            _need(t.dtype == torch.uint8 and t.is_contiguous(),
                  "%s must be a contiguous uint8 tensor" % name)
            _need(t.numel() >= E * st, "%s holds %d bytes, %d experts at stride %d need %d"
                  % (name, t.numel(), E, st, E * st))
        if Wr is not None:
            _f32(Wr, "Wr")
            _need(Wr.is_contiguous() and tuple(Wr.shape) == (E, d), "Wr must be contiguous [E, d]")
        if bias is not None:
            _f32(bias, "bias")
            _need(bias.numel() == E, "bias must hold E = %d values" % E)
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
    _check_io(layer, x2, y, residual, ws)
    _check_routing_out(idx, wts, B, k)
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
    _need(layer.Wr is not None, "the layer has no router (Wr)")
    _check_io(layer, x2, y, residual, ws)
    _check_routing_out(idx, wts, B, k)
    _check(lib.moe_layer_decode(ctypes.byref(layer.c), _ptr(layer.Wr), _ptr(layer.bias), _ptr(x2),
                                x2.stride(0), B, k, _ptr(idx), _ptr(wts), _ptr(residual), _ptr(y),
                                y.stride(0), _ptr(ws), ws.numel(), _stream(stream)))
    return idx, wts, y


def moe_layer_decode_noalloc(layer, x, k, idx, wts, y, residual=None, err=None, stream=None):
    """moe_layer_decode on the library's fixed scratch (no workspace): for
    callers that cannot allocate.  Every output is the caller's (nothing is
    allocated here or in the library); err is an optional device int32 [1]
    that receives the sticky device error bits."""
    x2 = x if x.dim() == 2 else x.view(1, -1)
    B = x2.shape[0]
    _need(layer.Wr is not None, "the layer has no router (Wr)")
    _f32(x2, "x")
    _need(x2.shape[1] >= layer.d, "x rows hold %d elements, need d = %d" % (x2.shape[1], layer.d))
    _f32(y, "y")
    _rows(y, "y", B, layer.d)
    if residual is not None:
        r2 = residual if residual.dim() == 2 else residual.view(1, -1)
        _f32(r2, "residual")
        _rows(r2, "residual", B, layer.d)
        _need(B == 1 or r2.stride(0) == y.stride(0),
              "residual row stride %d differs from y's %d" % (r2.stride(0), y.stride(0)))
    _check_routing_out(idx, wts, B, k)
    _check(lib.moe_layer_decode_noalloc(ctypes.byref(layer.c), _ptr(layer.Wr), _ptr(layer.bias),
                                        _ptr(x2), x2.stride(0), B, k, _ptr(idx), _ptr(wts),
                                        _ptr(residual), _ptr(y), y.stride(0), _ptr(err),
                                        _stream(stream)))
    return idx, wts, y


# ------------------------------------------------------------------ host CPU execution

def _host_array(a, name, dtype):
    """(pointer, numpy view) of a host buffer: a numpy array or a CPU torch
    tensor (pinned or not), C-contiguous along its rows."""
    import numpy as np
    if hasattr(a, "is_cuda"):
        _need(not a.is_cuda, "%s must be host memory" % name)
        arr = a.numpy()
    else:
        arr = np.asarray(a)
    _need(arr.dtype == dtype, "%s must be %s, got %s" % (name, np.dtype(dtype), arr.dtype))
    _need(arr.ndim <= 1 or arr.strides[-1] == arr.itemsize, "%s must have unit stride" % name)
    return ctypes.c_void_p(arr.ctypes.data), arr


def hfq4_gemv_host(W, rows, K, x, residual=None, y=None, nthreads=0):
    """y[b] = residual[b] + W x[b] on the host CPU (every buffer host memory;
    numpy arrays or CPU torch tensors).  Returns y (numpy, float32)."""
    import numpy as np
    wp, Wa = _host_array(W, "W", np.uint8)
    _need(Wa.size >= hfq4_packed_bytes(rows, K), "W holds %d bytes, need %d"
          % (Wa.size, hfq4_packed_bytes(rows, K)))
    xp, xa = _host_array(x, "x", np.float32)
    xa2 = xa.reshape(1, -1) if xa.ndim == 1 else xa
    batch = xa2.shape[0]
    _need(xa2.shape[1] >= K, "x rows hold %d elements, need K = %d" % (xa2.shape[1], K))
    if y is None:
        y = np.empty((batch, rows), dtype=np.float32)
    yp, ya = _host_array(y, "y", np.float32)
    ya2 = ya.reshape(1, -1) if ya.ndim == 1 else ya
    rp, ldr = None, rows
    if residual is not None:
        rp, ra = _host_array(residual, "residual", np.float32)
        ra2 = ra.reshape(1, -1) if ra.ndim == 1 else ra
        ldr = ra2.strides[0] // 4
    _check(lib.hfq4_gemv_host(wp, rows, K, xp, xa2.strides[0] // 4, batch, rp, ldr, yp,
                              ya2.strides[0] // 4, int(nthreads)))
    return y


HOST_KERNELS = {"best": 0, "avx512": 1, "avx2": 2, "portable": 3}


def set_host_kernel(name="best"):
    """Row kernel of the host CPU entry points for later calls (process-wide):
    'best' (the default), 'avx512', 'avx2' or 'portable'.  Returns the name
    of the kernel now in use; raises Hfq4Error if the CPU lacks it."""
    used = ctypes.c_int(0)
    _check(lib.hfq4_debug_set_host_kernel(HOST_KERNELS[name], ctypes.byref(used)))
    return {v: k for k, v in HOST_KERNELS.items()}[used.value]


class HostMoeLayer:
    """One MoE layer's experts in host memory for moe_expert_decode_host:
    gate/up [E * packed(F, d)] and down [E * packed(d, F)] uint8 buffers
    (numpy arrays or CPU torch tensors, pinned or not)."""

    def __init__(self, gate, up, down, E, d, F):
        import numpy as np
        self.E, self.d, self.F = E, d, F
        gb, db = hfq4_packed_bytes(F, d), hfq4_packed_bytes(d, F)
        ptrs = []
        self._keep = []
        for t, name, need in ((gate, "gate", E * gb), (up, "up", E * gb), (down, "down", E * db)):
            p, a = _host_array(t, name, np.uint8)
            _need(a.size >= need, "%s holds %d bytes, need %d" % (name, a.size, need))
            ptrs.append(p.value)
            self._keep.append(t)
        self.c = MoeLayerC(ptrs[0], ptrs[1], ptrs[2], E, d, F, gb, gb, db, 0, 0)


def moe_expert_decode_host(layer, x, idx, wts, residual=None, y=None, nthreads=0):
    """The expert half of a layer on the host CPU.  Returns (y, error bits)."""
    import numpy as np
    xp, xa = _host_array(x, "x", np.float32)
    xa2 = xa.reshape(1, -1) if xa.ndim == 1 else xa
    B = xa2.shape[0]
    ip, ia = _host_array(idx, "idx", np.int32)
    wp, wa = _host_array(wts, "wts", np.float32)
    k = ia.shape[-1]
    _need(ia.size == B * k and wa.size == B * k, "idx and wts must be [B, k]")
    if y is None:
        y = np.empty((B, layer.d), dtype=np.float32)
    yp, ya = _host_array(y, "y", np.float32)
    ya2 = ya.reshape(1, -1) if ya.ndim == 1 else ya
    rp = None
    if residual is not None:
        rp, ra = _host_array(residual, "residual", np.float32)
        ra2 = ra.reshape(1, -1) if ra.ndim == 1 else ra
        _need(B == 1 or ra2.strides[0] == ya2.strides[0], "residual row stride differs from y's")
    err = ctypes.c_uint32(0)
    _check(lib.moe_expert_decode_host(ctypes.byref(layer.c), xp, xa2.strides[0] // 4, B, ip, wp, k,
                                      rp, yp, ya2.strides[0] // 4, int(nthreads),
                                      ctypes.byref(err)))
    return y, err.value


def hfq4_offload_choice(pcie_seconds, cpu_seconds):
    """True when the CPU path is at least 15% faster than the PCIe path."""
    out = ctypes.c_int()
    _check(lib.hfq4_offload_choice(float(pcie_seconds), float(cpu_seconds), ctypes.byref(out)))
    return bool(out.value)


# ------------------------------------------------------------------ expert cache

def moe_place_experts(mode, layers, E, expert_bytes, fixed_bytes, budget_bytes, heat=None):
    """Placement of layers x E experts into an HBM budget (see the C ABI).
    Returns (resident uint8 [layers, E] numpy, placed bytes); raises
    Hfq4Error(HFQ4_E_NOFIT) naming the bytes short when it does not fit."""
    import numpy as np
    res = np.zeros((layers, E), dtype=np.uint8)
    hp = None
    if heat is not None:
        heat = np.ascontiguousarray(heat, dtype=np.uint64)
        _need(heat.shape == (layers, E), "heat must be [layers, E]")
        hp = ctypes.c_void_p(heat.ctypes.data)
    placed = ctypes.c_uint64()
    _check(lib.moe_place_experts(int(mode), layers, E, hp, int(expert_bytes), int(fixed_bytes),
                                 int(budget_bytes), ctypes.c_void_p(res.ctypes.data),
                                 ctypes.byref(placed)))
    return res, placed.value


def moe_layer_decode_table(tlayer, x, k, ws, residual=None, y=None, idx=None, wts=None, hits=None,
                           stream=None):
    """One token through a table layer (cache.TableLayer).  Returns (idx, wts, y)."""
    import torch
    x2 = x if x.dim() == 2 else x.view(1, -1)
    _need(x2.shape[0] == 1, "table layers take one token per call")
    _f32(x2, "x")
    _need(x2.is_contiguous() and x2.shape[1] == tlayer.d, "x must be a contiguous [1, d] tensor")
    if y is None:
        y = torch.empty((1, tlayer.d), dtype=torch.float32, device=x.device)
    if idx is None:
        idx = torch.empty((1, k), dtype=torch.int32, device=x.device)
    if wts is None:
        wts = torch.empty((1, k), dtype=torch.float32, device=x.device)
    _f32(y, "y")
    _need(y.is_contiguous() and y.numel() == tlayer.d, "y must be a contiguous [1, d] tensor")
    if residual is not None:
        _need(residual.is_contiguous() and residual.numel() == tlayer.d and
              residual.dtype == torch.float32, "residual must be a contiguous [1, d] float32 tensor")
    _check_routing_out(idx, wts, 1, k)
    if hits is not None:
        _need(hits.dtype == torch.int64 and hits.numel() >= 2, "hits must be an int64 [2] tensor")
    _need(ws.dtype == torch.uint8, "ws must be a uint8 tensor")
    _check(lib.moe_layer_decode_table(ctypes.byref(tlayer.c), _ptr(tlayer.Wr), _ptr(tlayer.bias),
                                      _ptr(x2), 1, k, _ptr(idx), _ptr(wts), _ptr(residual), _ptr(y),
                                      _ptr(hits), _ptr(ws), ws.numel(), _stream(stream)))
    return idx, wts, y


# ------------------------------------------------------------------ TurboQuant KV codec

def turbo_record_bytes(n, bits):
    out = ctypes.c_size_t()
    _check(lib.turbo_record_bytes(n, bits, ctypes.byref(out)))
    return out.value


def turbo_levels(n, bits):
    """The library's level table (numpy float32, 2^bits ascending)."""
    import numpy as np
    out = np.zeros(1 << bits, dtype=np.float32)
    _check(lib.turbo_levels(n, bits, ctypes.c_void_p(out.ctypes.data)))
    return out


def turbo_encode(v, bits, out=None, stream=None):
    """Encode f32 vectors v [count, n] (device) into records (uint8 [count,
    record bytes])."""
    import torch
    _f32(v, "v")
    count, n = v.shape
    rec = turbo_record_bytes(n, bits)
    if out is None:
        out = torch.empty((count, rec), dtype=torch.uint8, device=v.device)
    _need(out.dtype == torch.uint8 and out.is_contiguous() and out.numel() >= count * rec,
          "out must be a contiguous uint8 tensor of %d bytes" % (count * rec))
    _check(lib.turbo_encode(_ptr(v), count, n, v.stride(0), bits, _ptr(out), out.numel(),
                            _stream(stream)))
    return out


def turbo_decode(records, n, bits, v=None, stream=None):
    """Decode records (uint8 [count, record bytes], device) into f32 [count, n]."""
    import torch
    rec = turbo_record_bytes(n, bits)
    _need(records.dtype == torch.uint8 and records.is_contiguous(), "records must be contiguous uint8")
    count = records.numel() // rec
    if v is None:
        v = torch.empty((count, n), dtype=torch.float32, device=records.device)
    _f32(v, "v")
    _need(v.shape[0] >= count and v.shape[1] >= n, "v must be [count, n]")
    _check(lib.turbo_decode(_ptr(records), records.numel(), count, n, bits, _ptr(v), v.stride(0),
                            _stream(stream)))
    return v


def workspace_error(ws):
    """Sticky device error word of a workspace (synchronises the device)."""
    return int(ws[:4].view(__import__("torch").int32).item())
