"""Python binding of libmoe.so: the low-bit sparse-MoE layer on MI355X (gfx950).

The functions below have the C ABI's names (include/moe.h) and only marshal
arguments: torch tensors become device pointers, the current torch stream
becomes the hipStream_t.  Every step of the computation runs in the HIP
kernels of libmoe.so; there is no other implementation in this package.  If
the library has not been built, importing works but the first call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP, MOE_ERR_DATA = 0, 1, 2, 3, 4, 5
TIMING_GATE_UP, TIMING_DOWN, TIMING_ROUTER, TIMING_PREFILL_GATE_UP, TIMING_PREFILL_DOWN = 0, 1, 2, 3, 4
TIMING_PREFILL_ROUTER = 5
TIMING_PERSIST = 6
MAX_TOK_DECODE_KERNELS = 8  # one layer of at most this many tokens runs the decode kernels
MAX_TOK_F16ACT = 16  # tokens per call of the fp16-activation decode entry points

EXPORTED = ("moe_last_error", "moe_packed_bytes", "moe_pack_experts", "moe_layer_release", "moe_layer_get_desc",
            "moe_route_topk", "moe_workspace_bytes", "moe_workspace_init", "moe_layer_forward",
            "moe_stack_forward", "moe_rmsnorm", "moe_debug_unpack", "moe_timing_start", "moe_timing_stop",
            "moe_group_workspace_bytes", "moe_group_tokens", "moe_layer_forward_f16act",
            "moe_stack_forward_f16act", "moe_debug_unpack_path", "moe_layer_forward_noalloc",
            "moe_workspace_status", "moe_layer_workspace_bytes", "moe_pack_experts_cb")


class MoeError(RuntimeError):
    def __init__(self, code: int, fn: str, msg: str):
        super().__init__(f"{fn} failed with code {code}: {msg}")
        self.code = code


class LayerDesc(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("d_ff_shared", ctypes.c_int32), ("top_k", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("block", ctypes.c_int32), ("codebook", ctypes.c_int32)]


class RouteIO(ctypes.Structure):
    _fields_ = [("in_idx", ctypes.c_void_p), ("in_w", ctypes.c_void_p), ("out_logits", ctypes.c_void_p),
                ("out_idx", ctypes.c_void_p), ("out_w", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_packed_bytes.argtypes = [P, ctypes.POINTER(S)]
        L.moe_pack_experts.argtypes = [P, P, P, P, P, P, S, ctypes.POINTER(P), P]
        L.moe_pack_experts_cb.argtypes = [P, P, P, P, P, P, P, S, ctypes.POINTER(P), P]
        L.moe_layer_release.argtypes = [P]
        L.moe_layer_get_desc.argtypes = [P, P]
        L.moe_route_topk.argtypes = [P, I, I, I, P, P, P]
        L.moe_workspace_bytes.argtypes = [P, I, ctypes.POINTER(S)]
        L.moe_layer_workspace_bytes.argtypes = [P, I, ctypes.POINTER(S)]
        L.moe_workspace_init.argtypes = [P, S, P]
        L.moe_layer_forward.argtypes = [P, P, I, P, P, P, S, P]
        L.moe_stack_forward.argtypes = [P, I, P, I, ctypes.c_float, P, P, P, P, P, S, P]
        L.moe_layer_forward_f16act.argtypes = [P, P, I, P, P, P, S, P]
        L.moe_layer_forward_noalloc.argtypes = [P, P, I, P, P, P]
        L.moe_workspace_status.argtypes = [P, S, ctypes.POINTER(I), P]
        L.moe_stack_forward_f16act.argtypes = [P, I, P, I, ctypes.c_float, P, P, P, P, P, S, P]
        L.moe_rmsnorm.argtypes = [P, I, I, ctypes.c_float, P, P]
        L.moe_debug_unpack.argtypes = [P, I, I, P, P, P, P]
        L.moe_debug_unpack_path.argtypes = [P, I, I, I, P, P, P, P]
        L.moe_timing_start.argtypes = [I, I]
        L.moe_timing_stop.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int)]
        L.moe_group_workspace_bytes.argtypes = [I, I, I, ctypes.POINTER(S)]
        L.moe_group_tokens.argtypes = [P, I, I, I, P, P, P, P, S, P]
        for name in EXPORTED:
            if name != "moe_last_error":
                getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int, fn: str):
    if rc != MOE_OK:
        raise MoeError(rc, fn, (lib().moe_last_error() or b"").decode())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream=None):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_desc(d_model, n_experts, d_ff, d_ff_shared, top_k, bits, block=32, codebook=False) -> LayerDesc:
    return LayerDesc(d_model, n_experts, d_ff, d_ff_shared, top_k, bits, block, int(bool(codebook)))


# ---------------------------------------------------------------------------
# C ABI, one wrapper per entry point
# ---------------------------------------------------------------------------
def moe_last_error() -> str:
    return (lib().moe_last_error() or b"").decode()


def moe_packed_bytes(desc: LayerDesc) -> int:
    n = ctypes.c_size_t()
    _check(lib().moe_packed_bytes(ctypes.byref(desc), ctypes.byref(n)), "moe_packed_bytes")
    return n.value


def moe_pack_experts(desc: LayerDesc, experts_canon, shared_canon, router_w, router_bias, packed, stream=None) -> int:
    """Returns the opaque layer handle (an integer)."""
    h = ctypes.c_void_p()
    _check(lib().moe_pack_experts(ctypes.byref(desc), _ptr(experts_canon), _ptr(shared_canon), _ptr(router_w),
                                  _ptr(router_bias), _ptr(packed), packed.numel() * packed.element_size(),
                                  ctypes.byref(h), _stream(stream)), "moe_pack_experts")
    return h.value


def moe_pack_experts_cb(desc: LayerDesc, experts_canon, shared_canon, grid, router_w, router_bias, packed,
                        stream=None) -> int:
    """Codebook blocks: as moe_pack_experts plus the grid (uint8 [512, 4] on the device)."""
    h = ctypes.c_void_p()
    _check(lib().moe_pack_experts_cb(ctypes.byref(desc), _ptr(experts_canon), _ptr(shared_canon), _ptr(grid),
                                     _ptr(router_w), _ptr(router_bias), _ptr(packed),
                                     packed.numel() * packed.element_size(), ctypes.byref(h), _stream(stream)),
           "moe_pack_experts_cb")
    return h.value


def moe_layer_release(handle: int):
    _check(lib().moe_layer_release(handle), "moe_layer_release")


def moe_layer_get_desc(handle: int) -> LayerDesc:
    d = LayerDesc()
    _check(lib().moe_layer_get_desc(handle, ctypes.byref(d)), "moe_layer_get_desc")
    return d


def moe_route_topk(logits, k: int, idx, w, stream=None):
    T, E = logits.shape
    _check(lib().moe_route_topk(_ptr(logits), T, E, k, _ptr(idx), _ptr(w), _stream(stream)), "moe_route_topk")


def moe_workspace_bytes(handle: int, T: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().moe_workspace_bytes(handle, T, ctypes.byref(n)), "moe_workspace_bytes")
    return n.value


def moe_layer_workspace_bytes(handle: int, T: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().moe_layer_workspace_bytes(handle, T, ctypes.byref(n)), "moe_layer_workspace_bytes")
    return n.value


def moe_workspace_init(ws, stream=None):
    _check(lib().moe_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "moe_workspace_init")


def moe_layer_forward(handle: int, x, y, ws, route: RouteIO | None = None, stream=None):
    T = x.shape[0]
    _check(lib().moe_layer_forward(handle, _ptr(x), T, _ptr(y), ctypes.byref(route) if route is not None else None,
                                   _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "moe_layer_forward")


def moe_layer_forward_noalloc(handle: int, x, y, route: RouteIO | None = None, stream=None):
    T = x.shape[0]
    _check(lib().moe_layer_forward_noalloc(handle, _ptr(x), T, _ptr(y),
                                           ctypes.byref(route) if route is not None else None, _stream(stream)),
           "moe_layer_forward_noalloc")


NOALLOC_SCRATCH_BYTES = 16 << 20


def moe_layer_forward_f16act(handle: int, x, y, ws, route: RouteIO | None = None, stream=None):
    T = x.shape[0]
    _check(lib().moe_layer_forward_f16act(handle, _ptr(x), T, _ptr(y),
                                          ctypes.byref(route) if route is not None else None, _ptr(ws),
                                          ws.numel() * ws.element_size(), _stream(stream)), "moe_layer_forward_f16act")


def moe_stack_forward_f16act(handles, x, y, ws, eps: float = 1e-6, y_layers=None, idx_layers=None, w_layers=None,
                             stream=None):
    arr = (ctypes.c_void_p * len(handles))(*handles)
    T = x.shape[0]
    _check(lib().moe_stack_forward_f16act(arr, len(handles), _ptr(x), T, eps, _ptr(y), _ptr(y_layers),
                                          _ptr(idx_layers), _ptr(w_layers), _ptr(ws),
                                          ws.numel() * ws.element_size(), _stream(stream)),
           "moe_stack_forward_f16act")


def moe_stack_forward(handles, x, y, ws, eps: float = 1e-6, y_layers=None, idx_layers=None, w_layers=None,
                      stream=None):
    arr = (ctypes.c_void_p * len(handles))(*handles)
    T = x.shape[0]
    _check(lib().moe_stack_forward(arr, len(handles), _ptr(x), T, eps, _ptr(y), _ptr(y_layers), _ptr(idx_layers),
                                   _ptr(w_layers), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "moe_stack_forward")


def moe_group_workspace_bytes(T: int, E: int, k: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().moe_group_workspace_bytes(T, E, k, ctypes.byref(n)), "moe_group_workspace_bytes")
    return n.value


def moe_group_tokens(idx, E: int, counts, offsets, perm, ws, stream=None):
    T, k = idx.shape
    _check(lib().moe_group_tokens(_ptr(idx), T, E, k, _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream)), "moe_group_tokens")


def moe_rmsnorm(x, y, eps: float = 1e-6, stream=None):
    T, d = x.shape
    _check(lib().moe_rmsnorm(_ptr(x), T, d, eps, _ptr(y), _stream(stream)), "moe_rmsnorm")


def moe_debug_unpack(handle: int, expert: int, mat: int, codes=None, w_f32=None, w_f16=None, stream=None):
    _check(lib().moe_debug_unpack(handle, expert, mat, _ptr(codes), _ptr(w_f32), _ptr(w_f16), _stream(stream)),
           "moe_debug_unpack")


def moe_debug_unpack_path(handle: int, expert: int, mat: int, path: int, codes=None, w_f32=None, w_f16=None,
                          stream=None):
    _check(lib().moe_debug_unpack_path(handle, expert, mat, path, _ptr(codes), _ptr(w_f32), _ptr(w_f16),
                                       _stream(stream)), "moe_debug_unpack_path")


def moe_workspace_status(ws, stream=None) -> int:
    st = ctypes.c_int()
    _check(lib().moe_workspace_status(_ptr(ws), ws.numel() * ws.element_size(), ctypes.byref(st), _stream(stream)),
           "moe_workspace_status")
    return st.value


def moe_timing_start(kernel_class: int, max_launches: int):
    _check(lib().moe_timing_start(kernel_class, max_launches), "moe_timing_start")


def moe_timing_stop():
    ms = ctypes.c_double()
    n = ctypes.c_int()
    _check(lib().moe_timing_stop(ctypes.byref(ms), ctypes.byref(n)), "moe_timing_stop")
    return ms.value, n.value


# ---------------------------------------------------------------------------
# Owning helpers
# ---------------------------------------------------------------------------
class PackedLayer:
    """A packed layer: owns its device buffer (torch uint8) and host handle."""

    def __init__(self, desc: LayerDesc, experts_canon, shared_canon, router_w, router_bias, device="cuda",
                 grid=None):
        self.desc = desc
        n = moe_packed_bytes(desc)
        self.buffer = torch.empty(n, dtype=torch.uint8, device=device)
        if desc.codebook:
            self.handle = moe_pack_experts_cb(desc, experts_canon, shared_canon, grid, router_w, router_bias,
                                              self.buffer)
        else:
            self.handle = moe_pack_experts(desc, experts_canon, shared_canon, router_w, router_bias, self.buffer)

    def workspace_bytes(self, T: int) -> int:
        return moe_workspace_bytes(self.handle, T)

    def layer_workspace_bytes(self, T: int) -> int:
        return moe_layer_workspace_bytes(self.handle, T)

    def close(self):
        if getattr(self, "handle", None):
            moe_layer_release(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def new_workspace(nbytes: int, device="cuda"):
    """A zero-initialised workspace tensor (control words cleared)."""
    ws = torch.empty(max(nbytes, 512), dtype=torch.uint8, device=device)
    moe_workspace_init(ws)
    return ws
