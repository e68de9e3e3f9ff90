"""CPU oracle for the low-bit sparse-MoE layer -- TEST INFRASTRUCTURE ONLY.

Thin ctypes wrapper around ``moe_oracle.c`` (plain single-threaded fp64 C).
Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package; the product library never does, and it
shares no code with the HIP path.

Every function documents the step of the method it follows; the C source
carries the citations of the pages and the readings taken where they are
silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

ORC_OK = 0
ORC_ERR_ARG = -1
ORC_ERR_MISSING_EXPERT = -2
ORC_ERR_NONFINITE = -3


def build(force: bool = False) -> str:
    """Compile moe_oracle.c with gcc (no FP contraction, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
             "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I = ctypes.c_int


def _declare(L):
    L.orc_half_to_double.argtypes = [ctypes.c_uint16]
    L.orc_half_to_double.restype = ctypes.c_double
    L.orc_double_to_half.argtypes = [ctypes.c_double]
    L.orc_double_to_half.restype = ctypes.c_uint16
    L.orc_double_to_half_array.argtypes = [_P, ctypes.c_long, _P]
    L.orc_double_to_half_array.restype = None
    L.orc_unpack_block.argtypes = [_P, _I, _P, _P]
    L.orc_unpack_block.restype = None
    L.orc_unpack_matrix.argtypes = [_P, _I, _I, _I, _P, _P]
    L.orc_dequant_matrix.argtypes = [_P, _I, _I, _I, _P]
    L.orc_exp64.argtypes = [ctypes.c_double]
    L.orc_exp64.restype = ctypes.c_double
    L.orc_exp64_coeff.argtypes = [_I]
    L.orc_exp64_coeff.restype = ctypes.c_double
    L.orc_exp64_ln2.argtypes = [_I]
    L.orc_exp64_ln2.restype = ctypes.c_double
    L.orc_router_logits.argtypes = [_P, _P, _P, _I, _I, _I, _P]
    L.orc_router_logits.restype = None
    L.orc_topk.argtypes = [_P, _I, _I, _I, _P, _P]
    L.orc_expert_bytes.argtypes = [_I, _I, _I]
    L.orc_expert_bytes.restype = ctypes.c_size_t
    L.orc_expert_ffn.argtypes = [_P, _I, _I, _I, _P, _P]
    L.orc_layer_forward.argtypes = [_P, _P, _I, _P, _P, _P, _P, _P, _P]
    L.orc_rmsnorm.argtypes = [_P, _I, _I, ctypes.c_double, _P]
    L.orc_group_tokens.argtypes = [_P, _I, _I, _I, _P, _P, _P]
    L.orc_group_tokens.restype = None
    L.orc_rmsnorm.restype = None
    L.orc_cb_block_bytes.argtypes = []
    L.orc_cb_unpack_block.argtypes = [_P, _P, _P, _P]
    L.orc_cb_unpack_block.restype = None
    L.orc_cb_unpack_matrix.argtypes = [_P, _I, _I, _P, _P, _P]
    L.orc_cb_dequant_matrix.argtypes = [_P, _I, _I, _P, _P]
    L.orc_cb_expert_bytes.argtypes = [_I, _I]
    L.orc_cb_expert_bytes.restype = ctypes.c_size_t
    L.orc_expert_ffn_any.argtypes = [_P, _I, _I, _I, _P, _P, _P]


class _Layer(ctypes.Structure):
    _fields_ = [("d", _I), ("E", _I), ("I", _I), ("Is", _I), ("k", _I), ("bits", _I),
                ("router_w", _P), ("router_bias", _P), ("experts", _P), ("shared", _P), ("grid", _P)]


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_P)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != ORC_OK:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


# ---------------------------------------------------------------------------
# scalar helpers
# ---------------------------------------------------------------------------
def half_to_double(bits: int) -> float:
    return lib().orc_half_to_double(bits)


def double_to_half(v: float) -> int:
    """Binary16 bit pattern nearest to v (ties to even)."""
    return lib().orc_double_to_half(v)


def double_to_half_array(v):
    """Binary16 bit patterns (uint16) nearest to each value (ties to even)."""
    v = _c(v, np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().orc_double_to_half_array(_ptr(v), v.size, _ptr(out))
    return out


def exp64(z):
    """Deterministic fp64 exp used for the gate weights (vectorised over z)."""
    L = lib()
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    flat_in, flat_out = z.reshape(-1), out.reshape(-1)
    for i in range(flat_in.size):
        flat_out[i] = L.orc_exp64(float(flat_in[i]))
    return out


def exp64_coefficients():
    L = lib()
    return [L.orc_exp64_coeff(i) for i in range(14)]


def exp64_ln2_parts():
    L = lib()
    return L.orc_exp64_ln2(0), L.orc_exp64_ln2(1), L.orc_exp64_ln2(2)


def block_bytes(bits: int, grid=None) -> int:
    """Bytes of one canonical block: b-bit codes, or a codebook block when a
    grid is given."""
    return int(lib().orc_cb_block_bytes()) if grid is not None else 2 + 4 * bits


def expert_bytes(d: int, I: int, bits: int) -> int:
    return int(lib().orc_expert_bytes(d, I, bits))


# ---------------------------------------------------------------------------
# unpack / dequant
# ---------------------------------------------------------------------------
def unpack_block(blk: bytes, bits: int):
    """Return (codes[32] int8, scale float) of one canonical block."""
    b = _c(np.frombuffer(bytes(blk), dtype=np.uint8), np.uint8)
    codes = np.empty(32, dtype=np.int8)
    s = ctypes.c_double()
    lib().orc_unpack_block(_ptr(b), bits, _ptr(codes), ctypes.byref(s))
    return codes, s.value


def unpack_matrix(canon, rows: int, cols: int, bits: int):
    """Canonical matrix bytes -> (codes [rows, cols] int8, scales [rows, cols/32] f64)."""
    c = _c(canon, np.uint8)
    codes = np.empty((rows, cols), dtype=np.int8)
    scales = np.empty((rows, cols // 32), dtype=np.float64)
    _check(lib().orc_unpack_matrix(_ptr(c), rows, cols, bits, _ptr(codes), _ptr(scales)), "unpack_matrix")
    return codes, scales


def dequant_matrix(canon, rows: int, cols: int, bits: int):
    """Canonical matrix bytes -> dequantised fp64 weights [rows, cols]."""
    c = _c(canon, np.uint8)
    w = np.empty((rows, cols), dtype=np.float64)
    _check(lib().orc_dequant_matrix(_ptr(c), rows, cols, bits, _ptr(w)), "dequant_matrix")
    return w


# ---------------------------------------------------------------------------
# codebook blocks (grid [512, 4] uint8 of magnitudes)
# ---------------------------------------------------------------------------
def cb_unpack_block(blk: bytes, grid):
    """Return (codes[32] int8, scale float) of one canonical codebook block."""
    b = _c(np.frombuffer(bytes(blk), dtype=np.uint8), np.uint8)
    g = _c(grid, np.uint8)
    codes = np.empty(32, dtype=np.int8)
    s = ctypes.c_double()
    lib().orc_cb_unpack_block(_ptr(b), _ptr(g), _ptr(codes), ctypes.byref(s))
    return codes, s.value


def cb_unpack_matrix(canon, rows: int, cols: int, grid):
    c = _c(canon, np.uint8)
    g = _c(grid, np.uint8)
    codes = np.empty((rows, cols), dtype=np.int8)
    scales = np.empty((rows, cols // 32), dtype=np.float64)
    _check(lib().orc_cb_unpack_matrix(_ptr(c), rows, cols, _ptr(g), _ptr(codes), _ptr(scales)),
           "cb_unpack_matrix")
    return codes, scales


def cb_dequant_matrix(canon, rows: int, cols: int, grid):
    c = _c(canon, np.uint8)
    g = _c(grid, np.uint8)
    w = np.empty((rows, cols), dtype=np.float64)
    _check(lib().orc_cb_dequant_matrix(_ptr(c), rows, cols, _ptr(g), _ptr(w)), "cb_dequant_matrix")
    return w


def unpack_any(canon, rows: int, cols: int, bits: int, grid=None):
    return cb_unpack_matrix(canon, rows, cols, grid) if grid is not None else unpack_matrix(canon, rows, cols, bits)


def dequant_any(canon, rows: int, cols: int, bits: int, grid=None):
    return cb_dequant_matrix(canon, rows, cols, grid) if grid is not None else dequant_matrix(canon, rows, cols, bits)


def split_expert(canon, d: int, I: int, bits: int, grid=None):
    """Byte ranges of gate [I][d], up [I][d], down [d][I] inside one expert."""
    bb = block_bytes(bits, grid)
    g = I * (d // 32) * bb
    dn = d * (I // 32) * bb
    c = np.asarray(canon, dtype=np.uint8)
    return c[:g], c[g:2 * g], c[2 * g:2 * g + dn]


# ---------------------------------------------------------------------------
# router, top-k, FFN, layer
# ---------------------------------------------------------------------------
def router_logits(x, W, bias=None):
    x = _c(x, np.float32)
    W = _c(W, np.float32)
    T, d = x.shape
    E = W.shape[0]
    b = None if bias is None else _c(bias, np.float32)
    out = np.empty((T, E), dtype=np.float32)
    lib().orc_router_logits(_ptr(x), _ptr(W), _ptr(b), T, d, E, _ptr(out))
    return out


def topk(logits, k: int):
    """(idx [T,k] int32 in rank order, w [T,k] fp32 gate weights)."""
    l = _c(logits, np.float32)
    T, E = l.shape
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    _check(lib().orc_topk(_ptr(l), T, E, k, _ptr(idx), _ptr(w)), "topk")
    return idx, w


def expert_ffn(canon, d: int, I: int, bits: int, x, grid=None):
    c = _c(canon, np.uint8)
    xv = _c(x, np.float64)
    y = np.empty(d, dtype=np.float64)
    if grid is None:
        _check(lib().orc_expert_ffn(_ptr(c), d, I, bits, _ptr(xv), _ptr(y)), "expert_ffn")
    else:
        g = _c(grid, np.uint8)
        _check(lib().orc_expert_ffn_any(_ptr(c), d, I, bits, _ptr(g), _ptr(xv), _ptr(y)), "expert_ffn")
    return y


class Layer:
    """One MoE layer as the oracle sees it.

    ``experts`` maps expert id -> canonical bytes (numpy uint8).  Experts that
    the routing never selects may be left out.
    """

    def __init__(self, d, E, I, Is, k, bits, router_w, router_bias, experts, shared=None, grid=None):
        self.d, self.E, self.I, self.Is, self.k, self.bits = d, E, I, Is, k, bits
        self.grid = None if grid is None else _c(grid, np.uint8)
        self.router_w = _c(router_w, np.float32)
        self.router_bias = None if router_bias is None else _c(router_bias, np.float32)
        self.experts = {int(e): _c(v, np.uint8) for e, v in dict(experts).items()}
        self.shared = None if shared is None else _c(shared, np.uint8)

    def _struct(self):
        ptrs = (_P * self.E)()
        for e, v in self.experts.items():
            ptrs[e] = v.ctypes.data
        s = _Layer(self.d, self.E, self.I, self.Is, self.k, self.bits,
                   _ptr(self.router_w), _ptr(self.router_bias),
                   ctypes.cast(ptrs, _P), _ptr(self.shared), _ptr(self.grid))
        return s, ptrs


def layer_forward(layer: Layer, x, force_idx=None, force_w=None):
    """Returns (y [T,d] f32, logits [T,E] f32, idx [T,k] i32, w [T,k] f32).

    With ``force_idx``/``force_w`` the router's choice is replaced (teacher
    forcing with the GPU's own routing); logits are still computed.
    """
    x = _c(x, np.float32)
    T = x.shape[0]
    y = np.empty((T, layer.d), dtype=np.float32)
    logits = np.empty((T, layer.E), dtype=np.float32)
    idx = np.empty((T, layer.k), dtype=np.int32)
    w = np.empty((T, layer.k), dtype=np.float32)
    fi = None if force_idx is None else _c(force_idx, np.int32)
    fw = None if force_w is None else _c(force_w, np.float32)
    s, keep = layer._struct()
    rc = lib().orc_layer_forward(ctypes.byref(s), _ptr(x), T, _ptr(fi), _ptr(fw),
                                 _ptr(logits), _ptr(idx), _ptr(w), _ptr(y))
    del keep
    _check(rc, "layer_forward")
    return y, logits, idx, w


def rmsnorm(x, eps: float = 1e-6):
    x = _c(x, np.float32)
    T, d = x.shape
    y = np.empty_like(x)
    lib().orc_rmsnorm(_ptr(x), T, d, float(eps), _ptr(y))
    return y


def group_tokens(idx, E: int):
    """Counting sort of the (token, slot) pairs of a routing idx [T][k] by
    expert (see orc_group_tokens): returns (counts [E], offsets [E+1],
    perm [T*k]) as int32 arrays."""
    idx = _c(idx, np.int32)
    T, k = idx.shape
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    perm = np.zeros(T * k, np.int32)
    lib().orc_group_tokens(_ptr(idx), T, E, k, _ptr(counts), _ptr(offsets), _ptr(perm))
    return counts, offsets, perm
