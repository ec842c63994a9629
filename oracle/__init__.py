"""CPU oracle for the W4A16 routed-expert MoE layer (Python side).

TEST INFRASTRUCTURE ONLY: only tests/, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It wraps the plain C oracle in
moe_oracle.c (fp64 arithmetic, FP16 rounding at the layer's explicit rounding
points, exact router logits rounded once to FP32) with numpy-friendly calls.
It shares no code with the HIP library and never imports it.

Every function cites the page passage it follows in the C source.
Parity pins live in tests/test_oracle_pins.py.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_i32p = ctypes.POINTER(ctypes.c_int32)


def build() -> str:
    """Compile moe_oracle.c into liboracle.so (gcc, no fast-math, no FP contraction)."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-Wall",
                           "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        L.oracle_half_to_double.restype = ctypes.c_double
        L.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_double_to_half.restype = ctypes.c_uint16
        L.oracle_double_to_half.argtypes = [ctypes.c_double]
        L.oracle_weight.restype = ctypes.c_double
        L.oracle_weight.argtypes = [_u8p, _u16p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        L.oracle_dequant_matrix.argtypes = [_u8p, _u16p, ctypes.c_int, ctypes.c_int, _dp]
        L.oracle_row_offsets.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t),
                                         ctypes.POINTER(ctypes.c_size_t)]
        L.oracle_exact_dot_rn32.restype = ctypes.c_float
        L.oracle_exact_dot_rn32.argtypes = [_u16p, _u16p, ctypes.c_int, ctypes.c_int]
        L.oracle_router_logits.argtypes = [_u16p, _u16p, _fp, ctypes.c_int, ctypes.c_int, ctypes.c_int, _fp]
        L.oracle_topk_softmax.argtypes = [_fp, ctypes.c_int, ctypes.c_int, ctypes.c_int, _i32p, _dp]
        L.oracle_group.argtypes = [_i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _i32p, _i32p, _i32p,
                                   _i32p, _i32p]
        L.oracle_swiglu_dense.argtypes = [_dp, _dp, _dp, ctypes.c_int, ctypes.c_int, _u16p, _u16p, _dp]
        L.oracle_dequant_expert.argtypes = [_u8p, ctypes.c_int, ctypes.c_int, _dp, _dp, _dp]
        L.oracle_shared_ffn.argtypes = [_u16p, _u16p, _u16p, _u16p, _u16p, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, _dp, _dp]
        L.oracle_combine.argtypes = [_dp, _dp, _dp, _dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, _u16p]
        L.oracle_layer.restype = ctypes.c_int
        L.oracle_layer.argtypes = [_u16p, _u16p, _fp, _u8p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, _dp, _dp, _u16p, _fp, _i32p,
                                   _dp, _u16p, _dp]
        L.oracle_layer_fp16_slots.restype = ctypes.c_int
        L.oracle_layer_fp16_slots.argtypes = L.oracle_layer.argtypes
        L.oracle_dequant_expert_fp16.argtypes = [_u8p, ctypes.c_int, ctypes.c_int, _dp, _dp, _dp]
        L.oracle_halves_to_doubles.argtypes = [_u16p, _dp, ctypes.c_size_t]
        L.oracle_doubles_to_halves.argtypes = [_dp, _u16p, ctypes.c_size_t]
        _lib = L
    return _lib


def _ptr(a: np.ndarray, ctype):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _h(a) -> np.ndarray:
    """FP16 array (or its uint16 bits) -> contiguous uint16 bits."""
    a = np.asarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    assert a.dtype == np.uint16
    return np.ascontiguousarray(a)


# ------------------------------------------------------------------ FP16
def half_to_double(bits) -> np.ndarray:
    b = _h(bits)
    out = np.empty(b.shape, dtype=np.float64)
    lib().oracle_halves_to_doubles(_ptr(b, ctypes.c_uint16), _ptr(out, ctypes.c_double), b.size)
    return out


def double_to_half(v) -> np.ndarray:
    """fp64 -> FP16 bits (uint16), round to nearest even."""
    d = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(d.shape, dtype=np.uint16)
    lib().oracle_doubles_to_halves(_ptr(d, ctypes.c_double), _ptr(out, ctypes.c_uint16), d.size)
    return out


# ------------------------------------------------------------ qpacked read
def row_offsets(H: int, I: int):
    off = (ctypes.c_size_t * 6)()
    rb = ctypes.c_size_t()
    lib().oracle_row_offsets(H, I, off, ctypes.byref(rb))
    names = ("gate_q", "up_q", "down_q", "gate_s", "up_s", "down_s")
    d = {n: int(off[i]) for i, n in enumerate(names)}
    d["row_bytes"] = int(rb.value)
    return d


def weight(nib: np.ndarray, scales: np.ndarray, R: int, K: int, row: int, col: int) -> float:
    nib = np.ascontiguousarray(nib, dtype=np.uint8)
    sc = _h(scales)
    return lib().oracle_weight(_ptr(nib, ctypes.c_uint8), _ptr(sc, ctypes.c_uint16), R, K, row, col)


def dequant_matrix(nib: np.ndarray, scales, R: int, K: int) -> np.ndarray:
    nib = np.ascontiguousarray(nib, dtype=np.uint8)
    sc = _h(scales)
    assert nib.size == R * K // 2
    out = np.empty((R, K), dtype=np.float64)
    lib().oracle_dequant_matrix(_ptr(nib, ctypes.c_uint8), _ptr(sc, ctypes.c_uint16), R, K,
                                _ptr(out, ctypes.c_double))
    return out


def dequant_expert(row: np.ndarray, H: int, I: int, fp16: bool = False):
    """The three matrices of a qpacked expert row as doubles; fp16=True gives the offload-qpacked
    profile's FP16 execution-slot values (each weight rounded to FP16)."""
    row = np.ascontiguousarray(row, dtype=np.uint8)
    Wg = np.empty((I, H)); Wu = np.empty((I, H)); Wd = np.empty((H, I))
    f = lib().oracle_dequant_expert_fp16 if fp16 else lib().oracle_dequant_expert
    f(_ptr(row, ctypes.c_uint8), H, I, _ptr(Wg, ctypes.c_double), _ptr(Wu, ctypes.c_double),
      _ptr(Wd, ctypes.c_double))
    return Wg, Wu, Wd


# --------------------------------------------------------------- routing
def exact_dot_rn32(a, b) -> np.float32:
    a = _h(a); b = _h(b)
    assert a.size == b.size
    return np.float32(lib().oracle_exact_dot_rn32(_ptr(a, ctypes.c_uint16), _ptr(b, ctypes.c_uint16), a.size, 1))


def router_logits(x, wr, bias=None) -> np.ndarray:
    x = _h(x); wr = _h(wr)
    T, H = x.shape
    H2, E = wr.shape
    assert H == H2
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    out = np.empty((T, E), dtype=np.float32)
    lib().oracle_router_logits(_ptr(x, ctypes.c_uint16), _ptr(wr, ctypes.c_uint16), _ptr(b, ctypes.c_float),
                               T, H, E, _ptr(out, ctypes.c_float))
    return out


def topk_softmax(logits: np.ndarray, k: int):
    l = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = l.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    lib().oracle_topk_softmax(_ptr(l, ctypes.c_float), T, E, k, _ptr(ids, ctypes.c_int32), _ptr(w, ctypes.c_double))
    return ids, w


def group(ids: np.ndarray, E: int):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    n = T * k
    offsets = np.empty(E + 1, dtype=np.int32)
    sorted_pairs = np.empty(n, dtype=np.int32)
    pair_pos = np.empty(n, dtype=np.int32)
    active = np.full(E, -1, dtype=np.int32)
    n_active = np.zeros(1, dtype=np.int32)
    lib().oracle_group(_ptr(ids, ctypes.c_int32), T, E, k, _ptr(offsets, ctypes.c_int32),
                       _ptr(sorted_pairs, ctypes.c_int32), _ptr(pair_pos, ctypes.c_int32),
                       _ptr(active, ctypes.c_int32), _ptr(n_active, ctypes.c_int32))
    return dict(offsets=offsets, sorted_pairs=sorted_pairs, pair_pos=pair_pos,
                active=active[:int(n_active[0])].copy(), n_active=int(n_active[0]))


# ------------------------------------------------------------ expert FFN
def swiglu_dense(Wg, Wu, Wd, x_row):
    Wg = np.ascontiguousarray(Wg, dtype=np.float64)
    Wu = np.ascontiguousarray(Wu, dtype=np.float64)
    Wd = np.ascontiguousarray(Wd, dtype=np.float64)
    I, H = Wg.shape
    x = _h(x_row)
    h = np.empty(I, dtype=np.uint16)
    o = np.empty(H, dtype=np.float64)
    lib().oracle_swiglu_dense(_ptr(Wg, ctypes.c_double), _ptr(Wu, ctypes.c_double), _ptr(Wd, ctypes.c_double),
                              H, I, _ptr(x, ctypes.c_uint16), _ptr(h, ctypes.c_uint16), _ptr(o, ctypes.c_double))
    return h, o


def shared_ffn(x, Wsg, Wsu, Wsd, wgate):
    x = _h(x); Wsg = _h(Wsg); Wsu = _h(Wsu); Wsd = _h(Wsd); wgate = _h(wgate)
    T, H = x.shape
    Is = Wsg.shape[0]
    os_ = np.empty((T, H), dtype=np.float64)
    sig = np.empty(T, dtype=np.float64)
    lib().oracle_shared_ffn(_ptr(x, ctypes.c_uint16), _ptr(Wsg, ctypes.c_uint16), _ptr(Wsu, ctypes.c_uint16),
                            _ptr(Wsd, ctypes.c_uint16), _ptr(wgate, ctypes.c_uint16), T, H, Is,
                            _ptr(os_, ctypes.c_double), _ptr(sig, ctypes.c_double))
    return os_, sig


def combine(o, w, os_=None, sigma=None):
    o = np.ascontiguousarray(o, dtype=np.float64)
    w = np.ascontiguousarray(w, dtype=np.float64)
    T, k = w.shape
    H = o.shape[1]
    y = np.empty((T, H), dtype=np.uint16)
    os_p = None if os_ is None else np.ascontiguousarray(os_, dtype=np.float64)
    sg_p = None if sigma is None else np.ascontiguousarray(sigma, dtype=np.float64)
    lib().oracle_combine(_ptr(o, ctypes.c_double), _ptr(w, ctypes.c_double), _ptr(os_p, ctypes.c_double),
                         _ptr(sg_p, ctypes.c_double), T, H, k, _ptr(y, ctypes.c_uint16))
    return y


# ------------------------------------------------------------ whole layer
def layer(x, wr, rows: np.ndarray, H: int, I: int, E: int, k: int, bias=None, shared=None, want_h=False,
          fp16_slots=False):
    """Oracle of the whole routed-expert layer.

    rows: uint8 [E, row_bytes] qpacked expert rows (expert e = rows[e]).
    shared: None or (Wsg, Wsu, Wsd, wgate) FP16 shared expert.
    fp16_slots: the offload-qpacked profile (expert weights rounded to FP16 before use).
    Returns dict(y=FP16 bits [T,H], logits, ids, w, o [T*k,H] by pair t*k+j, h (opt.), and grouping).
    """
    x = _h(x); wr = _h(wr)
    rows = np.ascontiguousarray(rows, dtype=np.uint8)
    T = x.shape[0]
    n = T * k
    row_bytes = rows.shape[1]
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    os_, sig = (None, None) if shared is None else shared_ffn(x, *shared)
    y = np.empty((T, H), dtype=np.uint16)
    logits = np.empty((T, E), dtype=np.float32)
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    o = np.empty((n, H), dtype=np.float64)
    h = np.empty((n, I), dtype=np.uint16) if want_h else None
    f = lib().oracle_layer_fp16_slots if fp16_slots else lib().oracle_layer
    rc = f(_ptr(x, ctypes.c_uint16), _ptr(wr, ctypes.c_uint16), _ptr(b, ctypes.c_float),
                            _ptr(rows, ctypes.c_uint8), row_bytes, T, H, I, E, k,
                            _ptr(os_, ctypes.c_double), _ptr(sig, ctypes.c_double),
                            _ptr(y, ctypes.c_uint16), _ptr(logits, ctypes.c_float), _ptr(ids, ctypes.c_int32),
                            _ptr(w, ctypes.c_double), _ptr(h, ctypes.c_uint16), _ptr(o, ctypes.c_double))
    if rc != 0:
        raise MemoryError("oracle_layer: allocation failed")
    out = dict(y=y, logits=logits, ids=ids, w=w, o=o, h=h, shared_os=os_, shared_sigma=sig)
    out.update(group(ids, E))
    return out
