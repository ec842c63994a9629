"""Thin ctypes binding of libmoe_w4a16.so (include/moe_w4a16.h).

Argument marshalling only: every step of the layer runs in the HIP kernels of
the library.  Functions carry the C names; tensors are torch CUDA tensors (or
raw device addresses as ints), `stream` a torch.cuda.Stream, a raw hipStream_t
address, or None for torch's current stream.  A non-zero status raises
MoeError with the library's message.  If the library is not built, loading it
raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_w4a16.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE = 3
MOE_ERR_CAPACITY = 4
MOE_ERR_HIP = 5
MOE_ERR_FAULTED = 6
MOE_ERR_ABSENT_EXPERT = 7
MOE_ERR_SOURCE = 8
MOE_ERR_TIMEOUT = 9

MOE_SLOT_QPACKED = 0
MOE_SLOT_FP16 = 1

MOE_FFN_PATH_AUTO = 0
MOE_FFN_PATH_STREAM = 1
MOE_FFN_PATH_GEMM = 2
MOE_FFN_PATH_KSPLIT = 3
MOE_FFN_PATH_ONE_LAUNCH = 4

# Every symbol the header declares (checked by the CPU test suite).
EXPORTS = (
    "moe_version", "moe_last_error", "moe_expert_row_bytes",
    "moe_route_workspace_size", "moe_route", "moe_route_exact", "moe_route_static_max_bytes", "moe_route_static",
    "moe_w4a16_gateup", "moe_w4a16_down", "moe_w4a16_expert_ffn",
    "moe_combine", "moe_shared_ffn_workspace_size", "moe_shared_ffn", "moe_pack_fp16_tile8",
    "moe_layer_workspace_size", "moe_layer_forward", "moe_layer_forward_shared", "moe_residual_add",
    "moe_expert_row_bytes_fp16", "moe_dequant_expert_rows", "moe_fp16_expert_ffn",
    "moe_row_digest", "moe_table_create", "moe_table_destroy", "moe_table_device", "moe_table_misses",
    "moe_upload_expert_rows", "moe_table_prefetch", "moe_table_acquire", "moe_table_release", "moe_table_verify_source",
    "moe_table_stats", "moe_table_published",
)


class TableDesc(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int), ("H", ctypes.c_int), ("I", ctypes.c_int), ("capacity", ctypes.c_int),
                ("spare_rows", ctypes.c_int), ("staging_rows", ctypes.c_int), ("top_k", ctypes.c_int),
                ("max_tokens", ctypes.c_int), ("host_source", ctypes.c_void_p),
                ("host_row_stride", ctypes.c_size_t), ("initial_resident", ctypes.c_void_p),
                ("row_digests", ctypes.c_void_p), ("slot_format", ctypes.c_int)]


class LayerBuffers(ctypes.Structure):
    _fields_ = [("logits", ctypes.c_void_p), ("topk_ids", ctypes.c_void_p), ("topk_w", ctypes.c_void_p),
                ("expert_offsets", ctypes.c_void_p), ("sorted_pairs", ctypes.c_void_p), ("pair_pos", ctypes.c_void_p),
                ("active_list", ctypes.c_void_p), ("n_active", ctypes.c_void_p), ("h", ctypes.c_void_p),
                ("pair_out", ctypes.c_void_p), ("status", ctypes.c_void_p), ("ws", ctypes.c_void_p),
                ("ws_bytes", ctypes.c_size_t)]


class TableCounters(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in ("steps", "hits", "misses", "evictions", "h2d_bytes", "staging_waits",
                                               "expert_d2h_bytes", "host_writes", "generation", "open_leases",
                                               "failed_uploads", "prefetched", "prefetch_hits",
                                               "prefetch_unused", "direct_copies")]


class TableLease(ctypes.Structure):
    _fields_ = [("generation", ctypes.c_uint64), ("rows_dev", ctypes.c_void_p), ("row_stride", ctypes.c_size_t),
                ("slot_map_dev", ctypes.c_void_p)]


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[moe status {code}] {msg}")
        self.code = code


_lib = None
_vp = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t


def load(path: str = LIB_PATH):
    """Load the HIP library (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() (hipcc, gfx950) first")
    L = ctypes.CDLL(path)
    L.moe_version.restype = _i
    L.moe_version.argtypes = []
    L.moe_last_error.restype = ctypes.c_char_p
    L.moe_last_error.argtypes = []
    L.moe_expert_row_bytes.restype = _sz
    L.moe_expert_row_bytes.argtypes = [_i, _i, ctypes.POINTER(_sz)]
    L.moe_route_workspace_size.restype = _sz
    L.moe_route_workspace_size.argtypes = [_i, _i, _i]
    L.moe_route.restype = _i
    L.moe_route.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
    L.moe_route_exact.restype = _i
    L.moe_route_exact.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                  _vp]
    L.moe_route_static_max_bytes.restype = _sz
    L.moe_route_static_max_bytes.argtypes = []
    L.moe_route_static.restype = _i
    L.moe_route_static.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
    L.moe_w4a16_gateup.restype = _i
    L.moe_w4a16_gateup.argtypes = [_vp, _i, _i, _i, _i, _i, _vp, _sz, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp]
    L.moe_w4a16_down.restype = _i
    L.moe_w4a16_down.argtypes = [_i, _i, _i, _i, _i, _vp, _sz, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp]
    L.moe_w4a16_expert_ffn.restype = _i
    L.moe_w4a16_expert_ffn.argtypes = [_vp, _i, _i, _i, _i, _i, _vp, _sz, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                       _i, _vp]
    L.moe_combine.restype = _i
    L.moe_combine.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _vp, _vp]
    L.moe_shared_ffn_workspace_size.restype = _sz
    L.moe_shared_ffn_workspace_size.argtypes = [_i, _i, _i]
    L.moe_pack_fp16_tile8.restype = _i
    L.moe_pack_fp16_tile8.argtypes = [_vp, _vp, _i, _i, _vp]
    L.moe_shared_ffn.restype = _i
    L.moe_shared_ffn.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _vp, _vp, _vp, _sz, _vp]
    L.moe_row_digest.restype = ctypes.c_uint64
    L.moe_row_digest.argtypes = [_vp, _sz]
    L.moe_layer_workspace_size.restype = _sz
    L.moe_layer_workspace_size.argtypes = [_i, _i, _i, _i, _i]
    L.moe_layer_forward.restype = _i
    L.moe_layer_forward.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _sz, _vp, _vp, _vp, _vp, _vp,
                                    ctypes.POINTER(LayerBuffers), _i, _vp]
    L.moe_layer_forward_shared.restype = _i
    L.moe_layer_forward_shared.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _sz, _vp, _vp, _vp, _vp, _vp,
                                           _i, _vp, _vp, _vp, _sz, _vp, ctypes.POINTER(LayerBuffers), _i, _vp]
    L.moe_expert_row_bytes_fp16.restype = _sz
    L.moe_expert_row_bytes_fp16.argtypes = [_i, _i]
    L.moe_dequant_expert_rows.restype = _i
    L.moe_dequant_expert_rows.argtypes = [_vp, _sz, _vp, _sz, _i, _i, _i, _vp]
    L.moe_fp16_expert_ffn.restype = _i
    L.moe_fp16_expert_ffn.argtypes = [_vp, _i, _i, _i, _i, _i, _vp, _sz, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      _vp]
    L.moe_residual_add.restype = _i
    L.moe_residual_add.argtypes = [_vp, _vp, _vp, ctypes.c_longlong, _vp]
    L.moe_table_create.restype = _i
    L.moe_table_create.argtypes = [ctypes.POINTER(_vp), ctypes.POINTER(TableDesc), _vp]
    L.moe_table_destroy.restype = None
    L.moe_table_destroy.argtypes = [_vp]
    L.moe_table_device.restype = _i
    L.moe_table_device.argtypes = [_vp, ctypes.POINTER(_vp), ctypes.POINTER(_sz), ctypes.POINTER(_vp)]
    L.moe_table_misses.restype = _i
    L.moe_table_misses.argtypes = [_vp, _vp, _i, _vp, ctypes.POINTER(_i)]
    L.moe_upload_expert_rows.restype = _i
    L.moe_upload_expert_rows.argtypes = [_vp, _vp, _i, _vp]
    L.moe_table_prefetch.restype = _i
    L.moe_table_prefetch.argtypes = [_vp, _vp, _i]
    L.moe_table_acquire.restype = _i
    L.moe_table_acquire.argtypes = [_vp, _vp, ctypes.POINTER(TableLease)]
    L.moe_table_release.restype = _i
    L.moe_table_release.argtypes = [_vp, ctypes.POINTER(TableLease), _vp]
    L.moe_table_verify_source.restype = _i
    L.moe_table_verify_source.argtypes = [_vp]
    L.moe_table_stats.restype = _i
    L.moe_table_stats.argtypes = [_vp, ctypes.POINTER(TableCounters)]
    L.moe_table_published.restype = _i
    L.moe_table_published.argtypes = [_vp, _vp]
    _lib = L
    return L


def _p(t):
    """Device address of a tensor (or an int address, or None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _s(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int):
    if rc != MOE_OK:
        raise MoeError(rc, load().moe_last_error().decode())


# ------------------------------------------------------------------ queries
def moe_version() -> int:
    return load().moe_version()


def moe_last_error() -> str:
    return load().moe_last_error().decode()


def moe_expert_row_bytes(H: int, I: int):
    """(row_bytes, dict of the six section offsets)."""
    off = (_sz * 6)()
    rb = load().moe_expert_row_bytes(H, I, off)
    names = ("gate_q", "up_q", "down_q", "gate_s", "up_s", "down_s")
    return int(rb), {n: int(off[i]) for i, n in enumerate(names)}


def moe_route_workspace_size(T: int, H: int, E: int) -> int:
    return int(load().moe_route_workspace_size(T, H, E))


# ------------------------------------------------------------------ compute
def moe_route(x, w_router, bias, T, H, E, k, logits, topk_ids, topk_w, expert_offsets, sorted_pairs, pair_pos,
              active_list, n_active, ws, ws_bytes, stream=None):
    _check(load().moe_route(_p(x), _p(w_router), _p(bias), T, H, E, k, _p(logits), _p(topk_ids), _p(topk_w),
                            _p(expert_offsets), _p(sorted_pairs), _p(pair_pos), _p(active_list), _p(n_active),
                            _p(ws), ws_bytes, _s(stream)))


def moe_route_exact(x, w_router, bias, T, H, E, k, logits, topk_ids, topk_w, expert_offsets, sorted_pairs,
                    pair_pos, active_list, n_active, ws=None, ws_bytes=0, stream=None):
    _check(load().moe_route_exact(_p(x), _p(w_router), _p(bias), T, H, E, k, _p(logits), _p(topk_ids), _p(topk_w),
                                  _p(expert_offsets), _p(sorted_pairs), _p(pair_pos), _p(active_list),
                                  _p(n_active), _p(ws), ws_bytes, _s(stream)))


def moe_route_static_max_bytes() -> int:
    return int(load().moe_route_static_max_bytes())


def moe_route_static(x, w_router, bias, T, H, E, k, logits, topk_ids, topk_w, expert_offsets, sorted_pairs,
                     pair_pos, active_list, n_active, stream=None):
    _check(load().moe_route_static(_p(x), _p(w_router), _p(bias), T, H, E, k, _p(logits), _p(topk_ids),
                                   _p(topk_w), _p(expert_offsets), _p(sorted_pairs), _p(pair_pos),
                                   _p(active_list), _p(n_active), _s(stream)))


def moe_w4a16_gateup(x, T, H, I, E, k, rows, row_stride, slot_map, expert_offsets, sorted_pairs, active_list,
                     n_active, h, status=None, mode=MOE_FFN_PATH_AUTO, stream=None):
    _check(load().moe_w4a16_gateup(_p(x), T, H, I, E, k, _p(rows), row_stride, _p(slot_map), _p(expert_offsets),
                                   _p(sorted_pairs), _p(active_list), _p(n_active), _p(h), _p(status), mode,
                                   _s(stream)))


def moe_w4a16_down(T, H, I, E, k, rows, row_stride, slot_map, expert_offsets, active_list, n_active, h, pair_out,
                   status=None, mode=MOE_FFN_PATH_AUTO, stream=None):
    _check(load().moe_w4a16_down(T, H, I, E, k, _p(rows), row_stride, _p(slot_map), _p(expert_offsets),
                                 _p(active_list), _p(n_active), _p(h), _p(pair_out), _p(status), mode, _s(stream)))


def moe_w4a16_expert_ffn(x, T, H, I, E, k, rows, row_stride, slot_map, expert_offsets, sorted_pairs, active_list,
                         n_active, h, pair_out, status=None, mode=MOE_FFN_PATH_AUTO, stream=None):
    _check(load().moe_w4a16_expert_ffn(_p(x), T, H, I, E, k, _p(rows), row_stride, _p(slot_map),
                                       _p(expert_offsets), _p(sorted_pairs), _p(active_list), _p(n_active), _p(h),
                                       _p(pair_out), _p(status), mode, _s(stream)))


def moe_combine(pair_out, pair_pos, topk_w, shared_out, shared_gate, T, H, k, y, stream=None):
    _check(load().moe_combine(_p(pair_out), _p(pair_pos), _p(topk_w), _p(shared_out), _p(shared_gate), T, H, k,
                              _p(y), _s(stream)))


def moe_shared_ffn_workspace_size(T, H, Is) -> int:
    return int(load().moe_shared_ffn_workspace_size(T, H, Is))


def moe_shared_ffn(x, w_gate, w_up, w_down, w_sgate, T, H, Is, shared_out, shared_gate, ws, ws_bytes, stream=None):
    _check(load().moe_shared_ffn(_p(x), _p(w_gate), _p(w_up), _p(w_down), _p(w_sgate), T, H, Is, _p(shared_out),
                                 _p(shared_gate), _p(ws), ws_bytes, _s(stream)))


def moe_pack_fp16_tile8(src, dst, R, K, stream=None):
    _check(load().moe_pack_fp16_tile8(_p(src), _p(dst), R, K, _s(stream)))


def pack_tile8(w):
    """A new device tensor holding the tile8 layout of the row-major float16 device matrix w [R, K]
    (moe_pack_fp16_tile8 on the current stream)."""
    import torch
    R, K = w.shape
    out = torch.empty(R * K, dtype=torch.float16, device=w.device)
    moe_pack_fp16_tile8(w.contiguous(), out, R, K, torch.cuda.current_stream())
    return out


def moe_layer_workspace_size(T, H, I, E, k) -> int:
    return int(load().moe_layer_workspace_size(T, H, I, E, k))


def layer_buffers(logits, topk_ids, topk_w, expert_offsets, sorted_pairs, pair_pos, active_list, n_active, h,
                  pair_out, status, ws, ws_bytes) -> LayerBuffers:
    return LayerBuffers(_p(logits), _p(topk_ids), _p(topk_w), _p(expert_offsets), _p(sorted_pairs), _p(pair_pos),
                        _p(active_list), _p(n_active), _p(h), _p(pair_out), _p(status), _p(ws), ws_bytes)


def moe_layer_forward(x, w_router, bias, T, H, I, E, k, rows, row_stride, slot_map, shared_out, shared_gate,
                      shared_ready_event, y, buffers: LayerBuffers, mode=MOE_FFN_PATH_AUTO, stream=None):
    """shared_ready_event: a torch.cuda.Event, a raw hipEvent_t address, or None."""
    ev = shared_ready_event
    if ev is not None and not isinstance(ev, int):
        ev = ev.cuda_event
    _check(load().moe_layer_forward(_p(x), _p(w_router), _p(bias), T, H, I, E, k, _p(rows), row_stride,
                                    _p(slot_map), _p(shared_out), _p(shared_gate), ev, _p(y),
                                    ctypes.byref(buffers), mode, _s(stream)))


def moe_layer_forward_shared(x, w_router, bias, T, H, I, E, k, rows, row_stride, slot_map, w_sgate_proj, w_sup,
                             w_sdown, w_sgate, Is, shared_out, shared_gate, shared_ws, shared_ws_bytes, y,
                             buffers: LayerBuffers, mode=MOE_FFN_PATH_AUTO, stream=None):
    _check(load().moe_layer_forward_shared(_p(x), _p(w_router), _p(bias), T, H, I, E, k, _p(rows), row_stride,
                                           _p(slot_map), _p(w_sgate_proj), _p(w_sup), _p(w_sdown), _p(w_sgate), Is,
                                           _p(shared_out), _p(shared_gate), _p(shared_ws), shared_ws_bytes, _p(y),
                                           ctypes.byref(buffers), mode, _s(stream)))


def moe_expert_row_bytes_fp16(H: int, I: int) -> int:
    return int(load().moe_expert_row_bytes_fp16(H, I))


def moe_dequant_expert_rows(q_rows, q_stride, f_rows, f_stride, n, H, I, stream=None):
    _check(load().moe_dequant_expert_rows(_p(q_rows), q_stride, _p(f_rows), f_stride, n, H, I, _s(stream)))


def moe_fp16_expert_ffn(x, T, H, I, E, k, rows, row_stride, slot_map, expert_offsets, sorted_pairs, active_list,
                        n_active, h, pair_out, status=None, stream=None):
    _check(load().moe_fp16_expert_ffn(_p(x), T, H, I, E, k, _p(rows), row_stride, _p(slot_map),
                                      _p(expert_offsets), _p(sorted_pairs), _p(active_list), _p(n_active), _p(h),
                                      _p(pair_out), _p(status), _s(stream)))


def moe_residual_add(a, b, out, n, stream=None):
    _check(load().moe_residual_add(_p(a), _p(b), _p(out), n, _s(stream)))


# ------------------------------------------------------------------ resident expert table
def moe_row_digest(a) -> int:
    """Digest of a host buffer (numpy array), the identity moe_table_create checks."""
    import numpy as np
    a = np.ascontiguousarray(a)
    return int(load().moe_row_digest(a.ctypes.data, a.nbytes))


def moe_table_create(E, H, I, capacity, spare_rows, staging_rows, top_k, max_tokens, host_source, host_row_stride,
                     initial_resident=None, row_digests=None, stream=None, slot_format=MOE_SLOT_QPACKED):
    """host_source: a C-contiguous uint8 numpy array [E, host_row_stride] that must outlive the table.
    Returns the table handle (an int)."""
    import numpy as np
    init = None if initial_resident is None else np.ascontiguousarray(initial_resident, dtype=np.int32)
    dig = None if row_digests is None else np.ascontiguousarray(row_digests, dtype=np.uint64)
    d = TableDesc(E, H, I, capacity, spare_rows, staging_rows, top_k, max_tokens, host_source.ctypes.data,
                  host_row_stride, None if init is None else init.ctypes.data, None if dig is None else dig.ctypes.data,
                  slot_format)
    out = _vp()
    _check(load().moe_table_create(ctypes.byref(out), ctypes.byref(d), _s(stream)))
    return out.value


def moe_table_destroy(table):
    load().moe_table_destroy(table)


def moe_table_device(table):
    """(rows device address, row stride, slot map device address)."""
    rows, stride, smap = _vp(), _sz(), _vp()
    _check(load().moe_table_device(table, ctypes.byref(rows), ctypes.byref(stride), ctypes.byref(smap)))
    return rows.value, stride.value, smap.value


def moe_table_misses(table, active):
    """active: host int32 array of expert ids.  Returns the int32 array of misses."""
    import numpy as np
    act = np.ascontiguousarray(active, dtype=np.int32)
    miss = np.empty(max(len(act), 1), dtype=np.int32)
    n = _i()
    _check(load().moe_table_misses(table, act.ctypes.data if len(act) else None, len(act), miss.ctypes.data,
                                   ctypes.byref(n)))
    return miss[:n.value].copy()


def moe_upload_expert_rows(table, expert_ids, stream=None):
    import numpy as np
    ids = np.ascontiguousarray(expert_ids, dtype=np.int32)
    _check(load().moe_upload_expert_rows(table, ids.ctypes.data if len(ids) else None, len(ids), _s(stream)))


def moe_table_prefetch(table, expert_ids):
    import numpy as np
    ids = np.ascontiguousarray(expert_ids, dtype=np.int32)
    _check(load().moe_table_prefetch(table, ids.ctypes.data if len(ids) else None, len(ids)))


def moe_table_acquire(table, stream=None) -> TableLease:
    lease = TableLease()
    _check(load().moe_table_acquire(table, _s(stream), ctypes.byref(lease)))
    return lease


def moe_table_release(table, lease: TableLease, stream=None):
    _check(load().moe_table_release(table, ctypes.byref(lease), _s(stream)))


def moe_table_verify_source(table):
    _check(load().moe_table_verify_source(table))


def moe_table_stats(table) -> dict:
    c = TableCounters()
    _check(load().moe_table_stats(table, ctypes.byref(c)))
    return {n: int(getattr(c, n)) for n, _ in TableCounters._fields_}


def moe_table_published(table, E):
    import numpy as np
    m = np.empty(E, dtype=np.int32)
    _check(load().moe_table_published(table, m.ctypes.data))
    return m
