"""Python binding of libpion_prefix.so: attention over a resident KV-cache prefix on
MI355X (gfx950).

Thin marshalling only: each function checks tensor device, dtype, contiguity and shape,
then calls the C entry point of the same name (include/pion_prefix.h) with raw device
pointers and the current HIP stream. Every step of the computation runs in the
library's HIP kernels; there is no fallback - if the library is missing, importing a
function that needs it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PION_OK = 0
PION_ERR_NOT_FOUND = -1
PION_ERR_INVALID = -2
PION_ERR_UNSUPPORTED = -3
PION_ERR_NOMEM = -4
PION_ERR_HIP = -5
PION_ERR_COLDMISS = -6
PION_ERR_SCRATCH = -7
PION_KV_FP16 = 0
PION_KV_MLX4G32 = 1
PION_KV_FP32 = 2

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpion_prefix.so")

# Every symbol include/pion_prefix.h declares, with its ctypes signature.
_c_char_p, _int, _vp = ctypes.c_char_p, ctypes.c_int, ctypes.c_void_p
SIGNATURES = {
    "pion_prefix_store": (_int, [_c_char_p, _int, _int, _int, _int, _vp, _vp, _int, _vp]),
    "pion_prefix_lookup": (_int, [_c_char_p, _int]),
    "pion_prefix_drop": (_int, [_c_char_p, _int]),
    "pion_prefix_info": (_int, [_c_char_p, _int, _vp, _vp, _vp, _vp]),
    "pion_prefix_stats": (_int, [_vp]),
    "pion_prefix_set_capacity": (_int, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]),
    "pion_prefix_query": (_int, [_c_char_p, _int, _int, _int, _int, _vp, _vp, _vp, _vp, _vp]),
    "pion_prefix_query_noalloc": (_int, [_c_char_p, _int, _int, _int, _int, _vp, _vp, _vp, _vp,
                                         _vp]),
    "pion_prefix_query_layers": (_int, [_c_char_p, _int, _int, _int, _int, _int, _vp, _vp, _vp,
                                        _vp, _vp]),
    "pion_prefix_query_fused": (_int, [_c_char_p, _int, _int, _int, _int, _int, _int,
                                       _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "pion_prefix_query_sparse_auto": (_int, [_c_char_p, _int, _int, _int, _int, _int, _int,
                                             _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "pion_prefix_query_sparse": (_int, [_c_char_p, _int, _int, _int, _int, _vp, _vp, _vp, _vp,
                                        _vp, _vp]),
    "pion_kv_quantize_mlx4g32": (_int, [_vp, ctypes.c_int64, _int, _vp, _vp, _vp, _vp]),
    "pion_vstore_fetch_f32": (_int, [_vp, _int, ctypes.c_int64, _int, ctypes.c_int64,
                                     ctypes.c_int64, _vp, _vp]),
    "pion_prefix_warm": (_int, [_c_char_p, _int, _int, _int, _int, _int, _vp, _vp, _int, _vp]),
    "pion_status_str": (ctypes.c_char_p, [_int]),
    "pion_prefix_last_plan": (ctypes.c_char_p, []),
    "pion_bench_stream_read": (_int, [_vp, ctypes.c_int64, _vp, _vp]),
    "pion_bench_mfma_peak": (_int, [_int, _vp, _vp, _vp]),
}

_lib = None


class PionError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} ({status})")


def lib() -> ctypes.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run kv_cache_prefix_amd/build.py")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def status_str(status: int) -> str:
    return lib().pion_status_str(status).decode()


def _check(rc: int, where: str) -> int:
    if rc < 0:
        raise PionError(rc, where)
    return rc


def _sid(sid) -> bytes:
    return sid.encode() if isinstance(sid, str) else bytes(sid)


def _stream(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t, dtype, name, shape=None):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _head_map(head_map, H_q):
    if head_map is None:
        return None, None
    import numpy as np
    arr = np.ascontiguousarray(np.asarray(head_map, dtype=np.int32))
    if arr.shape != (H_q,):
        raise ValueError("head_map must hold one int32 per q-head")
    return arr, arr.ctypes.data


def _fmt_dtype(kv_format: int):
    """Element type of the arrays a call passes for a slot of this format."""
    import torch
    return torch.float32 if kv_format == PION_KV_FP32 else torch.float16


def _slot_dtype(sid, layer: int):
    """Element type of Q and the suffix for the slot (sid, layer); fp16 if it has no warm
    slot (the call itself then reports the status)."""
    fmt = ctypes.c_int(PION_KV_FP16)
    lib().pion_prefix_info(_sid(sid), layer, None, None, None, ctypes.byref(fmt))
    return _fmt_dtype(fmt.value)


def pion_prefix_store(sid, layer: int, K, V, kv_format: int = PION_KV_FP16, stream=None) -> int:
    """ATTEND.PREFIX.STORE: K, V [H, N, D] device tensors (fp16; fp32 for PION_KV_FP32)
    -> resident slot."""
    if K.dim() != 3 or V.shape != K.shape:
        raise ValueError("K and V must both be [H, N, D]")
    H, N, D = K.shape
    dt = _fmt_dtype(kv_format)
    rc = lib().pion_prefix_store(_sid(sid), layer, H, N, D, _dev(K, dt, "K"), _dev(V, dt, "V"),
                                 kv_format, _stream(stream))
    return _check(rc, "pion_prefix_store")


def pion_prefix_lookup(sid, layer: int) -> int:
    return _check(lib().pion_prefix_lookup(_sid(sid), layer), "pion_prefix_lookup")


def pion_prefix_drop(sid, layer: int = -1) -> int:
    return _check(lib().pion_prefix_drop(_sid(sid), layer), "pion_prefix_drop")


def pion_prefix_info(sid, layer: int):
    vals = [ctypes.c_int() for _ in range(4)]
    rc = lib().pion_prefix_info(_sid(sid), layer, *[ctypes.byref(v) for v in vals])
    _check(rc, "pion_prefix_info")
    return tuple(v.value for v in vals)   # (H, N, D, kv_format)


class _Stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "warm_slots", "cold_slots", "demotions", "rehydrates", "resident_bytes",
        "max_slots", "max_bytes", "cold_capacity")]


def pion_prefix_stats() -> dict:
    """Slot-table telemetry: warm/cold counts, lifetime demotions and rehydrates,
    resident K/V bytes and the capacity in force."""
    st = _Stats()
    _check(lib().pion_prefix_stats(ctypes.byref(st)), "pion_prefix_stats")
    return {n: getattr(st, n) for n, _ in _Stats._fields_}


def pion_prefix_set_capacity(max_slots: int, max_bytes: int = 0, cold_slots: int = 1024) -> int:
    return _check(lib().pion_prefix_set_capacity(max_slots, max_bytes, cold_slots),
                  "pion_prefix_set_capacity")


def _vstore_rows(rows, fmt: int, kv_dim: int, name: str) -> int:
    """Pointer of a layer's V-store rows: fp16 [n, kv_dim] or uint8 mlx4g32 records
    [n, 5 * kv_dim / 8]."""
    import torch
    fp16 = fmt == PION_KV_FP16
    width = kv_dim if fp16 else kv_dim * 5 // 8
    if rows.dim() != 2 or rows.shape[1] != width:
        raise ValueError(f"{name} must be [n, {width}]")
    return _dev(rows, torch.float16 if fp16 else torch.uint8, name)


def pion_vstore_fetch_f32(rows, fmt: int, kv_dim: int, start: int, end: int, out,
                          stream=None) -> int:
    """V.FETCH RANGE: a layer's V-store rows (fp16 [n, kv_dim], or uint8 mlx4g32 records
    [n, 5 * kv_dim / 8]) -> out fp32 [end - start, kv_dim]."""
    import torch
    rp = _vstore_rows(rows, fmt, kv_dim, "rows")
    op = _dev(out, torch.float32, "out", (max(end - start, 0), kv_dim))
    rc = lib().pion_vstore_fetch_f32(rp, fmt, rows.shape[0], kv_dim, start, end, op,
                                     _stream(stream))
    return _check(rc, "pion_vstore_fetch_f32")


def pion_prefix_warm(sid, layer: int, H: int, D: int, K_rows, V_rows, src_format: int,
                     kv_format: int = PION_KV_FP16, stream=None) -> int:
    """KV.PREFIX.WARM for one layer: V-store rows of K and V (N tokens, src_format) ->
    slot (sid, layer) in kv_format, layout [H, N, D]."""
    kp_ = _vstore_rows(K_rows, src_format, H * D, "K_rows")
    vp_ = _vstore_rows(V_rows, src_format, H * D, "V_rows")
    if V_rows.shape != K_rows.shape:
        raise ValueError("K_rows and V_rows must have the same shape")
    rc = lib().pion_prefix_warm(_sid(sid), layer, H, K_rows.shape[0], D, src_format, kp_, vp_,
                                kv_format, _stream(stream))
    return _check(rc, "pion_prefix_warm")


def pion_prefix_query(sid, layer: int, Q, out, lse=None, head_map=None, stream=None) -> int:
    """ATTEND.PREFIX.QUERY (M >= 1): Q [H_q, M, D] (fp16; fp32 on an fp32 slot) ->
    out fp32 [H_q, M, D], lse [H_q, M]."""
    import torch
    H_q, M, D = Q.shape
    qt = _slot_dtype(sid, layer)
    hm, hm_ptr = _head_map(head_map, H_q)
    rc = lib().pion_prefix_query(
        _sid(sid), layer, H_q, D, M, _dev(Q, qt, "Q"), hm_ptr,
        _dev(out, torch.float32, "out", (H_q, M, D)),
        None if lse is None else _dev(lse, torch.float32, "lse", (H_q, M)), _stream(stream))
    return _check(rc, "pion_prefix_query")


def pion_prefix_query_layers(sid, layer0: int, Q, out, lse=None, head_map=None,
                             stream=None) -> int:
    """Layers layer0 .. layer0 + n - 1 in one launch: Q [n, H_q, M, D] (the slots'
    precision) -> out fp32 [n, H_q, M, D], lse fp32 [n, H_q, M]."""
    import torch
    n, H_q, M, D = Q.shape
    qt = _slot_dtype(sid, layer0)
    hm, hm_ptr = _head_map(head_map, H_q)
    rc = lib().pion_prefix_query_layers(
        _sid(sid), layer0, n, H_q, D, M, _dev(Q, qt, "Q"), hm_ptr,
        _dev(out, torch.float32, "out", (n, H_q, M, D)),
        None if lse is None else _dev(lse, torch.float32, "lse", (n, H_q, M)), _stream(stream))
    return _check(rc, "pion_prefix_query_layers")


def pion_prefix_query_fused(sid, layer: int, Q, K_suf, V_suf, out, lse=None, head_map=None,
                            H_kv: Optional[int] = None, stream=None) -> int:
    """ATTEND.PREFIX.QUERY_FUSED: Q [H_q, M, D], K_suf/V_suf [H_kv, S_suf, D] (fp16; fp32
    on an fp32 slot)."""
    import torch
    H_q, M, D = Q.shape
    qt = _slot_dtype(sid, layer)
    if K_suf is not None:
        H_kv_s, S_suf, _ = K_suf.shape
        H_kv = H_kv_s if H_kv is None else H_kv
        ks = _dev(K_suf, qt, "K_suf", (H_kv, S_suf, D))
        vs = _dev(V_suf, qt, "V_suf", (H_kv, S_suf, D))
    else:
        if H_kv is None:
            raise ValueError("H_kv is required without a suffix")
        S_suf, ks, vs = 0, None, None
    hm, hm_ptr = _head_map(head_map, H_q)
    rc = lib().pion_prefix_query_fused(
        _sid(sid), layer, H_q, D, M, S_suf, H_kv, _dev(Q, qt, "Q"), ks, vs, hm_ptr,
        _dev(out, torch.float32, "out", (H_q, M, D)),
        None if lse is None else _dev(lse, torch.float32, "lse", (H_q, M)), _stream(stream))
    return _check(rc, "pion_prefix_query_fused")


def pion_prefix_query_sparse_auto(sid, layer: int, Q, B: int, K_top: int, out, lse=None,
                                  blocks_out=None, K_suf=None, V_suf=None, head_map=None,
                                  H_kv: Optional[int] = None, stream=None) -> int:
    """ATTEND.PREFIX.QUERY_SPARSE_AUTO(_FUSED): Q [H_q, 1, D] (fp16; fp32 on an fp32 slot)
    -> out fp32 [H_q, D]."""
    import torch
    H_q, M, D = Q.shape
    qt = _slot_dtype(sid, layer)
    if M != 1:
        raise ValueError("sparse-auto takes one query row per head")
    if K_suf is not None:
        H_kv_s, S_suf, _ = K_suf.shape
        H_kv = H_kv_s if H_kv is None else H_kv
        ks = _dev(K_suf, qt, "K_suf", (H_kv, S_suf, D))
        vs = _dev(V_suf, qt, "V_suf", (H_kv, S_suf, D))
    else:
        if H_kv is None:
            raise ValueError("H_kv is required without a suffix")
        S_suf, ks, vs = 0, None, None
    hm, hm_ptr = _head_map(head_map, H_q)
    rc = lib().pion_prefix_query_sparse_auto(
        _sid(sid), layer, H_q, D, B, K_top, H_kv, S_suf, _dev(Q, qt, "Q"), ks, vs,
        hm_ptr, _dev(out, torch.float32, "out", (H_q, D)),
        None if lse is None else _dev(lse, torch.float32, "lse", (H_q,)),
        None if blocks_out is None else _dev(blocks_out, torch.int32, "blocks_out", (H_kv, K_top)),
        _stream(stream))
    return _check(rc, "pion_prefix_query_sparse_auto")


def pion_prefix_query_sparse(sid, layer: int, Q, indices, counts, out, lse=None,
                             stream=None) -> int:
    """ATTEND.PREFIX.QUERY_SPARSE: Q [H, 1, D] (fp16; fp32 on an fp32 slot), indices int32
    [H, K_sparse_max], counts int32 [H] -> out fp32 [H, D], lse fp32 [H]."""
    import torch
    H, M, D = Q.shape
    qt = _slot_dtype(sid, layer)
    if M != 1:
        raise ValueError("QUERY_SPARSE takes one query row per head")
    K_sparse_max = indices.shape[1]
    rc = lib().pion_prefix_query_sparse(
        _sid(sid), layer, H, D, K_sparse_max, _dev(Q, qt, "Q"),
        _dev(indices, torch.int32, "indices", (H, K_sparse_max)),
        _dev(counts, torch.int32, "counts", (H,)), _dev(out, torch.float32, "out", (H, D)),
        None if lse is None else _dev(lse, torch.float32, "lse", (H,)), _stream(stream))
    return _check(rc, "pion_prefix_query_sparse")


def pion_kv_quantize_mlx4g32(x, codes, scales, biases, stream=None) -> int:
    """mlx4g32 encoder: x fp16 [rows, D] -> codes int32 (uint32 bits) [rows, D/8],
    scales, biases fp16 [rows, D/32]."""
    import torch
    rows, D = x.shape
    rc = lib().pion_kv_quantize_mlx4g32(
        _dev(x, torch.float16, "x"), rows, D,
        _dev(codes, torch.int32, "codes", (rows, D // 8)),
        _dev(scales, torch.float16, "scales", (rows, D // 32)),
        _dev(biases, torch.float16, "biases", (rows, D // 32)), _stream(stream))
    return _check(rc, "pion_kv_quantize_mlx4g32")


def pion_prefix_last_plan() -> str:
    """Kernel names the calling thread's most recent library call enqueued ("" if none)."""
    return lib().pion_prefix_last_plan().decode()


def pion_bench_stream_read(buf, sink, stream=None) -> int:
    """Measurement aid: one plain streaming read of the whole device tensor `buf` (its
    byte size a multiple of 16); sink is a 1-element int32 device tensor."""
    import torch
    if not isinstance(buf, torch.Tensor) or not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous GPU tensor")
    rc = lib().pion_bench_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(),
                                      _dev(sink, torch.int32, "sink", (1,)), _stream(stream))
    return _check(rc, "pion_bench_stream_read")


def pion_bench_mfma_peak(iters, sink, stream=None) -> float:
    """Measurement aid: one launch of `iters` rounds of fp16 MFMA products on every SIMD;
    returns the launch's flop count. sink is a 1-element int32 device tensor."""
    import torch
    flops = ctypes.c_double(0.0)
    rc = lib().pion_bench_mfma_peak(int(iters), ctypes.byref(flops),
                                    _dev(sink, torch.int32, "sink", (1,)), _stream(stream))
    _check(rc, "pion_bench_mfma_peak")
    return flops.value


__all__ = [n for n in SIGNATURES if n != "pion_status_str"] + [
    "lib", "status_str", "PionError", "PION_KV_FP16", "PION_KV_MLX4G32", "LIB_PATH"]
