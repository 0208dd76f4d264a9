"""Oracle for the V-store side of the prefix cache: the per-token mlx4g32 record, the
dequantizing range fetch, and the rehydrate relayout into a resident slot.

TEST INFRASTRUCTURE ONLY (tests, smoke check, bench CPU baseline).

Sources:
  * V-store page, "The mlx4g32 tier" (same text in Shared KV Cache Serving,
    "Quantized tier - mlx4g32"): per token and layer, with kv_dim = H * D, a record
    of kv_dim/8 packed uint32 code words, then kv_dim/32 fp16 scales, then kv_dim/32
    fp16 biases (640 B at kv_dim = 1024). An fp16 V-store row is kv_dim fp16 values.
  * Shared KV Cache Serving, V.FETCH ... RANGE: one call returns the concatenated,
    dequantized fp32 values of a token range.
  * Shared KV Cache Serving, KV.PREFIX.WARM: per layer, dequantize the V-store rows to
    fp32, transpose [N, H*D] -> [H, N, D] (the STORE layout) and store them.

Readings where the pages are silent:
  * multi-byte fields are little-endian (the host order of the pages' machine);
  * dequantized fp32 = the exact s*q + b (fp64 here, where it is exact) rounded once to
    fp32; an fp16-resident slot then holds that fp32 value rounded to fp16 (RNE);
  * a rehydrate into an mlx4g32-resident slot keeps the record's codes, scales and
    biases as they are (no second quantization), so it equals storing the original
    fp16 K/V with the mlx4g32 format.
"""
from __future__ import annotations

import numpy as np

from .mlx4g32 import GROUP, dequantize, record_bytes

FP16, MLX4G32 = 0, 1


def pack_records(codes, scales, biases) -> np.ndarray:
    """Encoder output for N tokens (codes uint32 [N, kv/8], scales and biases fp16
    [N, kv/32]) -> records uint8 [N, record_bytes(kv)]."""
    codes = np.ascontiguousarray(codes, dtype="<u4")
    scales = np.ascontiguousarray(scales, dtype="<f2")
    biases = np.ascontiguousarray(biases, dtype="<f2")
    N = codes.shape[0]
    return np.concatenate([codes.view(np.uint8).reshape(N, -1),
                           scales.view(np.uint8).reshape(N, -1),
                           biases.view(np.uint8).reshape(N, -1)], axis=1)


def unpack_records(rec, kv_dim: int):
    """records uint8 [N, record_bytes(kv_dim)] -> (codes u32 [N, kv/8], scales f16
    [N, kv/32], biases f16 [N, kv/32])."""
    rec = np.ascontiguousarray(rec, dtype=np.uint8)
    N = rec.shape[0]
    assert rec.shape[1] == record_bytes(kv_dim)
    nc, ng = 4 * (kv_dim // 8), 2 * (kv_dim // GROUP)
    codes = rec[:, :nc].copy().view("<u4").reshape(N, kv_dim // 8)
    scales = rec[:, nc:nc + ng].copy().view("<f2").reshape(N, kv_dim // GROUP)
    biases = rec[:, nc + ng:].copy().view("<f2").reshape(N, kv_dim // GROUP)
    return codes, scales, biases


def fetch_f32(rows, fmt: int, kv_dim: int, start: int, end: int) -> np.ndarray:
    """V.FETCH RANGE: fp32 [end - start, kv_dim] of tokens start .. end - 1 of a V-store
    layer given as fp16 rows [N, kv_dim] (fmt FP16) or records (fmt MLX4G32)."""
    if fmt == FP16:
        return np.asarray(rows[start:end], np.float16).astype(np.float32)
    codes, scales, biases = unpack_records(rows[start:end], kv_dim)
    return dequantize(codes, scales, biases).astype(np.float32)


def warm_fp16(rows, fmt: int, H: int, D: int) -> np.ndarray:
    """KV.PREFIX.WARM into an fp16-resident slot: the [H, N, D] fp16 values it holds."""
    N = rows.shape[0]
    x = fetch_f32(rows, fmt, H * D, 0, N).astype(np.float16)
    return np.ascontiguousarray(x.reshape(N, H, D).transpose(1, 0, 2))
