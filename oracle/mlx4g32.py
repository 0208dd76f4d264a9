"""Oracle for the mlx4g32 K/V encoding: int4 codes, group 32, affine, fp16 scale and bias.

TEST INFRASTRUCTURE ONLY (tests, smoke check, bench CPU baseline).

Source: Shared KV Cache Serving, "Quantized tier - mlx4g32", and the V-store page,
"The mlx4g32 tier". The pages fix: 4-bit codes in groups of 32, affine (a per-group
scale AND bias), fp16 scales and biases, element j of a group at bits 4*(j%8) of a
uint32, and that the scale is rounded to fp16 before the codes are chosen. They do
not print the constants; the reading taken here (15 levels, bias = group minimum,
scale = (max - min) / 15, codes by round-half-even and clamped to [0, 15]) is one
encoding that satisfies every stated fact. The steps run in fp32, in this order,
each op IEEE-rounded (numpy float32 arithmetic):

  1. mn = min_j x_j, mx = max_j x_j                      (exact)
  2. s32 = (mx - mn) / 15                                (two fp32 ops)
  3. s16 = fp16_rne(s32); s = float(s16)                 (the fp16 round trip)
  4. b16 = fp16_rne(mn);  b = float(b16)                 (exact: mn is an fp16 value)
  5. s16 == 0: every code 0; else t_j = (x_j - b) / s (two fp32 ops),
     q_j = clamp(rint_half_even(t_j), 0, 15)
  6. row element i -> word i // 8, bits 4 * (i % 8); group G's scale and bias at index G
  7. reader: x_hat = s * q + b  (fp64 here, where it is exact)

Two readings where the pages are silent, both part of the encoding here:
  * signed zeros: -0 orders below +0 (the minimum / maximum operations of IEEE 754-2019),
    so a group whose minimum is zero has bias -0 (bits 0x8000) when it holds a -0 and
    +0 otherwise, and a group whose maximum is zero has maximum +0 when it holds a +0;
    the scale (max - min) / 15 is then +0 for an all-zero group whatever its signs;
  * non-finite input (inf, NaN) is outside the encoder's domain: it is rejected here and
    the device encoder's result for such a group is unspecified.
"""
from __future__ import annotations

import numpy as np

GROUP = 32


def quantize(x16):
    """x16: fp16 [rows, D], D % 32 == 0 -> (codes uint32 [rows, D/8],
    scales fp16 [rows, D/32], biases fp16 [rows, D/32])."""
    x16 = np.asarray(x16)
    if x16.dtype != np.float16:
        raise TypeError("mlx4g32 input is fp16")
    rows, D = x16.shape
    if D % GROUP:
        raise ValueError("D must be a multiple of 32")
    if not np.all(np.isfinite(x16)):
        raise ValueError("mlx4g32 input must be finite")
    x = x16.astype(np.float32).reshape(rows, D // GROUP, GROUP)
    mn = x.min(axis=-1)                                   # step 1
    mx = x.max(axis=-1)
    # -0 below +0: a zero minimum is -0 if the group holds a -0, a zero maximum +0 if it
    # holds a +0 (numpy's reduction would return whichever zero it met first)
    is_zero = x == 0
    neg_zero = (is_zero & np.signbit(x)).any(axis=-1)
    pos_zero = (is_zero & ~np.signbit(x)).any(axis=-1)
    mn = np.where(mn == 0, np.where(neg_zero, np.float32(-0.0), np.float32(0.0)), mn)
    mx = np.where(mx == 0, np.where(pos_zero, np.float32(0.0), np.float32(-0.0)), mx)
    mn, mx = mn.astype(np.float32), mx.astype(np.float32)
    s32 = (mx - mn) / np.float32(15.0)                    # step 2 (fp32 / fp32)
    assert s32.dtype == np.float32
    s16 = s32.astype(np.float16)                          # step 3 (RNE)
    b16 = mn.astype(np.float16)                           # step 4
    s = s16.astype(np.float32)[..., None]
    b = b16.astype(np.float32)[..., None]
    zero = (s16 == 0)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (x - b) / np.where(zero, np.float32(1.0), s)  # step 5, fp32
    assert t.dtype == np.float32
    q = np.clip(np.rint(t), 0, 15)                        # rint: round half to even
    q = np.where(zero, 0, q).astype(np.uint32)
    q = q.reshape(rows, D // 8, 8)                        # step 6
    codes = np.zeros((rows, D // 8), dtype=np.uint32)
    for k in range(8):
        codes |= q[..., k] << np.uint32(4 * k)
    return codes, s16, b16


def unpack_codes(codes, D: int) -> np.ndarray:
    """codes uint32 [rows, D/8] -> int codes [rows, D] (element i at word i//8, bits 4*(i%8))."""
    codes = np.asarray(codes, dtype=np.uint32)
    rows = codes.shape[0]
    q = np.zeros((rows, D // 8, 8), dtype=np.int64)
    for k in range(8):
        q[..., k] = (codes >> np.uint32(4 * k)) & np.uint32(0xF)
    return q.reshape(rows, D)


def dequantize(codes, scales, biases) -> np.ndarray:
    """Reader side: x_hat = s * q + b per element, in fp64 (exact for fp16 s, b and q <= 15)."""
    scales = np.asarray(scales)
    rows, ng = scales.shape
    D = ng * GROUP
    q = unpack_codes(codes, D).astype(np.float64).reshape(rows, ng, GROUP)
    s = scales.astype(np.float64)[..., None]
    b = np.asarray(biases).astype(np.float64)[..., None]
    return (s * q + b).reshape(rows, D)


def record_bytes(D: int) -> int:
    """Bytes per token (per layer, per K or V side) of the record
    [uint32 x D/8][fp16 scales x D/32][fp16 biases x D/32]."""
    return 4 * (D // 8) + 2 * (D // GROUP) + 2 * (D // GROUP)
