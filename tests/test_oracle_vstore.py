"""Pins of the V-store oracle: the record layout the pages print (V-store page, "The
mlx4g32 tier"), checked byte by byte against the hand-worked group fixture packed with
`struct`; the dequantizing fetch against that fixture's hand-worked codes and the
quantizer's half-step bound; the WARM relayout against an element-by-element loop."""
import struct

import numpy as np
import pytest
from conftest import read_golden

from oracle import mlx4g32 as q4
from oracle import vstore


def golden_group():
    g = read_golden("mlx4g32_group.txt")
    x = np.array([float(v) for v in g["x"]], np.float16)[None, :]
    words = [int(w, 16) for w in g["words"]]
    return g, x, words, int(g["scale_bits"][0], 16), int(g["bias_bits"][0], 16)


def test_record_of_the_hand_worked_group_byte_by_byte():
    g, x, words, sbits, bbits = golden_group()
    rec = vstore.pack_records(*q4.quantize(x))
    assert rec.shape == (1, 20)
    assert rec[0].tobytes() == struct.pack("<4IHH", *words, sbits, bbits)


def test_record_size_and_field_order_at_kv_1024():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 1024)).astype(np.float16)
    codes, s, b = q4.quantize(x)
    rec = vstore.pack_records(codes, s, b)
    assert rec.shape == (3, 640)                                   # the printed 640 B/token
    for t in range(3):
        raw = rec[t].tobytes()
        assert struct.unpack("<128I", raw[:512]) == tuple(int(w) for w in codes[t])
        assert struct.unpack("<32H", raw[512:576]) == tuple(int(v) for v in s[t].view(np.uint16))
        assert struct.unpack("<32H", raw[576:]) == tuple(int(v) for v in b[t].view(np.uint16))
    back = vstore.unpack_records(rec, 1024)
    for u, v in zip(back, (codes, s, b)):
        np.testing.assert_array_equal(np.asarray(u).view(np.uint8), np.asarray(v).view(np.uint8))


def test_fetch_dequantizes_to_the_hand_worked_values():
    g, x, words, _, _ = golden_group()
    rec = vstore.pack_records(*q4.quantize(x))
    got = vstore.fetch_f32(rec, vstore.MLX4G32, 32, 0, 1)
    want = 0.5 * np.array([int(c) for c in g["codes"]], np.float64) - 2.0   # s * q + b
    assert got.dtype == np.float32
    np.testing.assert_array_equal(got[0], want.astype(np.float32))
    assert np.max(np.abs(got[0] - x[0].astype(np.float32))) == float(g["max_abs_dequant_error"][0])


@pytest.mark.parametrize("kv", [32, 96, 512])
def test_fetch_ranges_and_error_bound(kv):
    rng = np.random.default_rng(kv)
    x = (rng.standard_normal((50, kv)) * rng.lognormal(0, 1, (1, kv))).astype(np.float16)
    codes, s, b = q4.quantize(x)
    rec = vstore.pack_records(codes, s, b)
    full = vstore.fetch_f32(rec, vstore.MLX4G32, kv, 0, 50)
    np.testing.assert_array_equal(vstore.fetch_f32(rec, vstore.MLX4G32, kv, 7, 31), full[7:31])
    assert vstore.fetch_f32(rec, vstore.MLX4G32, kv, 9, 9).shape == (0, kv)
    # within half a quantization step (plus fp32 rounding) of the original value
    step = np.repeat(s.astype(np.float64), 32, axis=1)
    err = np.abs(full.astype(np.float64) - x.astype(np.float64))
    assert np.all(err <= step / 2 + 1e-6 * np.abs(x.astype(np.float64)) + 1e-30)
    # fp16 rows: the exact values
    np.testing.assert_array_equal(vstore.fetch_f32(x, vstore.FP16, kv, 3, 40),
                                  x[3:40].astype(np.float32))


@pytest.mark.parametrize("fmt", [vstore.FP16, vstore.MLX4G32])
def test_warm_relayout_matches_elementwise_loop(fmt):
    H, N, D = 3, 5, 64
    rng = np.random.default_rng(fmt)
    x = rng.standard_normal((N, H * D)).astype(np.float16)
    rows = x if fmt == vstore.FP16 else vstore.pack_records(*q4.quantize(x))
    got = vstore.warm_fp16(rows, fmt, H, D)
    vals = vstore.fetch_f32(rows, fmt, H * D, 0, N)
    assert got.shape == (H, N, D) and got.dtype == np.float16
    for h in range(H):
        for n in range(N):
            for d in range(D):
                assert got[h, n, d] == np.float16(vals[n, h * D + d])
    if fmt == vstore.FP16:
        np.testing.assert_array_equal(got.reshape(H, N * D)[1, :D], x[0, D:2 * D])
