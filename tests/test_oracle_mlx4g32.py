"""Pins for the mlx4g32 oracle: the hand-worked group (tests/golden), the closed-form
record size the pages print, the dequantization error bound (at most half a step),
exact-rational brute force of each code, and the degenerate groups."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from conftest import read_golden


def test_hand_worked_group_bits():
    g = read_golden("mlx4g32_group.txt")
    x = np.array([float(v) for v in g["x"]], np.float16)[None, :]
    assert np.all(x.astype(np.float64) == np.array([float(v) for v in g["x"]]))
    codes, s16, b16 = oracle.quantize(x)
    assert [hex(int(w)) for w in codes[0]] == [w.lower() for w in g["words"]]
    assert int(s16.view(np.uint16)[0, 0]) == int(g["scale_bits"][0], 16)
    assert int(b16.view(np.uint16)[0, 0]) == int(g["bias_bits"][0], 16)
    assert list(oracle.unpack_codes(codes, 32)[0]) == [int(c) for c in g["codes"]]
    err = np.abs(oracle.dequantize(codes, s16, b16) - x.astype(np.float64)).max()
    assert err == float(g["max_abs_dequant_error"][0])


def test_record_size_closed_form():
    g = read_golden("mlx4g32_size.txt")
    D = int(g["D"][0])
    assert oracle.record_bytes(D) == int(g["mlx4g32_bytes_per_token"][0])
    assert 2 * D == int(g["fp16_bytes_per_token"][0])
    assert round(2 * D / oracle.record_bytes(D), 1) == 3.2
    # and the layout the quantizer actually emits has that many bytes
    codes, s, b = oracle.quantize(np.zeros((1, D), np.float16))
    assert codes.nbytes + s.nbytes + b.nbytes == oracle.record_bytes(D)


def _groups(n_rows, D, seed, outliers=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n_rows, D))
    if outliers:
        x = x * rng.lognormal(0, 0.5, size=(1, D))
    return x.astype(np.float16)


@pytest.mark.parametrize("D", [32, 64, 128, 256])
def test_dequant_error_at_most_half_a_step(D):
    x = _groups(2000, D, D)
    codes, s16, b16 = oracle.quantize(x)
    xh = oracle.dequantize(codes, s16, b16).reshape(2000, D // 32, 32)
    xd = x.astype(np.float64).reshape(2000, D // 32, 32)
    s = s16.astype(np.float64)[..., None]
    # half a step, plus the fp32 rounding of (x - b) and of the division (2 ulp of t)
    slack = s * 2.0 * 2.0 ** -23 * 16
    assert np.all(np.abs(xh - xd) <= s / 2 + slack)
    # the bound is tight: some element sits near half a step
    assert np.max(np.abs(xh - xd) / s) > 0.49


def test_each_code_is_the_nearest_level_brute_force():
    x = _groups(300, 64, 7)
    codes, s16, b16 = oracle.quantize(x)
    q = oracle.unpack_codes(codes, 64).reshape(300, 2, 32)
    xg = x.reshape(300, 2, 32)
    checked = 0
    for r in range(300):
        for G in range(2):
            s = Fraction(float(s16[r, G]))
            b = Fraction(float(b16[r, G]))
            if s == 0:
                assert np.all(q[r, G] == 0)
                continue
            for j in range(32):
                xv = Fraction(float(xg[r, G, j]))
                dist = [abs(xv - (s * c + b)) for c in range(16)]
                best = min(dist)
                cands = [c for c in range(16) if dist[c] == best]
                c = int(q[r, G, j])
                t = (xv - b) / s
                near_tie = abs(abs(t - round(t)) - Fraction(1, 2)) < Fraction(1, 2 ** 18)
                if len(cands) == 2:
                    assert c == [k for k in cands if k % 2 == 0][0]   # ties to even
                elif not near_tie:
                    assert c == cands[0]
                checked += 1
    assert checked > 15000


def test_constant_group_has_zero_scale_and_zero_codes():
    x = np.full((3, 32), 1.25, np.float16)
    codes, s16, b16 = oracle.quantize(x)
    assert np.all(codes == 0) and np.all(s16.view(np.uint16) == 0)
    np.testing.assert_array_equal(oracle.dequantize(codes, s16, b16), x.astype(np.float64))


def test_scale_underflowing_fp16_gives_zero_codes():
    # range 2^-26: (max-min)/15 rounds to fp16 zero, so codes are 0 and the reader sees min
    x = np.zeros((1, 32), np.float16)
    x[0, 5] = np.float16(2.0 ** -24)
    codes, s16, b16 = oracle.quantize(x)
    assert float(s16[0, 0]) == 0.0 and np.all(codes == 0)


def test_scale_is_rounded_to_fp16_before_codes():
    # (max-min)/15 = 1.1/15 is not an fp16 value; codes must use the fp16 scale the
    # reader sees, so a value at max maps back within half of THAT step.
    x = np.linspace(0, 1.1, 32).astype(np.float16)[None, :]
    codes, s16, b16 = oracle.quantize(x)
    s32 = (np.float32(x.max()) - np.float32(x.min())) / np.float32(15)
    assert float(s16[0, 0]) != float(s32)
    xh = oracle.dequantize(codes, s16, b16)
    assert np.abs(xh - x.astype(np.float64)).max() <= float(s16[0, 0]) / 2 * (1 + 1e-6)


def test_group_layout_matches_row_form_per_token_head():
    # groups never straddle heads (D_head % 32 == 0): quantizing [N, H*D] rows and
    # [H, N, D] rows gives the same bits
    inp = synth.generate(synth.MLX4_DECODE, N=64, H_q=6, H_kv=2, D=64)
    K = inp.K                                     # [H, N, D]
    c1, s1, b1 = oracle.quantize(K.reshape(-1, 64))
    rowform = np.ascontiguousarray(K.transpose(1, 0, 2)).reshape(64, 2 * 64)
    c2, s2, b2 = oracle.quantize(rowform)
    np.testing.assert_array_equal(c1.reshape(2, 64, 8), c2.reshape(64, 2, 8).transpose(1, 0, 2))
    np.testing.assert_array_equal(s1.reshape(2, 64, 2), s2.reshape(64, 2, 2).transpose(1, 0, 2))


def _fp16_ulp(v: Fraction) -> Fraction:
    if v < Fraction(1, 2 ** 14):
        return Fraction(1, 2 ** 24)
    e = 0
    while Fraction(2) ** (e + 1) <= v:
        e += 1
    while Fraction(2) ** e > v:
        e -= 1
    return Fraction(2) ** (e - 10)


def test_scale_is_within_half_an_fp16_ulp_of_exact_range_over_15():
    # Exact rationals: s16 must be the fp16 nearest (max-min)/15, up to the fp32
    # intermediate rounding (a 2^-24 relative window around fp16 midpoints).
    x = _groups(3000, 32, 11)
    _, s16, _ = oracle.quantize(x)
    xd = x.astype(np.float64)
    for r in range(3000):
        exact = (Fraction(float(xd[r].max())) - Fraction(float(xd[r].min()))) / 15
        s = Fraction(float(s16[r, 0]))
        half = _fp16_ulp(exact) / 2
        assert abs(s - exact) <= half * (1 + Fraction(1, 2 ** 12)), (r, float(s), float(exact))
