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


def _fl(v: Fraction, mant: int, emin: int) -> Fraction:
    """v rounded to the binary format with `mant` fraction bits and minimum normal
    exponent `emin`, nearest with ties to even (gradual underflow below 2^emin)."""
    if v == 0:
        return Fraction(0)
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** (max(e, emin) - mant)
    r = round(a / quantum) * quantum        # Fraction.__round__: half to even
    return r if v > 0 else -r


def fl32(v):
    return _fl(v, 23, -126)


def fl16(v):
    r = _fl(v, 10, -14)
    assert abs(r) <= 65504
    return r


def _model_group(xs):
    """The encoder's steps on one group of fp16 values, each fp32 / fp16 operation
    rounded by hand from exact rationals: mn, mx exact; s32 = fl32(fl32(mx - mn) / 15);
    s = fl16(s32); b = fl16(mn); t_j = fl32(fl32(x_j - b) / s); q_j = clamp(rint(t_j)).
    Returns (codes, s, b) as rationals (codes a list of ints)."""
    fx = [Fraction(float(v)) for v in xs]
    mn, mx = min(fx), max(fx)
    s = fl16(fl32(fl32(mx - mn) / 15))
    b = fl16(mn)
    if s == 0:
        return [0] * len(fx), s, b
    codes = []
    for v in fx:
        t = fl32(fl32(v - b) / s)
        codes.append(min(max(round(t), 0), 15))
    return codes, s, b


def _near_tie_groups(n, seed):
    """Groups whose quotients (x - b) / s lie on, or one fp16 step either side of, the
    half-integers k + 0.5 for random fp16 scales: where any other fp32 evaluation order
    than (x - b) / s, or a product with 1 / s, can round to the other code."""
    rng = np.random.default_rng(seed)
    s = (2.0 ** rng.integers(-12, 6, n)) * rng.choice([1.0, 1.5, 1.25, 1.75, 1.375, 3.0 / 7], n)
    base = -rng.integers(0, 40, n) * s * (np.arange(n) % 2)   # bias 0 or -j s
    x = np.zeros((n, 32), np.float64)
    x[:, 0] = base
    x[:, 1] = base + 15.0 * s
    x[:, 2:] = base[:, None] + (rng.integers(0, 15, (n, 30)) + 0.5) * s[:, None]
    x16 = x.astype(np.float16)
    step = rng.integers(-1, 2, x16[:, 2:].shape)
    x16[:, 2:] = np.where(step < 0, np.nextafter(x16[:, 2:], np.float16(-np.inf)),
                          np.where(step > 0, np.nextafter(x16[:, 2:], np.float16(np.inf)),
                                   x16[:, 2:]))
    return x16


def test_each_code_is_the_nearest_level_brute_force():
    # the mathematical pin: every code is the level nearest x (ties to even), except
    # where the fp32 quotient lies within its rounding error of a half-integer; there the
    # exact-rational model of the fp32 steps below decides
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


@pytest.mark.parametrize("kind", ["random", "near_tie", "subnormal"])
def test_encoding_equals_exact_rational_model_of_the_fp32_steps(kind):
    # every element, near-ties included: codes, scale and bias equal a model that rounds
    # each fp32 (and fp16) operation by hand from exact rationals, so the op order
    # (x - b) / s with a correctly rounded divide is pinned, not only numpy's float32
    if kind == "random":
        x = _groups(160, 32, 21)
    elif kind == "near_tie":
        x = _near_tie_groups(400, 22)
    else:
        rng = np.random.default_rng(23)
        x = (rng.standard_normal((160, 32)) * 2.0 ** -16).astype(np.float16)
    codes, s16, b16 = oracle.quantize(x)
    q = oracle.unpack_codes(codes, 32)
    near = 0
    for r in range(len(x)):
        mc, ms, mb = _model_group(x[r])
        assert Fraction(float(s16[r, 0])) == ms and Fraction(float(b16[r, 0])) == mb, r
        assert list(q[r]) == mc, r
        if ms != 0:
            for v in x[r]:
                t = (Fraction(float(v)) - mb) / ms
                near += abs(abs(t - round(t)) - Fraction(1, 2)) < Fraction(1, 2 ** 18)
    if kind == "near_tie":
        assert near > 3000   # the window the nearest-level pin leaves to this model


def test_model_rounds_like_ieee_binary32():
    # the hand rounding itself: against exactly known binary32 results
    assert fl32(Fraction(1, 3)) == Fraction(float(np.float32(1) / np.float32(3)))
    assert fl32(Fraction(1) + Fraction(1, 2 ** 24)) == 1                    # tie -> even
    assert fl32(Fraction(1) + Fraction(3, 2 ** 24)) == 1 + Fraction(1, 2 ** 22)
    assert fl32(Fraction(1, 2 ** 150)) == 0 and fl32(Fraction(3, 2 ** 150)) == Fraction(1, 2 ** 148)
    assert fl16(Fraction(1, 3)) == Fraction(float(np.float16(1 / 3)))
    assert fl16(Fraction(3, 2 ** 26)) == Fraction(1, 2 ** 24)                # subnormal


def test_signed_zero_minimum_and_maximum():
    # -0 orders below +0: a zero minimum is -0 (bias bits 0x8000) if the group holds a -0,
    # whichever zero comes first; an all-zero group has scale +0 and all codes 0
    nz, pz = np.float16(-0.0), np.float16(0.0)
    x = np.zeros((6, 32), np.float16)
    x[0, 0], x[0, 1] = pz, nz            # +0 then -0
    x[1, 0], x[1, 1] = nz, pz            # -0 then +0
    x[2, :] = nz                         # all -0
    x[3, :] = pz                         # all +0
    x[4, :] = nz
    x[4, 7] = np.float16(2.5)            # -0 minimum with a positive range
    x[5, :] = np.float16(-1.0)
    x[5, 9], x[5, 10] = nz, pz           # zero maximum, negative minimum
    codes, s16, b16 = oracle.quantize(x)
    assert list(b16.view(np.uint16)[:, 0]) == [0x8000, 0x8000, 0x8000, 0x0000, 0x8000, 0xBC00]
    assert list(s16.view(np.uint16)[:, 0][:4]) == [0, 0, 0, 0]
    assert np.all(codes[:4] == 0)
    assert float(s16[4, 0]) == float(np.float16(np.float32(2.5) / np.float32(15)))
    xh = oracle.dequantize(codes, s16, b16)
    assert np.all(np.abs(xh - x.astype(np.float64)) <= s16.astype(np.float64).repeat(32, 1) / 2)


@pytest.mark.parametrize("bad", [np.inf, -np.inf, np.nan])
def test_non_finite_input_is_rejected(bad):
    x = np.zeros((2, 32), np.float16)
    x[1, 4] = bad
    with pytest.raises(ValueError):
        oracle.quantize(x)


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
