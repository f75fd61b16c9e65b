"""Pins of the oracle's element and scale rules (E2M1 decode/encode, E8M0).

Each check compares the oracle with something other than itself: the generic
minifloat definition of E2M1, torch's own E8M0 decoder, exact rational
arithmetic, a closed-form threshold encoder, or hand-derived values.
Format source: the MX specification named on the Quark page ("What is MXFP4
and why does it eliminate dequantization overhead?"); power-of-two E8M0 scale
and group size 32: "Bridging the Gap ..." page, "Probleemstelling".
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- E2M1 ---

def minifloat_e2m1(code: int) -> Fraction:
    """Generic IEEE-style minifloat with 2 exponent bits (bias 1), 1 mantissa
    bit, subnormals at exponent field 0, no Inf/NaN."""
    s = (code >> 3) & 1
    ef = (code >> 1) & 3
    mf = code & 1
    if ef == 0:
        mag = Fraction(mf, 2)                       # 2^(1-bias) * 0.m
    else:
        mag = Fraction(2) ** (ef - 1) * (1 + Fraction(mf, 2))
    return -mag if s else mag


def load_golden_e2m1():
    rows = []
    with open(os.path.join(GOLDEN, "e2m1_codes.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                c, v = line.split()
                rows.append((int(c, 16), Fraction(v)))
    return rows


def test_e2m1_decode_all_codes_match_minifloat_definition():
    for code in range(16):
        assert Fraction(oracle.e2m1_value(code)) == minifloat_e2m1(code), code


def test_e2m1_decode_matches_golden_table():
    rows = load_golden_e2m1()
    assert len(rows) == 16
    for code, val in rows:
        assert Fraction(oracle.e2m1_value(code)) == val
    # the eight magnitudes of the element format
    mags = sorted({abs(v) for _, v in rows})
    assert mags == [Fraction(x) for x in ("0", "1/2", "1", "3/2", "2", "3", "4", "6")]


def e2m1_rne_exact(t: Fraction) -> int:
    """Round t >= 0 into E2M1 by the IEEE rule: spacing of t's binade,
    round-half-even on the exact quotient, saturate at the largest finite
    magnitude.  Returns the magnitude index 0..7."""
    assert t >= 0
    if t < 1:
        spacing = Fraction(1, 2)
    elif t < 2:
        spacing = Fraction(1, 2)
    elif t < 4:
        spacing = Fraction(1)
    else:
        spacing = Fraction(2)
    r = round(t / spacing) * spacing          # Fraction round: half to even
    if r > 6:
        r = Fraction(6)
    mags = [Fraction(x) for x in ("0", "1/2", "1", "3/2", "2", "3", "4", "6")]
    return mags.index(r)


def threshold_index(t: np.ndarray) -> np.ndarray:
    """Closed form of RNE + saturation into E2M1 (ties 0.25->0, 0.75->1,
    1.25->1, 1.75->2, 2.5->2, 3.5->4, 5->4)."""
    t = t.astype(np.float64)
    return ((t > 0.25).astype(np.int32) + (t >= 0.75) + (t > 1.25) + (t >= 1.75)
            + (t > 2.5) + (t >= 3.5) + (t > 5.0)).astype(np.uint8)


def all_bf16_finite_nonneg() -> np.ndarray:
    h = np.arange(0, 0x7F80, dtype=np.uint32)          # +0 .. largest finite
    return (h << 16).view(np.float32)


def test_e2m1_index_exhaustive_bf16_against_exact_rne():
    t = all_bf16_finite_nonneg()
    got = oracle.e2m1_index_array(t)
    # exact-rational IEEE rounding on the part of the range where it matters
    sel = t < 16
    for tv, g in zip(t[sel], got[sel]):
        assert g == e2m1_rne_exact(Fraction(float(tv))), float(tv)
    # everything at or above 16 saturates
    assert (got[~sel] == 7).all()


def test_e2m1_index_dense_fp32_sweep_against_threshold_form():
    # every fp32 in [0, 8) with the low 8 mantissa bits dropped, plus each
    # tie point and its two fp32 neighbours
    u = np.arange(0, 0x41000000, 256, dtype=np.uint32)
    t = u.view(np.float32)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, 8.0], np.float32)
    nb = np.concatenate([ties, np.nextafter(ties, np.float32(0)), np.nextafter(ties, np.float32(100))])
    t = np.concatenate([t, nb.astype(np.float32)])
    assert np.array_equal(oracle.e2m1_index_array(t), threshold_index(t))


def test_e2m1_ties_go_to_even_mantissa():
    expect = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for t, i in expect.items():
        assert oracle.e2m1_index(t) == i, t
    # saturation
    for t in (6.0, 6.5, 7.0, 7.999):
        assert oracle.e2m1_index(t) == 7


def test_e2m1_encode_sign_and_zero():
    assert oracle.e2m1_encode(0.0, 0) == 0x0
    assert oracle.e2m1_encode(-0.0, 0) == 0x8          # signed zero
    assert oracle.e2m1_encode(-0.1, 0) == 0x8          # rounds to -0
    assert oracle.e2m1_encode(0.1, 0) == 0x0
    for code in range(16):
        v = float(minifloat_e2m1(code))
        if code == 8:
            v = -0.0                       # Fraction has no signed zero
        for e in (-127, -20, 0, 20, 125):
            y = np.float32(math.ldexp(v, e))
            if y == 0 and code & 7:
                continue
            assert oracle.e2m1_encode(y, e) == code, (code, e)


def test_worked_block_amax_seven():
    # amax = 7: floor(log2 7) = 2, so e = 0 and the values are their own t.
    # 7 -> 6 (saturating; 7 is the 6|8 midpoint, rounds up to 8, clamps to 6)
    # 5 -> 4 (tie between 4 and 6, the even mantissa is 4)
    # 0.25 -> 0 (tie between 0 and 0.5)
    # -0.75 -> -1 (tie between 0.5 and 1, even mantissa is 1.0)
    assert oracle.e8m0_from_amax(7.0) == 127
    assert oracle.e2m1_encode(7.0, 0) == 0x7
    assert oracle.e2m1_encode(5.0, 0) == 0x6
    assert oracle.e2m1_encode(0.25, 0) == 0x0
    assert oracle.e2m1_encode(-0.75, 0) == 0xA


# ----------------------------------------------------------------- E8M0 ---

def test_e8m0_value_matches_torch_decoder():
    b = torch.arange(0, 255, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = np.array([oracle.e8m0_value(i) for i in range(255)])
    assert np.array_equal(got, ref)
    assert math.isnan(oracle.e8m0_value(255))


def exact_floor_log2(a: Fraction) -> int:
    """Largest integer n with 2^n <= a, by exact comparisons."""
    n = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** n > a:
        n -= 1
    while Fraction(2) ** (n + 1) <= a:
        n += 1
    return n


def test_e8m0_top_element_lands_in_top_binade():
    """Defining property of the shared exponent: with 2^e the block scale the
    largest magnitude maps into E2M1's top binade [4, 8) (emax = 2), unless
    the E8M0 range clamps (amax < 2^-125)."""
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        all_bf16_finite_nonneg()[1:],
        np.abs(rng.standard_normal(20000).astype(np.float32)) * np.float32(2.0) ** rng.integers(-140, 120, 20000).astype(np.float32),
    ]).astype(np.float32)
    vals = vals[(vals > 0) & np.isfinite(vals)]
    got = oracle.e8m0_from_amax_array(vals)
    for a, byte in zip(vals[::7], got[::7]):
        fa = Fraction(float(a))
        e = int(byte) - 127
        t = fa / Fraction(2) ** e
        if exact_floor_log2(fa) - 2 >= -127:
            assert Fraction(4) <= t < 8, (float(a), byte)
        else:
            assert e == -127 and t < 4


def test_e8m0_powers_of_two_and_neighbours():
    for k in range(-149, 128):
        a = np.float32(math.ldexp(1.0, k))
        fl = exact_floor_log2(Fraction(float(a)))
        assert fl == k
        assert oracle.e8m0_from_amax(a) == max(k - 2, -127) + 127
        dn = np.nextafter(a, np.float32(0))
        if dn > 0:
            assert oracle.e8m0_from_amax(dn) == max(k - 3, -127) + 127
        up = np.nextafter(a, np.float32(np.inf))
        if np.isfinite(up):
            assert oracle.e8m0_from_amax(up) == max(k - 2, -127) + 127


def test_e8m0_hand_values():
    # amax -> byte, derived by hand from floor(log2(amax)) - 2 + 127
    cases = {1.0: 125, 3.99: 126, 4.0: 127, 6.0: 127, 7.0: 127, 8.0: 128,
             0.5: 124, 1e-40: 0, 0.0: 0, 3.4e38: 252}
    for a, byte in cases.items():
        assert oracle.e8m0_from_amax(a) == byte, a
