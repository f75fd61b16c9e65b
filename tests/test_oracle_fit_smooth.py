"""Pins of the oracle's MXFP4 scale fitting and per-channel smoothing.

Scale fitting ("Bridging the Gap Between Promise and Performance for
Microscaling FP4 Quantization", "Methodologie: MR-GPTQ" item 2 names it; the
rule is a reading): per block, the exponent among e0 - 1, e0, e0 + 1 (e0 the
E8M0 rule) with the smallest squared error; ties keep e0, then prefer e0 + 1.
Pinned against an independent exact computation (Python fractions over the
candidates' codes from the already-pinned scalar encoder), a hand-worked
block, and invariants (never worse than the plain rule; grid-exact blocks keep
e0).

Smoothing (the per-channel scaling the KroQuant page compares against): one
fp32 multiply by a per-channel factor before quantizing.  Pinned against numpy's
fp32 multiply followed by the unrotated quantizer, and against exact
power-of-two scaling.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads

E2M1 = [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def code_value(c: int) -> Fraction:
    v = Fraction(E2M1[c & 7]).limit_denominator()
    return -v if c & 8 else v


def exact_sse(v32: np.ndarray, e: int):
    """Codes of the block at exponent e (scalar encoder) and the exact squared
    error as a fraction."""
    codes = oracle.e2m1_encode_array(v32, e)
    s = Fraction(0)
    for x, c in zip(v32.tolist(), codes.tolist()):
        d = Fraction(x) - code_value(int(c)) * Fraction(2) ** e
        s += d * d
    return codes, s


def expected_fit(v32: np.ndarray):
    """Fitted exponent by the stated rule, with exact errors; also whether the
    decision is a near tie (relative gap below 1e-12)."""
    e0 = int(oracle.e8m0_from_amax(np.max(np.abs(v32)))) - 127
    cands = [e0, e0 + 1] + ([e0 - 1] if e0 > -127 else [])
    errs = {e: exact_sse(v32, e)[1] for e in cands}
    best = e0
    for e in cands[1:]:
        if errs[e] < errs[best]:
            best = e
    vals = sorted(errs.values())
    near = len(vals) > 1 and vals[1] - vals[0] <= abs(vals[1]) * Fraction(1, 10 ** 12) and vals[1] != vals[0]
    return best, errs, near


def unpack(codes_row: np.ndarray) -> np.ndarray:
    """Packed bytes -> one 4-bit code per element (low nibble first)."""
    out = np.empty(codes_row.size * 2, np.uint8)
    out[0::2] = codes_row & 0xF
    out[1::2] = codes_row >> 4
    return out


def test_fit_worked_example():
    # 7.9 and 31 x 0.3: at e = 0 the error is 1.9^2 + 31 * 0.2^2 = 4.85; at
    # e = 1 it is 0.1^2 + 31 * 0.3^2 = 2.80; at e = -1 7.9 saturates to 3.
    x = np.full((1, 32), 0.3, np.float32)
    x[0, 5] = 7.9
    c0, s0 = oracle.quantize(x)
    c1, s1 = oracle.quantize(x, fit=True)
    assert s0[0, 0] == 127 and s1[0, 0] == 128
    codes = unpack(c1[0])
    assert codes[5] == 0x6                       # 7.9 / 2 = 3.95 -> 4  (value 8)
    assert (np.delete(codes, 5) == 0).all()      # 0.3 / 2 = 0.15 -> 0
    _, errs, _ = expected_fit(x[0])
    assert float(errs[0]) == pytest.approx(4.85) and float(errs[1]) == pytest.approx(2.80)


def test_fit_chooses_the_finer_grid():
    # 4.0 and 31 x 0.75: e0 = 0, where 0.75 is a tie rounded to 1.0 (error
    # 31 * 0.25^2 = 1.9375); at e0 - 1 the 0.75 are exact and 4.0 saturates to
    # 3.0 (error 1.0); at e0 + 1 0.75 rounds to 1.0 as well (error 1.9375).
    x = np.full((1, 32), 0.75, np.float32)
    x[0, 0] = 4.0
    _, s0 = oracle.quantize(x)
    c1, s1 = oracle.quantize(x, fit=True)
    assert s0[0, 0] == 127 and s1[0, 0] == 126
    codes = unpack(c1[0])
    assert codes[0] == 0x7 and (codes[1:] == 0x3).all()   # 3.0 = 6 * 2^-1, 0.75 = 1.5 * 2^-1
    best, errs, _ = expected_fit(x[0])
    assert best == -1 and errs[-1] == 1 and errs[0] == Fraction(31, 16)


@pytest.mark.parametrize("seed", range(4))
def test_fit_matches_exact_argmin(seed):
    rng = np.random.default_rng(100 + seed)
    rows, k = 24, 256
    x = workloads.bf16_to_f32(workloads.bf16_bits(workloads.random_blocks(rng, rows, k)))
    if seed % 2:
        x[rng.random(x.shape) < 0.05] *= 9.0      # some outliers inside blocks
    codes, scales = oracle.quantize(x, fit=True)
    dcodes, dscales = oracle.quantize(x)
    near_ties = 0
    for r in range(rows):
        for b in range(k // 32):
            blk = x[r, 32 * b:32 * b + 32]
            best, errs, near = expected_fit(blk)
            if near:
                near_ties += 1
                continue
            assert scales[r, b] == best + 127, (r, b, errs)
            want = exact_sse(blk, best)[0]
            assert np.array_equal(unpack(codes[r, 16 * b:16 * b + 16]), want)
            # never worse than the plain rule
            assert errs[best] <= errs[int(dscales[r, b]) - 127]
    assert near_ties == 0


def test_fit_keeps_grid_exact_blocks():
    rng = np.random.default_rng(7)
    rows, k = 16, 512
    ac, as_ = workloads.random_mxfp4(rng, rows, k, -10, 10)
    x = oracle.dequantize(ac, as_).astype(np.float32)   # exactly representable blocks
    c0, s0 = oracle.quantize(x)
    c1, s1 = oracle.quantize(x, fit=True)
    assert np.array_equal(c0, c1) and np.array_equal(s0, s1)
    assert np.array_equal(oracle.dequantize(c1, s1), x.astype(np.float64))


def test_fit_edge_blocks():
    x = np.zeros((3, 32), np.float32)
    x[1, :] = np.float32(1e-45)                  # smallest subnormal: e0 = -127, no e0 - 1
    x[2, :] = np.float32(3.0e38)                 # near FLT_MAX: e0 = 125, e0 + 1 = 126
    c, s = oracle.quantize(x, fit=True)
    assert s[0, 0] == 0 and not c[0].any()
    assert s[1, 0] == 0
    assert s[2, 0] in (252, 253)
    best, _, _ = expected_fit(x[2])
    assert s[2, 0] == best + 127


def test_fit_with_rotation_never_worse():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((16, 256)).astype(np.float32)
    y = oracle.rotate(x, "h32")
    c0, s0 = oracle.quantize(x, rot="h32")
    c1, s1 = oracle.quantize(x, rot="h32", fit=True)
    e0 = (oracle.dequantize(c0, s0) - y) ** 2
    e1 = (oracle.dequantize(c1, s1) - y) ** 2
    blk0 = e0.reshape(16, -1, 32).sum(axis=2)
    blk1 = e1.reshape(16, -1, 32).sum(axis=2)
    assert (blk1 <= blk0 * (1 + 1e-12)).all()
    assert blk1.sum() < blk0.sum()


# --------------------------------------------------------------- smoothing ---

def test_smooth_unit_factors_is_identity():
    rng = np.random.default_rng(3)
    x = workloads.random_blocks(rng, 8, 256)
    r = np.ones(256, np.float32)
    assert all(np.array_equal(a, b) for a, b in zip(oracle.quantize(x, rot=("smooth", r)), oracle.quantize(x)))


def test_smooth_power_of_two_factors_are_exact():
    rng = np.random.default_rng(4)
    x = workloads.random_blocks(rng, 8, 256)
    j = rng.integers(-6, 7, 256)
    r = np.exp2(j).astype(np.float32)
    scaled = (x.astype(np.float64) * np.exp2(j)).astype(np.float32)   # exact
    got = oracle.quantize(x, rot=("smooth", r))
    want = oracle.quantize(scaled)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])


@pytest.mark.parametrize("bf16", [False, True])
def test_smooth_is_one_fp32_multiply(bf16):
    rng = np.random.default_rng(5 + bf16)
    x = workloads.random_blocks(rng, 16, 512)
    r = (0.25 + rng.random(512) * 4).astype(np.float32)
    if bf16:
        bits = workloads.bf16_bits(x)
        got = oracle.quantize(bits, rot=("smooth", r), bf16=True)
        xf = workloads.bf16_to_f32(bits)
    else:
        got = oracle.quantize(x, rot=("smooth", r))
        xf = x
    want = oracle.quantize(np.multiply(xf, r[None, :], dtype=np.float32))   # numpy's IEEE fp32 multiply
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
    # the rotation-only entry point applies the same multiply
    assert np.array_equal(oracle.rotate(xf, ("smooth", r)), np.multiply(xf, r[None, :], dtype=np.float32))


# ------------------------------------------------ smoothing, weight side ---
# The weight side of smoothing multiplies W by the reciprocal of the
# activation factor ("KroQuant: ...", the SmoothQuant comparison: the scaling
# the activations lose is folded into the weights).  The oracle forms it in
# binary64 and rounds to fp32; pinned here against the exact rational
# reciprocal, correctly rounded (ties to even), computed with fractions.

def correctly_rounded_reciprocal(r: float) -> float:
    q = 1 / Fraction(r)
    f = np.float32(float(q))          # within one fp32 step of the exact value
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    dist = [abs(Fraction(float(c)) - q) for c in cands]
    best = min(dist)
    ties = [c for c, d in zip(cands, dist) if d == best]
    if len(ties) > 1:                 # midpoint: the even significand wins
        ties = [c for c in ties if (int(np.float32(c).view(np.uint32)) & 1) == 0]
    return np.float32(ties[0])


def test_smooth_weight_factors_are_correctly_rounded_reciprocals():
    rng = np.random.default_rng(21)
    mant = rng.random(3000) + 1.0
    ex = rng.integers(-120, 121, 3000)
    r = (mant * np.exp2(ex) * rng.choice([-1.0, 1.0], 3000)).astype(np.float32)
    got = oracle.smooth_weight_factors(r)
    want = np.array([correctly_rounded_reciprocal(float(v)) for v in r], np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_smooth_weight_factors_worked_values():
    r = np.array([3.0, 0.1, 7.0, -0.75, 1.0], np.float32)
    got = oracle.smooth_weight_factors(r).view(np.uint32)
    # 1/3 rounds up to 0x3EAAAAAB; 1/0.1f is 9.99999985..., nearest fp32 is 10;
    # 1/7 = 0x3E124925; -1/0.75 = -4/3 = 0xBFAAAAAB; 1/1 = 1
    assert got.tolist() == [0x3EAAAAAB, 0x41200000, 0x3E124925, 0xBFAAAAAB, 0x3F800000]


def test_smooth_weight_factors_powers_of_two_exact():
    j = np.arange(-127, 128)
    r = np.exp2(j).astype(np.float32)
    got = oracle.smooth_weight_factors(r)
    assert np.array_equal(got, np.exp2(-j).astype(np.float32))


@pytest.mark.parametrize("bad", [0.0, -0.0, np.inf, -np.inf, np.nan, 2.0 ** -149])
def test_smooth_weight_factors_reject_unusable_factors(bad):
    with pytest.raises(ValueError):
        oracle.smooth_weight_factors(np.array([1.0, bad], np.float32))


def test_smooth_fold_preserves_block_products():
    """Unquantized, (x * r) . (w / r) = x . w to binary32 rounding."""
    rng = np.random.default_rng(22)
    k = 256
    x = rng.standard_normal((4, k)).astype(np.float32)
    w = rng.standard_normal((5, k)).astype(np.float32)
    r = (0.25 + 4 * rng.random(k)).astype(np.float32)
    wr = oracle.smooth_weight_factors(r)
    xs = oracle.rotate(x, ("smooth", r)).astype(np.float64)
    ws = np.multiply(w, wr[None, :], dtype=np.float32).astype(np.float64)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    bound = 4 * 2.0 ** -24 * (np.abs(x).astype(np.float64) @ np.abs(w).astype(np.float64).T)
    assert np.all(np.abs(xs @ ws.T - ref) <= bound)
