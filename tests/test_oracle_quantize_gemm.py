"""Pins of the oracle's block quantizer and GEMM.

Quantizer: 32-element blocks, one shared power-of-two scale, 4-bit elements
(Quark page, "What is MXFP4 and why does it eliminate dequantization
overhead?"; "Bridging the Gap ..." page, "Probleemstelling").  GEMM on MXFP4
operands with no dequantization pass (Quark page, "MXFP4 quantization for
diffusion models").
"""
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import workloads

MAGS = [Fraction(x) for x in ("0", "1/2", "1", "3/2", "2", "3", "4", "6")]


def decode_independent(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Decode with the minifloat definition, written separately from the
    oracle: low nibble = even element."""
    rows, kh = codes.shape
    k = 2 * kh
    nib = np.empty((rows, k), np.int64)
    nib[:, 0::2] = codes & 0xF
    nib[:, 1::2] = codes >> 4
    ef = (nib >> 1) & 3
    mf = nib & 1
    mag = np.where(ef == 0, 0.5 * mf, np.exp2(ef - 1.0) * (1.0 + 0.5 * mf))
    val = np.where(nib & 8, -mag, mag)
    return val * np.exp2(np.repeat(scales.astype(np.float64) - 127.0, 32, axis=1))


# --------------------------------------------------------------- quantizer ---

def test_quantize_error_bounds_and_scale_property():
    rng = np.random.default_rng(11)
    x = workloads.random_blocks(rng, 64, 512)
    codes, scales = oracle.quantize(x)
    xh = oracle.dequantize(codes, scales)
    assert np.array_equal(xh, decode_independent(codes, scales))
    xb = x.astype(np.float64).reshape(64, 16, 32)
    xhb = xh.reshape(64, 16, 32)
    s = np.exp2(scales.astype(np.float64) - 127.0)[:, :, None]
    t = np.abs(xb) / s
    amax_t = t.max(axis=2)
    assert ((amax_t >= 4) & (amax_t < 8)).all()             # top binade
    assert (np.abs(xhb) <= 6 * s).all()                      # saturating
    # half a grid step at the element's binade (elements below saturation)
    half = np.where(t < 2, 0.25, np.where(t < 4, 0.5, 1.0)) * s
    unsat = t <= 6
    assert (np.abs(xhb - xb)[unsat] <= half[unsat]).all()
    assert (np.abs(xhb[~unsat]) == 6 * np.broadcast_to(s, t.shape)[~unsat]).all()
    # sign always kept (code sign bit equals the input's sign bit)
    nib = np.empty(x.shape, np.int64)
    nib[:, 0::2] = codes & 0xF
    nib[:, 1::2] = codes >> 4
    assert np.array_equal((nib >> 3) & 1, np.signbit(x).astype(np.int64))


def test_grid_values_reproduce_exactly():
    rng = np.random.default_rng(12)
    for e in (-100, -3, 0, 7, 90):
        idx = rng.integers(0, 16, 32)
        idx[5] = 7                                            # 6 * 2^e sets amax
        vals = np.array([float(MAGS[i & 7]) * (-1 if i & 8 else 1) for i in idx])
        x = (vals * 2.0 ** e).astype(np.float32)[None, :]
        codes, scales = oracle.quantize(x)
        assert scales[0, 0] == e + 127
        assert np.array_equal(oracle.dequantize(codes, scales)[0], x[0].astype(np.float64))


def test_nibble_order_low_first():
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 0.5        # code 1 -> low nibble of byte 0
    x[0, 1] = 1.0        # code 2 -> high nibble of byte 0
    x[0, 31] = -6.0      # code 0xF -> high nibble of byte 15; sets amax, e = 0
    codes, scales = oracle.quantize(x)
    assert scales[0, 0] == 127
    assert codes[0, 0] == 0x21
    assert codes[0, 15] == 0xF0


def test_edge_blocks():
    x = np.zeros((6, 32), np.float32)
    x[1, :] = -0.0
    x[2, :] = np.float32(1e-45)                                    # min subnormal
    x[3, :] = np.float32(3.0e38)
    x[3, 1] = np.float32(-3.0e38)
    x[4, ::2] = np.float32(2.0 ** -130)                            # subnormal amax
    x[4, 1::2] = np.float32(2.0 ** -131)
    x[5, :] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0] * 4, np.float32)
    codes, scales = oracle.quantize(x)
    assert scales[0, 0] == 0 and (codes[0] == 0).all()
    assert scales[1, 0] == 0 and (codes[1] == 0x88).all()
    assert scales[2, 0] == 0                                       # clamp at 2^-127
    # min subnormal * 2^127 = 2^-22 -> rounds to 0
    assert (codes[2] == 0).all()
    assert scales[3, 0] == 252                                     # floor(log2 3e38) = 127
    assert codes[3, 0] == 0xF7                                     # +6, -6 (3e38/2^125 = 7.05)
    assert scales[4, 0] == 0
    # t = 2^-130 * 2^127 = 1/8 -> 0; 2^-131 -> 0
    assert (codes[4] == 0).all()
    # ties at e = 0: 0.25->0, 0.75->1, 1.25->1, 1.75->2, 2.5->2, 3.5->4, 5->4, 7->6
    assert scales[5, 0] == 127
    expect = [0x0, 0x2, 0x2, 0x4, 0x4, 0x6, 0x6, 0x7] * 4
    got = np.empty(32, np.int64)
    got[0::2] = codes[5] & 0xF
    got[1::2] = codes[5] >> 4
    assert got.tolist() == expect


def test_bf16_and_f32_entry_points_agree():
    rng = np.random.default_rng(13)
    x32 = workloads.random_blocks(rng, 16, 256)
    xb = workloads.bf16_bits(x32)
    xw = workloads.bf16_to_f32(xb)
    for rot in (None, "h32"):
        a = oracle.quantize(xb, rot=rot, bf16=True)
        b = oracle.quantize(xw, rot=rot)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_rotation_then_quantize_equals_quantize_of_rotated():
    rng = np.random.default_rng(14)
    x = rng.standard_normal((8, 128)).astype(np.float32)
    a = (np.eye(4) + 0.1 * rng.standard_normal((4, 4))).astype(np.float32)
    b = (np.eye(8) + 0.1 * rng.standard_normal((8, 8))).astype(np.float32)
    for rot in ("h32", ("kron", a, b)):
        c1, s1 = oracle.quantize(x, rot=rot)
        c2, s2 = oracle.quantize(oracle.rotate(x, rot))
        assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


@settings(max_examples=200, deadline=None)
@given(st.lists(st.floats(min_value=-2.0**100, max_value=2.0**100, allow_nan=False, width=32),
                min_size=32, max_size=32))
def test_property_roundtrip_error(vals):
    x = np.array(vals, np.float32)[None, :]
    codes, scales = oracle.quantize(x)
    xh = oracle.dequantize(codes, scales)[0]
    s = 2.0 ** (int(scales[0, 0]) - 127)
    assert np.all(np.abs(xh) <= 6 * s)
    amax = float(np.max(np.abs(x)))
    if amax > 2.0 ** -120:
        # error at most one grid step of the top binade
        assert np.all(np.abs(xh - x[0].astype(np.float64)) <= 2 * s + 1e-300)


# -------------------------------------------------------------------- GEMM ---

def exact_gemm(a_codes, a_scales, b_codes, b_scales):
    """Exact rational result: each product is an integer multiple of a power
    of two; sum with Fractions."""
    def vals(codes, scales):
        rows, kh = codes.shape
        out = []
        for r in range(rows):
            row = []
            for c in range(2 * kh):
                nib = (codes[r, c // 2] >> 4) if c & 1 else (codes[r, c // 2] & 0xF)
                v = MAGS[nib & 7] * (-1 if nib & 8 else 1)
                row.append(v * Fraction(2) ** (int(scales[r, c // 32]) - 127))
            out.append(row)
        return out
    av, bv = vals(a_codes, a_scales), vals(b_codes, b_scales)
    return [[sum((x * y for x, y in zip(ar, br)), Fraction(0)) for br in bv] for ar in av]


@pytest.mark.parametrize("m,n,k", [(1, 1, 32), (3, 5, 64), (8, 8, 128), (7, 2, 96)])
def test_gemm_tiny_against_exact_rationals(m, n, k):
    rng = np.random.default_rng(100 + m * n + k)
    ac, as_ = workloads.random_mxfp4(rng, m, k)
    bc, bs = workloads.random_mxfp4(rng, n, k)
    ref = exact_gemm(ac, as_, bc, bs)
    full = oracle.gemm(ac, as_, bc, bs)
    mi, ni = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
    ent = oracle.gemm_entries(ac, as_, bc, bs, mi.ravel(), ni.ravel()).reshape(m, n)
    absum = np.abs(decode_independent(ac, as_)) @ np.abs(decode_independent(bc, bs)).T
    for i in range(m):
        for j in range(n):
            tol = k * 2.0 ** -53 * absum[i, j]
            assert abs(Fraction(float(ent[i, j])) - ref[i][j]) <= Fraction(tol)
            assert abs(Fraction(float(full[i, j])) - ref[i][j]) <= Fraction(tol)


def test_gemm_unit_scales_match_numpy_matmul_of_decoded():
    rng = np.random.default_rng(15)
    ac = rng.integers(0, 256, (16, 64), dtype=np.uint8)
    bc = rng.integers(0, 256, (24, 64), dtype=np.uint8)
    s_a = np.full((16, 4), 127, np.uint8)
    s_b = np.full((24, 4), 127, np.uint8)
    ref = decode_independent(ac, s_a) @ decode_independent(bc, s_b).T
    # with unit scales all partial sums are multiples of 1/4 below 2^53: exact
    assert np.array_equal(oracle.gemm(ac, s_a, bc, s_b), ref)


def test_gemm_closed_form_constant_operands():
    k = 256
    ac = np.full((4, k // 2), 0x22, np.uint8)        # every element 1.0
    bc = np.full((5, k // 2), 0x11, np.uint8)        # every element 0.5
    s_a = np.full((4, k // 32), 127, np.uint8)
    s_b = np.full((5, k // 32), 127, np.uint8)
    assert (oracle.gemm(ac, s_a, bc, s_b) == k / 2).all()
    # scales multiply: 2^3 on A and 2^-5 on B -> K/2 * 2^-2
    assert (oracle.gemm(ac, s_a + 3, bc, s_b - 5) == k / 8).all()


def test_gemm_entries_match_full_at_samples():
    rng = np.random.default_rng(16)
    ac, as_ = workloads.random_mxfp4(rng, 40, 320)
    bc, bs = workloads.random_mxfp4(rng, 33, 320)
    full = oracle.gemm(ac, as_, bc, bs)
    mi = rng.integers(0, 40, 200)
    ni = rng.integers(0, 33, 200)
    ent = oracle.gemm_entries(ac, as_, bc, bs, mi, ni)
    np.testing.assert_allclose(ent, full[mi, ni], rtol=1e-14, atol=0)
