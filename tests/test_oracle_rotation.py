"""Pins of the oracle's block rotations.

Hadamard-32: "Bridging the Gap Between Promise and Performance for Microscaling
FP4 Quantization", "Methodologie: MR-GPTQ" item 1 (block-wise Hadamard on
weights and activations) and "GPU Kernel Ondersteuning (QuTLASS)" (online).
Kronecker transform: "KroQuant: ...", abstract and "Tiefenanalyse" (learned
Kronecker-structured invertible transform per 32-element block),
"Hintergrund" (its inverse goes on the weights).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle

U32 = 2.0 ** -24          # unit roundoff of binary32


def sylvester(n: int) -> np.ndarray:
    h = np.array([[1]], dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def popcount_hadamard(n: int) -> np.ndarray:
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    par = np.vectorize(lambda v: bin(int(v)).count("1") & 1)(i & j)
    return np.where(par == 1, -1, 1).astype(np.int64)


# ---------------------------------------------------------------- Hadamard ---

def test_hadamard_orthogonality_in_integers():
    hu = sylvester(32)
    assert np.array_equal(hu @ hu.T, 32 * np.eye(32, dtype=np.int64))
    assert np.array_equal(hu, hu.T)


def test_hadamard_kronecker_structure():
    h2 = np.array([[1, 1], [1, -1]], dtype=np.int64)
    k5 = h2
    for _ in range(4):
        k5 = np.kron(k5, h2)
    assert np.array_equal(k5, sylvester(32))
    assert np.array_equal(np.kron(sylvester(4), sylvester(8)), sylvester(32))
    assert np.array_equal(popcount_hadamard(32), sylvester(32))


def test_normalisation_constant_is_nearest_fp32():
    c = np.float32(1.0 / np.sqrt(32.0))
    assert c.view(np.uint32) == 0x3E3504F3
    # c is the fp32 nearest to 1/sqrt(32): compare squares exactly
    cf = Fraction(float(c))
    up = Fraction(float(np.nextafter(c, np.float32(1))))
    dn = Fraction(float(np.nextafter(c, np.float32(0))))
    target_sq = Fraction(1, 32)
    # 1/sqrt(32) lies within half an ulp of c
    lo = (cf + dn) / 2
    hi = (cf + up) / 2
    assert lo * lo < target_sq < hi * hi
    # and the oracle uses it: e_0 maps to c in every position
    y = oracle.fwht32(np.eye(32, dtype=np.float32)[0])
    assert (y.view(np.uint32) == 0x3E3504F3).all()


def test_fwht_of_unit_vectors_is_hadamard_column_times_c():
    c = np.float32(1.0 / np.sqrt(32.0))
    hu = sylvester(32)
    for j in range(32):
        e = np.zeros(32, np.float32)
        e[j] = 1.0
        y = oracle.fwht32(e)
        assert np.array_equal(y, (hu[:, j] * c).astype(np.float32)), j


def test_fwht_integer_inputs_exact():
    # small integers: every butterfly sum is exact, so before the final
    # multiply by c the result must equal Hu @ x exactly
    rng = np.random.default_rng(3)
    hu = sylvester(32)
    c = np.float32(1.0 / np.sqrt(32.0))
    for _ in range(50):
        x = rng.integers(-1000, 1000, 32)
        y = oracle.fwht32(x.astype(np.float32))
        assert np.array_equal(y, ((hu @ x).astype(np.float32) * c).astype(np.float32))


def test_fwht_matches_dense_within_fp32_bound():
    rng = np.random.default_rng(4)
    h = sylvester(32).astype(np.float64) / np.sqrt(32.0)
    for _ in range(200):
        x = (rng.standard_t(3, 32) * 2.0 ** rng.integers(-20, 20)).astype(np.float32)
        y = oracle.fwht32(x).astype(np.float64)
        ref = h @ x.astype(np.float64)
        # 5 rounded butterfly levels + rounded constant + rounded product
        bound = 8 * U32 * np.abs(x.astype(np.float64)).sum() / np.sqrt(32.0)
        assert np.max(np.abs(y - ref)) <= bound


def test_fwht_twice_is_identity_within_bound():
    rng = np.random.default_rng(5)
    for _ in range(100):
        x = rng.standard_normal(32).astype(np.float32)
        z = oracle.fwht32(oracle.fwht32(x)).astype(np.float64)
        bound = 20 * U32 * np.abs(x.astype(np.float64)).sum()
        assert np.max(np.abs(z - x)) <= bound


def test_rotate_h32_is_per_block():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((3, 96)).astype(np.float32)
    y = oracle.rotate(x, "h32")
    for r in range(3):
        for b in range(3):
            assert np.array_equal(y[r, 32 * b:32 * b + 32], oracle.fwht32(x[r, 32 * b:32 * b + 32]))


# --------------------------------------------------------------- Kronecker ---

def kron_bound(a, b, x, p, q):
    t_abs = np.kron(np.abs(a.astype(np.float64)), np.abs(b.astype(np.float64)))
    return (p + q + 2) * U32 * (t_abs @ np.abs(x.astype(np.float64)))


@pytest.mark.parametrize("p,q", [(4, 8), (8, 4), (2, 16), (1, 32), (32, 1)])
def test_kron_integer_inputs_exact(p, q):
    # small integer factors and inputs: every product and sum is exact in
    # fp32, so the oracle must equal (A (x) B) x exactly -- catches any
    # transposed factor or mixed-up index
    rng = np.random.default_rng(10 + p)
    for _ in range(20):
        a = rng.integers(-3, 4, (p, p))
        b = rng.integers(-3, 4, (q, q))
        x = rng.integers(-50, 50, 32)
        y = oracle.kron_apply(a.astype(np.float32), b.astype(np.float32), x.astype(np.float32))
        assert np.array_equal(y.astype(np.int64), np.kron(a, b) @ x)


@pytest.mark.parametrize("p,q", [(4, 8), (8, 4), (2, 16), (1, 32), (32, 1)])
def test_kron_matches_dense_within_fp32_bound(p, q):
    rng = np.random.default_rng(20 + p)
    for _ in range(50):
        a = (np.eye(p) + 0.1 * rng.standard_normal((p, p))).astype(np.float32)
        b = (np.eye(q) + 0.1 * rng.standard_normal((q, q))).astype(np.float32)
        x = rng.standard_normal(32).astype(np.float32)
        y = oracle.kron_apply(a, b, x).astype(np.float64)
        ref = np.kron(a.astype(np.float64), b.astype(np.float64)) @ x.astype(np.float64)
        assert np.all(np.abs(y - ref) <= kron_bound(a, b, x, p, q))


def test_kron_reproduces_hadamard_as_special_case():
    # H32 = H4 (x) H8 in Sylvester order; 1/2 * 1/sqrt(8) = 1/sqrt(32)
    a = (sylvester(4) / 2.0).astype(np.float32)
    b = (sylvester(8) / np.sqrt(8.0)).astype(np.float32)
    rng = np.random.default_rng(7)
    for _ in range(50):
        x = rng.standard_normal(32).astype(np.float32)
        yk = oracle.kron_apply(a, b, x).astype(np.float64)
        yh = oracle.fwht32(x).astype(np.float64)
        assert np.max(np.abs(yk - yh)) <= 24 * U32 * np.abs(x).sum()


def test_kron_identities_fp64():
    rng = np.random.default_rng(8)
    a = np.eye(4) + 0.1 * rng.standard_normal((4, 4))
    b = np.eye(8) + 0.1 * rng.standard_normal((8, 8))
    c = np.eye(4) + 0.1 * rng.standard_normal((4, 4))
    d = np.eye(8) + 0.1 * rng.standard_normal((8, 8))
    t = np.kron(a, b)
    assert np.allclose(np.linalg.inv(t), np.kron(np.linalg.inv(a), np.linalg.inv(b)), atol=1e-13, rtol=0)
    assert np.allclose(t @ np.kron(c, d), np.kron(a @ c, b @ d), atol=1e-13, rtol=0)
    assert np.allclose(np.linalg.inv(t).T, np.kron(np.linalg.inv(a).T, np.linalg.inv(b).T), atol=1e-13, rtol=0)


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32])
def test_inverse_transpose_against_library(n):
    rng = np.random.default_rng(30 + n)
    m = (np.eye(n) + 0.1 * rng.standard_normal((n, n))).astype(np.float32)
    got = oracle.inverse_transpose(m)
    ref = np.linalg.inv(m.astype(np.float64)).T
    # fp32 rounding of the fp64 inverse: within one fp32 ulp of the library's
    assert np.all(np.abs(got - ref) <= 1.0001 * np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64))
    # M^T * M^-T = I
    assert np.allclose(m.astype(np.float64).T @ got.astype(np.float64), np.eye(n), atol=1e-5)


def test_inverse_transpose_of_permutation_is_exact():
    p = np.eye(8, dtype=np.float32)[[3, 0, 7, 1, 2, 6, 5, 4]]
    assert np.array_equal(oracle.inverse_transpose(p), p)      # P^-T = P
    d = np.diag(np.array([2, 4, 0.5, 8, 1, 0.25, 16, 2], np.float32))
    assert np.array_equal(oracle.inverse_transpose(d), np.diag(1.0 / np.diag(d)).astype(np.float32))


def test_weight_fold_preserves_products():
    """(T x) . (T^-T w) = x . w: the activation transform and the weight-side
    factors A^-T, B^-T cancel in every block (before quantization)."""
    rng = np.random.default_rng(9)
    a = (np.eye(4) + 0.1 * rng.standard_normal((4, 4))).astype(np.float32)
    b = (np.eye(8) + 0.1 * rng.standard_normal((8, 8))).astype(np.float32)
    ait, bit = oracle.inverse_transpose(a), oracle.inverse_transpose(b)
    x = rng.standard_normal((8, 256)).astype(np.float32)
    w = rng.standard_normal((6, 256)).astype(np.float32)
    xt = oracle.rotate(x, ("kron", a, b)).astype(np.float64)
    wt = oracle.rotate(w, ("kron", ait, bit)).astype(np.float64)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    got = xt @ wt.T
    scale = np.abs(x).astype(np.float64) @ np.abs(w).astype(np.float64).T
    assert np.max(np.abs(got - ref) / scale) < 1e-5
