"""CPU oracle for the W4A4 MXFP4 linear layer -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow reference that the HIP path is checked
against.  Only the test-suite, the smoke check and the CPU-baseline leg of the
benchmark may import it; the product path never does, and this package never
imports the product.  The arithmetic lives in ``mxfp4_oracle.c`` (plain C,
strict IEEE, no contraction); this module only marshals numpy arrays.

What it computes (page titles and sections as the pages give them):
  * MXFP4 block format -- "AMD Quark delivers MXFP4 quantization for FLUX.1-dev
    on Instinct MI350 with 1.92x speedup", section "What is MXFP4 and why does
    it eliminate dequantization overhead?" (32-element blocks, 4-bit elements,
    a shared scale; the OCP MX specification it names fixes E2M1 and E8M0).
  * power-of-two E8M0 scale, group size 32 -- "Bridging the Gap Between Promise
    and Performance for Microscaling FP4 Quantization", Technische
    samenvatting, "Probleemstelling".
  * block-wise Hadamard micro-rotation -- same page, "Methodologie: MR-GPTQ"
    item 1, and "GPU Kernel Ondersteuning (QuTLASS)" (online, fused).
  * Kronecker-factored block transform, inverse folded into the weights --
    "KroQuant: Effiziente Post-Training-Quantisierung fuer Diffusion
    Transformers mittels Kronecker-Produkt-Struktur", abstract, "Hintergrund"
    and "Tiefenanalyse".
  * the GEMM on MXFP4 operands -- the Quark page, section "MXFP4 quantization
    for diffusion models" (no dequantization pass; output written as
    bf16/fp32).
  * per-channel smoothing (the SmoothQuant baseline the KroQuant page compares
    against): one fp32 multiply per element by a per-channel factor; the
    weight side multiplies by the correctly rounded reciprocal.
  * MXFP4 scale fitting -- "Bridging the Gap ...", "Methodologie: MR-GPTQ"
    item 2: the block exponent re-fitted among e0 - 1, e0, e0 + 1 by the
    smallest binary64 squared error (the rule is a reading; see the C source).

Every function is pinned by the ``-m "not gpu"`` tests (tests/test_oracle_*).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle_mxfp4.so")
_lib = None

ROT_NONE, ROT_H32, ROT_KRON, ROT_SMOOTH = 0, 1, 2, 3

_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64
_int = ctypes.c_int


def _load():
    global _lib
    if _lib is not None:
        return _lib
    src = os.path.join(_HERE, "mxfp4_oracle.c")
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        from . import build as _b  # compiling the checker is not using it
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    sig = {
        "oracle_e2m1_value": (ctypes.c_double, [_int]),
        "oracle_e8m0_value": (ctypes.c_double, [_int]),
        "oracle_e8m0_from_amax": (_int, [ctypes.c_float]),
        "oracle_e2m1_index": (_int, [ctypes.c_float]),
        "oracle_e2m1_encode": (_int, [ctypes.c_float, _int]),
        "oracle_fwht32": (None, [_f32p, _f32p]),
        "oracle_kron_apply": (None, [_f32p, _int, _f32p, _int, _f32p, _f32p]),
        "oracle_inverse_transpose": (_int, [_f32p, _int, _f32p]),
        "oracle_smooth_weight_factors": (_int, [_f32p, _i64, _f32p]),
        "oracle_quantize_f32": (_int, [_f32p, _i64, _i64, _i64, _int, _f32p, _int, _f32p, _int, _u8p, _u8p]),
        "oracle_quantize_bf16": (_int, [_u16p, _i64, _i64, _i64, _int, _f32p, _int, _f32p, _int, _u8p, _u8p]),
        "oracle_quantize_f32_ex": (_int, [_f32p, _i64, _i64, _i64, _int, _f32p, _int, _f32p, _int, _int,
                                          _u8p, _u8p]),
        "oracle_quantize_bf16_ex": (_int, [_u16p, _i64, _i64, _i64, _int, _f32p, _int, _f32p, _int, _int,
                                           _u8p, _u8p]),
        "oracle_rotate_f32": (_int, [_f32p, _i64, _i64, _int, _f32p, _int, _f32p, _int, _f32p]),
        "oracle_dequantize": (None, [_u8p, _u8p, _i64, _i64, _f64p]),
        "oracle_gemm_entries": (None, [_u8p, _u8p, _u8p, _u8p, _i64, _i64p, _i64p, _i64, _f64p]),
        "oracle_e2m1_index_array": (None, [_f32p, _i64, _u8p]),
        "oracle_e2m1_encode_array": (None, [_f32p, _i64, _int, _u8p]),
        "oracle_e8m0_from_amax_array": (None, [_f32p, _i64, _u8p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


# ---------------------------------------------------------------- scalars ---

def e2m1_value(code: int) -> float:
    return _load().oracle_e2m1_value(int(code))


def e8m0_value(byte: int) -> float:
    return _load().oracle_e8m0_value(int(byte))


def e8m0_from_amax(amax) -> int:
    return _load().oracle_e8m0_from_amax(float(np.float32(amax)))


def e2m1_index(t) -> int:
    return _load().oracle_e2m1_index(float(np.float32(t)))


def e2m1_encode(y, e: int) -> int:
    return _load().oracle_e2m1_encode(float(np.float32(y)), int(e))


def e2m1_index_array(t: np.ndarray) -> np.ndarray:
    t = np.ascontiguousarray(t, dtype=np.float32).ravel()
    out = np.empty(t.size, np.uint8)
    _load().oracle_e2m1_index_array(t, t.size, out)
    return out


def e2m1_encode_array(y: np.ndarray, e: int) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float32).ravel()
    out = np.empty(y.size, np.uint8)
    _load().oracle_e2m1_encode_array(y, y.size, int(e), out)
    return out


def e8m0_from_amax_array(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32).ravel()
    out = np.empty(a.size, np.uint8)
    _load().oracle_e8m0_from_amax_array(a, a.size, out)
    return out


# -------------------------------------------------------------- rotations ---

def fwht32(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.shape == (32,)
    y = np.empty(32, np.float32)
    _load().oracle_fwht32(x, y)
    return y


def kron_apply(a: np.ndarray, b: np.ndarray, x: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    x = np.ascontiguousarray(x, dtype=np.float32)
    p, q = a.shape[0], b.shape[0]
    assert a.shape == (p, p) and b.shape == (q, q) and p * q == 32 and x.shape == (32,)
    y = np.empty(32, np.float32)
    _load().oracle_kron_apply(a, p, b, q, x, y)
    return y


def inverse_transpose(m: np.ndarray) -> np.ndarray:
    m = np.ascontiguousarray(m, dtype=np.float32)
    n = m.shape[0]
    out = np.empty((n, n), np.float32)
    if _load().oracle_inverse_transpose(m, n, out) != 0:
        raise ValueError("singular matrix")
    return out


def smooth_weight_factors(r: np.ndarray) -> np.ndarray:
    """Weight side of per-channel smoothing: fp32(1/r[c]) for the activation
    factors r (the quotient formed in binary64)."""
    r = np.ascontiguousarray(r, dtype=np.float32).ravel()
    out = np.empty(r.size, np.float32)
    if _load().oracle_smooth_weight_factors(r, r.size, out) != 0:
        raise ValueError("smoothing factors must be finite, nonzero, with finite fp32 reciprocals")
    return out


def _rot_args(rot):
    dummy = np.zeros(1, np.float32)
    if rot is None or rot == "none":
        return ROT_NONE, dummy, 1, dummy, 1
    if rot == "h32":
        return ROT_H32, dummy, 1, dummy, 1
    if rot[0] == "smooth":
        r = np.ascontiguousarray(rot[1], dtype=np.float32).ravel()
        return ROT_SMOOTH, r, 1, dummy, 1
    kind, a, b = rot
    assert kind == "kron"
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    return ROT_KRON, a, a.shape[0], b, b.shape[0]


def rotate(x: np.ndarray, rot) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, k = x.shape
    kind, a, p, b, q = _rot_args(rot)
    if kind == ROT_SMOOTH:
        assert a.size == k
    y = np.empty_like(x)
    if _load().oracle_rotate_f32(x, rows, k, kind, a, p, b, q, y) != 0:
        raise ValueError("bad arguments")
    return y


# -------------------------------------------------------------- quantizer ---

def quantize(x: np.ndarray, rot=None, bf16: bool = False, fit: bool = False):
    """Quantize rows of x to MXFP4.  x: float32 [rows, k], or uint16 bf16 bit
    patterns [rows, k] with bf16=True.  rot: None, "h32", ("kron", A, B) or
    ("smooth", r) with r the k per-channel factors.  fit: fitted block
    exponents instead of the E8M0 rule.  Returns (codes [rows, k/2] uint8,
    scales [rows, k/32] uint8)."""
    rows, k = x.shape
    kind, a, p, b, q = _rot_args(rot)
    if kind == ROT_SMOOTH:
        assert a.size == k
    codes = np.empty((rows, k // 2), np.uint8)
    scales = np.empty((rows, k // 32), np.uint8)
    if bf16:
        x = np.ascontiguousarray(x, dtype=np.uint16)
        rc = _load().oracle_quantize_bf16_ex(x, rows, k, k, kind, a, p, b, q, int(fit), codes, scales)
    else:
        x = np.ascontiguousarray(x, dtype=np.float32)
        rc = _load().oracle_quantize_f32_ex(x, rows, k, k, kind, a, p, b, q, int(fit), codes, scales)
    if rc != 0:
        raise ValueError("bad arguments")
    return codes, scales


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows, k = codes.shape[0], codes.shape[1] * 2
    assert scales.shape == (rows, k // 32)
    out = np.empty((rows, k), np.float64)
    _load().oracle_dequantize(codes, scales, rows, k, out)
    return out


# ------------------------------------------------------------------- GEMM ---

def gemm(a_codes, a_scales, b_codes, b_scales) -> np.ndarray:
    """Y = A_hat * B_hat^T in binary64: dequantize both operands exactly, then
    one library matmul in float64."""
    return dequantize(a_codes, a_scales) @ dequantize(b_codes, b_scales).T


def gemm_entries(a_codes, a_scales, b_codes, b_scales, mi, ni) -> np.ndarray:
    """Y[mi[t], ni[t]] in binary64 for sampled index pairs, one dot product
    each (usable at any size)."""
    a_codes = np.ascontiguousarray(a_codes, dtype=np.uint8)
    b_codes = np.ascontiguousarray(b_codes, dtype=np.uint8)
    a_scales = np.ascontiguousarray(a_scales, dtype=np.uint8)
    b_scales = np.ascontiguousarray(b_scales, dtype=np.uint8)
    k = a_codes.shape[1] * 2
    assert b_codes.shape[1] * 2 == k
    mi = np.ascontiguousarray(mi, dtype=np.int64)
    ni = np.ascontiguousarray(ni, dtype=np.int64)
    assert mi.shape == ni.shape
    assert (mi >= 0).all() and (mi < a_codes.shape[0]).all()
    assert (ni >= 0).all() and (ni < b_codes.shape[0]).all()
    out = np.empty(mi.size, np.float64)
    _load().oracle_gemm_entries(a_codes, a_scales, b_codes, b_scales, k, mi, ni, mi.size, out)
    return out
