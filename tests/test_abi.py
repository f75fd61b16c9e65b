"""Boundary checks that need no GPU: the library loads, exports every symbol
include/mxfp4.h declares, and rejects bad arguments synchronously (before any
device work).  The host-side Kronecker fold helper is compared with the
oracle's.  No compute call reaches the device here."""
import ctypes
import os
import re

import numpy as np
import pytest

import mxfp4_w4a4_quantized_amd as mx
import oracle
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxfp4.h")

NULL = None
ALIGNED = 1 << 20          # arbitrary aligned address: never dereferenced
MISALIGNED = ALIGNED + 4


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"MXFP4_API\s+[\w\s\*]+?\b(mxfp4_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    syms = declared_symbols()
    assert syms == sorted(mx.EXPORTED)
    assert {"mxfp4_quantize_rotate", "mxfp4_gemm"} <= set(syms)


def test_library_loads_and_exports_every_declared_symbol():
    L = mx.lib()
    for s in declared_symbols():
        assert hasattr(L, s), s
    out = os.popen(f"nm -D --defined-only {mx.LIB_PATH}").read()
    exported = set(re.findall(r"\bT (mxfp4_\w+)", out))
    assert exported == set(declared_symbols())


def test_abi_version_and_status_strings():
    assert mx.lib().mxfp4_abi_version() == 4
    for s in range(4):
        assert mx.status_string(s).startswith("MXFP4_")
    assert "unknown" in mx.status_string(99)


def q(*args):
    return mx.lib().mxfp4_quantize_rotate(*args)


def g(*args):
    return mx.lib().mxfp4_gemm(*args)


def test_quantize_argument_errors():
    INV, UNS, OK = mx.MXFP4_ERR_INVALID_ARG, mx.MXFP4_ERR_UNSUPPORTED, mx.MXFP4_OK
    A, R, T = ALIGNED, mx.ROWMAJOR, mx.TILED
    assert q(A, 7, 4, 64, 64, None, R, A, A, None) == INV      # bad dtype
    assert q(A, 1, 4, 48, 64, None, R, A, A, None) == INV      # k % 32
    assert q(A, 1, 4, 0, 64, None, R, A, A, None) == INV       # k == 0
    assert q(A, 1, -1, 64, 64, None, R, A, A, None) == INV     # rows < 0
    assert q(A, 1, 4, 64, 32, None, R, A, A, None) == INV      # ld < k
    assert q(A, 1, 4, 64, 64, None, 2, A, A, None) == INV      # bad layout
    assert q(A, 1, 4, 64, 64, None, T, A, A, None) == INV      # tiled: k % 128
    assert q(NULL, 1, 4, 64, 64, None, R, A, A, None) == INV   # null x
    assert q(A, 1, 4, 64, 64, None, R, NULL, A, None) == INV   # null codes
    assert q(A, 1, 4, 64, 64, None, R, A, NULL, None) == INV   # null scales
    assert q(NULL, 1, 0, 64, 64, None, R, NULL, NULL, None) == OK   # rows == 0: no-op
    assert q(MISALIGNED, 1, 4, 64, 64, None, R, A, A, None) == UNS
    assert q(A, 1, 4, 64, 68, None, R, A, A, None) == UNS      # bf16 row stride not 16 B
    assert q(A, 1, 4, 64, 64, None, R, A + 8, A, None) == UNS  # codes not 16 B aligned
    assert q(A, 1, 4, 128, 128, None, T, A, A + 2, None) == UNS   # tiled scales not 4 B aligned
    assert q(A, 1, 1 << 30, 4096, 4096, None, R, A, A, None) == UNS   # too many blocks
    bad = mx.RotationDesc(9, 0, 0, 0, None, None)
    assert q(A, 1, 4, 64, 64, ctypes.byref(bad), R, A, A, None) == INV
    kr = mx.RotationDesc(mx.ROT_KRON, 4, 4, 0, A, A)
    assert q(A, 1, 4, 64, 64, ctypes.byref(kr), R, A, A, None) == INV     # p*q != 32
    kr = mx.RotationDesc(mx.ROT_KRON, 4, 8, 0, None, A)
    assert q(A, 1, 4, 64, 64, ctypes.byref(kr), R, A, A, None) == INV     # null factor
    kr = mx.RotationDesc(mx.ROT_KRON, 4, 8, 1, A, A)
    assert q(A, 1, 4, 64, 64, ctypes.byref(kr), R, A, A, None) == INV     # reserved != 0


def test_smooth_and_fit_argument_errors():
    INV, UNS = mx.MXFP4_ERR_INVALID_ARG, mx.MXFP4_ERR_UNSUPPORTED
    A, R = ALIGNED, mx.ROWMAJOR
    sm = mx.RotationDesc(mx.ROT_SMOOTH, 0, 0, 0, None, None)
    assert q(A, 1, 4, 64, 64, ctypes.byref(sm), R, A, A, None) == INV        # null factors
    sm = mx.RotationDesc(mx.ROT_SMOOTH, 0, 0, 0, A + 4, None)
    assert q(A, 1, 4, 64, 64, ctypes.byref(sm), R, A, A, None) == UNS        # factors not 16 B aligned
    fit = mx.lib().mxfp4_quantize_fit
    assert fit(A, 7, 4, 64, 64, None, R, A, A, None) == INV                  # same checks as quantize
    assert fit(A, 1, 4, 48, 64, None, R, A, A, None) == INV
    assert fit(NULL, 1, 4, 64, 64, None, R, A, A, None) == INV
    assert fit(MISALIGNED, 1, 4, 64, 64, None, R, A, A, None) == UNS
    assert fit(NULL, 1, 0, 64, 64, None, R, NULL, NULL, None) == mx.MXFP4_OK


def test_gemm_argument_errors():
    INV, UNS, OK = mx.MXFP4_ERR_INVALID_ARG, mx.MXFP4_ERR_UNSUPPORTED, mx.MXFP4_OK
    A, R, T = ALIGNED, mx.ROWMAJOR, mx.TILED
    assert g(A, A, 4, A, A, 4, 64, R, A, 5, 4, None) == INV     # bad dtype
    assert g(A, A, 4, A, A, 4, 48, R, A, 0, 4, None) == INV     # k % 32
    assert g(A, A, 4, A, A, 4, 0, R, A, 0, 4, None) == INV      # k == 0
    assert g(A, A, -4, A, A, 4, 64, R, A, 0, 4, None) == INV    # m < 0
    assert g(A, A, 4, A, A, -4, 64, R, A, 0, 4, None) == INV    # n < 0
    assert g(A, A, 4, A, A, 8, 64, R, A, 0, 4, None) == INV     # ld_y < n
    assert g(A, A, 4, A, A, 4, 64, 3, A, 0, 4, None) == INV     # bad layout
    assert g(A, A, 4, A, A, 4, 64, T, A, 0, 4, None) == INV     # tiled: k % 128
    assert g(NULL, A, 4, A, A, 4, 64, R, A, 0, 4, None) == INV
    assert g(A, NULL, 4, A, A, 4, 64, R, A, 0, 4, None) == INV
    assert g(A, A, 4, NULL, A, 4, 64, R, A, 0, 4, None) == INV
    assert g(A, A, 4, A, NULL, 4, 64, R, A, 0, 4, None) == INV
    assert g(A, A, 4, A, A, 4, 64, R, NULL, 0, 4, None) == INV
    assert g(NULL, NULL, 0, NULL, NULL, 4, 64, R, NULL, 0, 4, None) == OK   # m == 0
    assert g(NULL, NULL, 4, NULL, NULL, 0, 64, R, NULL, 0, 0, None) == OK   # n == 0
    assert g(A + 4, A, 4, A, A, 4, 64, R, A, 0, 4, None) == UNS   # misaligned codes
    assert g(A, A, 4, A + 8, A, 4, 64, R, A, 0, 4, None) == UNS
    assert g(A, A, 4, A, A, 4, 64, R, A + 2, 0, 4, None) == UNS   # fp32 y misaligned
    assert g(A, A + 1, 4, A, A, 4, 128, T, A, 0, 4, None) == UNS   # tiled scales misaligned
    assert g(A, A, 1 << 30, A, A, 4, 64, R, A, 0, 4, None) == UNS


def ls(*args):
    return mx.lib().mxfp4_linear_small(*args)


def test_linear_small_argument_errors():
    """Synchronous validation of the fused small-M linear entry point (no
    device access happens on any of these paths)."""
    INV, UNS, OK = mx.MXFP4_ERR_INVALID_ARG, mx.MXFP4_ERR_UNSUPPORTED, mx.MXFP4_OK
    A, R, T, BF, F = ALIGNED, mx.ROWMAJOR, mx.TILED, mx.MXFP4_BF16, mx.MXFP4_F32
    assert ls(A, 7, 4, 64, 64, None, A, A, 8, R, A, F, 8, NULL, 0, None) == INV    # bad x dtype
    assert ls(A, BF, 4, 64, 64, None, A, A, 8, R, A, 9, 8, NULL, 0, None) == INV   # bad y dtype
    assert ls(A, BF, 4, 64, 64, None, A, A, 8, 2, A, F, 8, NULL, 0, None) == INV   # bad layout
    assert ls(A, BF, 4, 48, 64, None, A, A, 8, R, A, F, 8, NULL, 0, None) == INV   # k % 32
    assert ls(A, BF, 4, 64, 64, None, A, A, 8, T, A, F, 8, NULL, 0, None) == INV   # tiled: k % 128
    assert ls(A, BF, 4, 64, 32, None, A, A, 8, R, A, F, 8, NULL, 0, None) == INV   # ld_x < k
    assert ls(A, BF, 4, 64, 64, None, A, A, 8, R, A, F, 4, NULL, 0, None) == INV   # ld_y < n
    assert ls(A, BF, -1, 64, 64, None, A, A, 8, R, A, F, 8, NULL, 0, None) == INV  # m < 0
    assert ls(NULL, BF, 4, 64, 64, None, A, A, 8, R, A, F, 8, NULL, 0, None) == INV
    assert ls(A, BF, 4, 64, 64, None, NULL, A, 8, R, A, F, 8, NULL, 0, None) == INV
    assert ls(A, BF, 4, 64, 64, None, A, A, 8, R, NULL, F, 8, NULL, 0, None) == INV
    assert ls(NULL, BF, 0, 64, 64, None, NULL, NULL, 8, R, NULL, F, 8, NULL, 0, None) == OK   # m == 0
    assert ls(A, BF, 65, 64, 64, None, A, A, 8, R, A, F, 8, NULL, 0, None) == UNS  # m > 64
    assert ls(A, F, 4, 64, 64, None, A, A, 8, R, A, F, 8, NULL, 0, None) == UNS    # fp32 activations
    assert ls(MISALIGNED, BF, 4, 64, 64, None, A, A, 8, R, A, F, 8, NULL, 0, None) == UNS
    assert ls(A, BF, 4, 64, 68, None, A, A, 8, R, A, F, 8, NULL, 0, None) == UNS   # row stride not 16 B
    assert ls(A, BF, 4, 64, 64, None, A + 8, A, 8, R, A, F, 8, NULL, 0, None) == UNS
    assert ls(A, BF, 4, 128, 128, None, A, A + 2, 8, T, A, F, 8, NULL, 0, None) == UNS   # tiled scales
    for p_, q_ in ((1, 32), (32, 1)):
        kr = mx.RotationDesc(mx.ROT_KRON, p_, q_, 0, A, A)
        assert ls(A, BF, 4, 64, 64, ctypes.byref(kr), A, A, 8, R, A, F, 8, NULL, 0, None) == UNS
    kr = mx.RotationDesc(mx.ROT_KRON, 4, 4, 0, A, A)
    assert ls(A, BF, 4, 64, 64, ctypes.byref(kr), A, A, 8, R, A, F, 8, NULL, 0, None) == INV   # p*q != 32


def test_linear_small_workspace():
    """Workspace size of the fused layer: 4 KiB of handoff counters plus 1152
    bytes per 16 activation rows and 128 columns (the quantized activations
    in operand order); a missing or short workspace is rejected
    synchronously."""
    INV, UNS = mx.MXFP4_ERR_INVALID_ARG, mx.MXFP4_ERR_UNSUPPORTED
    A, T, BF, F = ALIGNED, mx.TILED, mx.MXFP4_BF16, mx.MXFP4_F32
    b = ctypes.c_int64()
    W = mx.lib().mxfp4_linear_small_workspace
    assert mx.linear_small_workspace_bytes(16, 14336, 4096) == 4096 + 32 * 1152
    assert mx.linear_small_workspace_bytes(16, 14336, 1024) == 4096 + 8 * 1152
    assert mx.linear_small_workspace_bytes(1, 300, 4128) == 4096 + 33 * 1152      # ragged K: 33 steps
    assert mx.linear_small_workspace_bytes(17, 300, 96) == 4096 + 2 * 1152        # two M groups, one step
    assert mx.linear_small_workspace_bytes(64, 7, 4096) == 4096 + 4 * 32 * 1152
    assert mx.linear_small_workspace_bytes(0, 300, 4096) == 0
    assert mx.linear_small_workspace_bytes(16, 0, 4096) == 0
    assert W(65, 300, 4096, ctypes.byref(b)) == UNS
    assert W(64, 300, 1 << 29, ctypes.byref(b)) == UNS               # activation image past 2 GiB
    assert ls(A, BF, 64, 1 << 29, 1 << 29, None, A, A, 8, T, A, F, 8, A, 1 << 40, None) == UNS
    assert W(4, 300, 48, ctypes.byref(b)) == INV
    assert W(4, 300, 64, None) == INV
    need = mx.linear_small_workspace_bytes(16, 512, 4096)
    assert ls(A, BF, 16, 4096, 4096, None, A, A, 512, T, A, F, 512, NULL, 0, None) == INV        # missing
    assert ls(A, BF, 16, 4096, 4096, None, A, A, 512, T, A, F, 512, A, need - 4, None) == INV    # short
    assert ls(A, BF, 16, 4096, 4096, None, A, A, 512, T, A, F, 512, A + 16, need, None) == UNS   # alignment
    assert ls(A, BF, 16, 1024, 1024, None, A, A, 512, T, A, F, 512, NULL, 0, None) == INV        # any K needs one


def test_linear_small_noalloc_rejects_before_any_device_work():
    """The allocation-free fused layer checks its arguments and its 4 MiB
    scratch limit synchronously, before looking up or touching the scratch."""
    INV, UNS, OK = mx.MXFP4_ERR_INVALID_ARG, mx.MXFP4_ERR_UNSUPPORTED, mx.MXFP4_OK
    A, T, BF, F = ALIGNED, mx.TILED, mx.MXFP4_BF16, mx.MXFP4_F32
    na = mx.lib().mxfp4_linear_small_noalloc
    assert mx.linear_small_workspace_bytes(16, 512, 465536) <= 4 << 20
    assert mx.linear_small_workspace_bytes(16, 512, 465536 + 128) > 4 << 20
    assert mx.linear_small_workspace_bytes(64, 512, 116352) <= 4 << 20
    assert na(A, BF, 16, 465664, 465664, None, A, A, 512, T, A, F, 512, None) == UNS     # past 4 MiB
    assert na(A, BF, 64, 116480, 116480, None, A, A, 512, T, A, F, 512, None) == UNS     # past 4 MiB
    assert na(A, BF, 65, 4096, 4096, None, A, A, 512, T, A, F, 512, None) == UNS         # m > 64
    assert na(A, BF, 16, 4096, 4096, None, NULL, A, 512, T, A, F, 512, None) == INV      # null weights
    assert na(NULL, BF, 0, 4096, 4096, None, NULL, NULL, 512, T, NULL, F, 512, None) == OK   # m == 0


def test_gemm_requant_argument_errors():
    INV, UNS, OK = mx.MXFP4_ERR_INVALID_ARG, mx.MXFP4_ERR_UNSUPPORTED, mx.MXFP4_OK
    A, R, T = ALIGNED, mx.ROWMAJOR, mx.TILED
    gq = mx.lib().mxfp4_gemm_requant
    assert gq(A, A, 4, A, A, 256, 128, 2, A, A, R, None) == INV       # bad operand layout
    assert gq(A, A, 4, A, A, 256, 128, R, A, A, 5, None) == INV       # bad output layout
    assert gq(A, A, 4, A, A, 256, 48, R, A, A, R, None) == INV        # k % 32
    assert gq(A, A, -1, A, A, 256, 128, R, A, A, R, None) == INV
    assert gq(A, A, 4, A, A, 256, 128, R, NULL, A, R, None) == INV
    assert gq(NULL, NULL, 0, NULL, NULL, 256, 128, R, NULL, NULL, R, None) == OK   # m == 0
    assert gq(A, A, 4, A, A, 200, 128, R, A, A, R, None) == UNS       # n % 32
    assert gq(A, A, 4, A, A, 160, 128, R, A, A, T, None) == UNS       # tiled output: n % 128
    assert gq(A, A, 4, A, A, 256, 96, R, A, A, R, None) == UNS        # k % 128
    assert gq(A, A, 4, A, A, 256, 128, R, A + 8, A, R, None) == UNS   # codes not 16 B aligned
    assert gq(A, A, 4, A, A, 256, 128, R, A, A + 1, T, None) == UNS   # scales not 4 B aligned


def test_tiled_bytes():
    INV = mx.MXFP4_ERR_INVALID_ARG
    assert mx.tiled_bytes(1, 128) == (256 * 64, 256 * 4)
    assert mx.tiled_bytes(256, 3072) == (256 * 1536, 256 * 96)
    assert mx.tiled_bytes(257, 256) == (512 * 128, 512 * 8)
    assert mx.tiled_bytes(0, 128) == (0, 0)
    cb, sb = ctypes.c_int64(), ctypes.c_int64()
    assert mx.lib().mxfp4_tiled_bytes(4, 96, ctypes.byref(cb), ctypes.byref(sb)) == INV
    assert mx.lib().mxfp4_tiled_bytes(-1, 128, ctypes.byref(cb), ctypes.byref(sb)) == INV
    assert mx.lib().mxfp4_tiled_bytes(4, 128, None, ctypes.byref(sb)) == INV


@pytest.mark.parametrize("rows,k", [(1, 128), (255, 256), (256, 384), (700, 512)])
def test_host_tiling_roundtrip_and_definition(rows, k):
    """tile_host / untile_host are inverse permutations, and the tiled bytes
    sit where the header's layout definition puts them."""
    rng = np.random.default_rng(rows + k)
    c = rng.integers(0, 256, (rows, k // 2), dtype=np.uint8)
    s = rng.integers(0, 256, (rows, k // 32), dtype=np.uint8)
    tc, ts = mx.tile_host(c, s)
    assert tc.shape == (mx.padded_rows(rows), k // 2) and ts.shape == (mx.padded_rows(rows), k // 32)
    c2, s2 = mx.untile_host(tc, ts, rows)
    assert np.array_equal(c, c2) and np.array_equal(s, s2)
    flat_c, flat_s = tc.reshape(-1), ts.reshape(-1)
    S = k // 128
    for row in (0, rows - 1, rows // 2):
        for blk in (0, k // 32 - 1):
            t, r, st, cb = row // 256, row % 256, blk // 4, blk % 4
            p = cb ^ (((r >> 1) ^ (r >> 2)) & 3)
            base = (t * S + st) * 16384 + r * 64 + 16 * p
            assert np.array_equal(flat_c[base:base + 16], c[row, 16 * blk:16 * blk + 16])
            assert flat_s[(t * S + st) * 1024 + r * 4 + cb] == s[row, blk]
    if mx.padded_rows(rows) > rows:   # padding rows are zero
        pc, ps = mx.untile_host(tc, ts, mx.padded_rows(rows))
        assert not pc[rows:].any() and not ps[rows:].any()


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32])
def test_inverse_transpose_matches_oracle(n):
    """The library's weight-side Kronecker factors are the oracle's, bit for
    bit: both run Gauss-Jordan elimination with partial pivoting in binary64,
    the same operations in the same order, and round once to fp32."""
    for seed in range(40):
        rng = np.random.default_rng(1000 * n + seed)
        scale = 0.1 if seed % 2 == 0 else 1.0           # near-identity and general matrices
        m = (np.eye(n) + scale * rng.standard_normal((n, n))).astype(np.float32)
        got = mx.inverse_transpose(m)
        ref = oracle.inverse_transpose(m)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"n={n} seed={seed}"


def test_kron_workload_factors_match_oracle():
    inp = workloads.make("llm_decode_kron", m=1)
    for f in (inp["a"], inp["b"]):
        assert np.array_equal(mx.inverse_transpose(f).view(np.uint32), oracle.inverse_transpose(f).view(np.uint32))


def test_smooth_weight_factors_match_oracle():
    rng = np.random.default_rng(7)
    r = np.concatenate([(0.25 + 4 * rng.random(4096)),
                        rng.random(4096) * np.exp2(rng.integers(-100, 100, 4096)) + 1e-30,
                        np.exp2(np.arange(-126, 127))]).astype(np.float32)
    r[::3] *= -1
    got = mx.smooth_weight_factors(r)
    assert np.array_equal(got.view(np.uint32), oracle.smooth_weight_factors(r).view(np.uint32))


def test_smooth_weight_factors_errors():
    L = mx.lib()
    INV = mx.MXFP4_ERR_INVALID_ARG
    out = np.empty(4, np.float32)
    for bad in (0.0, np.inf, np.nan, 2.0 ** -149):
        r = np.array([1.0, 2.0, bad, 4.0], np.float32)
        assert L.mxfp4_smooth_weight_factors(r.ctypes.data, 4, out.ctypes.data) == INV
    r = np.ones(4, np.float32)
    assert L.mxfp4_smooth_weight_factors(None, 4, out.ctypes.data) == INV
    assert L.mxfp4_smooth_weight_factors(r.ctypes.data, 0, out.ctypes.data) == INV
    assert L.mxfp4_smooth_weight_factors(r.ctypes.data, 4, None) == INV
    with pytest.raises(mx.Mxfp4Error):
        mx.smooth_weight_factors(np.array([1.0, 0.0], np.float32))


def test_gemm_tiled_code_byte_limit():
    """TILED operands with m > 64 run on the kernel with 32-bit operand
    offsets: past 4 GiB of tiled code bytes the call returns UNSUPPORTED
    (synchronously, nothing launched)."""
    A, T, UNS, OK = ALIGNED, mx.TILED, mx.MXFP4_ERR_UNSUPPORTED, mx.MXFP4_OK
    k = 8192                                       # 4 KiB of codes per row
    big = (1 << 20)                                # 2^20 rows x 4 KiB = 4 GiB
    assert g(A, A, big, A, A, 256, k, T, A, 0, 256, None) == UNS      # A too large
    assert g(A, A, 256, A, A, big, k, T, A, 0, big, None) == UNS      # B too large
    assert g(A, A, big - 256, A, A, 256, k, T, NULL, 0, 256, None) == mx.MXFP4_ERR_INVALID_ARG  # just below: null y
    assert g(NULL, NULL, 0, NULL, NULL, big, k, T, NULL, 0, big, None) == OK   # m == 0: no-op


def test_binding_rejects_host_tensors():
    """The binding refuses tensors that are not on a GPU before any library
    call: a host pointer handed to a kernel would fault the device."""
    import torch
    x = torch.zeros((4, 64), dtype=torch.bfloat16)
    c = torch.zeros((4, 32), dtype=torch.uint8)
    s = torch.zeros((4, 2), dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU"):
        mx.quantize_rotate(x)
    with pytest.raises(ValueError, match="GPU"):
        mx.gemm(c, s, c, s)
    with pytest.raises(ValueError, match="GPU"):
        mx.gemm_requant(c, s, c, s)
    with pytest.raises(ValueError, match="GPU"):
        mx.linear_small(x, c, s)
    with pytest.raises(ValueError, match="GPU"):
        mx.linear(x, c, s)


def test_binding_checks_rotation_factors():
    """Kronecker factors must be p x p and q x q with p * q = 32; smoothing
    needs exactly k factors (checked on meta tensors: no memory, no device)."""
    import torch
    dev = torch.device("meta")
    f = lambda *shape: torch.empty(shape, dtype=torch.float32, device=dev)
    mx._rot_desc(mx.Kron(f(4, 4), f(8, 8)), dev, 64)
    for a, b in ((f(4, 4), f(4, 4)), (f(4, 8), f(8, 8)), (f(16), f(2, 2)), (f(4, 4), f(8, 4))):
        with pytest.raises(ValueError, match="Kron"):
            mx._rot_desc(mx.Kron(a, b), dev, 64)
    mx._rot_desc(mx.Smooth(f(64)), dev, 64)
    for r in (f(32), f(65)):
        with pytest.raises(ValueError, match="one factor per column"):
            mx._rot_desc(mx.Smooth(r), dev, 64)
    with pytest.raises(ValueError, match="input's device"):
        mx._rot_desc(mx.Smooth(torch.zeros(64)), dev, 64)


def test_inverse_transpose_errors():
    with pytest.raises(mx.Mxfp4Error):
        mx.inverse_transpose(np.zeros((4, 4), np.float32))      # singular
    assert mx.lib().mxfp4_inverse_transpose(None, 4, None) == mx.MXFP4_ERR_INVALID_ARG
    m = np.eye(4, dtype=np.float32)
    assert mx.lib().mxfp4_inverse_transpose(m.ctypes.data, 33, m.ctypes.data) == mx.MXFP4_ERR_INVALID_ARG


def test_measurement_library_loads_and_rejects_bad_arguments():
    # the benchmark's MFMA-rate kernel ships as a library of its own, outside
    # the MXFP4 ABI; argument errors return before any device call
    from mxfp4_w4a4_quantized_amd import build as hip_build
    L = ctypes.CDLL(hip_build.CEILING_LIB)
    out = os.popen(f"nm -D --defined-only {hip_build.CEILING_LIB}").read()
    assert set(re.findall(r"\bT (\w+)", out)) == {"mxfp4_ceiling_mfma", "mxfp4_ceiling_stream"}
    L.mxfp4_ceiling_mfma.restype = ctypes.c_int
    L.mxfp4_ceiling_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    for blocks, iters, o, c in ((0, 4, ALIGNED, ALIGNED), (4, 0, ALIGNED, ALIGNED), (4, 6, ALIGNED, ALIGNED),
                                (4, 4, NULL, ALIGNED), (4, 4, ALIGNED, NULL)):
        assert L.mxfp4_ceiling_mfma(blocks, iters, o, c, NULL) != 0
    L.mxfp4_ceiling_stream.restype = ctypes.c_int
    L.mxfp4_ceiling_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_void_p]
    for src, dst, waves, rk, wk in ((NULL, ALIGNED, 8, 4, 1), (ALIGNED, NULL, 8, 4, 1), (ALIGNED, ALIGNED, 0, 4, 1),
                                    (ALIGNED, ALIGNED, 8, 5, 1), (ALIGNED, ALIGNED, 8, 4, 5),
                                    (ALIGNED, ALIGNED, 8, 4, -1), (ALIGNED + 8, ALIGNED, 8, 4, 1)):
        assert L.mxfp4_ceiling_stream(src, dst, waves, rk, wk, NULL) != 0
