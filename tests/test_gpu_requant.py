"""GPU parity of the GEMM with an MXFP4 output (mxfp4_gemm_requant).

Exact parity: operands whose block exponents lie in [-1, 1] with K <= 4096 make
every partial sum of the GEMM a multiple of 2^-4 below 2^24 units, so Y is
exact in fp32 whatever the summation order.  Then the oracle's Y (binary64,
exact) is the kernel's Y, and the requantized output must equal the oracle's
quantizer applied to it, code for code and scale for scale.  Realistic
operands (wide exponents, Y rounded in fp32): the requantized output must
equal the oracle's quantizer applied to the fp32 Y that mxfp4_gemm returns for
the same operands -- the epilogue requantizes the same sums in the same
kernel.
"""
import numpy as np
import pytest
import torch

import mxfp4_w4a4_quantized_amd as mx
import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
R, T = mx.ROWMAJOR, mx.TILED


def announce(*what):
    print("[case]", *what, flush=True)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def operands(rng, rows, k, e_lo, e_hi, layout):
    c, s = workloads.random_mxfp4(rng, rows, k, e_lo, e_hi)
    dc, ds = (mx.tile_host(c, s) if layout == T else (c, s))
    return c, s, to_dev(dc), to_dev(ds)


SHAPES = [(256, 256, 128), (300, 512, 384), (1000, 768, 1024), (64, 256, 4096), (2304, 1280, 512),
          (130, 384, 256), (520, 640, 128)]


@pytest.mark.parametrize("out_layout", [R, T])
@pytest.mark.parametrize("layout", [R, T])
@pytest.mark.parametrize("m,n,k", SHAPES)
def test_requant_exact(m, n, k, layout, out_layout):
    rng = np.random.default_rng(m + 7 * n + k)
    ac, as_, dac, das = operands(rng, m, k, -1, 1, layout)
    bc, bs, dbc, dbs = operands(rng, n, k, -1, 1, layout)
    ref = oracle.gemm(ac, as_, bc, bs)
    y32 = ref.astype(np.float32)
    assert np.array_equal(y32.astype(np.float64), ref)          # Y is exact in fp32
    want = oracle.quantize(y32)
    announce("gemm_requant exact", m, n, k, layout, out_layout)
    qc, qs = mx.gemm_requant(dac, das, dbc, dbs, layout=layout, out_layout=out_layout, m=m, n=n)
    yg = mx.gemm(dac, das, dbc, dbs, torch.float32, layout=layout, m=m, n=n)
    torch.cuda.synchronize()
    assert np.array_equal(yg.cpu().numpy(), y32)
    got = (qc.cpu().numpy(), qs.cpu().numpy())
    if out_layout == T:
        got = mx.untile_host(got[0], got[1], m)
    assert np.array_equal(got[1], want[1]), f"{np.count_nonzero(got[1] != want[1])} scale bytes differ"
    assert np.array_equal(got[0], want[0]), f"{np.count_nonzero(got[0] != want[0])} code bytes differ"


def test_requant_rowmajor_ragged_n():
    # N a multiple of 32 but not of 128: only the row-major output takes it
    rng = np.random.default_rng(9)
    m, n, k = 270, 96 + 256, 256
    ac, as_, dac, das = operands(rng, m, k, -1, 1, R)
    bc, bs, dbc, dbs = operands(rng, n, k, -1, 1, R)
    ref = oracle.gemm(ac, as_, bc, bs).astype(np.float32)
    want = oracle.quantize(ref)
    announce("gemm_requant ragged n", m, n, k)
    qc, qs = mx.gemm_requant(dac, das, dbc, dbs)
    torch.cuda.synchronize()
    assert np.array_equal(qc.cpu().numpy(), want[0]) and np.array_equal(qs.cpu().numpy(), want[1])
    with pytest.raises(mx.Mxfp4Error):
        mx.gemm_requant(dac, das, dbc, dbs, out_layout=T)            # tiled output needs n % 128


def test_requant_tiled_padding_untouched():
    rng = np.random.default_rng(5)
    m, n, k = 300, 512, 256
    _, _, dac, das = operands(rng, m, k, -1, 1, R)
    _, _, dbc, dbs = operands(rng, n, k, -1, 1, R)
    rp = mx.padded_rows(m)
    qc = torch.full((rp, n // 2), 0xFF, dtype=torch.uint8, device=DEV)
    qs = torch.full((rp, n // 32), 0xFF, dtype=torch.uint8, device=DEV)
    announce("gemm_requant padding", m, n, k)
    mx.gemm_requant(dac, das, dbc, dbs, out_layout=T, y_codes=qc, y_scales=qs)
    torch.cuda.synchronize()
    pc, ps = mx.untile_host(qc.cpu().numpy(), qs.cpu().numpy(), rp)
    assert (pc[m:] == 0xFF).all() and (ps[m:] == 0xFF).all()


REALISTIC = [(520, 768, 1024, T, T), (520, 768, 1024, R, R), (300, 512, 3072, T, R),
             (16, 1024, 4096, T, T), (16, 1024, 4096, R, R), (64, 640, 1024, T, R), (5, 256, 512, R, T),
             (40, 384, 2048, T, T)]


@pytest.mark.parametrize("m,n,k,layout,out_layout", REALISTIC)
def test_requant_realistic_bit_exact(m, n, k, layout, out_layout):
    """Wide block exponents, so Y is rounded in fp32 and its summation order
    matters: the requantized bytes must equal the oracle's quantizer applied
    to the fp32 Y that mxfp4_gemm returns for the same operands (the decode
    kernel for m <= 64, the large-tile kernel above), bit for bit."""
    rng = np.random.default_rng(6 + m + n + k)
    _, _, dac, das = operands(rng, m, k, -20, 20, layout)
    _, _, dbc, dbs = operands(rng, n, k, -20, 20, layout)
    announce("gemm_requant realistic", m, n, k, layout, out_layout)
    qc, qs = mx.gemm_requant(dac, das, dbc, dbs, layout=layout, out_layout=out_layout, m=m, n=n)
    y = mx.gemm(dac, das, dbc, dbs, torch.float32, layout=layout, m=m, n=n)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    got = (qc.cpu().numpy(), qs.cpu().numpy())
    if out_layout == T:
        got = mx.untile_host(got[0], got[1], m)
    want = oracle.quantize(y)
    assert np.array_equal(got[1], want[1]), f"{np.count_nonzero(got[1] != want[1])} scale bytes differ"
    assert np.array_equal(got[0], want[0]), f"{np.count_nonzero(got[0] != want[0])} code bytes differ"
    # the case is not trivially exact: Y has rounded elements (inexact in any order)
    ac, as_ = (mx.untile_host(dac.cpu().numpy(), das.cpu().numpy(), m) if layout == T
               else (dac.cpu().numpy(), das.cpu().numpy()))
    bc, bs = (mx.untile_host(dbc.cpu().numpy(), dbs.cpu().numpy(), n) if layout == T
              else (dbc.cpu().numpy(), dbs.cpu().numpy()))
    assert np.count_nonzero(y.astype(np.float64) != oracle.gemm(ac, as_, bc, bs)) > 0


def test_requant_full_workload():
    """The flux_up GEMM (3584 x 3072 -> 12288) in the benchmark's tiled
    configuration with an MXFP4 output: bytes equal the oracle's quantizer on
    the same kernel's fp32 Y."""
    inp = workloads.make("flux_up")
    wl = inp["wl"]
    m, n, k = wl.m, wl.n, wl.k
    x = to_dev(inp["x"].view(np.int16)).view(torch.bfloat16)
    announce("gemm_requant flux_up", m, n, k)
    wc, ws = mx.quantize_weight(to_dev(inp["w"]), None, layout=T)
    xc, xs = mx.quantize_rotate(x, None, layout=T)
    qc, qs = mx.gemm_requant(xc, xs, wc, ws, layout=T, out_layout=T, m=m, n=n)
    y = mx.gemm(xc, xs, wc, ws, torch.float32, layout=T, m=m, n=n)
    torch.cuda.synchronize()
    got = mx.untile_host(qc.cpu().numpy(), qs.cpu().numpy(), m)
    want = oracle.quantize(y.cpu().numpy())
    assert np.array_equal(got[1], want[1]) and np.array_equal(got[0], want[0])


def test_requant_rejects_unsupported():
    z = torch.zeros((256, 64), dtype=torch.uint8, device=DEV)
    zs = torch.zeros((256, 4), dtype=torch.uint8, device=DEV)
    b = torch.zeros((200, 64), dtype=torch.uint8, device=DEV)
    bs = torch.zeros((200, 4), dtype=torch.uint8, device=DEV)
    with pytest.raises(mx.Mxfp4Error):
        mx.gemm_requant(z, zs, b, bs)                                # n = 200, not a multiple of 256
