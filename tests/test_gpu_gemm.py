"""GPU parity of the MXFP4 GEMM against the oracle's binary64 GEMM.

Tolerance (fp32 output): for every checked element,
    |Y_gpu - Y_oracle| <= 1e-5 * ||a_hat_m||_2 * ||b_hat_n||_2.
Derivation: inside one 32-element block every product of two E2M1 values is
a multiple of 1/4 below 36 in magnitude and the block sum is exact; the
kernel's only roundings are the fp32 accumulations across K (at most K/32 of
them, each with relative error 2^-24) and the block scaling, so the error is
below (K/32 + 1) * 2^-24 * sum_k |a_hat b_hat| <= (K/32 + 1) * 2^-24 *
||a_hat|| ||b_hat|| (Cauchy-Schwarz) -- 2.3e-5 in the worst case at
K = 12288, ~1e-6 in practice since the rounding errors do not align.
bf16 output: Y_bf16 must equal the round-to-nearest-even bf16 of the same
kernel's fp32 output bit for bit, and lie within half a bf16 ulp of the
oracle plus the fp32 bound.
"""
import numpy as np
import pytest
import torch

import mxfp4_w4a4_quantized_amd as mx
import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 1e-5


def announce(*what):
    print("[case]", *what, flush=True)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def row_norms(codes, scales):
    return np.sqrt((oracle.dequantize(codes, scales) ** 2).sum(axis=1))


def norm_err(got, ref, na, nb):
    den = np.outer(na, nb) if got.ndim == 2 else na * nb
    diff = np.abs(got.astype(np.float64) - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(den > 0, diff / den, np.where(diff == 0, 0.0, np.inf))
    return float(rel.max()) if rel.size else 0.0


def bf16_rne(y32: torch.Tensor) -> np.ndarray:
    return y32.to(torch.bfloat16).view(torch.int16).cpu().numpy().view(np.uint16)


def run_both(ac, as_, bc, bs):
    dac, das, dbc, dbs = map(to_dev, (ac, as_, bc, bs))
    y32 = mx.gemm(dac, das, dbc, dbs, torch.float32)
    y16 = mx.gemm(dac, das, dbc, dbs, torch.bfloat16)
    torch.cuda.synchronize()
    return y32, y16


def check_full(ac, as_, bc, bs, what):
    m, n = ac.shape[0], bc.shape[0]
    announce("gemm", what, m, n, ac.shape[1] * 2)
    y32, y16 = run_both(ac, as_, bc, bs)
    ref = oracle.gemm(ac, as_, bc, bs)
    na, nb = row_norms(ac, as_), row_norms(bc, bs)
    err = norm_err(y32.cpu().numpy(), ref, na, nb)
    assert err <= TOL, f"{what}: normalized error {err:.3e}"
    # bf16 epilogue: RNE of the same fp32 result
    assert np.array_equal(y16.view(torch.int16).cpu().numpy().view(np.uint16), bf16_rne(y32))
    yb = y16.float().cpu().numpy().astype(np.float64)
    half_ulp = np.abs(ref) * 2.0 ** -8 + 1e-300
    assert np.all(np.abs(yb - ref) <= half_ulp + TOL * np.outer(na, nb) + 1e-300)
    return err


# ------------------------------------------------------------ small cases ---

SHAPES = [
    (1, 1, 32), (16, 16, 128), (128, 128, 256), (17, 33, 96), (130, 260, 544),
    (257, 129, 1056), (300, 500, 2048), (64, 640, 4096), (5, 1000, 320),
]


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_random_operands(m, n, k):
    rng = np.random.default_rng(m * 131 + n * 7 + k)
    ac, as_ = workloads.random_mxfp4(rng, m, k)
    bc, bs = workloads.random_mxfp4(rng, n, k)
    check_full(ac, as_, bc, bs, "random")


# Shapes for the large-tile persistent kernel (K a multiple of 128, M > 64,
# at least 8 output tiles of 256 x 256; fewer tiles go to the small-M kernel,
# see FEW_TILE_SHAPES): one K stage, fewer stages than the load ring, ragged
# M and N, fewer tiles than CUs (grid not a multiple of 8), and more tiles
# than CUs (several tiles per workgroup, the load ring running across tile
# boundaries; 289, 432 and 560 tiles run as 2, 2 and 3 full rounds on 152,
# 216 and 192 workgroups).
LARGE_SHAPES = [
    (2304, 512, 128), (1030, 2100, 256), (520, 1030, 384), (96, 2048, 512),
    (2200, 100, 640), (1024, 768, 1024), (4352, 4352, 128), (2304, 4608, 384),
    (3000, 9000, 128), (5000, 7000, 256),
]


@pytest.mark.parametrize("m,n,k", LARGE_SHAPES)
def test_large_tile_shapes(m, n, k):
    rng = np.random.default_rng(m * 31 + n * 17 + k)
    ac, as_ = workloads.random_mxfp4(rng, m, k)
    bc, bs = workloads.random_mxfp4(rng, n, k)
    check_full(ac, as_, bc, bs, "large-tile")


# Shapes with M > 64 and fewer than 8 output tiles of 256 x 256: the small-M
# kernel with one grid row per 64 activation rows (tiny layers, where one
# large tile per workgroup would leave the chip idle), both layouts, K tails.
FEW_TILE_SHAPES = [(128, 128, 256), (256, 256, 128), (257, 300, 256), (700, 100, 640), (300, 500, 2048),
                   (130, 260, 544), (65, 1792, 4096), (768, 512, 96)]


@pytest.mark.parametrize("m,n,k", FEW_TILE_SHAPES)
def test_few_tile_shapes(m, n, k):
    rng = np.random.default_rng(m * 5 + n * 11 + k)
    ac, as_ = workloads.random_mxfp4(rng, m, k)
    bc, bs = workloads.random_mxfp4(rng, n, k)
    check_full(ac, as_, bc, bs, "few tiles")
    if k % 128 == 0:
        test_tiled_operands(m, n, k)


@pytest.mark.parametrize("dt,off", [(torch.float32, 4), (torch.float32, 1), (torch.bfloat16, 4), (torch.bfloat16, 8)],
                         ids=["f32-aligned", "f32-unaligned", "bf16-unaligned", "bf16-aligned"])
def test_large_tile_strided_output(dt, off):
    """Y inside a wider buffer (ld_y = n + 12) at an element offset, on a shape
    with edge tiles in both dimensions: rows that start 16-byte aligned (the
    staged epilogue's 16-byte stores, bounds-checked at the edges) and rows
    that do not (element stores).  fp32 Y is checked against the oracle; bf16
    Y must equal the kernel's own fp32 Y (contiguous) rounded to nearest even,
    bit for bit; nothing outside Y may be written."""
    rng = np.random.default_rng(80)
    m, n, k = 520, 2100, 256
    ac, as_ = workloads.random_mxfp4(rng, m, k)
    bc, bs = workloads.random_mxfp4(rng, n, k)
    fill = 7.0 if dt == torch.float32 else 3.0
    big = torch.full((m, n + 12), fill, dtype=dt, device=DEV)
    y = big[:, off:off + n]
    announce("gemm large strided", m, n, k, dt, off)
    ops = list(map(to_dev, (ac, as_, bc, bs)))
    mx.gemm(*ops, dt, y=y)
    y32 = mx.gemm(*ops, torch.float32)
    torch.cuda.synchronize()
    if dt == torch.float32:
        ref = oracle.gemm(ac, as_, bc, bs)
        assert norm_err(y.cpu().numpy(), ref, row_norms(ac, as_), row_norms(bc, bs)) <= TOL
        assert torch.equal(y, y32), "strided fp32 Y differs from the contiguous one"
    else:
        assert torch.equal(y.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16)), \
            "bf16 Y is not the round-to-nearest-even of the kernel's fp32 Y"
    host = big.float().cpu().numpy()
    assert (host[:, :off] == fill).all() and (host[:, off + n:] == fill).all()   # no stray writes


TILED_SHAPES = [
    (256, 256, 128), (257, 300, 256), (1000, 520, 384), (16, 1000, 256), (96, 2048, 512),
    (4352, 4352, 128), (2304, 4608, 384), (600, 2100, 256)]


@pytest.mark.parametrize("m,n,k", TILED_SHAPES)
def test_tiled_operands(m, n, k):
    """Both operands in the tiled layout (tiled on the host, a byte
    permutation), every output element checked against the oracle."""
    rng = np.random.default_rng(m * 13 + n * 5 + k)
    ac, as_ = workloads.random_mxfp4(rng, m, k)
    bc, bs = workloads.random_mxfp4(rng, n, k)
    announce("gemm tiled", m, n, k)
    ta, tas = mx.tile_host(ac, as_)
    tb, tbs = mx.tile_host(bc, bs)
    dev = [to_dev(t) for t in (ta, tas, tb, tbs)]
    y32 = mx.gemm(*dev, torch.float32, layout=mx.TILED, m=m, n=n)
    y16 = mx.gemm(*dev, torch.bfloat16, layout=mx.TILED, m=m, n=n)
    torch.cuda.synchronize()
    ref = oracle.gemm(ac, as_, bc, bs)
    err = norm_err(y32.cpu().numpy(), ref, row_norms(ac, as_), row_norms(bc, bs))
    assert err <= TOL, f"normalized error {err:.3e}"
    assert np.array_equal(y16.view(torch.int16).cpu().numpy().view(np.uint16), bf16_rne(y32))


# Shapes for the small-M kernel (M <= 64): every number of 16-row M groups,
# N not a multiple of 16 or of 4, K tails inside the last 128-element step,
# one to eight waves splitting K, and waves that loop over several register
# chunks of K steps.
SMALL_M_SHAPES = [
    (1, 14336, 4096), (7, 3, 32), (16, 2000, 4128), (33, 517, 12288), (48, 64, 160),
    (64, 130, 1024), (20, 4100, 20000), (2, 77, 96)]


@pytest.mark.parametrize("m,n,k", SMALL_M_SHAPES)
def test_small_m_shapes(m, n, k):
    rng = np.random.default_rng(m * 7 + n * 3 + k)
    ac, as_ = workloads.random_mxfp4(rng, m, k)
    bc, bs = workloads.random_mxfp4(rng, n, k)
    check_full(ac, as_, bc, bs, "small-m")


# K = 10240 at M = 16 gives each wave one whole 8-step chunk (scale bytes by
# dword loads) and one partial chunk (predicated loads); K = 8192 at M = 32
# covers two weight groups on whole chunks
SMALL_M_TILED = [(1, 300, 128), (33, 1000, 12288), (64, 256, 384), (50, 4097, 1024), (16, 14336, 4096),
                 (16, 520, 10240), (32, 777, 8192)]


@pytest.mark.parametrize("m,n,k", SMALL_M_TILED)
def test_small_m_tiled(m, n, k):
    test_tiled_operands(m, n, k)


def test_small_m_strided_output():
    rng = np.random.default_rng(81)
    m, n, k = 10, 90, 256
    ac, as_ = workloads.random_mxfp4(rng, m, k)
    bc, bs = workloads.random_mxfp4(rng, n, k)
    ref = oracle.gemm(ac, as_, bc, bs)
    for dt, off, fill in ((torch.float32, 4, 7.0), (torch.float32, 5, 7.0), (torch.bfloat16, 4, 3.0),
                          (torch.bfloat16, 5, 3.0)):
        big = torch.full((m, n + 12), fill, dtype=dt, device=DEV)
        y = big[:, off:off + n]
        announce("gemm small strided", m, n, k, dt, off)
        mx.gemm(*map(to_dev, (ac, as_, bc, bs)), dt, y=y)
        torch.cuda.synchronize()
        if dt == torch.float32:
            err = norm_err(y.cpu().numpy(), ref, row_norms(ac, as_), row_norms(bc, bs))
            assert err <= TOL
        host = big.float().cpu().numpy()
        assert (host[:, :off] == fill).all() and (host[:, off + n:] == fill).all()   # no stray writes


@pytest.mark.parametrize("m,n,k", [(20, 300, 256), (40, 70, 384), (300, 520, 256), (600, 2100, 256)])
def test_tiled_padding_is_ignored(m, n, k):
    """Padding rows of tiled operands hold garbage (code bytes 0xFF = -6, scale
    bytes 0xFF = NaN): no stored output may depend on them (small-M and
    large-tile kernels)."""
    rng = np.random.default_rng(m + n + k)
    ac, as_ = workloads.random_mxfp4(rng, m, k)
    bc, bs = workloads.random_mxfp4(rng, n, k)

    def padded(c, s):
        rp = mx.padded_rows(c.shape[0])
        pc = np.full((rp, c.shape[1]), 0xFF, np.uint8)
        ps = np.full((rp, s.shape[1]), 0xFF, np.uint8)
        pc[:c.shape[0]], ps[:s.shape[0]] = c, s
        return mx.tile_host(pc, ps)

    announce("gemm tiled padding garbage", m, n, k)
    dev = [to_dev(t) for t in (*padded(ac, as_), *padded(bc, bs))]
    y32 = mx.gemm(*dev, torch.float32, layout=mx.TILED, m=m, n=n)
    torch.cuda.synchronize()
    got = y32.cpu().numpy()
    assert np.isfinite(got).all()
    ref = oracle.gemm(ac, as_, bc, bs)
    assert norm_err(got, ref, row_norms(ac, as_), row_norms(bc, bs)) <= TOL


def test_extreme_scales():
    # scale bytes near both ends of the E8M0 range (products stay finite)
    rng = np.random.default_rng(77)
    m, n, k = 48, 80, 512
    ac, _ = workloads.random_mxfp4(rng, m, k)
    bc, _ = workloads.random_mxfp4(rng, n, k)
    as_ = rng.integers(0, 40, (m, k // 32)).astype(np.uint8)        # 2^-127 .. 2^-88
    bs = rng.integers(200, 254, (n, k // 32)).astype(np.uint8)      # 2^73 .. 2^126
    check_full(ac, as_, bc, bs, "extreme scales")


def test_zero_and_sign_codes():
    rng = np.random.default_rng(78)
    m, n, k = 40, 72, 256
    ac = np.full((m, k // 2), 0x88, np.uint8)                         # all -0
    ac[::3] = rng.integers(0, 256, (len(ac[::3]), k // 2), dtype=np.uint8)
    as_ = np.full((m, k // 32), 127, np.uint8)
    bc, bs = workloads.random_mxfp4(rng, n, k)
    check_full(ac, as_, bc, bs, "zeros")


def test_strided_output():
    rng = np.random.default_rng(79)
    m, n, k = 70, 90, 384
    ac, as_ = workloads.random_mxfp4(rng, m, k)
    bc, bs = workloads.random_mxfp4(rng, n, k)
    big = torch.full((m, n + 38), 7.0, dtype=torch.float32, device=DEV)
    y = big[:, 5:5 + n]                                                # ld_y = n + 38, offset 5
    announce("gemm strided", m, n, k)
    mx.gemm(*map(to_dev, (ac, as_, bc, bs)), torch.float32, y=y)
    torch.cuda.synchronize()
    ref = oracle.gemm(ac, as_, bc, bs)
    err = norm_err(y.cpu().numpy(), ref, row_norms(ac, as_), row_norms(bc, bs))
    assert err <= TOL
    host = big.cpu().numpy()
    assert (host[:, :5] == 7.0).all() and (host[:, 5 + n:] == 7.0).all()   # no stray writes


def test_empty_gemm_is_noop():
    z = torch.empty((0, 16), dtype=torch.uint8, device=DEV)
    zs = torch.empty((0, 1), dtype=torch.uint8, device=DEV)
    b = torch.zeros((8, 16), dtype=torch.uint8, device=DEV)
    bs = torch.zeros((8, 1), dtype=torch.uint8, device=DEV)
    y = mx.gemm(z, zs, b, bs, torch.float32)
    assert y.shape == (0, 8)


# -------------------------------------------------- linear layer, tiny ---

def test_tiny_linear_end_to_end():
    """The tiny workload end to end: both operands quantized on the device
    (bit-exact vs the oracle), then the GEMM checked on every element."""
    inp = workloads.make("tiny")
    x = to_dev(inp["x"])
    w = to_dev(inp["w"])
    wc, ws = mx.quantize_weight(w)
    xc, xs = mx.quantize_rotate(x)
    y = mx.gemm(xc, xs, wc, ws, torch.float32)
    yl = mx.linear(x, wc, ws, None, torch.float32)
    torch.cuda.synchronize()
    rxc, rxs = oracle.quantize(inp["x"])
    rwc, rws = oracle.quantize(inp["w"])
    assert np.array_equal(xc.cpu().numpy(), rxc) and np.array_equal(xs.cpu().numpy(), rxs)
    assert np.array_equal(wc.cpu().numpy(), rwc) and np.array_equal(ws.cpu().numpy(), rws)
    ref = oracle.gemm(rxc, rxs, rwc, rws)
    err = norm_err(y.cpu().numpy(), ref, row_norms(rxc, rxs), row_norms(rwc, rws))
    assert err <= TOL
    assert torch.equal(y, yl)


# --------------------------------------------------------- full workloads ---

def act_rot(inp):
    wl = inp["wl"]
    if wl.rot == "h32":
        return "h32"
    if wl.rot == "kron":
        return mx.Kron.from_host(inp["a"], inp["b"], DEV)
    return None


def oracle_weight_rot(inp):
    """The weight side of the workload's transform, from the oracle alone:
    Hadamard-32 is its own inverse transpose; for the Kronecker transform the
    oracle's own (A^-T, B^-T) ("KroQuant: ...", "Hintergrund": the inverse
    transform goes on the weights)."""
    wl = inp["wl"]
    if wl.rot == "kron":
        return ("kron", oracle.inverse_transpose(inp["a"]), oracle.inverse_transpose(inp["b"]))
    return wl.rot


# Every output element is compared where the full binary64 oracle GEMM fits in
# seconds of host time; flux_fused_h32 (7.6 TFLOP in binary64) is checked on
# 512 whole rows, every element of its first and last rows and columns, and
# 4096 random entries.
FULL_CHECK = {"flux_up", "flux_down_h32", "llm_decode_kron"}


@pytest.mark.parametrize("name,layout", [(n, "tiled") for n in workloads.WORKLOADS if n != "tiny"]
                         + [("flux_up", "rowmajor")])
def test_full_workload_linear(name, layout):
    """Full-size linear layer in the launch configuration the benchmark
    times (tiled layout): device quantization of X (activation side) and W
    (weight side), then the GEMM.  Operands are checked bit-exact against the
    oracle's quantizer (after untiling on the host), with the weight-side fold
    factors computed by the oracle; outputs against the oracle's binary64 GEMM
    of the oracle's operands."""
    inp = workloads.make(name)
    wl = inp["wl"]
    lay = mx.TILED if layout == "tiled" else mx.ROWMAJOR
    bf16 = wl.x_dtype == "bf16"
    x = to_dev(inp["x"].view(np.int16)).view(torch.bfloat16) if bf16 else to_dev(inp["x"])
    w = to_dev(inp["w"])
    rot = act_rot(inp)
    announce("linear", name, layout, wl.m, wl.n, wl.k)
    wc, ws = mx.quantize_weight(w, rot, layout=lay)
    out_dtype = torch.bfloat16 if wl.out_dtype == "bf16" else torch.float32
    xc, xs = mx.quantize_rotate(x, rot, layout=lay)
    y32 = mx.gemm(xc, xs, wc, ws, torch.float32, layout=lay, m=wl.m, n=wl.n)
    y = mx.gemm(xc, xs, wc, ws, out_dtype, layout=lay, m=wl.m, n=wl.n)
    torch.cuda.synchronize()
    hxc, hxs, hwc, hws = (t.cpu().numpy() for t in (xc, xs, wc, ws))
    if lay == mx.TILED:
        hxc, hxs = mx.untile_host(hxc, hxs, wl.m)
        hwc, hws = mx.untile_host(hwc, hws, wl.n)
    # operands: bit-exact against the oracle's quantizer
    orot = None if wl.rot is None else ("h32" if wl.rot == "h32" else ("kron", inp["a"], inp["b"]))
    rxc, rxs = oracle.quantize(inp["x"], rot=orot, bf16=bf16)
    assert np.array_equal(hxc, rxc) and np.array_equal(hxs, rxs)
    rwc, rws = oracle.quantize(inp["w"], rot=oracle_weight_rot(inp))
    assert np.array_equal(hwc, rwc) and np.array_equal(hws, rws)
    del hxc, hxs, hwc, hws
    m, n = wl.m, wl.n
    if name in FULL_CHECK:
        ref = oracle.gemm(rxc, rxs, rwc, rws)
        err = norm_err(y32.cpu().numpy(), ref, row_norms(rxc, rxs), row_norms(rwc, rws))
        print(f"[result] {name} {layout}: max normalized error {err:.3e} over all {m * n} outputs", flush=True)
        assert err <= TOL
        del ref
    else:
        rng = np.random.default_rng(1)
        rows = np.sort(rng.choice(m, 512, replace=False))
        ref = oracle.gemm(rxc[rows], rxs[rows], rwc, rws)
        na, nb = row_norms(rxc[rows], rxs[rows]), row_norms(rwc, rws)
        err = norm_err(y32[torch.from_numpy(rows).to(DEV)].cpu().numpy(), ref, na, nb)
        del ref
        mi = np.concatenate([rng.integers(0, m, 4096), np.zeros(n, np.int64), np.full(n, m - 1),
                             np.arange(m), np.arange(m)])
        ni = np.concatenate([rng.integers(0, n, 4096), np.arange(n), np.arange(n),
                             np.zeros(m, np.int64), np.full(m, n - 1)])
        ref = oracle.gemm_entries(rxc, rxs, rwc, rws, mi, ni)
        ua, ub = np.unique(mi), np.unique(ni)
        nmap_a = dict(zip(ua, row_norms(rxc[ua], rxs[ua])))
        nmap_b = dict(zip(ub, row_norms(rwc[ub], rws[ub])))
        den_a = np.array([nmap_a[i] for i in mi])
        den_b = np.array([nmap_b[j] for j in ni])
        g32 = y32[torch.from_numpy(mi).to(DEV), torch.from_numpy(ni).to(DEV)].cpu().numpy()
        err = max(err, norm_err(g32, ref, den_a, den_b))
        print(f"[result] {name} {layout}: max normalized error {err:.3e} on 512 rows and sampled entries",
              flush=True)
        assert err <= TOL
    if out_dtype == torch.bfloat16:
        assert torch.equal(y.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16))
