"""GPU parity of the MXFP4 quantizer: codes and scales must equal the CPU
oracle's bit for bit, on the same seeded inputs, for every rotation, input
dtype, ragged size, strided input, edge block and full-size workload."""
import numpy as np
import pytest
import torch

import mxfp4_w4a4_quantized_amd as mx
import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def announce(*what):
    print("[case]", *what, flush=True)


def dev_x(x_host: np.ndarray, bf16: bool) -> torch.Tensor:
    if bf16:
        return torch.from_numpy(np.ascontiguousarray(x_host).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x_host, np.float32)).to(DEV)


def gpu_quantize(x_host, bf16, rot=None):
    x = dev_x(x_host, bf16)
    c, s = mx.quantize_rotate(x, rot)
    torch.cuda.synchronize()
    return c.cpu().numpy(), s.cpu().numpy()


def oracle_rot(rot):
    if rot is None or rot == "h32":
        return rot
    return ("kron", rot.a.cpu().numpy(), rot.b.cpu().numpy())


def assert_same(got, ref, what):
    gc, gs = got
    rc, rs = ref
    bad_s = np.count_nonzero(gs != rs)
    bad_c = np.count_nonzero(gc != rc)
    assert bad_s == 0 and bad_c == 0, f"{what}: {bad_s} scale bytes and {bad_c} code bytes differ"


def check(x_host, bf16, rot=None, what=""):
    announce("quantize", what, x_host.shape, "bf16" if bf16 else "f32", rot if isinstance(rot, str) else type(rot).__name__)
    got = gpu_quantize(x_host, bf16, rot)
    ref = oracle.quantize(x_host, rot=oracle_rot(rot), bf16=bf16)
    assert_same(got, ref, what)


def rand_kron(p, q, seed):
    rng = np.random.default_rng(seed)
    a = (np.eye(p) + 0.1 * rng.standard_normal((p, p))).astype(np.float32)
    b = (np.eye(q) + 0.1 * rng.standard_normal((q, q))).astype(np.float32)
    return mx.Kron.from_host(a, b, DEV)


# ------------------------------------------------------------ small cases ---

@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("rot", [None, "h32"])
@pytest.mark.parametrize("rows,k", [(1, 32), (3, 96), (64, 256), (257, 544), (1000, 4096)])
def test_random_blocks(rows, k, rot, bf16):
    rng = np.random.default_rng(rows * 7 + k)
    x = workloads.random_blocks(rng, rows, k)
    if bf16:
        x = workloads.bf16_bits(x)
    check(x, bf16, rot, f"random {rows}x{k}")


# Up to 16384 blocks a Kronecker transform with p <= 16 runs on q lanes per
# block, above that on one lane per block: 129 x 320 (1290 blocks) and
# 700 x 1024 (22400 blocks) take one kernel each.
@pytest.mark.parametrize("rows,k", [(129, 320), (700, 1024)], ids=["q-lanes", "one-lane"])
@pytest.mark.parametrize("p,q", [(1, 32), (2, 16), (4, 8), (8, 4), (16, 2), (32, 1)])
@pytest.mark.parametrize("bf16", [False, True])
def test_kron_all_factorizations(p, q, bf16, rows, k):
    rng = np.random.default_rng(p * 100 + q + rows)
    x = workloads.random_blocks(rng, rows, k)
    if bf16:
        x = workloads.bf16_bits(x)
    check(x, bf16, rand_kron(p, q, p + 17 * q), f"kron {p}x{q}")


def edge_blocks(big: float = 3.0e38) -> np.ndarray:
    """Edge blocks; `big` is the near-overflow magnitude (kept small enough
    that a rotation's sums stay finite)."""
    rows = []
    z = np.zeros(32, np.float32)
    rows.append(z.copy())                                        # all zero
    rows.append(np.full(32, -0.0, np.float32))                   # all -0
    rows.append(np.full(32, 1e-45, np.float32))                  # min subnormal
    r = np.full(32, 2.0 ** -127, np.float32); r[3] = 2.0 ** -126; rows.append(r)   # subnormal elements, nonzero codes
    r = np.full(32, big, np.float32); r[1] = -big; rows.append(r)                   # near FLT_MAX
    rows.append(np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0] * 4, np.float32))   # ties, e = 0
    rows.append(-np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0] * 4, np.float32))
    r = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 4.0] * 4, np.float32) * np.float32(2.0 ** -60); rows.append(r)
    r = np.linspace(-7.99, 7.99, 32).astype(np.float32); rows.append(r)                # saturation band
    r = np.zeros(32, np.float32); r[17] = -1e-30; rows.append(r)                       # single tiny value
    r = np.full(32, 4.0, np.float32); rows.append(r)                                   # power-of-two amax
    r = np.full(32, np.nextafter(np.float32(4.0), np.float32(0)), np.float32); rows.append(r)
    r = np.full(32, np.nextafter(np.float32(8.0), np.float32(0)), np.float32); rows.append(r)
    x = np.stack(rows)
    return np.concatenate([x, x[::-1] * np.float32(0.5)], axis=1)   # 64 columns: two blocks per row


def test_edge_blocks_f32():
    check(edge_blocks(), False, None, "edge f32")
    check(edge_blocks(1.0e37), False, "h32", "edge f32 h32")


def test_edge_blocks_kron():
    check(edge_blocks(1.0e36), False, rand_kron(4, 8, 3), "edge kron")
    # 700 copies (36400 blocks): the one-lane kernel
    check(np.tile(edge_blocks(1.0e36), (700, 1)), False, rand_kron(4, 8, 3), "edge kron, one lane")
    check(edge_blocks(1.0e36), False, rand_kron(16, 2, 4), "edge kron 16x2")


def test_edge_blocks_bf16():
    check(workloads.bf16_bits(edge_blocks()), True, None, "edge bf16")
    check(workloads.bf16_bits(edge_blocks(1.0e37)), True, "h32", "edge bf16 h32")


def test_exhaustive_bf16_values():
    # every finite bf16 bit pattern appears, in blocks whose amax is fixed by
    # one large element so that codes cover the whole grid at many scales
    h = np.arange(0, 0x10000, dtype=np.uint32)
    h = h[((h >> 7) & 0xFF) != 0xFF].astype(np.uint16)      # drop Inf/NaN
    n = (h.size + 30) // 31 * 31
    h = np.concatenate([h, np.zeros(n - h.size, np.uint16)]).reshape(-1, 31)
    x = np.concatenate([h, np.full((h.shape[0], 1), 0x4100, np.uint16)], axis=1)   # 8.0
    check(np.ascontiguousarray(x), True, None, "all bf16")
    # rotated blocks must stay finite (sums of 32 values): below 2^120 only
    small = h[((h.astype(np.uint32) >> 7) & 0xFF).max(axis=1) < 127 + 120]
    xs = np.concatenate([small, np.full((small.shape[0], 1), 0x4100, np.uint16)], axis=1)
    check(np.ascontiguousarray(xs), True, "h32", "all bf16 below 2^120, h32")


def test_strided_input_rows():
    rng = np.random.default_rng(5)
    full = workloads.bf16_bits(workloads.random_blocks(rng, 40, 512))
    x = dev_x(full, True)[:, :256]                   # ld_x = 512 > k = 256
    announce("quantize strided", x.shape, x.stride())
    c, s = mx.quantize_rotate(x, "h32")
    ref = oracle.quantize(np.ascontiguousarray(full[:, :256]), rot="h32", bf16=True)
    assert_same((c.cpu().numpy(), s.cpu().numpy()), ref, "strided")


@pytest.mark.parametrize("rows,k,bf16,rot", [
    (1, 128, True, None), (255, 256, True, "h32"), (300, 384, False, None), (513, 512, True, "kron"),
    (1024, 3072, True, "h32"), (16, 4096, True, "kron"), (2000, 1024, True, "kron")])
def test_tiled_layout_matches_oracle(rows, k, bf16, rot):
    """Tiled output (the GEMM-native layout): untiled on the host it must equal
    the oracle's codes and scales bit for bit.  The padding rows of the last
    16-row group holding real rows are written as zeros; the padding rows past
    it are left untouched (here: the 0xFF the buffers were filled with)."""
    rng = np.random.default_rng(rows * 3 + k)
    x = workloads.random_blocks(rng, rows, k)
    if bf16:
        x = workloads.bf16_bits(x)
    r = rand_kron(4, 8, 9) if rot == "kron" else rot
    announce("quantize tiled", rows, k, "bf16" if bf16 else "f32", rot)
    rp = mx.padded_rows(rows)
    c = torch.full((rp, k // 2), 0xFF, dtype=torch.uint8, device=DEV)
    s = torch.full((rp, k // 32), 0xFF, dtype=torch.uint8, device=DEV)
    mx.quantize_rotate(dev_x(x, bf16), r, codes=c, scales=s, layout=mx.TILED)
    torch.cuda.synchronize()
    tc, ts = c.cpu().numpy(), s.cpu().numpy()
    got = mx.untile_host(tc, ts, rows)
    ref = oracle.quantize(x, rot=oracle_rot(r), bf16=bf16)
    assert_same(got, ref, f"tiled {rows}x{k}")
    pc, ps = mx.untile_host(tc, ts, rp)
    r16 = (rows + 15) // 16 * 16
    assert not pc[rows:r16].any() and not ps[rows:r16].any()
    assert (pc[r16:] == 0xFF).all() and (ps[r16:] == 0xFF).all()


# Strided activation rows (ld_x > k) with a Kronecker transform, on the
# q-lanes kernel (40 rows, 320 blocks) and on the one-lane kernel (1800 rows,
# 18000 blocks), in both layouts and input dtypes.
@pytest.mark.parametrize("rows", [40, 1800], ids=["q-lanes", "one-lane"])
@pytest.mark.parametrize("layout", [mx.ROWMAJOR, mx.TILED], ids=["rowmajor", "tiled"])
@pytest.mark.parametrize("bf16", [False, True])
def test_kron_strided_rows(rows, layout, bf16):
    k, ld = 1280, 1408
    rng = np.random.default_rng(rows + ld)
    full = workloads.random_blocks(rng, rows, ld)
    if bf16:
        full = workloads.bf16_bits(full)
    x = dev_x(full, bf16)[:, :k]
    r = rand_kron(8, 4, rows)
    announce("quantize kron strided", rows, k, ld, "bf16" if bf16 else "f32", layout)
    c, sc = mx.quantize_rotate(x, r, layout=layout)
    torch.cuda.synchronize()
    got = (c.cpu().numpy(), sc.cpu().numpy())
    if layout == mx.TILED:
        got = mx.untile_host(got[0], got[1], rows)
    ref = oracle.quantize(np.ascontiguousarray(full[:, :k]), rot=oracle_rot(r), bf16=bf16)
    assert_same(got, ref, "kron strided")


def test_tiled_strided_input():
    rng = np.random.default_rng(6)
    full = workloads.bf16_bits(workloads.random_blocks(rng, 70, 640))
    x = dev_x(full, True)[:, :256]                   # ld_x = 640 > k = 256
    announce("quantize tiled strided", x.shape, x.stride())
    c, s = mx.quantize_rotate(x, "h32", layout=mx.TILED)
    got = mx.untile_host(c.cpu().numpy(), s.cpu().numpy(), 70)
    ref = oracle.quantize(np.ascontiguousarray(full[:, :256]), rot="h32", bf16=True)
    assert_same(got, ref, "tiled strided")


def test_zero_rows_is_noop():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    c, s = mx.quantize_rotate(x)
    assert c.shape == (0, 32) and s.shape == (0, 2)


def test_errors_raise():
    x = torch.zeros((4, 48), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(mx.Mxfp4Error):
        mx.quantize_rotate(x)

# ------------------------------------------------- smoothing and scale fitting ---

def rand_smooth(k, seed):
    rng = np.random.default_rng(seed)
    return mx.Smooth.from_host((0.25 + 4 * rng.random(k)).astype(np.float32), DEV)


def oracle_rot_any(rot):
    if isinstance(rot, mx.Smooth):
        return ("smooth", rot.r.cpu().numpy())
    return oracle_rot(rot)


def make_rot(kind, k, seed):
    if kind == "kron":
        return rand_kron(4, 8, seed)
    if kind == "smooth":
        return rand_smooth(k, seed)
    return kind


def quantize_both(x_host, bf16, rot, layout, fit):
    rows, k = x_host.shape
    announce("quantize", "fit" if fit else "", rot if isinstance(rot, (str, type(None))) else type(rot).__name__,
             rows, k, "bf16" if bf16 else "f32", "tiled" if layout == mx.TILED else "rowmajor")
    c, s = mx.quantize_rotate(dev_x(x_host, bf16), rot, layout=layout, fit=fit)
    torch.cuda.synchronize()
    got = (c.cpu().numpy(), s.cpu().numpy())
    if layout == mx.TILED:
        got = mx.untile_host(got[0], got[1], rows)
    ref = oracle.quantize(x_host, rot=oracle_rot_any(rot), bf16=bf16, fit=fit)
    return got, ref


@pytest.mark.parametrize("layout", [mx.ROWMAJOR, mx.TILED])
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("rows,k", [(3, 128), (70, 512), (300, 3072)])
def test_smooth_matches_oracle(rows, k, bf16, layout):
    rng = np.random.default_rng(rows + k + bf16)
    x = workloads.random_blocks(rng, rows, k)
    if bf16:
        x = workloads.bf16_bits(x)
    got, ref = quantize_both(x, bf16, rand_smooth(k, rows * 3 + k), layout, False)
    assert_same(got, ref, f"smooth {rows}x{k}")


def test_smooth_strided_rows():
    # ld_x > k: the kernel's non-dense block addressing picks each block's factors
    rng = np.random.default_rng(12)
    full = workloads.bf16_bits(workloads.random_blocks(rng, 33, 640))
    r = rand_smooth(256, 13)
    x = dev_x(full, True)[:, :256]
    announce("quantize smooth strided", x.shape, x.stride())
    c, s = mx.quantize_rotate(x, r)
    ref = oracle.quantize(np.ascontiguousarray(full[:, :256]), rot=oracle_rot_any(r), bf16=True)
    assert_same((c.cpu().numpy(), s.cpu().numpy()), ref, "smooth strided")


@pytest.mark.parametrize("layout", [mx.ROWMAJOR, mx.TILED])
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("rot", [None, "h32", "kron", "smooth"])
def test_fit_matches_oracle(rot, bf16, layout):
    rng = np.random.default_rng(20 + bf16)
    rows, k = 257, 1024
    x = workloads.random_blocks(rng, rows, k)
    x[rng.random(x.shape) < 0.05] *= np.float32(9.0)      # outliers inside blocks
    if bf16:
        x = workloads.bf16_bits(x)
    got, ref = quantize_both(x, bf16, make_rot(rot, k, 31), layout, True)
    assert_same(got, ref, f"fit {rot}")
    # the fitted exponents differ from the plain rule somewhere (the test bites)
    plain = oracle.quantize(x, rot=oracle_rot_any(make_rot(rot, k, 31)), bf16=bf16)
    assert np.count_nonzero(plain[1] != ref[1]) > 0


def test_fit_edge_blocks():
    for bf16 in (False, True):
        x = edge_blocks()
        if bf16:
            x = workloads.bf16_bits(x)
        got, ref = quantize_both(x, bf16, None, mx.ROWMAJOR, True)
        assert_same(got, ref, "fit edge")


def test_smoothed_linear_matches_oracle():
    """A smoothed linear layer: activations multiplied by r per channel, the
    weights by 1/r (binary64 quotient rounded to fp32, the library's helper on
    the device side and the oracle's on the reference side); the GEMM of the
    two quantized operands against the oracle's."""
    rng = np.random.default_rng(40)
    m, n, k = 300, 260, 512
    x = workloads.bf16_bits(workloads.random_blocks(rng, m, k))
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    sm = rand_smooth(k, 41)
    announce("smoothed linear", m, n, k)
    wc, ws = mx.quantize_weight(torch.from_numpy(w).to(DEV), sm)
    y = mx.linear(dev_x(x, True), wc, ws, sm, torch.float32)
    torch.cuda.synchronize()
    xc, xs = oracle.quantize(x, rot=oracle_rot_any(sm), bf16=True)
    # weight side: the oracle's own reciprocal factors
    rwc, rws = oracle.quantize(w, rot=("smooth", oracle.smooth_weight_factors(sm.r.cpu().numpy())))
    assert np.array_equal(wc.cpu().numpy(), rwc) and np.array_equal(ws.cpu().numpy(), rws)
    ref = oracle.gemm(xc, xs, rwc, rws)
    den = np.outer(np.sqrt((oracle.dequantize(xc, xs) ** 2).sum(1)), np.sqrt((oracle.dequantize(rwc, rws) ** 2).sum(1)))
    assert (np.abs(y.cpu().numpy() - ref) <= 1e-5 * den).all()


# Full-size workloads (both operands, every code and scale byte) are checked
# in test_gpu_gemm.test_full_workload_linear, in the benchmark's launch setup.
