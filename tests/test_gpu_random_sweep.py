"""Seeded random sweep over the whole layer on the device: activation
quantization (with a drawn block transform), then the GEMM against MXFP4
weights, for shapes, layouts and dtypes drawn from one generator per case.

Each case draws
  * M (1..64 for the small-M kernels, 65..1299 otherwise), N (1..1599) and
    K (a multiple of 32 up to 3072; a multiple of 128 for the tiled layout and
    for half of the row-major cases, which sends M > 64 to the large-tile
    kernel);
  * the layout (row-major or tiled), the activation dtype (fp32 or bf16), the
    transform (none, Hadamard-32, Kronecker with a drawn p x q, per-channel
    smoothing) and the output dtype (fp32 or bf16).

Checks, the same bars as the fixed-shape tests:
  * activation codes and scales bit-exact against the oracle (tiled bytes
    untiled on the host first);
  * fp32 output within 1e-5 of the oracle's binary64 GEMM, normalized by the
    product of the dequantized row norms (the derivation is in the GEMM
    tests); bf16 output the round-to-nearest-even bf16 of the same kernel's
    fp32 output.

Three more draws use the same bars: the fused small-M layer (quantization
inside the GEMM; bf16 activations, M <= 64, Kronecker 2 <= p <= 16), the same
on wide weights (8000..24000 rows, K up to 8192; there the fused fp32 Y must
also equal the split path's bit for bit), and the
GEMM with an MXFP4 output on operands whose block exponents lie in [-1, 1],
where Y is exact in fp32 and the requantized bytes must equal the oracle
quantizer's on the oracle's Y.
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
CASES = 40
KRON_PQ = [(2, 16), (4, 8), (8, 4), (16, 2)]


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def row_norms(codes, scales):
    return np.sqrt((oracle.dequantize(codes, scales) ** 2).sum(axis=1))


def draw(i):
    rng = np.random.default_rng(7000 + i)
    small = rng.random() < 0.35
    m = int(rng.integers(1, 65)) if small else int(rng.integers(65, 1300))
    n = int(rng.integers(1, 1600))
    tiled = rng.random() < 0.5
    k = 32 * int(rng.integers(1, 97))
    if tiled or rng.random() < 0.5:
        k = 128 * max(1, k // 128)
    bf16 = rng.random() < 0.6
    rot = ["none", "h32", "kron", "smooth"][int(rng.integers(0, 4))]
    pq = KRON_PQ[int(rng.integers(0, len(KRON_PQ)))]
    out = torch.bfloat16 if rng.random() < 0.5 else torch.float32
    return rng, m, n, k, tiled, bf16, rot, pq, out


def make_rot(kind, pq, k, rng):
    """(device transform, oracle transform)"""
    if kind == "none":
        return None, None
    if kind == "h32":
        return "h32", "h32"
    if kind == "smooth":
        r = (0.25 + 4 * rng.random(k)).astype(np.float32)
        return mx.Smooth.from_host(r, DEV), ("smooth", r)
    p, q = pq
    a = (np.eye(p) + 0.1 * rng.standard_normal((p, p))).astype(np.float32)
    b = (np.eye(q) + 0.1 * rng.standard_normal((q, q))).astype(np.float32)
    return mx.Kron.from_host(a, b, DEV), ("kron", a, b)


@pytest.mark.parametrize("i", range(CASES))
def test_random_layer_case(i):
    rng, m, n, k, tiled, bf16, rot, pq, out = draw(i)
    layout = mx.TILED if tiled else mx.ROWMAJOR
    print(f"[case] sweep {i}: m={m} n={n} k={k} tiled={tiled} bf16={bf16} rot={rot}"
          f"{pq if rot == 'kron' else ''} out={out}", flush=True)
    x32 = workloads.random_blocks(rng, m, k)
    dev_rot, ref_rot = make_rot(rot, pq, k, rng)
    if bf16:
        xh = workloads.bf16_bits(x32)
        xd = to_dev(xh.view(np.int16)).view(torch.bfloat16)
        xc, xs = oracle.quantize(xh, rot=ref_rot, bf16=True)
    else:
        xd = to_dev(x32)
        xc, xs = oracle.quantize(x32, rot=ref_rot)
    wc, ws = workloads.random_mxfp4(rng, n, k)
    if tiled:
        wd = [to_dev(t) for t in mx.tile_host(wc, ws)]
    else:
        wd = [to_dev(wc), to_dev(ws)]

    ac, as_ = mx.quantize_rotate(xd, dev_rot, layout=layout)
    y = mx.gemm(ac, as_, *wd, out, layout=layout, m=m, n=n)
    y32 = y if out == torch.float32 else mx.gemm(ac, as_, *wd, torch.float32, layout=layout, m=m, n=n)
    torch.cuda.synchronize()

    gc, gs = ac.cpu().numpy(), as_.cpu().numpy()
    if tiled:
        gc, gs = mx.untile_host(gc, gs, m)
    assert np.array_equal(gc, xc), f"{np.count_nonzero(gc != xc)} code bytes differ"
    assert np.array_equal(gs, xs), f"{np.count_nonzero(gs != xs)} scale bytes differ"

    ref = oracle.gemm(xc, xs, wc, ws)
    den = np.outer(row_norms(xc, xs), row_norms(wc, ws))
    diff = np.abs(y32.cpu().numpy().astype(np.float64) - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(den > 0, diff / den, np.where(diff == 0, 0.0, np.inf))
    err = float(rel.max()) if rel.size else 0.0
    assert err <= TOL, f"normalized error {err:.3e}"
    if out == torch.bfloat16:
        assert torch.equal(y.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16))


FUSED_CASES = 24
FUSED_ROTS = ["none", "h32", "smooth", "kron"]


@pytest.mark.parametrize("i", range(FUSED_CASES))
def test_random_fused_small_m_case(i):
    rng = np.random.default_rng(9000 + i)
    m = int(rng.integers(1, 65))
    n = int(rng.integers(1, 3000))
    tiled = rng.random() < 0.5
    k = 32 * int(rng.integers(1, 129))
    if tiled:
        k = 128 * max(1, k // 128)
    rot = FUSED_ROTS[int(rng.integers(0, 4))]
    pq = KRON_PQ[int(rng.integers(0, len(KRON_PQ)))]
    out = torch.float32 if rng.random() < 0.5 else torch.bfloat16
    layout = mx.TILED if tiled else mx.ROWMAJOR
    print(f"[case] fused sweep {i}: m={m} n={n} k={k} tiled={tiled} rot={rot}"
          f"{pq if rot == 'kron' else ''} out={out}", flush=True)
    xh = workloads.bf16_bits(workloads.random_blocks(rng, m, k))
    dev_rot, ref_rot = make_rot(rot, pq, k, rng)
    wc, ws = workloads.random_mxfp4(rng, n, k)
    wd = [to_dev(t) for t in (mx.tile_host(wc, ws) if tiled else (wc, ws))]
    xd = to_dev(xh.view(np.int16)).view(torch.bfloat16)
    y32 = mx.linear_small(xd, *wd, dev_rot, torch.float32, layout=layout, n=n)
    y = mx.linear_small(xd, *wd, dev_rot, out, layout=layout, n=n)
    torch.cuda.synchronize()
    xc, xs = oracle.quantize(xh, rot=ref_rot, bf16=True)
    ref = oracle.gemm(xc, xs, wc, ws)
    den = np.outer(row_norms(xc, xs), row_norms(wc, ws))
    diff = np.abs(y32.cpu().numpy().astype(np.float64) - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(den > 0, diff / den, np.where(diff == 0, 0.0, np.inf))
    err = float(rel.max()) if rel.size else 0.0
    assert err <= TOL, f"normalized error {err:.3e}"
    if out == torch.bfloat16:
        assert torch.equal(y.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16))


WIDE_CASES = 6


@pytest.mark.parametrize("i", range(WIDE_CASES))
def test_random_fused_wide_case(i):
    """The fused layer on 8000..24000 weight rows and K up to 8192: grids of
    about a hundred to several hundred workgroups (past the CU count the
    producers sit in the compute workgroups), and up to 8 compute waves.  Its
    fp32 Y must equal the split path's (quantizer, then GEMM) bit for bit and
    be within the bound of the oracle."""
    rng = np.random.default_rng(50000 + i)
    m = int(rng.integers(1, 65))
    n = int(rng.integers(8000, 24000))
    tiled = rng.random() < 0.6
    k = 32 * int(rng.integers(1, 257))
    if tiled:
        k = 128 * max(1, k // 128)
    rot = FUSED_ROTS[int(rng.integers(0, 4))]
    pq = KRON_PQ[int(rng.integers(0, len(KRON_PQ)))]
    out = torch.float32 if rng.random() < 0.5 else torch.bfloat16
    layout = mx.TILED if tiled else mx.ROWMAJOR
    print(f"[case] fused wide {i}: m={m} n={n} k={k} tiled={tiled} rot={rot}"
          f"{pq if rot == 'kron' else ''} out={out}", flush=True)
    xh = workloads.bf16_bits(workloads.random_blocks(rng, m, k))
    dev_rot, ref_rot = make_rot(rot, pq, k, rng)
    wc, ws = workloads.random_mxfp4(rng, n, k)
    wd = [to_dev(t) for t in (mx.tile_host(wc, ws) if tiled else (wc, ws))]
    xd = to_dev(xh.view(np.int16)).view(torch.bfloat16)
    y32 = mx.linear_small(xd, *wd, dev_rot, torch.float32, layout=layout, n=n)
    y = mx.linear_small(xd, *wd, dev_rot, out, layout=layout, n=n)
    ac, as_ = mx.quantize_rotate(xd, dev_rot, layout=layout)
    ys = mx.gemm(ac, as_, *wd, torch.float32, layout=layout, m=m, n=n)
    torch.cuda.synchronize()
    assert torch.equal(ys.view(torch.int32), y32.view(torch.int32)), "fused and split fp32 Y differ"
    xc, xs = oracle.quantize(xh, rot=ref_rot, bf16=True)
    ref = oracle.gemm(xc, xs, wc, ws)
    den = np.outer(row_norms(xc, xs), row_norms(wc, ws))
    diff = np.abs(y32.cpu().numpy().astype(np.float64) - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(den > 0, diff / den, np.where(diff == 0, 0.0, np.inf))
    err = float(rel.max()) if rel.size else 0.0
    assert err <= TOL, f"normalized error {err:.3e}"
    if out == torch.bfloat16:
        assert torch.equal(y.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16))


REQUANT_CASES = 16


@pytest.mark.parametrize("i", range(REQUANT_CASES))
def test_random_requant_case(i):
    rng = np.random.default_rng(11000 + i)
    m = int(rng.integers(65, 1500))
    layout = mx.TILED if rng.random() < 0.5 else mx.ROWMAJOR
    out_layout = mx.TILED if rng.random() < 0.5 else mx.ROWMAJOR
    n = 128 * int(rng.integers(1, 12)) if out_layout == mx.TILED else 32 * int(rng.integers(1, 48))
    k = 128 * int(rng.integers(1, 33))
    print(f"[case] requant sweep {i}: m={m} n={n} k={k} layout={layout} out_layout={out_layout}", flush=True)
    ac, as_ = workloads.random_mxfp4(rng, m, k, -1, 1)
    bc, bs = workloads.random_mxfp4(rng, n, k, -1, 1)
    dev = [to_dev(t) for t in ((*mx.tile_host(ac, as_), *mx.tile_host(bc, bs)) if layout == mx.TILED
                               else (ac, as_, bc, bs))]
    ref = oracle.gemm(ac, as_, bc, bs)
    y32 = ref.astype(np.float32)
    assert np.array_equal(y32.astype(np.float64), ref)   # every partial sum is exact in fp32
    want_c, want_s = oracle.quantize(y32)
    qc, qs = mx.gemm_requant(*dev, layout=layout, out_layout=out_layout, m=m, n=n)
    torch.cuda.synchronize()
    gc, gs = qc.cpu().numpy(), qs.cpu().numpy()
    if out_layout == mx.TILED:
        gc, gs = mx.untile_host(gc, gs, m)
    assert np.array_equal(gs, want_s), f"{np.count_nonzero(gs != want_s)} scale bytes differ"
    assert np.array_equal(gc, want_c), f"{np.count_nonzero(gc != want_c)} code bytes differ"
