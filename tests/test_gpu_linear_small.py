"""GPU parity of the fused small-M linear layer (mxfp4_linear_small): the
activations are rotated and quantized inside the GEMM kernel.

Three kinds of check:
  * Exact pin of the in-GEMM quantization.  With W the K x K identity
    (quantized without rotation: each row has one element 1.0, encoded exactly
    as code 4.0 at scale 2^-2), every output element is a single exact product,
    Y[m][j] = x_hat[m][j].  So the fused kernel's fp32 output must equal the
    dequantized oracle codes of rot(X) bit for bit.
  * The layer against the oracle's binary64 GEMM of the oracle-quantized
    activations, at the normalized 1e-5 bound of the GEMM tests, for random
    MXFP4 weights; bf16 output equal to the round-to-nearest-even bf16 of the
    same kernel's fp32 output.
  * The layer against the unfused path (quantize_rotate, then gemm) on the
    same inputs: bit-identical Y, since both take the same K split and
    summation order.
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
LAYOUTS = {"rowmajor": mx.ROWMAJOR, "tiled": mx.TILED}


def announce(*what):
    print("[case]", *what, flush=True)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bf16_dev(x_bits):
    return to_dev(x_bits.view(np.int16)).view(torch.bfloat16)


def make_rot(r, seed=5, k=None):
    if r is None or r == "h32":
        return r
    if r == "smooth":
        rng = np.random.default_rng(seed)
        return mx.Smooth.from_host((0.25 + 4 * rng.random(k)).astype(np.float32), DEV)
    p, q = r
    rng = np.random.default_rng(seed)
    a = (np.eye(p) + 0.1 * rng.standard_normal((p, p))).astype(np.float32)
    b = (np.eye(q) + 0.1 * rng.standard_normal((q, q))).astype(np.float32)
    return mx.Kron.from_host(a, b, DEV)


def oracle_rot(rot):
    if rot is None or rot == "h32":
        return rot
    if isinstance(rot, mx.Smooth):
        return ("smooth", rot.r.cpu().numpy())
    return ("kron", rot.a.cpu().numpy(), rot.b.cpu().numpy())


def weights_dev(wc, ws, layout):
    if layout == mx.TILED:
        wc, ws = mx.tile_host(wc, ws)
    return to_dev(wc), to_dev(ws)


def row_norms(codes, scales):
    return np.sqrt((oracle.dequantize(codes, scales) ** 2).sum(axis=1))


def norm_err(got, ref, na, nb):
    den = np.outer(na, nb)
    diff = np.abs(got.astype(np.float64) - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(den > 0, diff / den, np.where(diff == 0, 0.0, np.inf))
    return float(rel.max()) if rel.size else 0.0


ROTS = [None, "h32", "smooth", (2, 16), (4, 8), (8, 4), (16, 2)]


@pytest.mark.parametrize("layout", ["rowmajor", "tiled"])
@pytest.mark.parametrize("m", [1, 16, 33, 64])
@pytest.mark.parametrize("rot", ROTS, ids=str)
def test_fused_quantization_is_bit_exact(rot, m, layout):
    k = 512
    rng = np.random.default_rng(m * 7 + k)
    x = workloads.bf16_bits(workloads.random_blocks(rng, m, k))
    r = make_rot(rot, k=k)
    xc, xs = oracle.quantize(x, rot=oracle_rot(r), bf16=True)
    want = oracle.dequantize(xc, xs)                       # exact in binary64 and in fp32
    wc, ws = oracle.quantize(np.eye(k, dtype=np.float32))  # identity weights, no rotation
    assert np.array_equal(oracle.dequantize(wc, ws), np.eye(k))
    announce("linear_small identity", rot, m, k, layout)
    lay = LAYOUTS[layout]
    dwc, dws = weights_dev(wc, ws, lay)
    y = mx.linear_small(bf16_dev(x), dwc, dws, r, torch.float32, layout=lay, n=k)
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    bad = np.count_nonzero(got != want)
    assert bad == 0, f"{bad} of {got.size} dequantized activations differ"


SHAPES = [
    (1, 300, 4096, "rowmajor"), (16, 1000, 4128, "rowmajor"), (7, 77, 96, "rowmajor"),
    (17, 513, 1024, "tiled"), (40, 256, 12288, "tiled"), (64, 130, 384, "rowmajor"),
    (16, 14336, 4096, "tiled"), (33, 70, 2048, "tiled")]


@pytest.mark.parametrize("rot", [None, "h32", "smooth", (4, 8)], ids=str)
@pytest.mark.parametrize("m,n,k,layout", SHAPES)
def test_fused_linear_matches_oracle(m, n, k, layout, rot):
    rng = np.random.default_rng(m + 3 * n + k)
    x = workloads.bf16_bits(workloads.random_blocks(rng, m, k))
    wc, ws = workloads.random_mxfp4(rng, n, k)
    r = make_rot(rot, k=k)
    lay = LAYOUTS[layout]
    announce("linear_small", m, n, k, layout, rot)
    dwc, dws = weights_dev(wc, ws, lay)
    xd = bf16_dev(x)
    y32 = mx.linear_small(xd, dwc, dws, r, torch.float32, layout=lay, n=n)
    y16 = mx.linear_small(xd, dwc, dws, r, torch.bfloat16, layout=lay, n=n)
    torch.cuda.synchronize()
    xc, xs = oracle.quantize(x, rot=oracle_rot(r), bf16=True)
    ref = oracle.gemm(xc, xs, wc, ws)
    err = norm_err(y32.cpu().numpy(), ref, row_norms(xc, xs), row_norms(wc, ws))
    assert err <= TOL, f"normalized error {err:.3e}"
    assert torch.equal(y16.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16))


def test_fused_strided_input_and_output():
    rng = np.random.default_rng(91)
    m, n, k = 12, 90, 256
    full = workloads.bf16_bits(workloads.random_blocks(rng, m, 640))
    x = bf16_dev(full)[:, :k]                                   # ld_x = 640 > k
    wc, ws = workloads.random_mxfp4(rng, n, k)
    xc, xs = oracle.quantize(np.ascontiguousarray(full[:, :k]), rot="h32", bf16=True)
    ref = oracle.gemm(xc, xs, wc, ws)
    for dt, off, fill in ((torch.float32, 4, 7.0), (torch.float32, 5, 7.0), (torch.bfloat16, 5, 3.0)):
        big = torch.full((m, n + 12), fill, dtype=dt, device=DEV)
        y = big[:, off:off + n]
        announce("linear_small strided", m, n, k, dt, off)
        mx.linear_small(x, to_dev(wc), to_dev(ws), "h32", dt, y=y)
        torch.cuda.synchronize()
        if dt == torch.float32:
            assert norm_err(y.cpu().numpy(), ref, row_norms(xc, xs), row_norms(wc, ws)) <= TOL
        host = big.float().cpu().numpy()
        assert (host[:, :off] == fill).all() and (host[:, off + n:] == fill).all()   # no stray writes


def test_fused_decode_workload():
    """The decode workload through the fused path: weights quantized on the
    device with the weight side of the Kronecker transform (bit-exact against
    the oracle), the layer against the oracle on every output element."""
    inp = workloads.make("llm_decode_kron")
    wl = inp["wl"]
    rot = mx.Kron.from_host(inp["a"], inp["b"], DEV)
    announce("linear_small workload", wl.name, wl.m, wl.n, wl.k)
    wc, ws = mx.quantize_weight(to_dev(inp["w"]), rot, layout=mx.TILED)
    y = mx.linear_small(bf16_dev(inp["x"]), wc, ws, rot, torch.float32, layout=mx.TILED, n=wl.n)
    y_split = mx.linear(bf16_dev(inp["x"]), wc, ws, rot, torch.float32, layout=mx.TILED, n=wl.n)
    torch.cuda.synchronize()
    hwc, hws = mx.untile_host(wc.cpu().numpy(), ws.cpu().numpy(), wl.n)
    # weight side: the oracle's own inverse-transpose factors
    rwc, rws = oracle.quantize(inp["w"], rot=("kron", oracle.inverse_transpose(inp["a"]),
                                              oracle.inverse_transpose(inp["b"])))
    assert np.array_equal(hwc, rwc) and np.array_equal(hws, rws)
    xc, xs = oracle.quantize(inp["x"], rot=("kron", inp["a"], inp["b"]), bf16=True)
    ref = oracle.gemm(xc, xs, hwc, hws)
    na, nb = row_norms(xc, xs), row_norms(hwc, hws)
    err = norm_err(y.cpu().numpy(), ref, na, nb)
    print(f"[result] fused decode: max normalized error {err:.3e}", flush=True)
    assert err <= TOL
    assert norm_err(y_split.cpu().numpy(), ref, na, nb) <= TOL


def test_fused_unsupported_cases_raise():
    x32 = torch.zeros((4, 64), dtype=torch.float32, device=DEV)
    wc = torch.zeros((8, 32), dtype=torch.uint8, device=DEV)
    ws = torch.zeros((8, 2), dtype=torch.uint8, device=DEV)
    with pytest.raises(mx.Mxfp4Error):
        mx.linear_small(x32, wc, ws)                             # fp32 activations
    x = torch.zeros((65, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(mx.Mxfp4Error):
        mx.linear_small(x, wc, ws)                               # m > 64


SAME_AS_SPLIT = [
    (16, 14336, 4096, "tiled", (4, 8)), (1, 300, 4128, "rowmajor", None), (33, 70, 2048, "tiled", "h32"),
    (64, 700, 12288, "tiled", "smooth"), (7, 77, 96, "rowmajor", (8, 4)), (24, 1000, 8192, "rowmajor", "h32"),
    (48, 513, 1024, "tiled", (2, 16)), (16, 4096, 14336, "tiled", (4, 8)), (30, 333, 8320, "rowmajor", (2, 16)),
    (5, 256, 16384, "tiled", (16, 2)),
    # on 256 CUs: 250 compute workgroups leave too few idle CUs for the 32
    # units (producers in the compute workgroups); 240 leave 16 (producer
    # workgroups with two producing waves each); 200 with 3-wave workgroups
    (16, 16000, 4096, "tiled", (4, 8)), (16, 15360, 4096, "tiled", "h32"), (9, 12800, 2048, "rowmajor", None)]


@pytest.mark.parametrize("m,n,k,layout,rot", SAME_AS_SPLIT, ids=str)
def test_fused_equals_split_layer_bit_for_bit(m, n, k, layout, rot):
    """The fused layer takes the small-M GEMM's K split and summation order,
    so its Y equals quantize_rotate followed by gemm bit for bit (fp32 and
    bf16), across M groups, the wave counts of long K (12288: 8 waves of 12
    steps; 14336 and 16384 with Kronecker transforms), ragged K (4128, 8320),
    both weight layouts, and both producer placements (workgroups of their own
    on idle CUs, or the compute workgroups' sync waves)."""
    rng = np.random.default_rng(3 * m + n + k)
    x = workloads.bf16_bits(workloads.random_blocks(rng, m, k))
    wc, ws = workloads.random_mxfp4(rng, n, k)
    r = make_rot(rot, k=k)
    lay = LAYOUTS[layout]
    announce("linear_small vs split", m, n, k, layout, rot)
    dwc, dws = weights_dev(wc, ws, lay)
    xd = bf16_dev(x)
    got = {}
    for dt, bits in ((torch.float32, torch.int32), (torch.bfloat16, torch.int16)):
        yf = mx.linear_small(xd, dwc, dws, r, dt, layout=lay, n=n)
        ys = mx.linear(xd, dwc, dws, r, dt, layout=lay, n=n)
        torch.cuda.synchronize()
        assert torch.equal(yf.view(bits), ys.view(bits)), f"{dt}: fused and split outputs differ"
        got[dt] = yf
    xc, xs = oracle.quantize(x, rot=oracle_rot(r), bf16=True)
    ref = oracle.gemm(xc, xs, wc, ws)
    assert norm_err(got[torch.float32].cpu().numpy(), ref, row_norms(xc, xs), row_norms(wc, ws)) <= TOL


@pytest.mark.parametrize("m,n,k,rot", [(16, 3000, 4096, (4, 8)), (64, 700, 12288, "h32"), (5, 256, 2048, None)],
                         ids=str)
def test_workspace_contract(m, n, k, rot):
    """With a caller-supplied zeroed workspace, two calls in a row give
    bit-identical Y, the handoff counters (the first 4 KiB, error word
    included) are back at zero after each call, the workspace holds the
    oracle's codes and scales in operand order, and Y meets the oracle
    bound."""
    rng = np.random.default_rng(m + n + k)
    x = workloads.bf16_bits(workloads.random_blocks(rng, m, k))
    wc, ws = workloads.random_mxfp4(rng, n, k)
    r = make_rot(rot, k=k)
    need = mx.linear_small_workspace_bytes(m, n, k)
    work = torch.zeros(need, dtype=torch.uint8, device=DEV)
    dwc, dws = weights_dev(wc, ws, mx.TILED)
    announce("linear_small workspace", m, n, k, rot)
    xd = bf16_dev(x)
    y1 = mx.linear_small(xd, dwc, dws, r, torch.float32, layout=mx.TILED, n=n, workspace=work)
    torch.cuda.synchronize()
    assert not work[:4096].any(), "handoff counters not reset"
    y2 = mx.linear_small(xd, dwc, dws, r, torch.float32, layout=mx.TILED, n=n, workspace=work)
    torch.cuda.synchronize()
    assert not work[:4096].any(), "handoff counters not reset"
    assert torch.equal(y1, y2)
    xc, xs = oracle.quantize(x, rot=oracle_rot(r), bf16=True)
    # the activation image: unit (M group g, step s) = 64 lanes x 16 code
    # bytes, lane l = block 4 s + l // 16 of row 16 g + l % 16; then per unit
    # 16 dwords of the step's 4 scale bytes of each row, in 128-byte slots
    img = work[4096:].cpu().numpy()
    groups, nsteps = -(-m // 16), -(-k // 128)
    units = groups * nsteps
    codes = img[:units * 1024].reshape(groups, nsteps, 4, 16, 16)        # [g][s][block][row][16 B]
    scales = img[units * 1024:units * 1152].reshape(groups, nsteps, 128)[:, :, :64].reshape(groups, nsteps, 16, 4)
    pad_rows = groups * 16
    xcp = np.zeros((pad_rows, nsteps * 64), np.uint8)
    xsp = np.zeros((pad_rows, nsteps * 4), np.uint8)
    xcp[:m, :k // 2] = xc
    xsp[:m, :k // 32] = xs
    want_c = xcp.reshape(groups, 16, nsteps, 4, 16).transpose(0, 2, 3, 1, 4)
    want_s = xsp.reshape(groups, 16, nsteps, 4).transpose(0, 2, 1, 3)
    assert np.array_equal(codes, want_c), "quantized activation codes in the workspace"
    assert np.array_equal(scales, want_s), "quantized activation scales in the workspace"
    ref = oracle.gemm(xc, xs, wc, ws)
    assert norm_err(y1.cpu().numpy(), ref, row_norms(xc, xs), row_norms(wc, ws)) <= TOL


def test_workspace_reused_across_shapes():
    """One workspace serves calls of different shapes in stream order: the
    counter region is the same for every shape and each call leaves it zero."""
    shapes = [(16, 3000, 4096), (7, 9000, 2048), (33, 500, 8192), (64, 300, 512), (16, 3000, 4096)]
    need = max(mx.linear_small_workspace_bytes(m, n, k) for m, n, k in shapes)
    work = torch.zeros(need, dtype=torch.uint8, device=DEV)
    for i, (m, n, k) in enumerate(shapes):
        rng = np.random.default_rng(400 + i)
        x = workloads.bf16_bits(workloads.random_blocks(rng, m, k))
        wc, ws = workloads.random_mxfp4(rng, n, k)
        announce("linear_small shared workspace", m, n, k)
        dwc, dws = weights_dev(wc, ws, mx.TILED)
        y = mx.linear_small(bf16_dev(x), dwc, dws, "h32", torch.float32, layout=mx.TILED, n=n, workspace=work)
        torch.cuda.synchronize()
        assert not work[:4096].any(), "counters not reset"
        xc, xs = oracle.quantize(x, rot="h32", bf16=True)
        ref = oracle.gemm(xc, xs, wc, ws)
        assert norm_err(y.cpu().numpy(), ref, row_norms(xc, xs), row_norms(wc, ws)) <= TOL


@pytest.mark.parametrize("rot", ["h32", (4, 8)], ids=str)
def test_back_to_back_calls_see_their_own_activations(rot):
    """Calls in a row on one workspace, with different activations and no
    synchronization between them, each read the activations they quantized,
    not a copy left in some L2 by the call before: every Y equals the unfused
    path's bit for bit.  Then the same through a captured graph of three
    calls, replayed three times with new activations copied in between."""
    m, n, k = 16, 3000, 4096
    rng = np.random.default_rng(77)
    wc, ws = workloads.random_mxfp4(rng, n, k)
    dwc, dws = weights_dev(wc, ws, mx.TILED)
    r = make_rot(rot, k=k)

    def fresh_x():
        return bf16_dev(workloads.bf16_bits(workloads.random_blocks(rng, m, k)))

    def split(x):
        return mx.linear(x, dwc, dws, r, torch.float32, layout=mx.TILED, n=n)

    work = torch.zeros(mx.linear_small_workspace_bytes(m, n, k), dtype=torch.uint8, device=DEV)
    xs = [fresh_x() for _ in range(8)]
    ys = [torch.empty(m, n, dtype=torch.float32, device=DEV) for _ in xs]
    announce("linear_small back to back", m, n, k, rot)
    for x, y in zip(xs, ys):
        mx.linear_small(x, dwc, dws, r, torch.float32, y=y, layout=mx.TILED, n=n, workspace=work)
    torch.cuda.synchronize()
    for i, (x, y) in enumerate(zip(xs, ys)):
        assert torch.equal(y, split(x)), f"call {i} of a back-to-back run"

    announce("linear_small graph replays", m, n, k, rot)
    xg = [fresh_x() for _ in range(3)]
    yg = [torch.empty(m, n, dtype=torch.float32, device=DEV) for _ in xg]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up outside the capture
        for x, y in zip(xg, yg):
            mx.linear_small(x, dwc, dws, r, torch.float32, y=y, layout=mx.TILED, n=n, workspace=work)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for x, y in zip(xg, yg):
            mx.linear_small(x, dwc, dws, r, torch.float32, y=y, layout=mx.TILED, n=n, workspace=work)
    for rep in range(3):
        for x in xg:
            x.copy_(fresh_x())
        graph.replay()
        torch.cuda.synchronize()
        assert not work[:4096].any(), "handoff counters not reset"
        for i, (x, y) in enumerate(zip(xg, yg)):
            assert torch.equal(y, split(x)), f"replay {rep}, call {i}"
