"""The allocation-free fused layer (mxfp4_linear_small_noalloc) against the
fused layer with a caller workspace (mxfp4_linear_small): the same kernel,
so the outputs must be bit-identical; both within the GEMM bound of the
oracle.  Two calls in a row, the second with a smaller input, share the
library's fixed scratch."""
import numpy as np
import pytest
import torch

import mxfp4_w4a4_quantized_amd as mx
import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 1e-5


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    rng0 = np.random.default_rng(77)
    kron = ("kron", (np.eye(4) + 0.1 * rng0.standard_normal((4, 4))).astype(np.float32),
            (np.eye(8) + 0.1 * rng0.standard_normal((8, 8))).astype(np.float32))
    cases = [(16, 14336, 4096, kron), (5, 3000, 2048, "h32")]     # the second call is smaller
    for i, (m, n, k, orot) in enumerate(cases):
        print(f"[case] linear_small_noalloc call {i}: m={m} n={n} k={k}", flush=True)
        rng = np.random.default_rng(500 + i)
        x = workloads.bf16_bits(workloads.random_blocks(rng, m, k))
        wc, ws = workloads.random_mxfp4(rng, n, k)
        rot = mx.Kron.from_host(orot[1], orot[2], DEV) if isinstance(orot, tuple) else orot
        tc, ts = mx.tile_host(wc, ws)
        dwc = torch.from_numpy(tc).to(DEV)
        dws = torch.from_numpy(ts).to(DEV)
        xd = torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
        work = torch.zeros(mx.linear_small_workspace_bytes(m, n, k), dtype=torch.uint8, device=DEV)
        y_ws = mx.linear_small(xd, dwc, dws, rot, torch.float32, layout=mx.TILED, n=n, workspace=work)
        y_na = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
        mx.linear_small_noalloc(xd, dwc, dws, y_na, rot, layout=mx.TILED)
        torch.cuda.synchronize()
        assert torch.equal(y_na, y_ws), f"call {i}: outputs differ"
        xc, xs = oracle.quantize(x, rot=orot, bf16=True)
        ref = oracle.gemm(xc, xs, wc, ws)
        den = np.outer(np.sqrt((oracle.dequantize(xc, xs) ** 2).sum(1)), np.sqrt((oracle.dequantize(wc, ws) ** 2).sum(1)))
        assert (np.abs(y_na.cpu().numpy().astype(np.float64) - ref) <= TOL * den).all(), f"call {i}: oracle bound"


def test_noalloc_back_to_back_calls():
    """Calls in a row on the fixed scratch, with different activations and no
    synchronization between them, each read the activations they quantized:
    every Y equals the workspace entry point's on the same input."""
    m, n, k = 16, 3000, 4096
    rng = np.random.default_rng(91)
    wc, ws = workloads.random_mxfp4(rng, n, k)
    tc, ts = mx.tile_host(wc, ws)
    dwc = torch.from_numpy(tc).to(DEV)
    dws = torch.from_numpy(ts).to(DEV)
    xs = [torch.from_numpy(workloads.bf16_bits(workloads.random_blocks(rng, m, k)).view(np.int16)).to(DEV)
          .view(torch.bfloat16) for _ in range(8)]
    print(f"[case] linear_small_noalloc back to back: m={m} n={n} k={k}", flush=True)
    ys = [torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV) for _ in xs]
    for x, y in zip(xs, ys):
        mx.linear_small_noalloc(x, dwc, dws, y, "h32", layout=mx.TILED)
    torch.cuda.synchronize()
    work = torch.zeros(mx.linear_small_workspace_bytes(m, n, k), dtype=torch.uint8, device=DEV)
    for i, (x, y) in enumerate(zip(xs, ys)):
        y_ws = mx.linear_small(x, dwc, dws, "h32", torch.float32, layout=mx.TILED, n=n, workspace=work)
        assert torch.equal(y, y_ws), f"call {i} of a back-to-back run"
