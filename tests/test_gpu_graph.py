"""The library's launches replayed from HIP graphs (how the benchmark runs
small steps): a captured quantize + GEMM step and a captured fused layer give,
on every replay, the same bytes as the same calls launched eagerly.  Between
replays the outputs are overwritten by eager work and the device is
synchronised, so a replay that reused stale results or skipped a node fails.
"""
import numpy as np
import pytest
import torch

import mxfp4_w4a4_quantized_amd as mx
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def announce(*what):
    print("[case]", *what, flush=True)


def bf16_dev(x_bits):
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def kron_rot(seed=3):
    rng = np.random.default_rng(seed)
    a = (np.eye(4) + 0.1 * rng.standard_normal((4, 4))).astype(np.float32)
    b = (np.eye(8) + 0.1 * rng.standard_normal((8, 8))).astype(np.float32)
    return mx.Kron.from_host(a, b, DEV)


@pytest.mark.parametrize("rot", [None, "h32", "kron"])
@pytest.mark.parametrize("m,n,k", [(300, 520, 512), (16, 384, 1024), (600, 2100, 512)])
def test_captured_step_matches_eager(m, n, k, rot):
    rng = np.random.default_rng(m + n + k)
    r = kron_rot() if rot == "kron" else rot
    x = bf16_dev(workloads.bf16_bits(rng.standard_normal((m, k), dtype=np.float32)))
    w = torch.from_numpy(rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)).to(DEV)
    wc, ws = mx.quantize_weight(w, r, layout=mx.TILED)
    announce("graph step", m, n, k, rot)
    xc0, xs0 = mx.quantize_rotate(x, r, layout=mx.TILED)
    y0 = mx.gemm(xc0, xs0, wc, ws, torch.bfloat16, layout=mx.TILED, m=m, n=n)
    xc = torch.empty_like(xc0)
    xs = torch.empty_like(xs0)
    y = torch.empty_like(y0)
    step = lambda: (mx.quantize_rotate(x, r, xc, xs, layout=mx.TILED),
                    mx.gemm(xc, xs, wc, ws, torch.bfloat16, y, layout=mx.TILED))
    step()                                   # warm the path before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    pad = mx.padded_rows(m)
    for rep in range(3):
        y.fill_(float("nan"))                # eager work between replays
        xc.fill_(0xAA)
        xs.fill_(0x55)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y0.view(torch.int16)), f"replay {rep}: Y differs"
        # codes and scales of the real rows (padding content is unspecified)
        hc, hs = mx.untile_host(xc.cpu().numpy(), xs.cpu().numpy(), pad)
        rc, rs = mx.untile_host(xc0.cpu().numpy(), xs0.cpu().numpy(), pad)
        assert np.array_equal(hc[:m], rc[:m]) and np.array_equal(hs[:m], rs[:m]), f"replay {rep}: codes differ"


def test_captured_fused_layer_matches_eager():
    rng = np.random.default_rng(17)
    m, n, k = 16, 1024, 2048
    r = kron_rot(5)
    x = bf16_dev(workloads.bf16_bits(rng.standard_normal((m, k), dtype=np.float32)))
    w = torch.from_numpy(rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)).to(DEV)
    wc, ws = mx.quantize_weight(w, r, layout=mx.TILED)
    announce("graph fused layer", m, n, k)
    y0 = mx.linear_small(x, wc, ws, r, torch.float32, layout=mx.TILED, n=n)
    y = torch.empty_like(y0)
    mx.linear_small(x, wc, ws, r, torch.float32, y, layout=mx.TILED, n=n)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mx.linear_small(x, wc, ws, r, torch.float32, y, layout=mx.TILED, n=n)
    torch.cuda.synchronize()
    for rep in range(3):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), y0.view(torch.int32)), f"replay {rep}: Y differs"
