"""Dense sweep of the device quantizer's E2M1 encoding at every E8M0 scale.

The quantizer converts each block with the hardware converter, whose operand
is the block scale 2^e ("AMD Quark delivers MXFP4 quantization for FLUX.1-dev
on Instinct MI350 with 1.92x speedup", "What is MXFP4 and why does it
eliminate dequantization overhead?": 32 elements share one power-of-two
scale).  This test checks that conversion against the oracle at every scale
byte a finite block can produce (0 .. 252; 253 and 254 would need an amax of
2^128 or more), not only at the scales that ordinary data reaches.

For each scale byte s (e = s - 127) the inputs are the fp32 values t * 2^e
for every fp32 t in [0, 8) whose low 8 mantissa bits are zero (4 259 840
values), both signs, plus each rounding midpoint of the E2M1 grid and the fp32
values on either side of it.  Every block holds one anchor element 4 * 2^e and
31 of these values, so its amax lies in [4 * 2^e, 8 * 2^e) and the block rule
gives exactly e.  Where t * 2^e is subnormal it is rounded on the host; the
oracle and the device see the same fp32 inputs.  Codes and scale bytes must
equal the oracle's bit for bit.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import mxfp4_w4a4_quantized_amd as mx
import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
K = 4096
MIDPOINTS = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
GRID = [0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def sweep_magnitudes() -> np.ndarray:
    t = (np.arange(0, 0x41000000 >> 8, dtype=np.uint32) << 8).view(np.float32)   # [0, 8), low 8 bits 0
    pts = np.array(MIDPOINTS + GRID, np.float32)
    near = np.concatenate([np.nextafter(pts, np.float32(0)), pts, np.nextafter(pts, np.float32(8))])
    mags = np.concatenate([t, near]).astype(np.float32)
    assert mags.max() < 8.0
    return np.concatenate([mags, -mags])


def blocks_at(vals: np.ndarray, e: int) -> np.ndarray:
    """[rows, K] fp32: blocks of one anchor 4 * 2^e followed by 31 values
    t * 2^e (the last row zero-padded: zero blocks are their own case)."""
    nb = -(-vals.size // 31)
    body = np.zeros(nb * 31, np.float32)
    body[:vals.size] = vals
    blk = np.empty((nb, 32), np.float32)
    blk[:, 0] = np.float32(np.ldexp(np.float32(4.0), e))
    blk[:, 1:] = np.ldexp(body.reshape(nb, 31), e).astype(np.float32)
    rows = -(-nb * 32 // K)
    x = np.zeros(rows * K, np.float32)
    x[:blk.size] = blk.ravel()
    return x.reshape(rows, K), nb


def oracle_parallel(x: np.ndarray, parts: int = 8):
    rows = x.shape[0]
    cuts = [rows * i // parts for i in range(parts + 1)]
    with ThreadPoolExecutor(parts) as ex:   # the C oracle releases the GIL
        res = list(ex.map(lambda i: oracle.quantize(x[cuts[i]:cuts[i + 1]]), range(parts)))
    return np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res])


def test_converter_every_scale_byte():
    vals = sweep_magnitudes()
    print(f"[case] converter sweep: {vals.size} values per scale byte, bytes 0..252", flush=True)
    for s in range(0, 253):
        e = s - 127
        x, nb = blocks_at(vals, e)
        assert np.isfinite(x).all()
        c, sc = mx.quantize_rotate(torch.from_numpy(x).to(DEV))
        torch.cuda.synchronize()
        gc, gs = c.cpu().numpy(), sc.cpu().numpy()
        rc, rs = oracle_parallel(x)
        # the anchored blocks all take scale byte s (the padding tail is zero blocks)
        assert (rs.reshape(-1)[:nb] == s).all()
        assert np.array_equal(gs, rs), f"scale byte {s}: {np.count_nonzero(gs != rs)} scale bytes differ"
        assert np.array_equal(gc, rc), f"scale byte {s}: {np.count_nonzero(gc != rc)} code bytes differ"
        if s % 32 == 0 or s == 252:
            print(f"[progress] scale byte {s} ok ({nb} blocks)", flush=True)


def test_bf16_converter_every_scale_byte():
    """bf16 activations (the quantizer converts their packed pairs directly
    when there is no transform): every bf16 value t in [0, 8), both signs,
    scaled by 2^e and rounded to bf16 on the host, at every reachable scale
    byte, in both output layouts and through the Hadamard path (which widens
    to fp32 first); codes and scales equal the oracle's on the same bf16
    inputs."""
    t = workloads.bf16_to_f32(np.arange(0, 0x4100, dtype=np.uint16))          # every bf16 in [0, 8)
    vals = np.concatenate([t, -t]).astype(np.float32)
    print(f"[case] bf16 converter sweep: {vals.size} values per scale byte, bytes 0..252", flush=True)
    for s in range(0, 253):
        e = s - 127
        x32, nb = blocks_at(vals, e)
        xb = workloads.bf16_bits(x32)                     # t * 2^e rounded to bf16 (exact above the subnormals)
        assert np.array_equal(workloads.bf16_to_f32(xb.reshape(-1)[::32][:nb]), x32.reshape(-1)[::32][:nb])
        xd = torch.from_numpy(xb.view(np.int16)).to(DEV).view(torch.bfloat16)
        rc, rs = oracle.quantize(xb, bf16=True)
        assert (rs.reshape(-1)[:nb] == s).all()
        for layout in (mx.ROWMAJOR, mx.TILED):
            c, sc = mx.quantize_rotate(xd, layout=layout)
            torch.cuda.synchronize()
            gc, gs = c.cpu().numpy(), sc.cpu().numpy()
            if layout == mx.TILED:
                gc, gs = mx.untile_host(gc, gs, xb.shape[0])
            assert np.array_equal(gs, rs), f"scale byte {s}: {np.count_nonzero(gs != rs)} scale bytes differ"
            assert np.array_equal(gc, rc), f"scale byte {s}: {np.count_nonzero(gc != rc)} code bytes differ"
        if s % 32 == 0:
            hc, hs = mx.quantize_rotate(xd, mx.HADAMARD32)
            torch.cuda.synchronize()
            rhc, rhs = oracle.quantize(xb, rot="h32", bf16=True)
            assert np.array_equal(hc.cpu().numpy(), rhc) and np.array_equal(hs.cpu().numpy(), rhs)
            print(f"[progress] bf16 scale byte {s} ok ({nb} blocks)", flush=True)
