"""Maximum sizes.  The large-tile GEMM addresses an operand's code bytes with
32-bit offsets and takes operands whose padded rows x k/2 stay below 4 GiB;
these tests put operands right under that limit (4 MiB short of it) through
the quantizer and the GEMM, in both layouts, and the small-M kernel through a
weight matrix of the same size.  Inputs are generated on the device from a
seeded torch generator; the checks copy sampled rows back (the first, the last
and random ones in between) and compare them with the oracle: codes and scales
bit for bit, GEMM rows within the normalized 1e-5 bound of the other GEMM
tests.  Each test holds 5-22 GB of device memory and runs in seconds.
"""
import numpy as np
import pytest
import torch

import mxfp4_w4a4_quantized_amd as mx
import oracle

DEV = "cuda:0"
TOL = 1e-5
K = 32768                       # 16 KiB of codes per row
ROWS = 1023 * 256 - 7           # padded to 1023 tiles: 1023 * 256 * 16 KiB = 4 GiB - 4 MiB


def announce(*what):
    print("[case]", *what, flush=True)


def gen(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


def random_operand(rows, k, seed):
    g = gen(seed)
    codes = torch.randint(0, 256, (rows, k // 2), dtype=torch.uint8, device=DEV, generator=g)
    scales = torch.randint(124, 131, (rows, k // 32), dtype=torch.uint8, device=DEV, generator=g)
    return codes, scales


def sample_rows(rows, count, seed):
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, rows - 1), size=count, replace=False)
    return np.unique(np.concatenate([[0, rows - 1], mid]))


def tiled_positions(rows_sel, k):
    """Byte positions, in a TILED operand ([T][S][256][64] codes, [T][S][256][4]
    scales, 16-byte chunk c of a row at c ^ ((r >> 1 ^ r >> 2) & 3)), of the
    given rows' codes and scales in row-major order."""
    S = k // 128
    r = np.asarray(rows_sel, np.int64)[:, None]
    t, rr = r // 256, r % 256
    blk = np.arange(k // 32, dtype=np.int64)[None, :]
    s, c = blk // 4, blk % 4
    swz = ((rr >> 1) ^ (rr >> 2)) & 3
    base = (t * S + s) * 256 + rr                                     # [rows, blocks]
    cpos = (base * 64 + 16 * (c ^ swz))[:, :, None] + np.arange(16, dtype=np.int64)[None, None, :]
    spos = base * 4 + c
    return cpos.reshape(len(rows_sel), k // 2), spos


def gather(flat_dev, pos):
    idx = torch.from_numpy(pos.reshape(-1)).to(DEV)
    return flat_dev.reshape(-1)[idx].cpu().numpy().reshape(pos.shape)


def rows_host(t, rows_sel):
    return t[torch.from_numpy(np.asarray(rows_sel)).to(DEV)].cpu().numpy()


def norm_err(got, ref, ac, as_, bc, bs):
    na = np.sqrt((oracle.dequantize(ac, as_) ** 2).sum(1))
    nb = np.sqrt((oracle.dequantize(bc, bs) ** 2).sum(1))
    den = np.outer(na, nb)
    return float(np.max(np.abs(got.astype(np.float64) - ref) / den))


def test_tiled_positions_match_untile():
    # (CPU) the test's own reading of the tiled layout against the binding's untile
    rng = np.random.default_rng(1)
    rows, k = 600, 512
    codes = rng.integers(0, 256, (rows, k // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, (rows, k // 32), dtype=np.uint8)
    tc, ts = mx.tile_host(codes, scales)
    sel = np.array([0, 1, 7, 255, 256, 300, 599])
    cpos, spos = tiled_positions(sel, k)
    assert np.array_equal(tc.reshape(-1)[cpos], codes[sel])
    assert np.array_equal(ts.reshape(-1)[spos], scales[sel])


@pytest.mark.gpu
def test_rowmajor_gemm_at_the_offset_limit():
    m, n = ROWS, 256
    # one more 256-row tile would reach 4 GiB
    assert mx.padded_rows(m) * (K // 2) < 1 << 32 <= (mx.padded_rows(m) + 256) * (K // 2)
    announce("row-major gemm at the limit", m, n, K)
    ac, as_ = random_operand(m, K, 11)
    bc, bs = random_operand(n, K, 12)
    y = mx.gemm(ac, as_, bc, bs, torch.float32)
    torch.cuda.synchronize()
    sel = sample_rows(m, 30, 13)
    hac, has = rows_host(ac, sel), rows_host(as_, sel)
    hbc, hbs = bc.cpu().numpy(), bs.cpu().numpy()
    ref = oracle.gemm(hac, has, hbc, hbs)
    err = norm_err(rows_host(y, sel), ref, hac, has, hbc, hbs)
    print(f"[result] rows {sel[:3]}..{sel[-1]}: normalized error {err:.3e}", flush=True)
    assert err <= TOL


@pytest.mark.gpu
def test_tiled_quantize_and_gemm_at_the_offset_limit():
    m, n = ROWS, 256
    announce("tiled quantize + gemm at the limit", m, n, K)
    g = gen(21)
    x = torch.randn((m, K), dtype=torch.bfloat16, device=DEV, generator=g)
    xc, xs = mx.quantize_rotate(x, mx.HADAMARD32, layout=mx.TILED)
    rng = np.random.default_rng(22)
    wc = rng.integers(0, 256, (n, K // 2), dtype=np.uint8)
    ws = rng.integers(124, 131, (n, K // 32), dtype=np.uint8)
    twc, tws = mx.tile_host(wc, ws)
    y = mx.gemm(xc, xs, torch.from_numpy(twc).to(DEV), torch.from_numpy(tws).to(DEV), torch.float32,
                layout=mx.TILED, m=m, n=n)
    torch.cuda.synchronize()
    sel = sample_rows(m, 24, 23)
    xh = rows_host(x.view(torch.int16), sel).view(np.uint16)
    rc, rs = oracle.quantize(xh, rot="h32", bf16=True)
    cpos, spos = tiled_positions(sel, K)
    gc, gs = gather(xc, cpos), gather(xs, spos)
    assert np.array_equal(gs, rs), f"{np.count_nonzero(gs != rs)} scale bytes differ"
    assert np.array_equal(gc, rc), f"{np.count_nonzero(gc != rc)} code bytes differ"
    ref = oracle.gemm(rc, rs, wc, ws)
    err = norm_err(rows_host(y, sel), ref, rc, rs, wc, ws)
    print(f"[result] tiled rows {sel[:3]}..{sel[-1]}: normalized error {err:.3e}", flush=True)
    assert err <= TOL
    del x, xc, xs, y
    torch.cuda.empty_cache()


@pytest.mark.gpu
def test_small_m_gemm_with_weights_at_the_limit():
    m, n = 16, ROWS
    announce("small-M gemm, weights at the limit", m, n, K)
    ac, as_ = random_operand(m, K, 31)
    bc, bs = random_operand(n, K, 32)
    y = mx.gemm(ac, as_, bc, bs, torch.float32)
    torch.cuda.synchronize()
    sel = sample_rows(n, 30, 33)
    hbc, hbs = rows_host(bc, sel), rows_host(bs, sel)
    hac, has = ac.cpu().numpy(), as_.cpu().numpy()
    ref = oracle.gemm(hac, has, hbc, hbs)
    got = y[:, torch.from_numpy(sel).to(DEV)].cpu().numpy()
    err = norm_err(got, ref, hac, has, hbc, hbs)
    print(f"[result] weight rows {sel[:3]}..{sel[-1]}: normalized error {err:.3e}", flush=True)
    assert err <= TOL
