"""Seeded synthetic inputs for the W4A4 MXFP4 linear layer.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no rotation, no scale rule, no encoding).  Both the CPU
oracle's tests and the GPU path's tests and benchmark take their inputs from
here, so the two sides see the same bytes.

Workloads (the pages measure FLUX.1-dev at 1024x768 and LLM decode; neither
model nor dataset is used -- these seeded tensors of the same shapes and
value distributions stand in for them):

  tiny            X fp32 [128, 256] ~ N(0,1), 2 outlier channels x50;
                  W fp32 [128, 256] ~ N(0, 0.02); no rotation; fp32 out.
  flux_up         X bf16 [3584, 3072] ~ N(0,1), 31 (1%) outlier channels x50;
                  W [12288, 3072] ~ N(0, 0.02) quantized without rotation;
                  bf16 out.  3584 = 3072 image tokens (1024x768 / 16^2) + 512
                  text tokens.
  flux_down_h32   X bf16 [3584, 12288] Student-t(3); W [3072, 12288] ~
                  N(0, 0.02); Hadamard-32 on both; bf16 out.
  flux_fused_h32  X bf16 [57344, 3072] (batch 16 x 3584 tokens) ~ N(0,1), 31
                  outlier channels x50; W [21504, 3072] (3 x 3072 QKV + 12288
                  MLP); Hadamard-32 on both; bf16 out.
  llm_decode_kron X bf16 [16, 4096] ~ N(0,1); W [14336, 4096] ~ N(0, 0.02);
                  Kronecker transform A (4x4) (x) B (8x8), A = I + 0.1 N(0,1),
                  B = I + 0.1 N(0,1); fp32 out.

Draw order from numpy.random.default_rng(seed): X, outlier channel indices,
W, A, B.  X and W are drawn as float32 standard normals (Student-t(3) is
drawn in float64 and rounded to float32); bf16 inputs are the float32 values
rounded to nearest-even.
"""
from dataclasses import dataclass
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    m: int
    k: int
    n: int
    x_dtype: str          # "f32" or "bf16"
    x_dist: str           # "normal" or "t3"
    outliers: int         # number of outlier channels (columns of X) scaled x50
    rot: Optional[str]    # None, "h32" or "kron"
    out_dtype: str        # "f32" or "bf16"
    p: int = 0            # Kronecker factor sizes (rot == "kron")
    q: int = 0


WORKLOADS = {
    "tiny": Workload("tiny", 128, 256, 128, "f32", "normal", 2, None, "f32"),
    "flux_up": Workload("flux_up", 3584, 3072, 12288, "bf16", "normal", 31, None, "bf16"),
    "flux_down_h32": Workload("flux_down_h32", 3584, 12288, 3072, "bf16", "t3", 0, "h32", "bf16"),
    "flux_fused_h32": Workload("flux_fused_h32", 57344, 3072, 21504, "bf16", "normal", 31, "h32", "bf16"),
    "llm_decode_kron": Workload("llm_decode_kron", 16, 4096, 14336, "bf16", "normal", 0, "kron", "f32", 4, 8),
}

OUTLIER_GAIN = 50.0
W_STD = 0.02
KRON_PERTURB = 0.1


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even.
    Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def make(name: str, seed: int = 0, m: Optional[int] = None) -> dict:
    """Inputs of one workload.  ``m`` overrides the number of X rows (a prefix
    of the same draw is NOT implied; the draw itself uses the given m).

    Returns a dict with: 'wl' (Workload), 'x' (float32 [m,k] or uint16 bf16
    bits [m,k]), 'x_f32' (float32 view of x's values), 'w' (float32 [n,k]),
    'outlier_cols', and for Kronecker workloads 'a' (p x p) and 'b' (q x q)
    float32."""
    wl = WORKLOADS[name]
    rows = wl.m if m is None else m
    rng = np.random.default_rng(seed)
    if wl.x_dist == "normal":
        x = rng.standard_normal((rows, wl.k), dtype=np.float32)
    elif wl.x_dist == "t3":
        x = rng.standard_t(3, size=(rows, wl.k)).astype(np.float32)
    else:
        raise ValueError(wl.x_dist)
    cols = np.sort(rng.choice(wl.k, wl.outliers, replace=False)) if wl.outliers else np.zeros(0, np.int64)
    if wl.outliers:
        x[:, cols] *= np.float32(OUTLIER_GAIN)
    w = rng.standard_normal((wl.n, wl.k), dtype=np.float32) * np.float32(W_STD)
    out = {"wl": wl, "outlier_cols": cols, "w": w}
    if wl.rot == "kron":
        out["a"] = (np.eye(wl.p) + KRON_PERTURB * rng.standard_normal((wl.p, wl.p))).astype(np.float32)
        out["b"] = (np.eye(wl.q) + KRON_PERTURB * rng.standard_normal((wl.q, wl.q))).astype(np.float32)
    if wl.x_dtype == "bf16":
        out["x"] = bf16_bits(x)
        out["x_f32"] = bf16_to_f32(out["x"])
    else:
        out["x"] = x
        out["x_f32"] = x
    return out


def random_mxfp4(rng: np.random.Generator, rows: int, k: int, e_lo: int = -20, e_hi: int = 20):
    """Random packed E2M1 codes (uniform over all 16 codes) and E8M0 scale
    bytes with exponents uniform in [e_lo, e_hi]."""
    codes = rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    scales = (rng.integers(e_lo, e_hi + 1, size=(rows, k // 32)) + 127).astype(np.uint8)
    return codes, scales


def random_blocks(rng: np.random.Generator, rows: int, k: int, dtype=np.float32) -> np.ndarray:
    """Blocks whose magnitudes span many binades: normal values times 2^u with
    u uniform in [-30, 30] per 32-block."""
    x = rng.standard_normal((rows, k)).astype(np.float64)
    e = rng.integers(-30, 31, size=(rows, k // 32))
    x *= np.exp2(np.repeat(e, 32, axis=1))
    return x.astype(dtype)
