"""W4A4 MXFP4 linear layer for MI355X (gfx950): a thin binding over libmxfp4.so.

Every step of the layer runs in the HIP library's kernels; this module only
marshals torch tensors (device memory and the current HIP stream) into the
C-ABI calls declared in include/mxfp4.h:

  quantize_rotate(x, rot, layout)    online MXFP4 quantization of activations,
                                     with an optional per-32-block rotation
  gemm(a_codes, a_scales, b_codes, b_scales, out_dtype, layout=...)
                                     Y = A * B^T on packed MXFP4 operands
  linear(x, w_codes, w_scales, rot)  the two above, back to back
  quantize_weight(w, rot)            offline weight quantization with the
                                     weight side of the rotation
  inverse_transpose(m)               host helper for the Kronecker weight fold

Layouts: ROWMAJOR (codes [rows, k/2], scales [rows, k/32]) or TILED, the
GEMM-native layout of include/mxfp4.h (256-row tiles x 128-element stages,
each stage stored as the GEMM's LDS image; tensors of padded_rows(rows) rows
holding the same bytes in tiled order).  tile_host / untile_host convert on
the host (a pure byte permutation, for tests and offline weight prep).

Rotations: None, HADAMARD32, or Kron(a, b) -- a learned Kronecker-factored
32x32 transform A (x) B ("KroQuant: ...", abstract and "Tiefenanalyse"); the
Hadamard-32 is the MR-GPTQ block rotation ("Bridging the Gap Between Promise
and Performance for Microscaling FP4 Quantization", "Methodologie: MR-GPTQ").

There is no fallback: if the library is missing, importing works but every
call raises.
"""
import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmxfp4.so")

MXFP4_OK, MXFP4_ERR_INVALID_ARG, MXFP4_ERR_UNSUPPORTED, MXFP4_ERR_HIP = 0, 1, 2, 3
MXFP4_F32, MXFP4_BF16 = 0, 1
ROT_NONE, ROT_HADAMARD32, ROT_KRON, ROT_SMOOTH = 0, 1, 2, 3
ROWMAJOR, TILED = 0, 1
TILE_ROWS, TILE_K = 256, 128

HADAMARD32 = "h32"

EXPORTED = ("mxfp4_quantize_rotate", "mxfp4_quantize_fit", "mxfp4_gemm", "mxfp4_gemm_requant",
            "mxfp4_linear_small", "mxfp4_linear_small_noalloc", "mxfp4_linear_small_workspace",
            "mxfp4_tiled_bytes",
            "mxfp4_inverse_transpose", "mxfp4_smooth_weight_factors", "mxfp4_status_string",
            "mxfp4_abi_version")
LINEAR_SMALL_MAX_M = 64


class Mxfp4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


class RotationDesc(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("p", ctypes.c_int32), ("q", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("a", ctypes.c_void_p), ("b", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with python -m mxfp4_w4a4_quantized_amd.build "
                           "(the MXFP4 path has no CPU fallback)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.mxfp4_quantize_rotate.restype = i32
    L.mxfp4_quantize_rotate.argtypes = [vp, i32, i64, i64, i64, ctypes.POINTER(RotationDesc), i32, vp, vp, vp]
    L.mxfp4_quantize_fit.restype = i32
    L.mxfp4_quantize_fit.argtypes = [vp, i32, i64, i64, i64, ctypes.POINTER(RotationDesc), i32, vp, vp, vp]
    L.mxfp4_gemm.restype = i32
    L.mxfp4_gemm.argtypes = [vp, vp, i64, vp, vp, i64, i64, i32, vp, i32, i64, vp]
    L.mxfp4_gemm_requant.restype = i32
    L.mxfp4_gemm_requant.argtypes = [vp, vp, i64, vp, vp, i64, i64, i32, vp, vp, i32, vp]
    L.mxfp4_linear_small.restype = i32
    L.mxfp4_linear_small.argtypes = [vp, i32, i64, i64, i64, ctypes.POINTER(RotationDesc), vp, vp, i64, i32,
                                     vp, i32, i64, vp, i64, vp]
    L.mxfp4_linear_small_noalloc.restype = i32
    L.mxfp4_linear_small_noalloc.argtypes = [vp, i32, i64, i64, i64, ctypes.POINTER(RotationDesc), vp, vp, i64,
                                             i32, vp, i32, i64, vp]
    L.mxfp4_linear_small_workspace.restype = i32
    L.mxfp4_linear_small_workspace.argtypes = [i64, i64, i64, ctypes.POINTER(i64)]
    L.mxfp4_tiled_bytes.restype = i32
    L.mxfp4_tiled_bytes.argtypes = [i64, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    L.mxfp4_inverse_transpose.restype = i32
    L.mxfp4_inverse_transpose.argtypes = [vp, i32, vp]
    L.mxfp4_smooth_weight_factors.restype = i32
    L.mxfp4_smooth_weight_factors.argtypes = [vp, i64, vp]
    L.mxfp4_status_string.restype = ctypes.c_char_p
    L.mxfp4_status_string.argtypes = [i32]
    L.mxfp4_abi_version.restype = i32
    L.mxfp4_abi_version.argtypes = []
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().mxfp4_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != MXFP4_OK:
        raise Mxfp4Error(status, what)


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


@dataclass
class Kron:
    """Kronecker-factored block transform T = A (x) B (A p x p, B q x q,
    p*q = 32), factors as fp32 device tensors."""
    a: torch.Tensor
    b: torch.Tensor

    @staticmethod
    def from_host(a: np.ndarray, b: np.ndarray, device="cuda") -> "Kron":
        return Kron(torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device),
                    torch.from_numpy(np.ascontiguousarray(b, np.float32)).to(device))

    def weight_side(self) -> "Kron":
        """Factors (A^-T, B^-T) of T^-T, for folding the inverse into W."""
        a = inverse_transpose(self.a.cpu().numpy())
        b = inverse_transpose(self.b.cpu().numpy())
        return Kron.from_host(a, b, self.a.device)


@dataclass
class Smooth:
    """Per-channel smoothing: column c is multiplied by r[c] before
    quantizing (r = 1 / s for smoothing factors s); fp32 device tensor of k
    factors."""
    r: torch.Tensor

    @staticmethod
    def from_host(r: np.ndarray, device="cuda") -> "Smooth":
        return Smooth(torch.from_numpy(np.ascontiguousarray(r, np.float32).ravel()).to(device))

    def weight_side(self) -> "Smooth":
        """Factors 1 / r[c] from the library (binary64 quotient rounded to
        fp32), for folding the inverse scaling into W."""
        return Smooth.from_host(smooth_weight_factors(self.r.cpu().numpy()), self.r.device)


def _on_device(device, **tensors):
    """Every tensor must live on one GPU, `device` (the first operand's):
    the library takes device pointers and would fault on host memory."""
    if device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU, got {device}")
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device} (all operands on one GPU)")


def _rot_desc(rot, device, k: int):
    """Rotation descriptor for a call over k columns, with its factor tensors
    (kept alive for the call) checked for shape, dtype and device."""
    if rot is None:
        return None, ()
    if isinstance(rot, str):
        if rot != HADAMARD32:
            raise ValueError(f"unknown rotation {rot!r}")
        return RotationDesc(ROT_HADAMARD32, 0, 0, 0, None, None), ()
    if isinstance(rot, Kron):
        a, b = rot.a, rot.b
        for t in (a, b):
            if t.dtype != torch.float32 or not t.is_contiguous() or t.device != device:
                raise ValueError("Kron factors must be contiguous fp32 tensors on the input's device")
        p, q = (a.shape[0] if a.dim() == 2 else 0), (b.shape[0] if b.dim() == 2 else 0)
        if tuple(a.shape) != (p, p) or tuple(b.shape) != (q, q) or p * q != 32:
            raise ValueError(f"Kron factors must be p x p and q x q with p * q = 32, got "
                             f"{tuple(a.shape)} and {tuple(b.shape)}")
        return RotationDesc(ROT_KRON, p, q, 0, a.data_ptr(), b.data_ptr()), (a, b)
    if isinstance(rot, Smooth):
        r = rot.r
        if r.dtype != torch.float32 or not r.is_contiguous() or r.device != device:
            raise ValueError("smoothing factors must be a contiguous fp32 tensor on the input's device")
        if r.numel() != k:
            raise ValueError(f"smoothing needs one factor per column: {r.numel()} factors for k = {k}")
        return RotationDesc(ROT_SMOOTH, 0, 0, 0, r.data_ptr(), None), (r,)
    raise TypeError(f"bad rotation {rot!r}")


def _dtype_code(dt) -> int:
    if dt == torch.float32:
        return MXFP4_F32
    if dt == torch.bfloat16:
        return MXFP4_BF16
    raise ValueError(f"unsupported dtype {dt}")


def padded_rows(rows: int) -> int:
    """Rows of a TILED operand: rows rounded up to the 256-row tile."""
    return (rows + TILE_ROWS - 1) // TILE_ROWS * TILE_ROWS


def tiled_bytes(rows: int, k: int):
    """(codes bytes, scales bytes) of a TILED operand, from the library."""
    cb, sb = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().mxfp4_tiled_bytes(rows, k, ctypes.byref(cb), ctypes.byref(sb)), "mxfp4_tiled_bytes")
    return cb.value, sb.value


def _out_shapes(rows: int, k: int, layout: int):
    r = padded_rows(rows) if layout == TILED else rows
    return (r, k // 2), (r, k // 32)


def quantize_rotate(x: torch.Tensor, rot=None, codes: torch.Tensor = None, scales: torch.Tensor = None,
                    layout: int = ROWMAJOR, fit: bool = False):
    """MXFP4-quantize the rows of x (fp32 or bf16, [rows, k], unit column
    stride) with an optional block transform (None, "h32", Kron, Smooth).
    fit=True fits each block exponent (mxfp4_quantize_fit).  Returns (codes,
    scales) uint8: [rows, k/2] and [rows, k/32] (ROWMAJOR), or the same shapes
    over padded_rows(rows) rows holding the tiled bytes (TILED)."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    rows, k = x.shape
    _on_device(x.device, codes=codes, scales=scales)
    desc, _keep = _rot_desc(rot, x.device, k)
    cshape, sshape = _out_shapes(rows, k, layout)
    if codes is None:
        codes = torch.empty(cshape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(sshape, dtype=torch.uint8, device=x.device)
    if not (codes.is_contiguous() and scales.is_contiguous()):
        raise ValueError("codes and scales must be contiguous")
    if codes.dtype != torch.uint8 or scales.dtype != torch.uint8:
        raise ValueError("codes and scales must be uint8")
    if tuple(codes.shape) != cshape or tuple(scales.shape) != sshape:
        raise ValueError(f"codes/scales must be {cshape} / {sshape}")
    fn = lib().mxfp4_quantize_fit if fit else lib().mxfp4_quantize_rotate
    st = fn(x.data_ptr(), _dtype_code(x.dtype), rows, k, x.stride(0),
            ctypes.byref(desc) if desc is not None else None, layout,
            codes.data_ptr(), scales.data_ptr(), _stream(x.device))
    _check(st, "mxfp4_quantize_fit" if fit else "mxfp4_quantize_rotate")
    return codes, scales


def gemm(a_codes: torch.Tensor, a_scales: torch.Tensor, b_codes: torch.Tensor, b_scales: torch.Tensor,
         out_dtype=torch.bfloat16, y: torch.Tensor = None, layout: int = ROWMAJOR, m: int = None, n: int = None):
    """Y = A * B^T with A [m, k] and B [n, k] in packed MXFP4 (both in
    `layout`); fp32 accumulation, fp32 or bf16 output [m, n].  For TILED
    operands the real row counts come from y, or from m and n."""
    k = a_codes.shape[1] * 2
    _on_device(a_codes.device, a_scales=a_scales, b_codes=b_codes, b_scales=b_scales, y=y)
    if y is not None:
        m, n = y.shape
    if m is None:
        m = a_codes.shape[0]
    if n is None:
        n = b_codes.shape[0]
    for rows, c, sc, name in ((m, a_codes, a_scales, "A"), (n, b_codes, b_scales, "B")):
        cshape, sshape = _out_shapes(rows, k, layout)
        if tuple(c.shape) != cshape or tuple(sc.shape) != sshape:
            raise ValueError(f"operand {name}: codes/scales must be {cshape} / {sshape}")
    for t in (a_codes, a_scales, b_codes, b_scales):
        if t.dtype != torch.uint8 or not t.is_contiguous():
            raise ValueError("codes and scales must be contiguous uint8 tensors")
    if y is None:
        y = torch.empty((m, n), dtype=out_dtype, device=a_codes.device)
    if y.dim() != 2 or y.shape != (m, n) or y.stride(1) != 1:
        raise ValueError("y must be [m, n] with unit column stride")
    st = lib().mxfp4_gemm(a_codes.data_ptr(), a_scales.data_ptr(), m,
                          b_codes.data_ptr(), b_scales.data_ptr(), n, k, layout,
                          y.data_ptr(), _dtype_code(y.dtype), y.stride(0), _stream(a_codes.device))
    _check(st, "mxfp4_gemm")
    return y


def gemm_requant(a_codes: torch.Tensor, a_scales: torch.Tensor, b_codes: torch.Tensor, b_scales: torch.Tensor,
                 layout: int = ROWMAJOR, out_layout: int = ROWMAJOR, m: int = None, n: int = None,
                 y_codes: torch.Tensor = None, y_scales: torch.Tensor = None):
    """Y = A * B^T requantized to MXFP4 in the GEMM epilogue (n % 32 == 0, or
    n % 128 == 0 for a TILED output; k % 128 == 0).  Returns (codes, scales) of Y in `out_layout`, the same
    bytes as quantize_rotate(fp32 Y)."""
    k = a_codes.shape[1] * 2
    _on_device(a_codes.device, a_scales=a_scales, b_codes=b_codes, b_scales=b_scales,
               y_codes=y_codes, y_scales=y_scales)
    if m is None:
        m = a_codes.shape[0]
    if n is None:
        n = b_codes.shape[0]
    for rows, c, sc, name in ((m, a_codes, a_scales, "A"), (n, b_codes, b_scales, "B")):
        cshape, sshape = _out_shapes(rows, k, layout)
        if tuple(c.shape) != cshape or tuple(sc.shape) != sshape:
            raise ValueError(f"operand {name}: codes/scales must be {cshape} / {sshape}")
    for t in (a_codes, a_scales, b_codes, b_scales):
        if t.dtype != torch.uint8 or not t.is_contiguous():
            raise ValueError("codes and scales must be contiguous uint8 tensors")
    cshape, sshape = _out_shapes(m, n, out_layout)
    if y_codes is None:
        y_codes = torch.empty(cshape, dtype=torch.uint8, device=a_codes.device)
    if y_scales is None:
        y_scales = torch.empty(sshape, dtype=torch.uint8, device=a_codes.device)
    if tuple(y_codes.shape) != cshape or tuple(y_scales.shape) != sshape:
        raise ValueError(f"output codes/scales must be {cshape} / {sshape}")
    for t in (y_codes, y_scales):
        if t.dtype != torch.uint8 or not t.is_contiguous():
            raise ValueError("output codes and scales must be contiguous uint8 tensors")
    st = lib().mxfp4_gemm_requant(a_codes.data_ptr(), a_scales.data_ptr(), m, b_codes.data_ptr(),
                                  b_scales.data_ptr(), n, k, layout, y_codes.data_ptr(), y_scales.data_ptr(),
                                  out_layout, _stream(a_codes.device))
    _check(st, "mxfp4_gemm_requant")
    return y_codes, y_scales


def linear(x: torch.Tensor, w_codes: torch.Tensor, w_scales: torch.Tensor, rot=None,
           out_dtype=torch.bfloat16, y: torch.Tensor = None, layout: int = ROWMAJOR, n: int = None) -> torch.Tensor:
    """One W4A4 MXFP4 linear layer: online quantization of x (with the
    activation side of `rot`) followed by the MXFP4 GEMM against
    pre-quantized weights (in the same layout; n = weight rows for TILED)."""
    a_codes, a_scales = quantize_rotate(x, rot, layout=layout)
    return gemm(a_codes, a_scales, w_codes, w_scales, out_dtype, y, layout=layout, m=x.shape[0], n=n)


def linear_small_workspace_bytes(m: int, n: int, k: int) -> int:
    """Device workspace that mxfp4_linear_small needs for (m, n, k): 4 KiB of
    counters plus the quantized activations (0 when m or n is 0)."""
    b = ctypes.c_int64()
    _check(lib().mxfp4_linear_small_workspace(m, n, k, ctypes.byref(b)), "mxfp4_linear_small_workspace")
    return b.value


_workspaces = {}


def _cached_workspace(device, stream: int, nbytes: int) -> torch.Tensor:
    """A zero-filled workspace per (device, stream), grown on demand.  The
    library leaves its counters at zero after every call, so one workspace
    serves every call on its stream; calls on other streams get their own."""
    key = (device.index, stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def linear_small(x: torch.Tensor, w_codes: torch.Tensor, w_scales: torch.Tensor, rot=None,
                 out_dtype=torch.bfloat16, y: torch.Tensor = None, layout: int = ROWMAJOR,
                 n: int = None, workspace: torch.Tensor = None) -> torch.Tensor:
    """Fused small-M linear layer (decode): bf16 x [m, k] with 1 <= m <= 64 is
    rotated and quantized inside the GEMM kernel (one launch; the quantized
    activations pass through `workspace`); the same bytes as linear() with
    the same layout.  `workspace` (uint8, zero-filled before its first use)
    defaults to one kept per device and stream."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    m, k = x.shape
    _on_device(x.device, w_codes=w_codes, w_scales=w_scales, y=y, workspace=workspace)
    desc, _keep = _rot_desc(rot, x.device, k)
    if n is None:
        n = w_codes.shape[0]
    cshape, sshape = _out_shapes(n, k, layout)
    if tuple(w_codes.shape) != cshape or tuple(w_scales.shape) != sshape:
        raise ValueError(f"weights: codes/scales must be {cshape} / {sshape}")
    for t in (w_codes, w_scales):
        if t.dtype != torch.uint8 or not t.is_contiguous():
            raise ValueError("codes and scales must be contiguous uint8 tensors")
    if y is None:
        y = torch.empty((m, n), dtype=out_dtype, device=x.device)
    if y.dim() != 2 or tuple(y.shape) != (m, n) or y.stride(1) != 1:
        raise ValueError("y must be [m, n] with unit column stride")
    stream = _stream(x.device)
    need = linear_small_workspace_bytes(m, n, k) if m <= LINEAR_SMALL_MAX_M else 0
    if workspace is None and need > 0:
        workspace = _cached_workspace(x.device, stream, need)
    if workspace is not None and (workspace.dtype != torch.uint8 or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous uint8 tensor")
    st = lib().mxfp4_linear_small(
        x.data_ptr(), _dtype_code(x.dtype), m, k, x.stride(0),
        ctypes.byref(desc) if desc is not None else None,
        w_codes.data_ptr(), w_scales.data_ptr(), n, layout,
        y.data_ptr(), _dtype_code(y.dtype), y.stride(0),
        workspace.data_ptr() if workspace is not None else None,
        workspace.numel() if workspace is not None else 0, stream)
    _check(st, "mxfp4_linear_small")
    return y


def linear_small_noalloc(x: torch.Tensor, w_codes: torch.Tensor, w_scales: torch.Tensor, y: torch.Tensor,
                         rot=None, layout: int = ROWMAJOR) -> torch.Tensor:
    """linear_small for callers that cannot allocate: the workspace is the
    library's fixed 4 MiB per-GPU scratch (mxfp4_linear_small_noalloc); y
    [m, n] is the caller's.  Calls that overlap in time on one GPU share that
    scratch and race."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    m, k = x.shape
    _on_device(x.device, w_codes=w_codes, w_scales=w_scales, y=y)
    desc, _keep = _rot_desc(rot, x.device, k)
    if y.dim() != 2 or y.shape[0] != m or y.stride(1) != 1:
        raise ValueError("y must be [m, n] with unit column stride")
    n = y.shape[1]
    cshape, sshape = _out_shapes(n, k, layout)
    if tuple(w_codes.shape) != cshape or tuple(w_scales.shape) != sshape:
        raise ValueError(f"weights: codes/scales must be {cshape} / {sshape}")
    for t in (w_codes, w_scales):
        if t.dtype != torch.uint8 or not t.is_contiguous():
            raise ValueError("codes and scales must be contiguous uint8 tensors")
    st = lib().mxfp4_linear_small_noalloc(
        x.data_ptr(), _dtype_code(x.dtype), m, k, x.stride(0),
        ctypes.byref(desc) if desc is not None else None,
        w_codes.data_ptr(), w_scales.data_ptr(), n, layout,
        y.data_ptr(), _dtype_code(y.dtype), y.stride(0), _stream(x.device))
    _check(st, "mxfp4_linear_small_noalloc")
    return y


def quantize_weight(w: torch.Tensor, rot=None, layout: int = ROWMAJOR, fit: bool = False):
    """Offline weight quantization with the weight side of `rot`: the same
    Hadamard-32 (it is its own inverse-transpose), the Kronecker factors
    (A^-T, B^-T), or the reciprocal smoothing factors, so that each block dot
    product is preserved.  fit=True fits the block exponents."""
    if isinstance(rot, (Kron, Smooth)):
        rot = rot.weight_side()
    return quantize_rotate(w, rot, layout=layout, fit=fit)


def _tiled_index(rows_pad: int, k: int):
    """For each byte of the tiled codes and scales, the flat index of the
    same byte in row-major codes [rows_pad, k/2] and scales [rows_pad, k/32]."""
    T, S = rows_pad // TILE_ROWS, k // TILE_K
    t, s, r, p, b = np.meshgrid(np.arange(T), np.arange(S), np.arange(TILE_ROWS), np.arange(4),
                                np.arange(16), indexing="ij")
    row = t * TILE_ROWS + r
    c = p ^ (((r >> 1) ^ (r >> 2)) & 3)          # block of the stage stored at position p
    cidx = row * (k // 2) + (4 * s + c) * 16 + b
    t2, s2, r2, c2 = np.meshgrid(np.arange(T), np.arange(S), np.arange(TILE_ROWS), np.arange(4), indexing="ij")
    sidx = (t2 * TILE_ROWS + r2) * (k // 32) + 4 * s2 + c2
    return cidx.reshape(-1), sidx.reshape(-1)


def tile_host(codes: np.ndarray, scales: np.ndarray):
    """Row-major (codes [rows, k/2], scales [rows, k/32]) -> TILED arrays of
    padded_rows(rows) rows (padding rows zero)."""
    rows, k = codes.shape[0], codes.shape[1] * 2
    rp = padded_rows(rows)
    c = np.zeros((rp, k // 2), np.uint8)
    sc = np.zeros((rp, k // 32), np.uint8)
    c[:rows], sc[:rows] = codes, scales
    ci, si = _tiled_index(rp, k)
    return c.reshape(-1)[ci].reshape(rp, k // 2), sc.reshape(-1)[si].reshape(rp, k // 32)


def untile_host(tcodes: np.ndarray, tscales: np.ndarray, rows: int):
    """TILED arrays -> row-major (codes [rows, k/2], scales [rows, k/32])."""
    rp, k = tcodes.shape[0], tcodes.shape[1] * 2
    ci, si = _tiled_index(rp, k)
    c = np.empty(rp * k // 2, np.uint8)
    sc = np.empty(rp * k // 32, np.uint8)
    c[ci] = np.ascontiguousarray(tcodes).reshape(-1)
    sc[si] = np.ascontiguousarray(tscales).reshape(-1)
    return c.reshape(rp, k // 2)[:rows], sc.reshape(rp, k // 32)[:rows]


def smooth_weight_factors(r: np.ndarray) -> np.ndarray:
    """fp32(1/r[c]) for activation smoothing factors r (library helper)."""
    r = np.ascontiguousarray(r, dtype=np.float32).ravel()
    out = np.empty(r.size, np.float32)
    _check(lib().mxfp4_smooth_weight_factors(r.ctypes.data, r.size, out.ctypes.data),
           "mxfp4_smooth_weight_factors")
    return out


def inverse_transpose(m: np.ndarray) -> np.ndarray:
    """M^-T rounded to fp32 (binary64 elimination in the library)."""
    m = np.ascontiguousarray(m, dtype=np.float32)
    n = m.shape[0]
    if m.shape != (n, n):
        raise ValueError("square matrix expected")
    out = np.empty((n, n), np.float32)
    st = lib().mxfp4_inverse_transpose(m.ctypes.data, n, out.ctypes.data)
    _check(st, "mxfp4_inverse_transpose")
    return out
