// C-ABI layer: argument validation, kernel selection, HIP error mapping.
// The declarations, layouts and error behaviour are documented in mxfp4.h.
#include "mxfp4.h"

#include <cmath>
#include <cstdint>

#include "internal.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

mxfp4_status from_hip(hipError_t e) { return e == hipSuccess ? MXFP4_OK : MXFP4_ERR_HIP; }

constexpr int64_t kMaxDim = int64_t(1) << 30;

struct Rot {
  int32_t kind = MXFP4_ROT_NONE, p = 0, q = 0;
  const float* fa = nullptr;
  const float* fb = nullptr;
};

// Validates a rotation descriptor (NULL = none).
mxfp4_status parse_rotation(const mxfp4_rotation* rot, Rot& r) {
  if (rot == nullptr) return MXFP4_OK;
  r.kind = rot->kind;
  if (r.kind != MXFP4_ROT_NONE && r.kind != MXFP4_ROT_HADAMARD32 && r.kind != MXFP4_ROT_KRON &&
      r.kind != MXFP4_ROT_SMOOTH)
    return MXFP4_ERR_INVALID_ARG;
  if (rot->reserved != 0) return MXFP4_ERR_INVALID_ARG;
  if (r.kind == MXFP4_ROT_KRON) {
    r.p = rot->p;
    r.q = rot->q;
    if (r.p < 1 || r.q < 1 || r.p * r.q != 32 || (r.p & (r.p - 1)) != 0) return MXFP4_ERR_INVALID_ARG;
    if (rot->a == nullptr || rot->b == nullptr) return MXFP4_ERR_INVALID_ARG;
    r.fa = rot->a;
    r.fb = rot->b;
    if (!aligned(r.fa, 4) || !aligned(r.fb, 4)) return MXFP4_ERR_UNSUPPORTED;
  }
  if (r.kind == MXFP4_ROT_SMOOTH) {
    if (rot->a == nullptr) return MXFP4_ERR_INVALID_ARG;
    r.fa = rot->a;
    if (!aligned(r.fa, 16)) return MXFP4_ERR_UNSUPPORTED;
  }
  return MXFP4_OK;
}

}  // namespace

namespace {

mxfp4_status quantize_impl(const void* x, int32_t x_dtype, int64_t rows, int64_t k, int64_t ld_x,
                           const mxfp4_rotation* rot, int32_t layout, uint8_t* codes, uint8_t* scales,
                           bool fit, void* stream) {
  if (x_dtype != MXFP4_F32 && x_dtype != MXFP4_BF16) return MXFP4_ERR_INVALID_ARG;
  if (layout != MXFP4_LAYOUT_ROWMAJOR && layout != MXFP4_LAYOUT_TILED) return MXFP4_ERR_INVALID_ARG;
  const bool tiled = layout == MXFP4_LAYOUT_TILED;
  if (rows < 0 || k <= 0 || (k % (tiled ? mxfp4::kTileK : 32)) != 0 || ld_x < k) return MXFP4_ERR_INVALID_ARG;
  Rot r;
  const mxfp4_status rs = parse_rotation(rot, r);
  if (rs != MXFP4_OK) return rs;
  if (rows == 0) return MXFP4_OK;
  if (x == nullptr || codes == nullptr || scales == nullptr) return MXFP4_ERR_INVALID_ARG;
  const int64_t elem = (x_dtype == MXFP4_BF16) ? 2 : 4;
  if (!aligned(x, 16) || ((ld_x * elem) % 16) != 0 || !aligned(codes, 16)) return MXFP4_ERR_UNSUPPORTED;
  if (tiled && !aligned(scales, 4)) return MXFP4_ERR_UNSUPPORTED;
  const int64_t rows_pad = tiled ? (rows + mxfp4::kTileRows - 1) / mxfp4::kTileRows * mxfp4::kTileRows : rows;
  if (rows_pad * (k / 32) >= (int64_t(1) << 31)) return MXFP4_ERR_UNSUPPORTED;

  mxfp4::QuantArgs a;
  a.x = x;
  a.ld_x = ld_x;
  a.rows = static_cast<uint32_t>(rows);
  a.nblk_row = static_cast<uint32_t>(k / 32);
  a.rot = r.kind;
  a.p = r.p;
  a.q = r.q;
  a.fa = r.fa;
  a.fb = r.fb;
  a.codes = codes;
  a.scales = scales;
  a.tiled = tiled;
  a.rows_pad = static_cast<uint32_t>(rows_pad);
  a.fit = fit;
  return from_hip(mxfp4::launch_quantize(a, x_dtype == MXFP4_BF16, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

MXFP4_API int32_t mxfp4_abi_version(void) { return MXFP4_ABI_VERSION; }

MXFP4_API const char* mxfp4_status_string(int32_t status) {
  switch (status) {
    case MXFP4_OK: return "MXFP4_OK";
    case MXFP4_ERR_INVALID_ARG: return "MXFP4_ERR_INVALID_ARG: invalid argument";
    case MXFP4_ERR_UNSUPPORTED: return "MXFP4_ERR_UNSUPPORTED: unsupported alignment or size";
    case MXFP4_ERR_HIP: return "MXFP4_ERR_HIP: HIP runtime or launch failure";
    default: return "MXFP4: unknown status";
  }
}

MXFP4_API mxfp4_status mxfp4_tiled_bytes(int64_t rows, int64_t k, int64_t* codes_bytes,
                                         int64_t* scales_bytes) {
  if (codes_bytes == nullptr || scales_bytes == nullptr || rows < 0 || k <= 0 || (k % mxfp4::kTileK) != 0)
    return MXFP4_ERR_INVALID_ARG;
  if (rows >= kMaxDim || k >= kMaxDim) return MXFP4_ERR_UNSUPPORTED;
  const int64_t rows_pad = (rows + mxfp4::kTileRows - 1) / mxfp4::kTileRows * mxfp4::kTileRows;
  *codes_bytes = rows_pad * (k / 2);
  *scales_bytes = rows_pad * (k / 32);
  return MXFP4_OK;
}

MXFP4_API mxfp4_status mxfp4_quantize_rotate(const void* x, int32_t x_dtype, int64_t rows, int64_t k,
                                             int64_t ld_x, const mxfp4_rotation* rot, int32_t layout,
                                             uint8_t* codes, uint8_t* scales, void* stream) {
  return quantize_impl(x, x_dtype, rows, k, ld_x, rot, layout, codes, scales, false, stream);
}

MXFP4_API mxfp4_status mxfp4_quantize_fit(const void* x, int32_t x_dtype, int64_t rows, int64_t k,
                                          int64_t ld_x, const mxfp4_rotation* rot, int32_t layout,
                                          uint8_t* codes, uint8_t* scales, void* stream) {
  return quantize_impl(x, x_dtype, rows, k, ld_x, rot, layout, codes, scales, true, stream);
}

MXFP4_API mxfp4_status mxfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, int64_t m,
                                  const uint8_t* b_codes, const uint8_t* b_scales, int64_t n, int64_t k,
                                  int32_t layout, void* y, int32_t y_dtype, int64_t ld_y, void* stream) {
  if (y_dtype != MXFP4_F32 && y_dtype != MXFP4_BF16) return MXFP4_ERR_INVALID_ARG;
  if (layout != MXFP4_LAYOUT_ROWMAJOR && layout != MXFP4_LAYOUT_TILED) return MXFP4_ERR_INVALID_ARG;
  const bool tiled = layout == MXFP4_LAYOUT_TILED;
  if (m < 0 || n < 0 || k <= 0 || (k % (tiled ? mxfp4::kTileK : 32)) != 0 || ld_y < n)
    return MXFP4_ERR_INVALID_ARG;
  if (m == 0 || n == 0) return MXFP4_OK;
  if (a_codes == nullptr || a_scales == nullptr || b_codes == nullptr || b_scales == nullptr ||
      y == nullptr)
    return MXFP4_ERR_INVALID_ARG;
  if (m >= kMaxDim || n >= kMaxDim || k >= kMaxDim) return MXFP4_ERR_UNSUPPORTED;
  if (!aligned(a_codes, 16) || !aligned(b_codes, 16)) return MXFP4_ERR_UNSUPPORTED;
  if (tiled && (!aligned(a_scales, 4) || !aligned(b_scales, 4))) return MXFP4_ERR_UNSUPPORTED;
  const int64_t ybytes = (y_dtype == MXFP4_BF16) ? 2 : 4;
  if (!aligned(y, ybytes)) return MXFP4_ERR_UNSUPPORTED;

  mxfp4::GemmArgs g;
  g.a_codes = a_codes;
  g.a_scales = a_scales;
  g.b_codes = b_codes;
  g.b_scales = b_scales;
  g.m = static_cast<int32_t>(m);
  g.n = static_cast<int32_t>(n);
  g.k = static_cast<int32_t>(k);
  g.y = y;
  g.ld_y = ld_y;
  g.y_bf16 = (y_dtype == MXFP4_BF16);
  g.tiled = tiled;
  // tiled operands with m > 64 run on the large-tile kernel only, whose
  // operand offsets are 32-bit: code bytes of each operand below 4 GiB
  if (tiled && !mxfp4::gemm_small_supported(g) && !mxfp4::gemm_large_supported(g)) return MXFP4_ERR_UNSUPPORTED;
  return from_hip(mxfp4::launch_gemm(g, static_cast<hipStream_t>(stream)));
}

MXFP4_API mxfp4_status mxfp4_gemm_requant(const uint8_t* a_codes, const uint8_t* a_scales, int64_t m,
                                          const uint8_t* b_codes, const uint8_t* b_scales, int64_t n, int64_t k,
                                          int32_t layout, uint8_t* y_codes, uint8_t* y_scales, int32_t y_layout,
                                          void* stream) {
  if (layout != MXFP4_LAYOUT_ROWMAJOR && layout != MXFP4_LAYOUT_TILED) return MXFP4_ERR_INVALID_ARG;
  if (y_layout != MXFP4_LAYOUT_ROWMAJOR && y_layout != MXFP4_LAYOUT_TILED) return MXFP4_ERR_INVALID_ARG;
  const bool tiled = layout == MXFP4_LAYOUT_TILED;
  if (m < 0 || n < 0 || k <= 0 || (k % (tiled ? mxfp4::kTileK : 32)) != 0) return MXFP4_ERR_INVALID_ARG;
  if (m == 0 || n == 0) return MXFP4_OK;
  if (a_codes == nullptr || a_scales == nullptr || b_codes == nullptr || b_scales == nullptr ||
      y_codes == nullptr || y_scales == nullptr)
    return MXFP4_ERR_INVALID_ARG;
  if (m >= kMaxDim || n >= kMaxDim || k >= kMaxDim) return MXFP4_ERR_UNSUPPORTED;
  if ((n % (y_layout == MXFP4_LAYOUT_TILED ? mxfp4::kTileK : 32)) != 0 || (k % mxfp4::kTileK) != 0)
    return MXFP4_ERR_UNSUPPORTED;
  if (!aligned(a_codes, 16) || !aligned(b_codes, 16) || !aligned(y_codes, 16)) return MXFP4_ERR_UNSUPPORTED;
  if (!aligned(a_scales, 4) || !aligned(b_scales, 4) || !aligned(y_scales, 4)) return MXFP4_ERR_UNSUPPORTED;

  mxfp4::GemmArgs g;
  g.a_codes = a_codes;
  g.a_scales = a_scales;
  g.b_codes = b_codes;
  g.b_scales = b_scales;
  g.m = static_cast<int32_t>(m);
  g.n = static_cast<int32_t>(n);
  g.k = static_cast<int32_t>(k);
  g.y = nullptr;
  g.ld_y = n;
  g.y_bf16 = false;
  g.tiled = tiled;
  g.q_out = true;
  g.q_tiled = (y_layout == MXFP4_LAYOUT_TILED);
  g.q_codes = y_codes;
  g.q_scales = y_scales;
  // the kernel that mxfp4_gemm takes for the same operands, so that the
  // requantized Y is the one mxfp4_gemm returns in fp32
  if (mxfp4::gemm_small_supported(g)) return from_hip(mxfp4::launch_gemm_small(g, static_cast<hipStream_t>(stream)));
  if (!mxfp4::gemm_large_supported(g)) return MXFP4_ERR_UNSUPPORTED;
  return from_hip(mxfp4::launch_gemm_large(g, static_cast<hipStream_t>(stream)));
}

MXFP4_API mxfp4_status mxfp4_linear_small_workspace(int64_t m, int64_t n, int64_t k, int64_t* bytes) {
  if (bytes == nullptr || m < 0 || n < 0 || k <= 0 || (k % 32) != 0) return MXFP4_ERR_INVALID_ARG;
  if (m > 64) return MXFP4_ERR_UNSUPPORTED;
  if (n >= kMaxDim || k >= kMaxDim) return MXFP4_ERR_UNSUPPORTED;
  const int64_t need = (m == 0 || n == 0) ? 0 : mxfp4::linear_small_workspace_bytes(m, k);
  // the quantized activations are addressed with 32-bit byte offsets
  if (need - mxfp4::kLinearCounterBytes >= (int64_t(1) << 31)) return MXFP4_ERR_UNSUPPORTED;
  *bytes = need;
  return MXFP4_OK;
}

}  // extern "C"

namespace {

// Validation and launch of the fused layer; ws == nullptr with
// use_static selects the library's fixed scratch.
mxfp4_status linear_small_impl(const void* x, int32_t x_dtype, int64_t m, int64_t k, int64_t ld_x,
                               const mxfp4_rotation* rot, const uint8_t* w_codes, const uint8_t* w_scales,
                               int64_t n, int32_t layout, void* y, int32_t y_dtype, int64_t ld_y, void* workspace,
                               int64_t workspace_bytes, bool use_static, void* stream) {
  if (x_dtype != MXFP4_F32 && x_dtype != MXFP4_BF16) return MXFP4_ERR_INVALID_ARG;
  if (y_dtype != MXFP4_F32 && y_dtype != MXFP4_BF16) return MXFP4_ERR_INVALID_ARG;
  if (layout != MXFP4_LAYOUT_ROWMAJOR && layout != MXFP4_LAYOUT_TILED) return MXFP4_ERR_INVALID_ARG;
  const bool tiled = layout == MXFP4_LAYOUT_TILED;
  if (m < 0 || n < 0 || k <= 0 || (k % (tiled ? mxfp4::kTileK : 32)) != 0 || ld_x < k || ld_y < n)
    return MXFP4_ERR_INVALID_ARG;
  Rot r;
  const mxfp4_status rs = parse_rotation(rot, r);
  if (rs != MXFP4_OK) return rs;
  if (m == 0 || n == 0) return MXFP4_OK;
  if (x == nullptr || w_codes == nullptr || w_scales == nullptr || y == nullptr) return MXFP4_ERR_INVALID_ARG;
  if (m > 64 || x_dtype != MXFP4_BF16) return MXFP4_ERR_UNSUPPORTED;
  if (r.kind == MXFP4_ROT_KRON && (r.p < 2 || r.p > 16)) return MXFP4_ERR_UNSUPPORTED;
  if (n >= kMaxDim || k >= kMaxDim || ld_x >= kMaxDim) return MXFP4_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || ((ld_x * 2) % 16) != 0 || !aligned(w_codes, 16)) return MXFP4_ERR_UNSUPPORTED;
  if (tiled && !aligned(w_scales, 4)) return MXFP4_ERR_UNSUPPORTED;
  const int64_t ybytes = (y_dtype == MXFP4_BF16) ? 2 : 4;
  if (!aligned(y, ybytes)) return MXFP4_ERR_UNSUPPORTED;
  const int64_t need = mxfp4::linear_small_workspace_bytes(m, k);
  // the quantized activations are addressed with 32-bit byte offsets
  if (need - mxfp4::kLinearCounterBytes >= (int64_t(1) << 31)) return MXFP4_ERR_UNSUPPORTED;
  if (use_static && need > mxfp4::kLinearStaticScratchBytes) return MXFP4_ERR_UNSUPPORTED;

  mxfp4::LinearArgs L;
  L.x = x;
  L.ld_x = ld_x;
  L.x_bf16 = true;
  L.rot = r.kind;
  L.p = r.p;
  L.q = r.q;
  L.fa = r.fa;
  L.fb = r.fb;
  L.g.a_codes = nullptr;
  L.g.a_scales = nullptr;
  L.g.b_codes = w_codes;
  L.g.b_scales = w_scales;
  L.g.m = static_cast<int32_t>(m);
  L.g.n = static_cast<int32_t>(n);
  L.g.k = static_cast<int32_t>(k);
  L.g.y = y;
  L.g.ld_y = ld_y;
  L.g.y_bf16 = (y_dtype == MXFP4_BF16);
  L.g.tiled = tiled;
  if (use_static) {
    const hipError_t e = mxfp4::linear_small_static_scratch(&workspace, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return MXFP4_ERR_HIP;
    workspace_bytes = mxfp4::kLinearStaticScratchBytes;
  }
  if (workspace == nullptr || workspace_bytes < need) return MXFP4_ERR_INVALID_ARG;
  if (!aligned(workspace, 256)) return MXFP4_ERR_UNSUPPORTED;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  L.counters = reinterpret_cast<uint32_t*>(ws);
  L.xq = ws + mxfp4::kLinearCounterBytes;
  return from_hip(mxfp4::launch_linear_small(L, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

MXFP4_API mxfp4_status mxfp4_linear_small(const void* x, int32_t x_dtype, int64_t m, int64_t k, int64_t ld_x,
                                          const mxfp4_rotation* rot, const uint8_t* w_codes,
                                          const uint8_t* w_scales, int64_t n, int32_t layout, void* y,
                                          int32_t y_dtype, int64_t ld_y, void* workspace,
                                          int64_t workspace_bytes, void* stream) {
  return linear_small_impl(x, x_dtype, m, k, ld_x, rot, w_codes, w_scales, n, layout, y, y_dtype, ld_y, workspace,
                           workspace_bytes, false, stream);
}

MXFP4_API mxfp4_status mxfp4_linear_small_noalloc(const void* x, int32_t x_dtype, int64_t m, int64_t k,
                                                  int64_t ld_x, const mxfp4_rotation* rot, const uint8_t* w_codes,
                                                  const uint8_t* w_scales, int64_t n, int32_t layout, void* y,
                                                  int32_t y_dtype, int64_t ld_y, void* stream) {
  return linear_small_impl(x, x_dtype, m, k, ld_x, rot, w_codes, w_scales, n, layout, y, y_dtype, ld_y, nullptr, 0,
                           true, stream);
}

// Reciprocals of the activation-side smoothing factors, for the weight fold:
// the quotient 1/r is formed in binary64 and rounded once to fp32.
MXFP4_API mxfp4_status mxfp4_smooth_weight_factors(const float* r, int64_t k, float* out) {
  if (r == nullptr || out == nullptr || k <= 0) return MXFP4_ERR_INVALID_ARG;
  for (int64_t c = 0; c < k; ++c) {
    const float v = r[c];
    if (!std::isfinite(v) || v == 0.0f) return MXFP4_ERR_INVALID_ARG;
    const float w = static_cast<float>(1.0 / static_cast<double>(v));
    if (!std::isfinite(w)) return MXFP4_ERR_INVALID_ARG;
    out[c] = w;
  }
  return MXFP4_OK;
}

// Binary64 Gauss-Jordan elimination with partial pivoting on [M | I]; the
// right half becomes M^-1, which is written transposed and rounded to fp32.
MXFP4_API mxfp4_status mxfp4_inverse_transpose(const float* m, int32_t n, float* out) {
  if (m == nullptr || out == nullptr || n < 1 || n > 32) return MXFP4_ERR_INVALID_ARG;
  double t[32][64];
  for (int r = 0; r < n; ++r)
    for (int c = 0; c < 2 * n; ++c) t[r][c] = (c < n) ? double(m[r * n + c]) : (c - n == r ? 1.0 : 0.0);
  for (int col = 0; col < n; ++col) {
    int piv = col;
    for (int r = col + 1; r < n; ++r)
      if (std::fabs(t[r][col]) > std::fabs(t[piv][col])) piv = r;
    if (t[piv][col] == 0.0) return MXFP4_ERR_INVALID_ARG;
    if (piv != col)
      for (int c = 0; c < 2 * n; ++c) {
        const double s = t[col][c];
        t[col][c] = t[piv][c];
        t[piv][c] = s;
      }
    const double d = t[col][col];
    for (int c = 0; c < 2 * n; ++c) t[col][c] /= d;
    for (int r = 0; r < n; ++r) {
      if (r == col || t[r][col] == 0.0) continue;
      const double f = t[r][col];
      for (int c = 0; c < 2 * n; ++c) t[r][c] -= f * t[col][c];
    }
  }
  for (int r = 0; r < n; ++r)
    for (int c = 0; c < n; ++c) out[r * n + c] = static_cast<float>(t[c][n + r]);
  return MXFP4_OK;
}

}  // extern "C"
