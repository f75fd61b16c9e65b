// Internal launch interface between the C-ABI layer (api.cpp) and the HIP
// kernels.  Arguments reaching these functions are already validated.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace mxfp4 {

struct QuantArgs {
  const void* x;
  int64_t ld_x;        // elements
  uint32_t rows;
  uint32_t nblk_row;   // k / 32
  int32_t rot;         // mxfp4_rot_kind
  int32_t p, q;        // Kronecker factor sizes
  const float* fa;     // p x p (Kronecker), or k per-channel factors (smoothing)
  const float* fb;     // q x q
  bool fit;            // fitted block exponents instead of the E8M0 rule
  uint8_t* codes;
  uint8_t* scales;
  bool tiled;          // MXFP4_LAYOUT_TILED outputs (nblk_row % 4 == 0)
  uint32_t rows_pad;   // rows rounded up to the 256-row tile (tiled only)
};

constexpr int kTileRows = 256;       // rows per tile of the tiled layout
constexpr int kTileK = 128;          // K elements per stage of the tiled layout

hipError_t launch_quantize(const QuantArgs& a, bool bf16, hipStream_t s);

struct GemmArgs {
  const uint8_t* a_codes;   // X side, m rows
  const uint8_t* a_scales;
  const uint8_t* b_codes;   // W side, n rows
  const uint8_t* b_scales;
  int32_t m, n, k;
  void* y;
  int64_t ld_y;
  bool y_bf16;
  bool tiled;               // both operands in MXFP4_LAYOUT_TILED
  // MXFP4 output (large-tile kernel only; n % 32 == 0, n % 128 == 0 when
  // q_tiled): Y requantized per 32-block along N into q_codes / q_scales
  // (y unused)
  bool q_out = false;
  bool q_tiled = false;     // output in MXFP4_LAYOUT_TILED
  uint8_t* q_codes = nullptr;
  uint8_t* q_scales = nullptr;
};

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s);

// Compute units of the current device (cached per device; 256 if the query
// fails).
int cu_count();

// Large-tile persistent kernel (gemm_large.hip): K a multiple of 128,
// 4-byte aligned scale pointers, operand code bytes below 4 GiB; the only
// kernel for tiled operands.
bool gemm_large_supported(const GemmArgs& a);
hipError_t launch_gemm_large(const GemmArgs& a, hipStream_t s);

// Small-M kernel (gemm_small.hip): either layout; the kernel for decode
// shapes (m <= 64), bound by streaming the weights from HBM, and for shapes
// with fewer than 8 output tiles of 256 x 256 (gemm_small_route).
bool gemm_small_route(int64_t m, int64_t n);
bool gemm_small_supported(const GemmArgs& a);
hipError_t launch_gemm_small(const GemmArgs& a, hipStream_t s);

// Fused small-M linear layer (gemm_small.hip): the activations are rotated
// and quantized inside the GEMM kernel, in the same launch (1 <= m <= 64; W
// in either layout, described by g.b_* / g.tiled; g.a_* unused).
struct LinearArgs {
  const void* x;       // [m][ld_x] fp32 or bf16
  int64_t ld_x;        // elements
  bool x_bf16;
  int32_t rot;         // mxfp4_rot_kind
  int32_t p, q;
  const float* fa;
  const float* fb;
  GemmArgs g;
  // workspace: handoff counters (zero between calls) and the quantized
  // activations in MFMA operand order
  uint32_t* counters = nullptr;
  uint8_t* xq = nullptr;
};
bool linear_small_supported(const LinearArgs& a);
hipError_t launch_linear_small(const LinearArgs& a, hipStream_t s);
// Workspace of the fused layer: a fixed region of counters (the same for
// every shape, so one workspace serves calls of any shape), then the
// quantized activations, 1152 bytes per 16 rows and 128 K elements.
constexpr int64_t kLinearCounterBytes = 4096;
int64_t linear_small_workspace_bytes(int64_t m, int64_t k);
// The fixed scratch of the allocation-free variant: its device address on
// the current device (looked up, and its counters cleared on `s`, on the
// first call per device).
constexpr int64_t kLinearStaticScratchBytes = int64_t(4) << 20;
hipError_t linear_small_static_scratch(void** ptr, hipStream_t s);

}  // namespace mxfp4
